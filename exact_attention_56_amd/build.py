"""Build libfa_mi355x.so (gfx950) in-tree with hipcc.

Usage: ``python -m exact_attention_56_amd.build`` or ``build()`` from Python.
Every translation unit is compiled for gfx950 only, with packed-FP32 code
generation disabled, then linked into one shared library next to this file.
"""

from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libfa_mi355x.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
# (source, extra flags).  headdim 64/128 keep S and O in arch VGPRs (MFMA VGPR form):
# the softmax reads S with plain VALU ops and the kernel fits two waves per SIMD.
# headdim 256 needs the accumulation registers, so it keeps the compiler's choice.
VGPR_FORM = ["-mllvm", "--amdgpu-mfma-vgpr-form"]
SOURCES = [
    ("fa_fwd_d64.hip", VGPR_FORM),
    ("fa_fwd_d128.hip", VGPR_FORM),
    ("fa_fwd_d256.hip", []),
    ("fa_fwd_launch.hip", []),
    # backward: the dQ pass keeps its accumulators in arch VGPRs (two waves per SIMD);
    # the dK/dV pass is left to the compiler's choice: accumulation registers at headdim 256
    # (one wave per SIMD), arch VGPRs at 128 (two waves per SIMD, V in LDS)
    ("fa_bwd_dq.hip", VGPR_FORM),
    ("fa_bwd.hip", []),
    ("fa_decode_kernel.hip", []),
    ("fa_api.hip", []),
    ("fa_noalloc.hip", []),
]
# host-only C++ (argument validation and launch planning): compiled by the host compiler
HOST_SOURCES = ["fa_validate.cpp"]
CXX = os.environ.get("CXX", "g++")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
OFFLOAD_ARCH = "gfx950"

COMMON_FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={OFFLOAD_ARCH}", "-fPIC",
    # no packed-FP32 (v_pk_*_f32) code generation
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


# host compiler flags: the ROCm headers (fa.h names hipStream_t) in their AMD form
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
              f"-I{INCLUDE}", f"-I{CSRC}"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature name; that warning is noise
    noise = "'-packed-fp32-ops' is not a recognized feature"
    out = "\n".join(l for l in res.stdout.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link the shared library; returns its path."""
    obj_dir = os.path.join(ROOT, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    objs = []
    jobs = []
    for src, extra in SOURCES:
        obj = os.path.join(obj_dir, src.replace(".hip", ".o"))
        objs.append(obj)
        jobs.append([HIPCC, *COMMON_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj])
    for src in HOST_SOURCES:
        obj = os.path.join(obj_dir, src.replace(".cpp", ".o"))
        objs.append(obj)
        jobs.append([CXX, *HOST_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    tmp = LIB_PATH + ".tmp"
    _run([HIPCC, f"--offload-arch={OFFLOAD_ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
