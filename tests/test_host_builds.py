"""Host-only builds against the C ABI (no GPU needed):

* tests/host/abi_from_c.c is compiled as C99 (-pedantic -Werror) against include/fa.h,
  linked with the built libfa_mi355x.so, and run: the header compiles as C and every
  entry point rejects invalid arguments (including grids past the runtime's 32-bit
  work-item count) with the documented code before any HIP call;
* tests/host/plan_checks.cpp is compiled together with the library's validation and
  launch planning (csrc/fa_validate.cpp) under AddressSanitizer and
  UndefinedBehaviorSanitizer and run: derived launch parameters, both sides of every
  grid limit, and a sweep of edge values through every planner.
"""

import os
import shutil
import subprocess

import pytest

import exact_attention_56_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST = os.path.join(ROOT, "tests", "host")
INCLUDE = os.path.join(ROOT, "include")
CSRC = os.path.join(ROOT, "exact_attention_56_amd", "csrc")
ROCM_INCLUDE = "/opt/rocm/include"


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=300, **kw)
    assert res.returncode == 0, f"{' '.join(cmd)}\nstdout:\n{res.stdout}\nstderr:\n{res.stderr}"
    return res.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no host C compiler")
def test_header_compiles_as_c_and_library_rejects_invalid_calls(tmp_path):
    if not os.path.exists(fa.LIB_PATH):
        pytest.fail("libfa_mi355x.so is not built (run __graft_entry__.build())")
    exe = str(tmp_path / "abi_from_c")
    libdir = os.path.dirname(fa.LIB_PATH)
    _run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-D__HIP_PLATFORM_AMD__",
          "-isystem", ROCM_INCLUDE, f"-I{INCLUDE}", os.path.join(HOST, "abi_from_c.c"), f"-L{libdir}", "-lfa_mi355x",
          f"-Wl,-rpath,{libdir}", "-Wl,-rpath,/opt/rocm/lib", "-lm", "-o", exe])
    out = _run([exe])
    assert out.startswith("ok ")


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_validation_under_address_and_ub_sanitizers(tmp_path):
    exe = str(tmp_path / "plan_checks")
    _run(["g++", "-std=c++17", "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__", "-isystem", ROCM_INCLUDE,
          f"-I{INCLUDE}", f"-I{CSRC}", os.path.join(CSRC, "fa_validate.cpp"), os.path.join(HOST, "plan_checks.cpp"),
          "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    out = _run([exe], env=env)
    assert out.startswith("ok ")
