#!/usr/bin/env python3
"""Benchmark of the attention forward on one MI355X.

Metric: attention forward TFLOP/s (bf16 inputs, fp32 accumulation) on the pages'
benchmark shape (hidden 2048 = 16 heads x headdim 128, seqlen 2048,
batch 16384 / seqlen = 8), as a fraction of the dense bf16 MFMA peak.

One step = fa_fwd non-causal + fa_fwd causal over one batch of seeded synthetic
Q/K/V already resident in HBM.  FLOPs are algorithmic: 4 * headdim per visible
(query, key) pair (Q K^T and P V); masked pairs the method skips are not counted.

Printed: ONE JSON line with the contract fields plus
  roofline      the forward kernel: algorithmic FLOPs per launch / mean launch time
                (HIP events on the launch stream), against the bf16 MFMA peak;
  cpu_baseline  the fp64 oracle on the host cores, on a bounded sample of the workload;
  extra         the seqlen sweep of the pages' recipe (non-causal, 4k/8k/16k), the
                long causal local ALiBi workload and the headdim-256 16k workload, the
                split-KV decode workload in HBM GB/s, a packed batch of causal
                sequences of mixed lengths with grouped K/V heads (fa_fwd_varlen), the
                backward (fa_bwd) on the benchmark shape and (fa_bwd_varlen) on the packed
                grouped-head batch, paged-KV-cache decode steps (fa_fwd_kvcache; 4 and
                1 K/V heads), and the benchmark shape with fp16 tensors.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import exact_attention_56_amd as fa  # noqa: E402
from exact_attention_56_amd.inputs import (VARLEN_GQA, WORKLOADS, Workload, make_alibi_slopes,  # noqa: E402
                                           make_qkv, make_varlen_qkv, sweep_workload)

METRIC = "attention fwd TFLOPS (bf16, 1 MI355X) at hd128 seqlen 2k-16k; % of MFMA peak"
# MI355X published dense peaks: 256 CUs x 2.4 GHz x 4096 bf16 flop/clk/CU, and HBM3E 8 TB/s.
PEAK_BF16_TFLOPS = 2516.6
PEAK_HBM_GBS = 8000.0


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "fa_fwd_hd128_bench_s2048_hbm_traffic.txt")
KERNEL_SOURCES = ["exact_attention_56_amd/csrc/fa_common.h", "exact_attention_56_amd/csrc/fa_fwd_kernel.h",
                  "exact_attention_56_amd/csrc/fa_fwd_d128.hip"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary,
    or None when that summary was taken on different kernel sources."""
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    t = re.search(r"traffic_bytes_per_launch:\s*(\d+)", text)
    hsh = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", text)
    if not t or not hsh or hsh.group(1) != kernel_source_hash():
        return None
    return int(t.group(1))


def fwd_waves(headdim: int, seqlen_q: int, causal: bool) -> int:
    """Waves per workgroup of the forward launch (the library's launch rule for a plain
    forward without a window: eight at headdim 128 from 2048 query rows unmasked and from
    8192 causal, else four)."""
    if headdim != 128:
        return 4
    return 8 if seqlen_q >= (8192 if causal else 2048) else 4


def visible_pairs(w: Workload) -> int:
    """(query, key) pairs the mask keeps, per (batch, head): bottom-right aligned
    position c = i + Sk - Sq, window [c - left, c + right] (right = 0 if causal)."""
    wr = 0 if w.causal else w.window_right
    total = 0
    for i in range(w.seqlen_q):
        c = i + w.seqlen_k - w.seqlen_q
        lo = 0 if w.window_left < 0 else max(0, c - w.window_left)
        hi = w.seqlen_k - 1 if wr < 0 else min(w.seqlen_k - 1, c + wr)
        total += max(0, hi - lo + 1)
    return total


def algorithmic_flops(w: Workload) -> float:
    return 4.0 * w.headdim * visible_pairs(w) * w.batch * w.nheads


def convention_flops(w: Workload) -> float:
    f = 4.0 * w.batch * w.nheads * w.seqlen_q * w.seqlen_k * w.headdim
    return f / 2 if w.causal else f


class FwdCase:
    """Device-resident inputs and outputs for repeated fa_fwd launches."""

    def __init__(self, w: Workload, q, k, v, slopes=None):
        self.w, self.q, self.k, self.v, self.slopes = w, q, k, v, slopes
        self.out = torch.empty_like(q)
        self.lse = torch.empty(w.batch, w.nheads, w.seqlen_q, dtype=torch.float32, device=q.device)
        self.flops = algorithmic_flops(w)

    def launch(self):
        fa.fwd(self.q, self.k, self.v, self.out, self.lse, self.w.softmax_scale, self.w.causal,
               (self.w.window_left, self.w.window_right), self.slopes)


def warm_up(fn, launches: int, min_seconds: float = 0.3) -> float:
    """Untimed launches of fn(): at least `launches`, and more until `min_seconds` of
    wall time have passed; returns the seconds spent.  A fixed handful of launches
    measured 10-20% slow while the clock ramps, and each extra workload draws fresh
    tensors whose first launches ran slow even on a warm GPU, so every workload (the
    headline step included) gets about the same settling time whatever its length."""
    t0 = time.perf_counter()
    for _ in range(launches):
        fn()
    torch.cuda.synchronize()
    while time.perf_counter() - t0 < min_seconds:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()
    return time.perf_counter() - t0


def time_events(fn, reps: int):
    """Mean and min duration (ms) of fn() over reps, HIP events on the current stream."""
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    ts = [a.elapsed_time(b) for a, b in evs]
    return sum(ts) / len(ts), min(ts)


CPU_WORKERS_MAX = 16  # the host-CPU share of one GPU on the measurement boxes


def _cpu_worker_init():
    """Each oracle worker runs single-threaded: the pool, not BLAS, spreads the work."""
    os.environ["OMP_NUM_THREADS"] = "1"
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except Exception:  # pragma: no cover - threadpoolctl missing: BLAS keeps its default
        pass


def _oracle_slice(task):
    """One (batch, head) slice of a workload through the fp64 oracle."""
    import oracle
    q, k, v, scale, causal, wl, wr = task
    oracle.attention_forward(q, k, v, scale, causal, wl, wr)
    return True


def start_cpu_pool():
    """Worker processes for cpu_baseline, forked before this process touches the GPU
    (the children inherit no GPU state).  Returns (pool, workers)."""
    import multiprocessing
    n = max(1, min(CPU_WORKERS_MAX, os.cpu_count() or 1))
    return multiprocessing.get_context("fork").Pool(n, initializer=_cpu_worker_init), n


def cpu_baseline(cases, budget_s: float, pool, workers: int):
    """The fp64 oracle, as it stands, on the host cores: whole (batch, head) slices of
    the workload, one per single-threaded worker process at a time, until every slice
    is done or `budget_s` has passed (slices already started are finished and counted)."""
    from collections import deque

    import oracle
    tasks = []
    n_pairs = cases[0].w.batch * cases[0].w.nheads
    for n in range(n_pairs):
        for case in cases:
            w = case.w
            b, h = n % w.batch, (n // w.batch) % w.nheads
            tasks.append((case, b, h))
    pending = deque()
    done_flops, done = 0.0, 0
    t0 = time.perf_counter()
    it = iter(tasks)
    while True:
        while len(pending) < 2 * workers and time.perf_counter() - t0 < budget_s:
            nxt = next(it, None)
            if nxt is None:
                break
            case, b, h = nxt
            w = case.w
            arg = (oracle.as_f64(case.q_cpu[b:b + 1, :, h:h + 1]), oracle.as_f64(case.k_cpu[b:b + 1, :, h:h + 1]),
                   oracle.as_f64(case.v_cpu[b:b + 1, :, h:h + 1]), w.softmax_scale, w.causal, w.window_left,
                   w.window_right)
            pending.append((pool.apply_async(_oracle_slice, (arg,)), case.flops / (w.batch * w.nheads)))
        if not pending:
            break
        res, fl = pending.popleft()
        res.get()
        done_flops += fl
        done += 1
    dt = time.perf_counter() - t0
    names = ", ".join(c.w.name for c in cases)
    return {"value": done_flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(workers), "kind": "oracle",
            "sample": f"{done} of the {len(tasks)} (batch, head) slices of {names} (full seqlen rows, fp64 NumPy), "
                      f"{dt:.1f} s on {workers} single-threaded worker processes; host has {os.cpu_count()} "
                      f"logical CPUs" + (f" ({cpu_model()})" if cpu_model() else "")}


def cpu_model() -> str:
    """The host CPU's model name (first 'model name' line of /proc/cpuinfo), or ''."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def sweep(dev, reps: int, warmup: int):
    res = {}
    for s in (4096, 8192, 16384):
        w = sweep_workload(s)
        q, k, v = make_qkv(w.batch, w.seqlen_q, w.seqlen_k, w.nheads, w.headdim, w.seed, device=dev)
        case = FwdCase(w, q, k, v)
        warm_up(case.launch, warmup)
        mean_ms, min_ms = time_events(case.launch, reps)
        tf = case.flops / (mean_ms * 1e-3) / 1e12
        res[w.name] = {"tflops": round(tf, 1), "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                       "mean_ms": round(mean_ms, 4), "min_ms": round(min_ms, 4),
                       "shape": [w.batch, w.nheads, w.seqlen_q, w.seqlen_k, w.headdim]}
        del q, k, v, case
    return res


def configs_bench(dev, reps: int, warmup: int):
    """The long causal local workload (headdim 64, window (1024, 0), ALiBi) and the
    headdim-256 16k workload.  TFLOP/s on the algorithmic count (visible pairs only)
    and, beside it, on the 4*B*H*Sq*Sk*d (halved when causal) convention."""
    res = {}
    for name in ("local_alibi_s8192", "hd256_s16384"):
        w = WORKLOADS[name]
        q, k, v = make_qkv(w.batch, w.seqlen_q, w.seqlen_k, w.nheads, w.headdim, w.seed, device=dev)
        slopes = make_alibi_slopes(w.nheads).to(dev) if w.alibi else None
        case = FwdCase(w, q, k, v, slopes)
        warm_up(case.launch, warmup)
        mean_ms, min_ms = time_events(case.launch, reps)
        tf = case.flops / (mean_ms * 1e-3) / 1e12
        res[name] = {"tflops": round(tf, 1), "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                     "convention_tflops": round(convention_flops(w) / (mean_ms * 1e-3) / 1e12, 1),
                     "mean_ms": round(mean_ms, 4), "min_ms": round(min_ms, 4),
                     "algorithmic_gflop": round(case.flops / 1e9, 2),
                     "shape": [w.batch, w.nheads, w.seqlen_q, w.seqlen_k, w.headdim]}
        del q, k, v, case
    return res


def decode_bench(dev, reps: int, warmup: int):
    w = WORKLOADS["decode_s32768"]
    q, k, v = make_qkv(w.batch, w.seqlen_q, w.seqlen_k, w.nheads, w.headdim, w.seed, device=dev)
    ns = w.num_splits
    op = torch.empty(ns, w.batch, w.nheads, w.seqlen_q, w.headdim, dtype=torch.float32, device=dev)
    lp = torch.empty(ns, w.batch, w.nheads, w.seqlen_q, dtype=torch.float32, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty(w.batch, w.nheads, w.seqlen_q, dtype=torch.float32, device=dev)

    def partial():
        fa.fwd_splitkv(q, k, v, op, lp, ns, w.softmax_scale, w.causal, (w.window_left, w.window_right))

    def both():
        partial()
        fa.combine(op, lp, out, lse)

    warm_up(both, warmup)
    p_mean, p_min = time_events(partial, reps)
    b_mean, _ = time_events(both, reps)
    kv_bytes = 2 * k.numel() * 2
    partial_bytes = kv_bytes + q.numel() * 2 + op.numel() * 4 + lp.numel() * 4
    pair_bytes = partial_bytes + op.numel() * 4 + lp.numel() * 4 + out.numel() * 2 + lse.numel() * 4
    return {"workload": "decode_s32768 (batch 8, 16 heads x 128, seqlen_q 1, seqlen_k 32768, causal, 16 splits)",
            "splitkv_gbs": round(partial_bytes / (p_mean * 1e-3) / 1e9, 1),
            "splitkv_frac_hbm_peak": round(partial_bytes / (p_mean * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "splitkv_mean_us": round(p_mean * 1e3, 2), "splitkv_min_us": round(p_min * 1e3, 2),
            "pair_mean_us": round(b_mean * 1e3, 2),
            "pair_gbs": round(pair_bytes / (b_mean * 1e-3) / 1e9, 1),
            "bytes_per_splitkv_launch": partial_bytes}


def varlen_bench(dev, reps: int, warmup: int):
    w = VARLEN_GQA
    q, k, v, cu = make_varlen_qkv(w, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty(w.nheads, q.shape[0], dtype=torch.float32, device=dev)
    mx = max(w.lengths)

    def launch():
        fa.fwd_varlen(q, k, v, out, lse, cu, cu, mx, mx, w.softmax_scale, w.causal)

    warm_up(launch, warmup)
    mean_ms, min_ms = time_events(launch, reps)
    # causal square sequences: S (S + 1) / 2 visible pairs, 4 * headdim flop per pair and head
    flops = sum(s * (s + 1) // 2 for s in w.lengths) * w.nheads * 4 * w.headdim
    tf = flops / (mean_ms * 1e-3) / 1e12
    return {"workload": f"{w.name}: {len(w.lengths)} sequences ({sum(w.lengths)} tokens, lengths "
                        f"{min(w.lengths)}..{mx}), {w.nheads} query heads over {w.nheads_k} K/V heads x "
                        f"{w.headdim}, causal",
            "tflops": round(tf, 1), "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "mean_ms": round(mean_ms, 4), "min_ms": round(min_ms, 4), "algorithmic_gflop": round(flops / 1e9, 2)}


def fp16_bench(dev, reps: int, warmup: int):
    """The benchmark shape (non-causal and causal) with fp16 q/k/v/out: the same kernels
    with the fp16 matrix-core instruction, against the same dense peak."""
    res = {}
    for name in ("bench_s2048", "bench_s2048_causal"):
        w = WORKLOADS[name]
        q, k, v = make_qkv(w.batch, w.seqlen_q, w.seqlen_k, w.nheads, w.headdim, w.seed, device=dev,
                           dtype=torch.float16)
        case = FwdCase(w, q, k, v)
        warm_up(case.launch, warmup)
        mean_ms, min_ms = time_events(case.launch, reps)
        tf = case.flops / (mean_ms * 1e-3) / 1e12
        res[name] = {"tflops": round(tf, 1), "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                     "mean_ms": round(mean_ms, 4), "min_ms": round(min_ms, 4)}
    return res


def kvcache_bench(dev, reps: int, warmup: int, hk: int = 4):
    """fa_fwd_kvcache on the decode workload's sizes with a paged cache: batch 8, 16 query
    heads over 4 K/V heads x 128 (hk), 32767 cached keys + 1 appended (rotary on q and the
    new key), 256-row blocks in shuffled order, automatic split count.  HBM bytes: the K/V
    rows read plus q, the appended row, partials and outputs."""
    w = WORKLOADS["decode_s32768"]
    b, h, d, page = w.batch, w.nheads, w.headdim, 256
    cached = w.seqlen_k - 1
    blocks = w.seqlen_k // page
    g = torch.Generator(device=dev).manual_seed(9)
    mk = lambda *shape: torch.randn(*shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    kc, vc = mk(b * blocks, page, hk, d), mk(b * blocks, page, hk, d)
    table = torch.randperm(b * blocks, generator=g, device=dev).to(torch.int32).view(b, blocks).contiguous()
    lens = torch.full((b,), cached, dtype=torch.int32, device=dev)
    q, knew, vnew = mk(b, 1, h, d), mk(b, 1, hk, d), mk(b, 1, hk, d)
    theta = torch.rand(w.seqlen_k + 8, d // 2, generator=g, device=dev) * 6.2831853
    cos, sin = torch.cos(theta), torch.sin(theta)
    out = torch.empty_like(q)
    lse = torch.empty(b, h, 1, dtype=torch.float32, device=dev)
    op = torch.empty(64, b, h, 1, d, dtype=torch.float32, device=dev)
    lp = torch.empty(64, b, h, 1, dtype=torch.float32, device=dev)

    def launch():
        fa.fwd_kvcache(q, kc, vc, lens, out, lse, op, lp, table, knew, vnew, cos, sin, w.softmax_scale, True)

    warm_up(launch, warmup)
    mean_ms, min_ms = time_events(launch, reps)
    nbytes = 2 * b * w.seqlen_k * hk * d * 2 + q.numel() * 2 * 2 + 2 * knew.numel() * 2 + out.numel() * 2
    return {"workload": f"paged KV cache: batch {b}, {h} query heads over {hk} K/V heads x {d}, {cached} cached + 1 "
                        f"appended key, {page}-row blocks, rotary, causal, automatic splits",
            "gbs": round(nbytes / (mean_ms * 1e-3) / 1e9, 1),
            "frac_hbm_peak": round(nbytes / (mean_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "mean_us": round(mean_ms * 1e3, 2), "min_us": round(min_ms * 1e3, 2), "bytes": nbytes}


def backward_bench(dev, reps: int, warmup: int):
    """fa_bwd on the benchmark shape, non-causal and causal, and on the headdim-256 16k
    workload.  Algorithmic FLOPs: the five products of the backward (S, dP, dV, dQ, dK)
    are 10 * headdim per visible pair, 2.5x the forward's count."""
    res = {}
    for name in ("bench_s2048", "bench_s2048_causal", "hd256_s16384"):
        w = WORKLOADS[name]
        q, k, v = make_qkv(w.batch, w.seqlen_q, w.seqlen_k, w.nheads, w.headdim, w.seed, device=dev)
        dout = torch.randn_like(q)
        out, lse = fa.flash_attn_func(q, k, v, w.softmax_scale, w.causal)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        delta = torch.empty(w.batch, w.nheads, w.seqlen_q, dtype=torch.float32, device=dev)

        def launch():
            fa.bwd(q, k, v, out, lse, dout, dq, dk, dv, delta, w.softmax_scale, w.causal)

        warm_up(launch, warmup)
        mean_ms, min_ms = time_events(launch, reps)
        flops = 2.5 * algorithmic_flops(w)
        tf = flops / (mean_ms * 1e-3) / 1e12
        res[name] = {"tflops": round(tf, 1), "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                     "mean_ms": round(mean_ms, 4), "min_ms": round(min_ms, 4),
                     "algorithmic_gflop": round(flops / 1e9, 2)}
        del q, k, v, dout, out, lse, dq, dk, dv, delta
    return res


def backward_varlen_bench(dev, reps: int, warmup: int):
    """fa_bwd_varlen on the packed grouped-head workload (the causal sequences of
    varlen_gqa, 32 query heads over 8 K/V heads x 128).  Algorithmic FLOPs: 10 * headdim
    per visible pair and query head (2.5x the forward's)."""
    w = VARLEN_GQA
    q, k, v, cu = make_varlen_qkv(w, device=dev)
    mx = max(w.lengths)
    out, lse = fa.flash_attn_varlen_func(q, k, v, cu, cu, mx, mx, w.softmax_scale, w.causal)
    dout = torch.randn_like(q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty(w.nheads, q.shape[0], dtype=torch.float32, device=dev)

    def launch():
        fa.bwd_varlen(q, k, v, out, lse, dout, dq, dk, dv, delta, cu, cu, mx, mx, w.softmax_scale, w.causal)

    warm_up(launch, warmup)
    mean_ms, min_ms = time_events(launch, reps)
    flops = 2.5 * sum(s * (s + 1) // 2 for s in w.lengths) * w.nheads * 4 * w.headdim
    tf = flops / (mean_ms * 1e-3) / 1e12
    return {"workload": f"{w.name} backward: {len(w.lengths)} sequences ({sum(w.lengths)} tokens), {w.nheads} query "
                        f"heads over {w.nheads_k} K/V heads x {w.headdim}, causal",
            "tflops": round(tf, 1), "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "mean_ms": round(mean_ms, 4), "min_ms": round(min_ms, 4), "algorithmic_gflop": round(flops / 1e9, 2)}


# extra workloads: name -> (function, timed repetitions, warm-up launches)
EXTRAS = {"sweep_noncausal": (sweep, 20, 10),
          "configs": (configs_bench, 10, 3),
          "decode": (decode_bench, 20, 3),
          "varlen_gqa": (varlen_bench, 10, 3),
          "backward": (backward_bench, 10, 5),
          "backward_varlen_gqa": (backward_varlen_bench, 10, 3),
          "kvcache_paged": (kvcache_bench, 20, 5),
          "kvcache_paged_mqa": (lambda dev, reps, warmup: kvcache_bench(dev, reps, warmup, hk=1), 20, 5),
          "fp16_fwd": (fp16_bench, 20, 10)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20, help="untimed steps first (at least)")
    ap.add_argument("--warmup-seconds", type=float, default=0.5,
                    help="and untimed steps until this much wall time has passed (the clock settles)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip every extra workload")
    ap.add_argument("--extra", default=",".join(EXTRAS),
                    help="comma-separated extra workloads to run (default: all of " + ", ".join(EXTRAS) + ")")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    unknown = [n for n in args.extra.split(",") if n not in EXTRAS]
    if unknown:
        ap.error(f"unknown extra workload(s) {unknown}; choose from {list(EXTRAS)}")

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this library has no multi-GPU path "
              "(each GPU would run fa_fwd on its own batch/head share).", file=sys.stderr)
        sys.exit(2)
    # the oracle's worker processes are forked before anything touches the GPU
    pool, workers = (None, 0) if args.no_cpu_baseline else start_cpu_pool()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    fa.load_library()

    base = WORKLOADS["bench_s2048"]
    causal = WORKLOADS["bench_s2048_causal"]
    q_cpu, k_cpu, v_cpu = make_qkv(base.batch, base.seqlen_q, base.seqlen_k, base.nheads, base.headdim, base.seed)
    q, k, v = q_cpu.to(dev), k_cpu.to(dev), v_cpu.to(dev)
    cases = [FwdCase(base, q, k, v), FwdCase(causal, q, k, v)]
    for c in cases:
        c.q_cpu, c.k_cpu, c.v_cpu = q_cpu, k_cpu, v_cpu

    def step():
        for c in cases:
            c.launch()

    warm_s = warm_up(step, args.warmup, args.warmup_seconds)

    # timed region: exactly K steps, wall clock bracketed by synchronisation, with
    # HIP events around every forward launch on the launch stream
    stream = torch.cuda.current_stream()
    evs = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for c in cases:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            c.launch()
            b.record(stream)
            evs.append((c, a, b))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    step_flops = sum(c.flops for c in cases)
    ms_per_step = wall * 1e3 / args.steps
    value = step_flops * args.steps / wall / 1e12
    launch_ms = [a.elapsed_time(b) for _, a, b in evs]
    launch_flops = [c.flops for c, _, _ in evs]
    achieved = sum(launch_flops) / (sum(launch_ms) * 1e-3) / 1e12
    per_case = {}
    for c in cases:
        ts = [a.elapsed_time(b) for cc, a, b in evs if cc is c]
        m = sum(ts) / len(ts)
        per_case[c.w.name] = {"mean_ms": round(m, 4), "median_ms": round(sorted(ts)[len(ts) // 2], 4),
                              "min_ms": round(min(ts), 4),
                              "tflops": round(c.flops / (m * 1e-3) / 1e12, 1),
                              "algorithmic_gflop": round(c.flops / 1e9, 2),
                              "convention_gflop": round(convention_flops(c.w) / 1e9, 2)}

    kernels = " and ".join(f"fa::fwd_kernel<{c.w.headdim},{fwd_waves(c.w.headdim, c.w.seqlen_q, c.w.causal)},"
                           f"false,false,__bf16,false> ({c.w.name})" for c in cases)
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_s": round(warm_s, 3),
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded iid N(0,1) Q/K/V rounded to bf16)",
        "config": {"workload": "bench_s2048: batch 8, 16 heads x headdim 128, seqlen_q = seqlen_k = 2048, "
                               "one non-causal + one causal fa_fwd per step",
                   "global_batch": base.batch, "seq_len": base.seqlen_q, "nheads": base.nheads,
                   "headdim": base.headdim, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(),
                     "kernel": kernels, "per_launch": per_case},
    }
    if not args.no_extra:
        result["extra"] = {}
        for name in args.extra.split(","):
            fn, reps, warmup = EXTRAS[name]
            result["extra"][name] = fn(dev, reps=reps, warmup=warmup)
    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = src.numel()
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cases, args.cpu_budget, pool, workers)
        pool.close()
        pool.join()
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
