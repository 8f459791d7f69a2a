"""Host-side checks of bench.py's accounting (no GPU needed)."""

import subprocess
import sys

import pytest

import bench
from exact_attention_56_amd.inputs import WORKLOADS, sweep_workload


@pytest.mark.parametrize("name,gflop", [
    ("tiny", 0.008388608), ("bench_s2048", 274.877906944), ("bench_s2048_causal", 137.506062336),
    ("local_alibi_s8192", 128.974848), ("hd256_s16384", 2199.023255552), ("decode_s32768", 2.147483648),
])
def test_algorithmic_flops(name, gflop):
    # 4 * headdim flops per visible (query, key) pair, closed forms:
    #  non-causal: Sq*Sk pairs; causal square: S(S+1)/2; window (1024,0) causal square:
    #  sum_i min(i,1024)+1; decode causal Sq=1: every key.
    assert bench.algorithmic_flops(WORKLOADS[name]) / 1e9 == pytest.approx(gflop, rel=1e-12)


def test_visible_pairs_closed_forms():
    w = WORKLOADS["bench_s2048_causal"]
    assert bench.visible_pairs(w) == 2048 * 2049 // 2
    w = WORKLOADS["local_alibi_s8192"]
    assert bench.visible_pairs(w) == sum(min(i, 1024) + 1 for i in range(8192))
    assert bench.visible_pairs(WORKLOADS["decode_s32768"]) == 32768


def test_sweep_recipe():
    for s in (2048, 4096, 8192, 16384):
        w = sweep_workload(s)
        assert w.batch * w.seqlen_q == 16384 and w.nheads * w.headdim == 2048
        assert bench.algorithmic_flops(w) == 4.0 * 128 * 16 * 16384 * s


def test_multi_gpu_refused():
    res = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], capture_output=True, text=True,
                         cwd=bench.ROOT, timeout=300)
    assert res.returncode == 2 and "one GPU" in res.stderr


def test_cpu_baseline_pool_reports_its_workers():
    """cpu_baseline runs whole (batch, head) slices on single-threaded worker processes
    and reports how many it used; on a tiny workload every slice finishes."""
    from exact_attention_56_amd.inputs import make_qkv

    class Case:
        pass

    w = WORKLOADS["tiny"]
    q, k, v = make_qkv(w.batch, w.seqlen_q, w.seqlen_k, w.nheads, w.headdim, w.seed)
    c = Case()
    c.w, c.flops, c.q_cpu, c.k_cpu, c.v_cpu = w, bench.algorithmic_flops(w), q, k, v
    import multiprocessing
    pool = multiprocessing.get_context("fork").Pool(2, initializer=bench._cpu_worker_init)
    try:
        res = bench.cpu_baseline([c], 30.0, pool, 2)
    finally:
        pool.close()
        pool.join()
    assert res["cores"] == 2 and res["kind"] == "oracle" and res["value"] > 0
    assert res["sample"].startswith(f"{w.batch * w.nheads} of the {w.batch * w.nheads} ")
    assert "2 single-threaded worker processes" in res["sample"]
