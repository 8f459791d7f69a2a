"""GPU parity at the full workload sizes, in the launch configuration the benchmark times.

The oracle cannot evaluate these problems whole, so it evaluates sampled output
rows one by one (first and last rows, query-tile and key-tile boundaries, and
seeded random rows); every output is also checked for properties that hold at
any size (all written, all finite, lse bounded below by the row max and above by
row max + ln |visible keys| is left to the sampled rows).
"""

import sys

import numpy as np
import pytest
import torch

import exact_attention_56_amd as fa
import oracle
from exact_attention_56_amd.inputs import WORKLOADS, workload_inputs
from tests.parity import check_lse, check_out

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
DEV = "cuda"
NSAMPLES = 48


def sample_rows(w, seed):
    rng = np.random.default_rng(seed)
    fixed_i = sorted({0, 1, 63, 64, 127, 128, 129, w.seqlen_q // 2, w.seqlen_q - 129, w.seqlen_q - 128,
                      w.seqlen_q - 2, w.seqlen_q - 1})
    fixed_i = [i for i in fixed_i if 0 <= i < w.seqlen_q]
    samples = set()
    for n, i in enumerate(fixed_i):
        samples.add((n % w.batch, (3 * n) % w.nheads, i))
    samples.add((w.batch - 1, w.nheads - 1, w.seqlen_q - 1))
    while len(samples) < NSAMPLES:
        samples.add((int(rng.integers(w.batch)), int(rng.integers(w.nheads)), int(rng.integers(w.seqlen_q))))
    return sorted(samples)


@pytest.mark.parametrize("name", [n for n in WORKLOADS])
def test_full_size_sampled(name):
    w = WORKLOADS[name]
    print(f"[case] full size {name}: {w}", file=sys.stderr, flush=True)
    q, k, v, slopes = workload_inputs(w)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    sd = None if slopes is None else slopes.to(DEV)
    scale = w.softmax_scale
    window = (w.window_left, w.window_right)
    if w.num_splits:
        out, lse = fa.decode(qd, kd, vd, w.num_splits, scale, w.causal, window, sd)
    else:
        out = torch.full_like(qd, float("nan"))
        lse = torch.full((w.batch, w.nheads, w.seqlen_q), float("nan"), device=DEV)
        fa.fwd(qd, kd, vd, out, lse, scale, w.causal, window, sd)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()), "non-finite or unwritten output"
    assert bool(torch.isfinite(lse).all()), "non-finite or unwritten lse (no row of these workloads is empty)"
    del qd, kd, vd

    samples = sample_rows(w, seed=w.seed)
    ref_out, ref_lse = oracle.attention_sampled(q, k, v, samples, scale, w.causal, w.window_left,
                                                w.window_right, slopes)
    idx_b = torch.tensor([s[0] for s in samples])
    idx_h = torch.tensor([s[1] for s in samples])
    idx_i = torch.tensor([s[2] for s in samples])
    out_c, lse_c = out.cpu(), lse.cpu()
    got_out = out_c[idx_b, idx_i, idx_h, :]
    got_lse = lse_c[idx_b, idx_h, idx_i]
    check_lse(got_lse, ref_lse)
    check_out(got_out, ref_out)


@pytest.mark.parametrize("name", ["bench_s2048", "bench_s2048_causal", "local_alibi_s8192"])
def test_full_size_backward_heads(name):
    """fa_bwd at the full workload size; two whole (batch, head) slices are compared with
    the exact oracle gradient of that head alone (heads are independent problems)."""
    from tests.test_gpu_backward import GRAD_REL
    w = WORKLOADS[name]
    print(f"[case] full-size backward {name}: {w}", file=sys.stderr, flush=True)
    q, k, v, slopes = workload_inputs(w)
    dout = torch.randn(q.shape, generator=torch.Generator().manual_seed(w.seed + 100)).to(torch.bfloat16)
    qd, kd, vd, gd = q.to(DEV), k.to(DEV), v.to(DEV), dout.to(DEV)
    sd = None if slopes is None else slopes.to(DEV)
    window = (w.window_left, w.window_right)
    out, lse = fa.flash_attn_func(qd, kd, vd, w.softmax_scale, w.causal, window, sd)
    dq, dk, dv = fa.attention_backward(qd, kd, vd, out, lse, gd, w.softmax_scale, w.causal, window, sd)
    torch.cuda.synchronize()
    for t, nm in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        assert bool(torch.isfinite(t).all()), f"{nm}: non-finite or unwritten values"
    for b, h in [(0, 0), (w.batch - 1, w.nheads - 1)]:
        sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
        hs = None if slopes is None else slopes[h:h + 1]
        rq, rk, rv = oracle.attention_backward(q[sl], k[sl], v[sl], dout[sl], w.softmax_scale, w.causal,
                                               w.window_left, w.window_right, hs)
        for got, ref, nm in ((dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv")):
            g = got[sl].cpu().double().numpy()
            err = float(np.abs(g - ref).max())
            bound = GRAD_REL * float(np.abs(ref).max())
            print(f"[case]   head ({b},{h}) {nm}: max err {err:.3e}, bound {bound:.3e}", file=sys.stderr, flush=True)
            assert err <= bound, f"{nm} of head ({b},{h}): max err {err:.3e} > {bound:.3e}"
