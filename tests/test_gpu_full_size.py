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
