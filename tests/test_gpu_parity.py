"""GPU parity: the HIP kernels (through the C ABI) against the fp64 oracle, element by element.

Shapes are small enough for the full oracle yet span several query and key tiles
(128 x 64) and ragged tails; each case names its shape and options in its id.
Outputs are poisoned with NaN before each call so an unwritten element fails.
"""

import math
import sys

import numpy as np
import pytest
import torch

import exact_attention_56_amd as fa
import oracle
from exact_attention_56_amd.inputs import make_alibi_slopes, make_qkv
from tests.parity import check_empty_rows_zero, check_lse, check_out

pytestmark = pytest.mark.gpu
DEV = "cuda"


def announce(msg):
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def inputs(b, h, sq, sk, d, alibi, seed):
    q, k, v = make_qkv(b, sq, sk, h, d, seed)
    slopes = make_alibi_slopes(h) if alibi else None
    return q, k, v, slopes


def gpu_fwd(q, k, v, scale, causal, wl, wr, slopes):
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    b, sq, h, d = q.shape
    out = torch.full_like(qd, float("nan"))
    lse = torch.full((b, h, sq), float("nan"), dtype=torch.float32, device=DEV)
    sd = None if slopes is None else slopes.to(DEV)
    fa.fwd(qd, kd, vd, out, lse, scale, causal, (wl, wr), sd)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def f32(x):
    return float(np.float32(x))


FWD_CASES = [
    # b, h, sq, sk, d, causal, wl, wr, alibi, scale (None = 1/sqrt(d))
    (1, 2, 128, 128, 64, False, -1, -1, False, None),
    (2, 3, 1, 1, 64, False, -1, -1, False, None),
    (1, 2, 17, 17, 128, True, -1, -1, False, None),
    (2, 2, 127, 129, 128, False, -1, -1, False, None),
    (1, 2, 129, 127, 256, True, -1, -1, False, None),
    (1, 2, 200, 1000, 128, True, -1, -1, False, None),
    (1, 2, 1000, 200, 64, True, -1, -1, False, None),
    (1, 3, 300, 300, 64, True, 50, 0, True, None),
    (1, 2, 256, 256, 128, False, 32, 16, False, None),
    (1, 2, 130, 70, 128, False, 5, 3, True, None),
    (1, 2, 64, 64, 256, False, 0, 0, False, None),
    (1, 2, 333, 517, 128, False, -1, -1, True, None),
    (2, 2, 257, 257, 256, True, -1, -1, True, None),
    (1, 2, 200, 300, 128, False, -1, -1, False, -0.09),
    (1, 2, 150, 150, 64, True, -1, -1, False, 0.0),
    (1, 1, 512, 512, 128, False, -1, 0, False, 1.5),
    (1, 2, 384, 768, 64, False, 100, -1, False, None),
    (1, 2, 96, 1200, 128, True, 700, 0, True, None),
    (1, 2, 1, 700, 128, True, -1, -1, True, None),
    # headdim 128 without a mask from 2048 query rows on, and with a plain causal mask
    # from 8192: eight-wave (256-row) workgroups in the ping-pong schedule
    (1, 1, 4096 + 77, 3001, 128, False, -1, -1, False, None),
    (1, 1, 4352, 4352, 128, False, -1, -1, True, None),
    (1, 1, 4095, 333, 128, False, -1, -1, False, None),
    (1, 1, 2047, 2100, 128, False, -1, -1, False, None),
    (2, 1, 2048, 1999, 128, False, -1, -1, False, None),
    (1, 1, 8192 + 40, 8192 + 40, 128, True, -1, -1, False, None),
    (1, 1, 8200, 9100, 128, True, -1, -1, True, None),
    (1, 1, 8191, 8191, 128, True, -1, -1, False, None),
    # ALiBi under a causal mask (key tiles right to left, no per-tile maximum): many tiles,
    # rows that see no key (Sq > Sk), a left window, a negative scale (scores that rise
    # from tile to tile refit the reference)
    (1, 8, 1500, 1500, 128, True, -1, -1, True, None),
    (1, 4, 700, 400, 64, True, -1, -1, True, None),
    (2, 8, 1030, 1100, 64, True, 256, 0, True, None),
    (1, 2, 600, 600, 64, True, -1, -1, True, -0.1),
]


def case_id(c):
    b, h, sq, sk, d, causal, wl, wr, alibi, scale = c
    return f"b{b}h{h}_sq{sq}_sk{sk}_d{d}{'_causal' if causal else ''}_w{wl},{wr}{'_alibi' if alibi else ''}_s{scale}"


@pytest.mark.parametrize("case", FWD_CASES, ids=[case_id(c) for c in FWD_CASES])
def test_fwd_matches_oracle(case):
    b, h, sq, sk, d, causal, wl, wr, alibi, scale = case
    announce(case_id(case))
    scale = f32(1.0 / math.sqrt(d) if scale is None else scale)
    q, k, v, slopes = inputs(b, h, sq, sk, d, alibi, seed=sq * 7 + sk)
    out, lse = gpu_fwd(q, k, v, scale, causal, wl, wr, slopes)
    ref_out, ref_lse = oracle.attention_forward(q, k, v, scale, causal, wl, wr, slopes)
    check_lse(lse, ref_lse)
    check_out(out, ref_out)
    check_empty_rows_zero(out, ref_lse)


VARLEN_CASES = [
    # lengths of q sequences, lengths of k sequences, H, H_k, d, causal, wl, wr, alibi
    ((100, 0, 257, 3), (130, 5, 200, 64), 4, 2, 128, True, -1, -1, False),
    ((1, 129, 64), (300, 129, 0), 2, 1, 64, False, -1, -1, True),
    ((300, 77), (77, 300), 8, 2, 128, False, 40, 10, True),
    ((200, 200), (200, 333), 4, 4, 256, True, -1, -1, False),
    ((520, 1), (700, 1000), 6, 3, 64, True, 100, 0, True),
    # a sequence of at least 4096 rows without a mask: the eight-wave launch, grouped heads
    ((4100, 50), (4100, 3000), 2, 1, 128, False, -1, -1, False),
    # causal with a sequence of at least 8192 rows: the eight-wave causal launch
    ((8197, 300), (8197, 300), 2, 1, 128, True, -1, -1, False),
]


def varlen_id(c):
    lq, lk, h, hk, d, causal, wl, wr, alibi = c
    return (f"q{'-'.join(map(str, lq))}_k{'-'.join(map(str, lk))}_h{h}kv{hk}_d{d}"
            f"{'_causal' if causal else ''}_w{wl},{wr}{'_alibi' if alibi else ''}")


@pytest.mark.parametrize("case", VARLEN_CASES, ids=[varlen_id(c) for c in VARLEN_CASES])
def test_varlen_gqa_matches_oracle(case):
    lq, lk, h, hk, d, causal, wl, wr, alibi = case
    announce("varlen " + varlen_id(case))
    cq = torch.tensor([0] + list(np.cumsum(lq)), dtype=torch.int32)
    ck = torch.tensor([0] + list(np.cumsum(lk)), dtype=torch.int32)
    total_q, total_k = int(cq[-1]), int(ck[-1])
    q, k, v = make_qkv(1, total_q, max(total_k, 1), h, d, seed=total_q * 3 + total_k, nheads_k=hk)
    q, k, v = q[0], k[0, :total_k], v[0, :total_k]
    slopes = make_alibi_slopes(h) if alibi else None
    scale = f32(1.0 / math.sqrt(d))
    qd, kd, vd = q.to(DEV), k.contiguous().to(DEV), v.contiguous().to(DEV)
    out = torch.full_like(qd, float("nan"))
    lse = torch.full((h, total_q), float("nan"), dtype=torch.float32, device=DEV)
    fa.fwd_varlen(qd, kd, vd, out, lse, cq.to(DEV), ck.to(DEV), max(lq), max(lk), scale, causal, (wl, wr),
                  None if slopes is None else slopes.to(DEV))
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle.attention_varlen(q, k, v, cq.numpy(), ck.numpy(), scale, causal, wl, wr, slopes)
    check_lse(lse.cpu(), ref_lse)
    check_out(out.cpu(), ref_out)
    check_empty_rows_zero(out.cpu()[None], ref_lse[None])


def test_fwd_deterministic():
    announce("determinism b2h4 sq300 sk700 d128 causal alibi")
    q, k, v, slopes = inputs(2, 4, 300, 700, 128, True, seed=11)
    o1, l1 = gpu_fwd(q, k, v, 0.1, True, -1, -1, slopes)
    o2, l2 = gpu_fwd(q, k, v, 0.1, True, -1, -1, slopes)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


SPLIT_CASES = [
    # b, h, sq, sk, d, causal, wl, wr, alibi, num_splits
    (2, 3, 1, 1000, 128, True, -1, -1, False, 16),
    (1, 2, 4, 513, 64, False, -1, -1, True, 3),
    (1, 2, 1, 300, 256, True, 100, 0, False, 64),
    (1, 2, 8, 2048, 128, True, -1, -1, False, 1),
    (1, 1, 1, 5, 64, True, -1, -1, False, 5),
    (1, 2, 9, 700, 128, True, -1, -1, False, 5),
    (1, 2, 200, 1000, 64, False, 64, 32, True, 7),
    (2, 2, 130, 333, 256, True, -1, -1, False, 3),
    (1, 2, 3, 100, 128, False, 10, 10, False, 16),
]


def split_id(c):
    b, h, sq, sk, d, causal, wl, wr, alibi, ns = c
    return f"b{b}h{h}_sq{sq}_sk{sk}_d{d}{'_causal' if causal else ''}_w{wl},{wr}{'_alibi' if alibi else ''}_splits{ns}"


@pytest.mark.parametrize("case", SPLIT_CASES, ids=[split_id(c) for c in SPLIT_CASES])
def test_splitkv_and_combine_match_oracle(case):
    b, h, sq, sk, d, causal, wl, wr, alibi, ns = case
    announce(split_id(case))
    scale = f32(1.0 / math.sqrt(d))
    q, k, v, slopes = inputs(b, h, sq, sk, d, alibi, seed=sk + ns)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    sd = None if slopes is None else slopes.to(DEV)
    op = torch.full((ns, b, h, sq, d), float("nan"), dtype=torch.float32, device=DEV)
    lp = torch.full((ns, b, h, sq), float("nan"), dtype=torch.float32, device=DEV)
    fa.fwd_splitkv(qd, kd, vd, op, lp, ns, scale, causal, (wl, wr), sd)
    out = torch.full_like(qd, float("nan"))
    lse = torch.full((b, h, sq), float("nan"), dtype=torch.float32, device=DEV)
    fa.combine(op, lp, out, lse)
    torch.cuda.synchronize()

    ref_op, ref_lp = oracle.splitkv_partials(q, k, v, scale, ns, causal, wl, wr, slopes)
    check_lse(lp.cpu(), ref_lp, "lse_partial")
    check_out(op.cpu(), ref_op, "out_partial")
    ref_out, ref_lse = oracle.attention_forward(q, k, v, scale, causal, wl, wr, slopes)
    check_lse(lse.cpu(), ref_lse)
    check_out(out.cpu(), ref_out)
    check_empty_rows_zero(out.cpu(), ref_lse)


def test_combine_on_oracle_partials():
    """fa_combine alone, fed partials written by the oracle (including empty splits)."""
    announce("combine on oracle partials")
    q, k, v, _ = inputs(2, 3, 5, 40, 64, False, seed=5)
    ref_op, ref_lp = oracle.splitkv_partials(q, k, v, 0.125, 12, True, 6, 0)
    op = torch.from_numpy(ref_op).float().to(DEV)
    lp = torch.from_numpy(ref_lp).float().to(DEV)
    out = torch.full((2, 5, 3, 64), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((2, 3, 5), float("nan"), dtype=torch.float32, device=DEV)
    fa.combine(op, lp, out, lse)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle.combine(ref_op.astype(np.float32), ref_lp.astype(np.float32))
    check_lse(lse.cpu(), ref_lse)
    check_out(out.cpu(), ref_out)
    # every split empty for a row: zero output, -inf lse
    lp_all = torch.full((3, 1, 1, 2), float("-inf"), device=DEV)
    op_all = torch.ones(3, 1, 1, 2, 64, device=DEV)
    out2 = torch.full((1, 2, 1, 64), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse2 = torch.full((1, 1, 2), float("nan"), device=DEV)
    fa.combine(op_all, lp_all, out2, lse2)
    torch.cuda.synchronize()
    assert torch.all(out2.cpu() == 0) and torch.all(torch.isneginf(lse2.cpu()))


def test_binding_errors_on_gpu():
    q = torch.zeros(1, 4, 2, 64, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        fa.flash_attn_func(q, q[:, :, :1], q[:, :, :1])
    with pytest.raises(ValueError):
        fa.flash_attn_func(q.transpose(1, 2), q, q)
    k = torch.zeros(1, 4, 2, 96, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(fa.FAError):
        fa.flash_attn_func(k, k, k)


# Scores that rise along the keys: key j is scaled by 1 + 4j/Sk and softmax_scale is 1,
# so every later key tile holds far larger scores than the first one.  Kernels without
# ALiBi keep the reference maximum from the first tile until a tile's exponentials
# grow past a threshold (or overflow), then refit it to that tile's row max; these
# cases run that refit on most tiles, in the four-wave (1000 rows) and eight-wave
# (4096 rows, headdim 128, unmasked) launches and under a causal mask.
RISING_CASES = [
    # b, h, sq, sk, d, causal
    (1, 2, 1000, 1000, 128, False),
    (1, 2, 4096, 4096, 128, False),
    (1, 2, 777, 1300, 64, True),
    (1, 1, 600, 900, 256, False),
]


@pytest.mark.parametrize("case", RISING_CASES, ids=[f"b{c[0]}h{c[1]}_sq{c[2]}_sk{c[3]}_d{c[4]}"
                                                     f"{'_causal' if c[5] else ''}" for c in RISING_CASES])
def test_rising_scores_match_oracle(case):
    b, h, sq, sk, d, causal = case
    announce(f"rising scores {case}")
    q, k, v = make_qkv(b, sq, sk, h, d, seed=sq + sk)
    ramp = (1.0 + 4.0 * torch.arange(sk, dtype=torch.float32) / sk).view(1, sk, 1, 1)
    k = (k.float() * ramp).to(torch.bfloat16)
    out, lse = gpu_fwd(q, k, v, 1.0, causal, -1, -1, None)
    ref_out, ref_lse = oracle.attention_forward(q, k, v, 1.0, causal)
    check_lse(lse, ref_lse)
    check_out(out, ref_out)


@pytest.mark.parametrize("d", [64, 128])
def test_far_negative_scores_under_window(d):
    """Every score near -1000: a row's exponentials against a reference of 0 all
    underflow.  Under a sliding window (and bottom-right alignment with Sq < Sk) many
    rows see no key in their block's first tiles, so they still have no reference when
    their first visible keys arrive; they must get one from those keys' scores."""
    b, h, sq, sk = 1, 2, 192, 450
    announce(f"far negative scores d{d}")
    g = torch.Generator().manual_seed(d)
    q = (4.0 + 0.05 * torch.randn(b, sq, h, d, generator=g)).to(torch.bfloat16)
    k = (-4.0 + 0.05 * torch.randn(b, sk, h, d, generator=g)).to(torch.bfloat16)
    v = torch.randn(b, sk, h, d, generator=g).to(torch.bfloat16)
    for wl, wr in ((30, 20), (100, 0)):
        out, lse = gpu_fwd(q, k, v, 1.0, False, wl, wr, None)
        ref_out, ref_lse = oracle.attention_forward(q, k, v, 1.0, False, wl, wr)
        check_lse(lse, ref_lse)
        check_out(out, ref_out)
