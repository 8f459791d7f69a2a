"""GPU parity for fp16 tensors and for ALiBi slopes given per (batch, head), through the
C ABI, against the fp64 oracle.

Every entry point takes both: the padded forward (four- and eight-wave launches), the
split pair, packed sequences, the backward and the KV-cache decode.  The comparison rule
is the bf16 one (tests/parity.py and the backward's bound): fp16 carries more mantissa
bits than bf16, so the same bounds hold with room to spare.  Inputs are N(0, 1) rounded
to the element type; slope tables come from make_alibi_slopes(nheads, batch).
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
from tests.test_gpu_backward import check_grad

pytestmark = pytest.mark.gpu
DEV = "cuda"
DTYPES = {"fp16": torch.float16, "bf16": torch.bfloat16}


def announce(msg):
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def slopes_for(kind, b, h):
    return None if kind == "none" else make_alibi_slopes(h) if kind == "head" else make_alibi_slopes(h, b)


def dev(t):
    return None if t is None else t.to(DEV)


FWD_CASES = [
    # b, h, sq, sk, d, causal, wl, wr, slopes (none / head / batch), dtype, scale (None = 1/sqrt(d))
    (1, 2, 128, 128, 64, False, -1, -1, "none", "fp16", None),
    (2, 2, 127, 129, 128, False, -1, -1, "batch", "fp16", None),
    (1, 2, 129, 127, 256, True, -1, -1, "none", "fp16", None),
    (2, 3, 300, 300, 64, True, 50, 0, "batch", "fp16", None),
    (1, 2, 200, 300, 128, False, -1, -1, "head", "fp16", -0.09),
    (1, 2, 1000, 200, 64, True, -1, -1, "none", "fp16", None),
    (2, 2, 257, 257, 256, True, -1, -1, "batch", "bf16", None),
    (3, 2, 333, 517, 128, False, 30, 60, "batch", "bf16", None),
    # causal ALiBi (keys right to left, the bias on the matrix cores) with fp16 operands:
    # the bias step split into fp16 parts, a negative scale
    (1, 4, 700, 700, 128, True, -1, -1, "head", "fp16", None),
    (2, 4, 1100, 1100, 64, True, 300, 0, "batch", "fp16", -0.2),
    # a tiny scale: the bias step per key in raw score units (slope / scale) is far past
    # the fp16 range, so the bias product runs in bf16
    (1, 4, 300, 300, 64, True, -1, -1, "head", "fp16", 1e-6),
    (1, 4, 300, 300, 128, True, 100, 0, "head", "fp16", 1e-6),
    # eight-wave (256-row) workgroups: headdim 128, no mask, >= 4096 query rows
    (1, 1, 4352, 4352, 128, False, -1, -1, "none", "fp16", None),
    (2, 1, 4100, 3001, 128, False, -1, -1, "batch", "fp16", None),
    (2, 1, 4097, 4097, 128, False, -1, -1, "batch", "bf16", None),
]


def fwd_id(c):
    b, h, sq, sk, d, causal, wl, wr, sl, dt, scale = c
    return f"{dt}_b{b}h{h}_sq{sq}_sk{sk}_d{d}{'_causal' if causal else ''}_w{wl},{wr}_slopes-{sl}_s{scale}"


@pytest.mark.parametrize("case", FWD_CASES, ids=[fwd_id(c) for c in FWD_CASES])
def test_fwd_fp16_and_batch_slopes(case):
    b, h, sq, sk, d, causal, wl, wr, sl, dt, scale = case
    announce("fwd " + fwd_id(case))
    scale = float(np.float32(1.0 / math.sqrt(d) if scale is None else scale))
    q, k, v = make_qkv(b, sq, sk, h, d, seed=sq * 11 + sk, dtype=DTYPES[dt])
    slopes = slopes_for(sl, b, h)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out = torch.full_like(qd, float("nan"))
    lse = torch.full((b, h, sq), float("nan"), dtype=torch.float32, device=DEV)
    fa.fwd(qd, kd, vd, out, lse, scale, causal, (wl, wr), dev(slopes))
    torch.cuda.synchronize()
    assert out.dtype == DTYPES[dt]
    ref_out, ref_lse = oracle.attention_forward(q, k, v, scale, causal, wl, wr, slopes)
    check_lse(lse.cpu(), ref_lse)
    check_out(out.cpu(), ref_out)
    check_empty_rows_zero(out.cpu(), ref_lse)


SPLIT_CASES = [
    # b, h, sq, sk, d, causal, wl, wr, slopes, dtype, num_splits
    (2, 3, 1, 1000, 128, True, -1, -1, "batch", "fp16", 16),
    (2, 2, 4, 513, 256, False, -1, -1, "none", "fp16", 3),
    (1, 2, 200, 1000, 64, False, 64, 32, "batch", "fp16", 7),
    (3, 2, 1, 700, 64, True, 100, 0, "batch", "bf16", 5),
]


def split_id(c):
    b, h, sq, sk, d, causal, wl, wr, sl, dt, ns = c
    return f"{dt}_b{b}h{h}_sq{sq}_sk{sk}_d{d}{'_causal' if causal else ''}_w{wl},{wr}_slopes-{sl}_splits{ns}"


@pytest.mark.parametrize("case", SPLIT_CASES, ids=[split_id(c) for c in SPLIT_CASES])
def test_splitkv_combine_fp16_and_batch_slopes(case):
    b, h, sq, sk, d, causal, wl, wr, sl, dt, ns = case
    announce("splitkv " + split_id(case))
    scale = float(np.float32(1.0 / math.sqrt(d)))
    q, k, v = make_qkv(b, sq, sk, h, d, seed=sq + 3 * sk, dtype=DTYPES[dt])
    slopes = slopes_for(sl, b, h)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    op = torch.full((ns, b, h, sq, d), float("nan"), dtype=torch.float32, device=DEV)
    lp = torch.full((ns, b, h, sq), float("nan"), dtype=torch.float32, device=DEV)
    fa.fwd_splitkv(qd, kd, vd, op, lp, ns, scale, causal, (wl, wr), dev(slopes))
    out = torch.full_like(qd, float("nan"))
    lse = torch.full((b, h, sq), float("nan"), dtype=torch.float32, device=DEV)
    fa.combine(op, lp, out, lse)
    torch.cuda.synchronize()
    ref_op, ref_lp = oracle.splitkv_partials(q, k, v, scale, ns, causal, wl, wr, slopes)
    check_lse(lp.cpu(), ref_lp, "lse_partial")
    check_out(op.cpu(), ref_op, "out_partial")
    ref_out, ref_lse = oracle.combine(ref_op, ref_lp)
    check_lse(lse.cpu(), ref_lse)
    check_out(out.cpu(), ref_out)


VARLEN_CASES = [
    # q lengths, k lengths, H, H_k, d, causal, wl, wr, slopes, dtype
    ((100, 0, 257, 3), (130, 5, 200, 64), 4, 2, 128, True, -1, -1, "batch", "fp16"),
    ((300, 77), (77, 300), 8, 2, 128, False, 40, 10, "batch", "bf16"),
    ((200, 200), (200, 333), 4, 4, 256, True, -1, -1, "none", "fp16"),
]


def varlen_id(c):
    lq, lk, h, hk, d, causal, wl, wr, sl, dt = c
    return (f"{dt}_q{'-'.join(map(str, lq))}_k{'-'.join(map(str, lk))}_h{h}kv{hk}_d{d}"
            f"{'_causal' if causal else ''}_w{wl},{wr}_slopes-{sl}")


@pytest.mark.parametrize("case", VARLEN_CASES, ids=[varlen_id(c) for c in VARLEN_CASES])
def test_varlen_fp16_and_sequence_slopes(case):
    lq, lk, h, hk, d, causal, wl, wr, sl, dt = case
    announce("varlen " + varlen_id(case))
    cq = torch.tensor([0] + list(np.cumsum(lq)), dtype=torch.int32)
    ck = torch.tensor([0] + list(np.cumsum(lk)), dtype=torch.int32)
    total_q, total_k = int(cq[-1]), int(ck[-1])
    q, k, v = make_qkv(1, total_q, total_k, h, d, seed=total_q + 7 * total_k, nheads_k=hk, dtype=DTYPES[dt])
    q, k, v = q[0], k[0], v[0]
    slopes = slopes_for(sl, len(lq), h)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out = torch.full_like(qd, float("nan"))
    lse = torch.full((h, total_q), float("nan"), dtype=torch.float32, device=DEV)
    fa.fwd_varlen(qd, kd, vd, out, lse, cq.to(DEV), ck.to(DEV), max(lq), max(lk), scale, causal, (wl, wr),
                  dev(slopes))
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle.attention_varlen(q, k, v, cq.numpy(), ck.numpy(), scale, causal, wl, wr, slopes)
    check_lse(lse.cpu(), ref_lse)
    check_out(out.cpu(), ref_out)
    check_empty_rows_zero(out.cpu()[None], ref_lse[None])


BWD_CASES = [
    # b, h, sq, sk, d, causal, wl, wr, slopes, dtype
    (1, 2, 128, 128, 64, False, -1, -1, "none", "fp16"),
    (2, 2, 200, 300, 128, True, -1, -1, "batch", "fp16"),
    (1, 3, 257, 129, 128, True, -1, -1, "none", "fp16"),
    (2, 2, 192, 450, 128, False, 30, 20, "head", "fp16"),
    (2, 2, 300, 300, 128, True, 40, 0, "batch", "bf16"),
    (3, 1, 100, 333, 64, True, -1, -1, "batch", "bf16"),
]


def bwd_id(c):
    b, h, sq, sk, d, causal, wl, wr, sl, dt = c
    return f"{dt}_b{b}h{h}_sq{sq}_sk{sk}_d{d}{'_causal' if causal else ''}_w{wl},{wr}_slopes-{sl}"


@pytest.mark.parametrize("case", BWD_CASES, ids=[bwd_id(c) for c in BWD_CASES])
def test_bwd_fp16_and_batch_slopes(case):
    b, h, sq, sk, d, causal, wl, wr, sl, dt = case
    announce("bwd " + bwd_id(case))
    scale = float(np.float32(1.0 / math.sqrt(d)))
    q, k, v = make_qkv(b, sq, sk, h, d, seed=sq * 13 + sk, dtype=DTYPES[dt])
    dout = make_qkv(b, sq, 1, h, d, seed=sq * 13 + sk + 1, dtype=DTYPES[dt])[0]
    slopes = slopes_for(sl, b, h)
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, dout))
    out, lse = fa.flash_attn_func(qd, kd, vd, scale, causal, (wl, wr), dev(slopes))
    dq, dk, dv_ = (torch.full_like(t, float("nan")) for t in (qd, kd, vd))
    delta = torch.full((b, h, sq), float("nan"), dtype=torch.float32, device=DEV)
    fa.bwd(qd, kd, vd, out, lse, gd, dq, dk, dv_, delta, scale, causal, (wl, wr), dev(slopes))
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_backward(q, k, v, dout, scale, causal, wl, wr, slopes)
    keep = oracle.visible_mask(sq, sk, causal, wl, wr)
    empty_rows, unseen_keys = ~keep.any(axis=1), ~keep.any(axis=0)
    check_grad(dq.cpu(), rq, "dq", empty_rows)
    check_grad(dk.cpu(), rk, "dk", unseen_keys)
    check_grad(dv_.cpu(), rv, "dv", unseen_keys)


KVC_CASES = [
    # batch, Sq, H, H_k, D, page (None: contiguous), max_blocks / capacity, cache lengths, S_new, rotary_dim,
    # causal, window_left, slopes, dtype
    (3, 1, 8, 2, 128, 64, 8, (100, 0, 447), 1, 128, True, -1, "batch", "fp16"),
    (2, 3, 4, 2, 128, None, 300, (0, 250), 3, 64, False, -1, "batch", "bf16"),
    (2, 1, 12, 4, 128, 64, 4, (150, 77), 1, 0, True, -1, "head", "fp16"),
    (2, 1, 4, 4, 64, 128, 4, (200, 5), 2, 32, True, 50, "batch", "fp16"),
]


def kvc_id(c):
    b, sq, h, hk, d, page, cap, lens, snew, rd, causal, wl, sl, dt = c
    return (f"{dt}_b{b}_sq{sq}_h{h}kv{hk}_d{d}_{'paged' + str(page) if page else 'contig'}"
            f"_lens{'-'.join(map(str, lens))}_new{snew}_rot{rd}{'_causal' if causal else ''}_wl{wl}_slopes-{sl}")


@pytest.mark.parametrize("case", KVC_CASES, ids=[kvc_id(c) for c in KVC_CASES])
def test_kvcache_fp16_and_batch_slopes(case):
    b, sq, h, hk, d, page, cap, lens, snew, rd, causal, wl, sl, dt = case
    announce("kvcache " + kvc_id(case))
    et = DTYPES[dt]
    g = torch.Generator().manual_seed(sum(lens) + 17 * d + snew)
    draw = lambda *shape: torch.randn(*shape, generator=g, dtype=torch.float32).to(et)
    q = draw(b, sq, h, d)
    if page is None:
        kc, vc, table = draw(b, cap, hk, d), draw(b, cap, hk, d), None
    else:
        kc, vc = draw(b * cap, page, hk, d), draw(b * cap, page, hk, d)
        table = torch.randperm(b * cap, generator=g).to(torch.int32).view(b, cap).contiguous()
    knew = draw(b, snew, hk, d) if snew else None
    vnew = draw(b, snew, hk, d) if snew else None
    cos = sin = None
    if rd:
        theta = torch.rand(4096, rd // 2, generator=g) * 2 * math.pi
        cos, sin = torch.cos(theta), torch.sin(theta)
    slopes = slopes_for(sl, b, h)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    kc_d, vc_d = kc.to(DEV), vc.to(DEV)
    out, lse = fa.kvcache_decode(q.to(DEV), kc_d, vc_d, torch.tensor(lens, dtype=torch.int32, device=DEV), dev(table),
                                 dev(knew), dev(vnew), dev(cos), dev(sin), scale, causal, (wl, -1), dev(slopes),
                                 max_splits=16)
    torch.cuda.synchronize()
    ref_out, ref_lse, k_app, _ = oracle.attention_kvcache(
        q, kc, vc, lens, scale, block_table=None if table is None else table.numpy(), k_new=knew, v_new=vnew,
        rotary_cos=cos, rotary_sin=sin, rotary_dim=rd, causal=causal, window_left=wl, alibi_slopes=slopes,
        storage=dt)
    assert out.dtype == et
    check_lse(lse.cpu(), ref_lse)
    check_out(out.cpu(), ref_out)
    check_empty_rows_zero(out.cpu(), ref_lse)
    kc_got, vc_got = kc_d.cpu(), vc_d.cpu()
    for bb in range(b):
        for i in range(snew):
            j = lens[bb] + i
            blk, row = (bb, j) if table is None else (int(table[bb, j // page]), j % page)
            assert torch.equal(vc_got[blk, row], vnew[bb, i])
            kg = kc_got[blk, row].view(torch.int16).int()
            kr = torch.from_numpy(k_app[bb, i]).to(et).view(torch.int16).int()
            assert int((kg - kr).abs().max()) <= 1, f"k row {bb},{i}: more than one {dt} step off"
