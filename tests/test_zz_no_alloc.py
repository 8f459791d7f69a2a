"""GPU check of fa_fwd_kvcache_noalloc (the KV-cache decode step whose split partials
live in the library's own device buffer) against fa_fwd_kvcache with caller-owned
partials, through the C ABI: two calls in a row on one GPU, the second with a smaller
input (so the buffer holds the first call's larger contents when the second runs).

Each call runs both entry points on their own copies of the cache.  Their outputs, lse
and caches must be bit-identical (same kernels, same split count), and the no-alloc
result must also meet the oracle tolerances.  A split count that does not fit the
buffer is rejected before any launch.
"""

import math
import sys

import numpy as np
import pytest
import torch

import exact_attention_56_amd as fa
import oracle
from exact_attention_56_amd.inputs import make_alibi_slopes
from tests.parity import check_lse, check_out

pytestmark = pytest.mark.gpu
DEV = "cuda"

# batch, Sq, H, H_k, D, page (None: contiguous), blocks / capacity, cache lengths, S_new, rotary_dim,
# causal, window_left, alibi, num_splits
LARGE = (4, 2, 16, 4, 128, 256, 16, (1000, 3000, 17, 2047), 2, 128, True, -1, False, 0)
SMALL = (2, 1, 8, 8, 64, None, 600, (300, 5), 1, 0, True, 50, True, 3)


def bf16(shape, g):
    return torch.randn(*shape, generator=g, dtype=torch.float32).to(torch.bfloat16)


def run_case(case, seed):
    b, sq, h, hk, d, page, cap, lens, snew, rd, causal, wl, alibi, ns = case
    print(f"[case] no-alloc kvcache b{b} sq{sq} h{h}/{hk} d{d} page{page} lens{lens} new{snew} rot{rd} ns{ns}",
          file=sys.stderr, flush=True)
    g = torch.Generator().manual_seed(seed)
    q = bf16((b, sq, h, d), g)
    if page is None:
        kc, vc = bf16((b, cap, hk, d), g), bf16((b, cap, hk, d), g)
        table = None
    else:
        kc, vc = bf16((b * cap, page, hk, d), g), bf16((b * cap, page, hk, d), g)
        table = torch.randperm(b * cap, generator=g).to(torch.int32).view(b, cap).contiguous()
    knew, vnew = bf16((b, snew, hk, d), g), bf16((b, snew, hk, d), g)
    cos = sin = None
    if rd:
        capacity = page * cap if page else cap
        theta = torch.rand(capacity, rd // 2, generator=g) * 2 * math.pi
        cos, sin = torch.cos(theta), torch.sin(theta)
    slopes = make_alibi_slopes(h) if alibi else None
    scale = float(np.float32(1.0 / math.sqrt(d)))
    lens_t = torch.tensor(lens, dtype=torch.int32)
    dv = lambda t: None if t is None else t.to(DEV)
    args = dict(block_table=dv(table), k_new=dv(knew), v_new=dv(vnew), rotary_cos=dv(cos), rotary_sin=dv(sin),
                softmax_scale=scale, causal=causal, window_size=(wl, -1), alibi_slopes=dv(slopes), num_splits=ns)

    # the existing entry point with caller-owned partials
    kc1, vc1 = kc.to(DEV), vc.to(DEV)
    out1 = torch.empty(b, sq, h, d, dtype=torch.bfloat16, device=DEV)
    lse1 = torch.empty(b, h, sq, dtype=torch.float32, device=DEV)
    op = torch.empty(64, b, h, sq, d, dtype=torch.float32, device=DEV)
    lp = torch.empty(64, b, h, sq, dtype=torch.float32, device=DEV)
    fa.fwd_kvcache(dv(q), kc1, vc1, dv(lens_t), out1, lse1, op, lp, **args)
    # the no-allocation entry point
    kc2, vc2 = kc.to(DEV), vc.to(DEV)
    out2 = torch.full((b, sq, h, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse2 = torch.full((b, h, sq), float("nan"), dtype=torch.float32, device=DEV)
    fa.fwd_kvcache_noalloc(dv(q), kc2, vc2, dv(lens_t), out2, lse2, **args)
    torch.cuda.synchronize()

    assert torch.equal(out2.cpu(), out1.cpu()), "out differs from fa_fwd_kvcache"
    assert torch.equal(lse2.cpu(), lse1.cpu()), "lse differs from fa_fwd_kvcache"
    assert torch.equal(kc2.cpu(), kc1.cpu()) and torch.equal(vc2.cpu(), vc1.cpu()), "caches differ"
    ref_out, ref_lse, _, _ = oracle.attention_kvcache(
        q, kc, vc, lens, scale, block_table=None if table is None else table.numpy(), k_new=knew, v_new=vnew,
        rotary_cos=cos, rotary_sin=sin, rotary_dim=rd, causal=causal, window_left=wl, alibi_slopes=slopes)
    check_lse(lse2.cpu(), ref_lse)
    check_out(out2.cpu(), ref_out)


def test_noalloc_matches_kvcache_twice_second_smaller():
    run_case(LARGE, seed=11)
    run_case(SMALL, seed=12)


def test_noalloc_rejects_split_count_past_buffer():
    # batch 8 x 16 heads x headdim 128: 254 splits fit in 16 MiB; 255 is refused before any launch
    q = torch.zeros(8, 1, 16, 128, dtype=torch.bfloat16, device=DEV)
    kc = torch.zeros(8, 1024, 16, 128, dtype=torch.bfloat16, device=DEV)
    lens = torch.zeros(8, dtype=torch.int32, device=DEV)
    out = torch.empty_like(q)
    lse = torch.empty(8, 16, 1, dtype=torch.float32, device=DEV)
    with pytest.raises(fa.FAError):
        fa.fwd_kvcache_noalloc(q, kc, kc, lens, out, lse, num_splits=255)
