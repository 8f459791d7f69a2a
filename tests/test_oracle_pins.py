"""Pins for the fp64 oracle: checks against what the pages and the mathematics fix.

None of these re-types the oracle's own formula.  Each pin is an independent
fact: a mask the page prints, a closed form, a special case that reduces to a
library routine, brute force with scalar loops, or an invariant.  The mutation
tests at the bottom plant plausible mistakes in the oracle (on the CPU) and
check that some pin catches each one.
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oa

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load_mask(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([int(x) for x in line.split()])
    return np.array(rows, dtype=bool)


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# --------------------------------------------------------------------------- pins


def pin_causal_2x5():
    """The page's printed v2.1 example (bottom-right) and not the v2.0 one (top-left)."""
    m = oracle.visible_mask(2, 5, causal=True)
    assert np.array_equal(m, load_mask("causal_mask_sq2_sk5_v21.txt"))
    assert not np.array_equal(m, load_mask("causal_mask_sq2_sk5_v20.txt"))


def pin_causal_5x2_zero_rows():
    """5x2 causal (reading of the lost example) and zero output for the empty rows."""
    m = oracle.visible_mask(5, 2, causal=True)
    assert np.array_equal(m, load_mask("causal_mask_sq5_sk2_v21.txt"))
    q, k, v = rand((1, 5, 1, 4), 1), rand((1, 2, 1, 4), 2), rand((1, 2, 1, 4), 3)
    out, lse = oracle.attention_forward(q, k, v, 0.5, causal=True)
    assert np.all(out[0, :3] == 0.0)
    assert np.all(np.isneginf(lse[0, 0, :3]))
    # row 3 sees only key 0: out = v_0 exactly, lse = its score
    assert np.allclose(out[0, 3, 0], v[0, 0, 0], atol=1e-15)
    assert abs(lse[0, 0, 3] - 0.5 * float(q[0, 3, 0] @ k[0, 0, 0])) < 1e-14
    assert np.all(np.isfinite(lse[0, 0, 3:]))


def pin_rows_sum_to_one(causal, wl, wr, slopes):
    """V = identity makes out = P itself: rows are a probability distribution on the visible set."""
    sq, sk = 7, 11
    q, k = rand((1, sq, 1, 5), 4), rand((1, sk, 1, 5), 5)
    v = np.eye(sk).reshape(1, sk, 1, sk)
    q5 = np.concatenate([q, np.zeros((1, sq, 1, sk - 5))], axis=3)
    k5 = np.concatenate([k, np.zeros((1, sk, 1, sk - 5))], axis=3)
    p, _ = oracle.attention_forward(q5, k5, v, 0.7, causal, wl, wr, slopes)
    p = p[0, :, 0, :]
    keep = oracle.visible_mask(sq, sk, causal, wl, wr)
    nonempty = keep.any(axis=1)
    assert np.all(p >= 0)
    assert np.all(p[~keep] == 0)
    assert np.allclose(p[nonempty].sum(axis=1), 1.0, atol=1e-12)
    assert np.all(p[~nonempty] == 0)


def pin_constant_v():
    """v_j = c for all j gives out_i = c on every non-empty row."""
    q, k = rand((2, 9, 3, 8), 6), rand((2, 13, 3, 8), 7)
    c = rand((8,), 8)
    v = np.broadcast_to(c, (2, 13, 3, 8)).copy()
    for causal, wl, wr in [(False, -1, -1), (True, -1, -1), (False, 2, 1), (True, 3, 0)]:
        out, lse = oracle.attention_forward(q, k, v, 0.3, causal, wl, wr, np.array([0.5, 0.25, 0.125]))
        keep = oracle.visible_mask(9, 13, causal, wl, wr)
        ne = keep.any(axis=1)
        assert np.allclose(out[:, ne], c, atol=1e-13)


def pin_scale_zero():
    """scale 0, no ALiBi: uniform weights, out = mean of visible v, lse = ln |V_i|."""
    sq = sk = 40
    q, k, v = rand((1, sq, 2, 4), 9), rand((1, sk, 2, 4), 10), rand((1, sk, 2, 4), 11)
    out, lse = oracle.attention_forward(q, k, v, 0.0, causal=True, window_left=10, window_right=0)
    for i in range(sq):
        lo = max(0, i - 10)
        assert abs(lse[0, 0, i] - math.log(min(i, 10) + 1)) < 1e-13
        assert np.allclose(out[0, i], v[0, lo:i + 1].mean(axis=0), atol=1e-14)


def pin_window_zero():
    """window (0, 0): only key c_i is visible, out_i = v_{c_i}, lse_i = s_{i, c_i}."""
    sq, sk = 6, 10
    q, k, v = rand((1, sq, 1, 8), 12), rand((1, sk, 1, 8), 13), rand((1, sk, 1, 8), 14)
    out, lse = oracle.attention_forward(q, k, v, 0.9, False, 0, 0)
    for i in range(sq):
        c = i + sk - sq
        assert np.array_equal(out[0, i, 0], v[0, c, 0])
        assert abs(lse[0, 0, i] - 0.9 * float(q[0, i, 0] @ k[0, c, 0])) < 1e-14


def pin_alibi_closed_form():
    """Q = 0 leaves only the ALiBi bias; lse is a geometric sum in r = e^-slope.

    Non-causal square: lse_i = ln[(1 - r^(i+1))/(1 - r) + r (1 - r^(S-1-i))/(1 - r)].
    Causal + window (wl, 0): lse_i = ln[(1 - r^(m+1))/(1 - r)] with m = min(i, wl).
    With Q = 0 the weights are r^|i-j| / Z, so out_i = sum_j r^|i-j| v_j / Z as well.
    """
    s, slope = 12, 0.37
    r = math.exp(-slope)
    q = np.zeros((1, s, 1, 4))
    k, v = rand((1, s, 1, 4), 15), rand((1, s, 1, 4), 16)
    # softmax_scale 0.5 multiplies Q.K^T only; the bias is added after scaling
    out, lse = oracle.attention_forward(q, k, v, 0.5, alibi_slopes=np.array([slope]))
    for i in range(s):
        z = (1 - r ** (i + 1)) / (1 - r) + r * (1 - r ** (s - 1 - i)) / (1 - r)
        assert abs(lse[0, 0, i] - math.log(z)) < 1e-13
        w = np.array([r ** abs(i - j) for j in range(s)]) / z
        assert np.allclose(out[0, i, 0], w @ v[0, :, 0], atol=1e-13)
    wl = 4
    out, lse = oracle.attention_forward(q, k, v, 0.5, causal=True, window_left=wl, window_right=0,
                                        alibi_slopes=np.array([slope]))
    for i in range(s):
        m = min(i, wl)
        assert abs(lse[0, 0, i] - math.log((1 - r ** (m + 1)) / (1 - r))) < 1e-13
    # Sq != Sk: the bias is measured from the bottom-right aligned position
    q2 = np.zeros((1, 3, 1, 4))
    _, lse2 = oracle.attention_forward(q2, k, v, 0.5, causal=True, alibi_slopes=np.array([slope]))
    for i in range(3):
        c = i + s - 3
        assert abs(lse2[0, 0, i] - math.log((1 - r ** (c + 1)) / (1 - r))) < 1e-13


def pin_sdpa_library():
    """Square, no window, no ALiBi: torch's scaled_dot_product_attention in fp64 on the CPU."""
    sdpa = torch.nn.functional.scaled_dot_product_attention
    for causal in (False, True):
        q, k, v = rand((2, 33, 3, 16), 17), rand((2, 33, 3, 16), 18), rand((2, 33, 3, 16), 19)
        out, _ = oracle.attention_forward(q, k, v, 0.21, causal)
        tq, tk, tv = (torch.from_numpy(x).permute(0, 2, 1, 3) for x in (q, k, v))
        ref = sdpa(tq, tk, tv, is_causal=causal, scale=0.21).permute(0, 2, 1, 3).numpy()
        assert np.allclose(out, ref, atol=1e-12, rtol=0)
    # Sq != Sk causal: bottom-right mask spelled as torch.tril with diagonal offset Sk - Sq
    sq, sk = 9, 21
    q, k, v = rand((1, sq, 2, 8), 20), rand((1, sk, 2, 8), 21), rand((1, sk, 2, 8), 22)
    out, _ = oracle.attention_forward(q, k, v, 0.4, causal=True)
    mask = torch.ones(sq, sk, dtype=torch.bool).tril(diagonal=sk - sq)
    tq, tk, tv = (torch.from_numpy(x).permute(0, 2, 1, 3) for x in (q, k, v))
    ref = sdpa(tq, tk, tv, attn_mask=mask, scale=0.4).permute(0, 2, 1, 3).numpy()
    assert np.allclose(out, ref, atol=1e-12, rtol=0)


BRUTE_CASES = [
    # (sq, sk, d, causal, wl, wr, alibi)
    (4, 4, 3, False, -1, -1, False),
    (4, 4, 3, True, -1, -1, False),
    (3, 7, 4, True, -1, -1, True),
    (7, 3, 4, True, -1, -1, False),
    (6, 8, 2, False, 2, 1, False),
    (8, 6, 5, False, 1, 3, True),
    (9, 9, 8, True, 3, -1, True),
    (5, 9, 3, False, -1, 0, False),
    (9, 5, 3, False, 0, -1, True),
    (1, 9, 8, True, -1, -1, True),
    (2, 5, 3, True, 2, 7, False),
]


def pin_brute_force(case):
    sq, sk, d, causal, wl, wr, alibi = case
    q, k, v = rand((2, sq, 2, d), 23), rand((2, sk, 2, d), 24), rand((2, sk, 2, d), 25)
    slopes = np.array([0.3, 0.05]) if alibi else None
    out, lse = oracle.attention_forward(q, k, v, 0.6, causal, wl, wr, slopes)
    bout, blse = oracle.brute_force(q, k, v, 0.6, causal, wl, wr, slopes)
    fin = np.isfinite(blse)
    assert np.array_equal(np.isneginf(lse), np.isneginf(blse))
    assert np.allclose(lse[fin], blse[fin], atol=1e-12, rtol=0)
    assert np.allclose(out, bout, atol=1e-12, rtol=0)


def pin_invariants():
    q, k, v = rand((1, 10, 2, 6), 26), rand((1, 14, 2, 6), 27), rand((1, 14, 2, 6), 28)
    base, base_lse = oracle.attention_forward(q, k, v, 0.5)
    # joint permutation of keys and values (non-causal, no window, no ALiBi)
    perm = np.random.default_rng(29).permutation(14)
    o2, l2 = oracle.attention_forward(q, k[:, perm], v[:, perm], 0.5)
    assert np.allclose(o2, base, atol=1e-13) and np.allclose(l2, base_lse, atol=1e-13)
    # max_j s_ij <= lse_i <= max_j s_ij + ln |V_i|
    s = 0.5 * np.einsum("bihd,bjhd->bhij", q, k)
    assert np.all(base_lse >= s.max(-1) - 1e-13)
    assert np.all(base_lse <= s.max(-1) + math.log(14) + 1e-13)
    # window equivalences
    for wl, wr in [(-1, -1), (14, 14), (100, -1)]:
        o, l = oracle.attention_forward(q, k, v, 0.5, False, wl, wr)
        assert np.allclose(o, base, atol=1e-14) and np.allclose(l, base_lse, atol=1e-14)
    oc, lc = oracle.attention_forward(q, k, v, 0.5, causal=True)
    ow, lw = oracle.attention_forward(q, k, v, 0.5, False, -1, 0)
    assert np.array_equal(oc, ow) and np.array_equal(lc, lw)
    # causal wins over a positive right window
    o3, l3 = oracle.attention_forward(q, k, v, 0.5, True, -1, 5)
    assert np.array_equal(o3, oc) and np.array_equal(l3, lc)
    # masked keys do not matter, however large their scores would be
    keep = oracle.visible_mask(10, 14, True, 3, 0)
    o5, l5 = oracle.attention_forward(q, k, v, 0.5, True, 3, 0)
    for i in (0, 4, 9):
        kb, vb = k.copy(), v.copy()
        kb[:, ~keep[i]] = 900.0 * np.sign(q[:, i:i + 1])
        vb[:, ~keep[i]] = 1e6
        o6, l6 = oracle.attention_forward(q, kb, vb, 0.5, True, 3, 0)
        assert np.allclose(o5[:, i], o6[:, i], atol=1e-13)
        assert np.allclose(l5[:, :, i], l6[:, :, i], atol=1e-13)
    # zero slope is no ALiBi
    o4, l4 = oracle.attention_forward(q, k, v, 0.5, alibi_slopes=np.zeros(2))
    assert np.allclose(o4, base, atol=1e-15) and np.allclose(l4, base_lse, atol=1e-15)


def pin_split_combine():
    """Merging per-split results reproduces the full row, for any partition of the keys."""
    q, k, v = rand((2, 5, 2, 4), 30), rand((2, 23, 2, 4), 31), rand((2, 23, 2, 4), 32)
    for causal, wl, wr, alibi in [(False, -1, -1, None), (True, -1, -1, np.array([0.2, 0.1])),
                                  (True, 6, 0, None), (False, 3, 2, np.array([0.4, 0.0]))]:
        full, full_lse = oracle.attention_forward(q, k, v, 0.8, causal, wl, wr, alibi)
        for ns in (1, 2, 3, 5, 8, 23):
            op, lp = oracle.splitkv_partials(q, k, v, 0.8, ns, causal, wl, wr, alibi)
            out, lse = oracle.combine(op, lp)
            assert np.allclose(out, full, atol=1e-13)
            fin = np.isfinite(full_lse)
            assert np.array_equal(np.isneginf(lse), np.isneginf(full_lse))
            assert np.allclose(lse[fin], full_lse[fin], atol=1e-13)
    # one key per split: each partial is that key's value and score, or empty
    op, lp = oracle.splitkv_partials(q, k, v, 0.8, 23, causal=True)
    for s in range(23):
        for i in range(5):
            c = i + 23 - 5
            if s <= c:
                assert np.array_equal(op[s, :, :, i], v[:, s])
                assert np.allclose(lp[s, :, :, i], 0.8 * np.einsum("bhd,bhd->bh", q[:, i], k[:, s]), atol=1e-14)
            else:
                assert np.all(op[s, :, :, i] == 0) and np.all(np.isneginf(lp[s, :, :, i]))
    # every split empty: out 0, lse -inf
    out, lse = oracle.combine(np.ones((3, 1, 1, 2, 4)), np.full((3, 1, 1, 2), -np.inf))
    assert np.all(out == 0) and np.all(np.isneginf(lse))
    # split bounds cover the keys once, in order, including a ragged last split
    assert oracle.split_bounds(10, 4) == [(0, 3), (3, 6), (6, 9), (9, 10)]
    assert oracle.split_bounds(9, 4) == [(0, 3), (3, 6), (6, 9), (9, 9)]


def pin_sampled_rows():
    """The sampled-row entry point agrees with the full forward row for row."""
    q, k, v = rand((2, 12, 3, 8), 33), rand((2, 17, 3, 8), 34), rand((2, 17, 3, 8), 35)
    slopes = np.array([0.5, 0.1, 0.02])
    full, full_lse = oracle.attention_forward(q, k, v, 0.3, True, 4, 0, slopes)
    samples = [(0, 0, 0), (1, 2, 11), (0, 1, 5), (1, 0, 3)]
    o, l = oracle.attention_sampled(q, k, v, samples, 0.3, True, 4, 0, slopes)
    for n, (b, h, i) in enumerate(samples):
        assert np.allclose(o[n], full[b, i, h], atol=1e-14) and abs(l[n] - full_lse[b, h, i]) < 1e-14


def pin_varlen_gqa():
    """A packed batch with grouped K/V heads equals, sequence by sequence, the scalar
    brute force on that sequence alone with each K/V head repeated for the query heads
    of its group (contiguous groups of H / H_k query heads share a K/V head)."""
    nheads, nheads_k, headdim = 4, 2, 5
    lens_q, lens_k = [3, 0, 6, 1, 2], [5, 2, 4, 1, 0]  # an empty query and an empty key sequence
    cq, ck = np.concatenate([[0], np.cumsum(lens_q)]), np.concatenate([[0], np.cumsum(lens_k)])
    q = rand((cq[-1], nheads, headdim), 40)
    k, v = rand((ck[-1], nheads_k, headdim), 41), rand((ck[-1], nheads_k, headdim), 42)
    heads = [0, 0, 1, 1]  # K/V head of each query head
    slopes = np.array([0.3, 0.1, 0.0, 0.2])
    for causal, wl, wr, al in [(False, -1, -1, None), (True, -1, -1, None), (True, 2, 0, slopes),
                               (False, 1, 2, slopes)]:
        out, lse = oracle.attention_varlen(q, k, v, cq, ck, 0.7, causal, wl, wr, al)
        assert out.shape == q.shape and lse.shape == (nheads, cq[-1])
        for b in range(len(lens_q)):
            if lens_q[b] == 0:
                continue
            rq, rk = slice(cq[b], cq[b + 1]), slice(ck[b], ck[b + 1])
            ob, lb = oracle.brute_force(q[None, rq], k[rk][:, heads][None], v[rk][:, heads][None], 0.7, causal,
                                        wl, wr, al)
            assert np.allclose(out[rq], ob[0], atol=1e-12)
            assert np.array_equal(np.isneginf(lse[:, rq]), np.isneginf(lb[0]))
            fin = np.isfinite(lb[0])
            assert np.allclose(lse[:, rq][fin], lb[0][fin], atol=1e-12)


BWD_MODES = [(False, -1, -1, None), (True, -1, -1, None), (True, 2, 0, [0.3, 0.05]), (False, 1, 2, [0.2, 0.7]),
             (False, -1, -1, [0.4, 0.0])]


def _loss(q, k, v, dout, scale, causal, wl, wr, al):
    out, _ = oracle.attention_forward(q, k, v, scale, causal, wl, wr, None if al is None else np.array(al))
    return float(np.sum(out * dout))


def pin_backward_finite_differences():
    """Every element of dq, dk, dv equals the central difference of sum(dout * out) with
    out from the (separately pinned) forward, in every mask mode; Sq > Sk leaves rows
    with no visible key under the causal mask."""
    eps = 1e-6
    for shape_q, shape_k in [((1, 4, 2, 3), (1, 6, 2, 3)), ((1, 5, 2, 3), (1, 3, 2, 3))]:
        q, k, v = rand(shape_q, 50), rand(shape_k, 51), rand(shape_k, 52)
        dout = rand(shape_q, 53)
        for causal, wl, wr, al in BWD_MODES:
            dq, dk, dv = oracle.attention_backward(q, k, v, dout, 0.6, causal, wl, wr,
                                                   None if al is None else np.array(al))
            for x, g in ((q, dq), (k, dk), (v, dv)):
                for idx in np.ndindex(*x.shape):
                    old = x[idx]
                    x[idx] = old + eps
                    up = _loss(q, k, v, dout, 0.6, causal, wl, wr, al)
                    x[idx] = old - eps
                    dn = _loss(q, k, v, dout, 0.6, causal, wl, wr, al)
                    x[idx] = old
                    fd = (up - dn) / (2 * eps)
                    assert abs(fd - g[idx]) <= 1e-7 * (1 + abs(fd)), (idx, fd, g[idx])


def pin_backward_autograd():
    """Square problems without window or ALiBi: torch autograd through
    scaled_dot_product_attention in fp64 on the CPU."""
    for causal in (False, True):
        q, k, v = (torch.tensor(rand((2, 3, 7, 5), s), requires_grad=True) for s in (54, 55, 56))
        dout = torch.tensor(rand((2, 3, 7, 5), 57))
        out = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal, scale=0.45)
        out.backward(dout)
        tr = lambda t: t.detach().numpy().transpose(0, 2, 1, 3)  # [B,H,S,D] -> [B,S,H,D]
        dq, dk, dv = oracle.attention_backward(tr(q), tr(k), tr(v), tr(dout), 0.45, causal)
        assert np.allclose(dq, tr(q.grad), atol=1e-12)
        assert np.allclose(dk, tr(k.grad), atol=1e-12)
        assert np.allclose(dv, tr(v.grad), atol=1e-12)


def pin_backward_closed_forms():
    """Rows of dS sum to zero, so the key gradients of every (batch, head) sum to zero;
    rows of P sum to one, so dV sums to the upstream gradient of the non-empty rows;
    scale 0 gives dq = dk = 0 and dv_j = sum over rows seeing j of dout_i / |visible_i|;
    rows with no visible key get dq = 0."""
    q, k, v, dout = rand((2, 6, 2, 4), 58), rand((2, 4, 2, 4), 59), rand((2, 4, 2, 4), 60), rand((2, 6, 2, 4), 61)
    for causal, wl, wr, al in BWD_MODES:
        al = None if al is None else np.array(al)
        dq, dk, dv = oracle.attention_backward(q, k, v, dout, 0.9, causal, wl, wr, al)
        keep = oracle.visible_mask(6, 4, causal, wl, wr)
        nonempty = keep.any(axis=1)
        assert np.allclose(dk.sum(axis=1), 0.0, atol=1e-12)
        assert np.allclose(dv.sum(axis=1), dout[:, nonempty].sum(axis=1), atol=1e-12)
        assert np.all(dq[:, ~nonempty] == 0)
        dq0, dk0, dv0 = oracle.attention_backward(q, k, v, dout, 0.0, causal, wl, wr)
        assert np.all(dq0 == 0) and np.all(dk0 == 0)
        cnt = np.maximum(keep.sum(axis=1), 1)
        expect = np.einsum("ij,bihd->bjhd", keep / cnt[:, None], dout)
        assert np.allclose(dv0, expect, atol=1e-13)


def _rot_complex(x, pos, cos, sin, rd):
    """Rotary as complex multiplication: (x_d + i x_{d+rd/2}) * (cos + i sin)."""
    half = rd // 2
    z = (x[..., :half] + 1j * x[..., half:rd]) * (cos[pos] + 1j * sin[pos])[:, None, :]
    y = np.array(x, dtype=np.float64, copy=True)
    y[..., :half], y[..., half:rd] = z.real, z.imag
    return y


def pin_kvcache(storage="bf16"):
    """KV-cache decode: rotary equals complex multiplication by e^{i theta}; a paged cache
    with a shuffled block table equals the contiguous cache; the result equals the scalar
    brute force on the explicitly gathered keys, with the new rows appended (rotated and
    rounded to the storage type when rotary tables are given); the appended rows are
    returned as stored."""
    rnd = oracle.round_bf16 if storage == "bf16" else oracle.round_fp16
    rng = np.random.default_rng(70)
    batch, sq, nh, nhk, d, page, rd = 3, 2, 4, 2, 8, 4, 6
    theta = rng.uniform(0, 2 * np.pi, (40, rd // 2))
    cos, sin = np.cos(theta), np.sin(theta)
    x = rand((5, 2, d), 71)
    assert np.allclose(oracle.rotary(x, np.arange(7, 12), cos, sin, rd), _rot_complex(x, np.arange(7, 12), cos, sin, rd),
                       atol=1e-14)
    lens = [5, 0, 9]
    cap = 12
    kc, vc = rand((batch, cap, nhk, d), 72), rand((batch, cap, nhk, d), 73)
    q = rand((batch, sq, nh, d), 74)
    knew, vnew = rand((batch, 2, nhk, d), 75), rand((batch, 2, nhk, d), 76)
    # the same cache, paged with 4-row blocks in shuffled physical order
    nblk = cap // page
    perm = rng.permutation(batch * nblk)
    kp, vp = np.zeros((batch * nblk, page, nhk, d)), np.zeros((batch * nblk, page, nhk, d))
    table = np.zeros((batch, nblk), dtype=np.int64)
    for b in range(batch):
        for n in range(nblk):
            table[b, n] = perm[b * nblk + n]
            kp[table[b, n]], vp[table[b, n]] = kc[b, n * page:(n + 1) * page], vc[b, n * page:(n + 1) * page]
    heads = [0, 0, 1, 1]
    for causal, wl, al, use_new, use_rot in [(True, -1, None, False, False), (True, 3, np.array([0.3, 0.1, 0.2, 0.05]),
                                                                              True, False),
                                             (False, -1, None, True, True), (True, -1, None, True, True)]:
        kw = dict(k_new=knew if use_new else None, v_new=vnew if use_new else None,
                  rotary_cos=cos if use_rot else None, rotary_sin=sin if use_rot else None, rotary_dim=rd,
                  causal=causal, window_left=wl, alibi_slopes=al, storage=storage)
        o1, l1, ka1, va1 = oracle.attention_kvcache(q, kc, vc, lens, 0.4, **kw)
        o2, l2, ka2, va2 = oracle.attention_kvcache(q, kp, vp, lens, 0.4, block_table=table, **kw)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
        for b in range(batch):
            kb, vb, qb = kc[b, :lens[b]], vc[b, :lens[b]], q[b]
            if use_new:
                kn = knew[b]
                if use_rot:
                    kn = rnd(_rot_complex(kn, lens[b] + np.arange(2), cos, sin, rd))
                assert np.array_equal(ka1[b], kn) and np.array_equal(va1[b], vnew[b])
                kb, vb = np.concatenate([kb, kn]), np.concatenate([vb, vnew[b]])
            if use_rot:
                qb = rnd(_rot_complex(qb, lens[b] + np.arange(sq), cos, sin, rd))
            ob, lb = oracle.brute_force(qb[None], kb[:, heads][None], vb[:, heads][None], 0.4, causal, wl, -1, al)
            assert np.allclose(o1[b], ob[0], atol=1e-12)
            assert np.array_equal(np.isneginf(l1[b]), np.isneginf(lb[0]))
            fin = np.isfinite(lb[0])
            assert np.allclose(l1[b][fin], lb[0][fin], atol=1e-12)


def pin_round_bf16():
    """Rounding to bf16 from first principles (8 exponent bits as in fp32, 7 stored
    mantissa bits), worked out by hand: spacing 2^-7 on [1, 2), ties to the even
    neighbour, a value just above a tie, a value whose rounding to fp32 first would
    create a false tie (1 + 2^-8 + 2^-40 must go up), negatives, the largest finite
    value (2 - 2^-7) * 2^127 with its overflow tie (2 - 2^-8) * 2^127 going to infinity,
    the subnormal spacing 2^-133 and the normal/subnormal boundary, and 0.1 (mantissa
    1.6 * 128 = 204.8 -> 205, i.e. 205 / 2048)."""
    big = (2 - 2.0 ** -7) * 2.0 ** 127
    tie_inf = (2 - 2.0 ** -8) * 2.0 ** 127
    cases = [(1 + 2.0 ** -8, 1.0), (1 + 3 * 2.0 ** -8, 1 + 2.0 ** -6), (1 + 2.0 ** -8 + 2.0 ** -30, 1 + 2.0 ** -7),
             (1 + 2.0 ** -8 + 2.0 ** -40, 1 + 2.0 ** -7), (1 + 2.0 ** -8 - 2.0 ** -30, 1.0),
             (-(1 + 2.0 ** -8), -1.0), (-(1 + 3 * 2.0 ** -8), -(1 + 2.0 ** -6)), (-(1 + 2.0 ** -8 + 2.0 ** -30),
                                                                               -(1 + 2.0 ** -7)),
             (3.0 + 2.0 ** -7, 3.0), (3.0 + 3 * 2.0 ** -7, 3.0 + 2.0 ** -5),
             (big, big), (tie_inf - 2.0 ** 100, big), (tie_inf, math.inf), (-tie_inf, -math.inf),
             (2.0 ** -133, 2.0 ** -133), (2.0 ** -134, 0.0), (3 * 2.0 ** -134, 2.0 ** -132),
             (2.0 ** -134 + 2.0 ** -160, 2.0 ** -133), (2.0 ** -126 - 2.0 ** -134, 2.0 ** -126),
             (2.0 ** -126 - 3 * 2.0 ** -134, 2.0 ** -126 - 2.0 ** -132),
             (0.1, 205.0 / 2048.0), (-0.1, -205.0 / 2048.0), (0.0, 0.0), (math.inf, math.inf)]
    x = np.array([c[0] for c in cases])
    got = oracle.round_bf16(x)
    want = np.array([c[1] for c in cases])
    assert np.array_equal(got, want), [(a, g, w) for a, g, w in zip(x, got, want) if g != w]
    assert np.isnan(oracle.round_bf16(np.array([math.nan]))[0])
    assert math.copysign(1.0, oracle.round_bf16(np.array([-0.0]))[0]) == -1.0
    # every value already on the bf16 grid is a fixed point (all 2^16 bit patterns but NaN)
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    pat = bits.view(np.float32)
    grid = pat[~np.isnan(pat)].astype(np.float64)
    assert np.array_equal(oracle.round_bf16(grid), grid)


def pin_round_fp16():
    """Rounding to IEEE binary16 from first principles: spacing 2^-10 on [1, 2), ties to
    the even neighbour, largest finite value 65504 (a tie at 65520 goes to infinity),
    subnormal spacing 2^-24."""
    cases = [(1 + 2.0 ** -11, 1.0), (1 + 3 * 2.0 ** -11, 1 + 2.0 ** -9), (1 + 2.0 ** -11 + 2.0 ** -30, 1 + 2.0 ** -10),
             (-(1 + 2.0 ** -11), -1.0), (65504.0, 65504.0), (65519.99, 65504.0), (65520.0, math.inf),
             (2.0 ** -25, 0.0), (3 * 2.0 ** -25, 2.0 ** -23), (2.0 ** -25 + 2.0 ** -40, 2.0 ** -24),
             (2.0 ** -14 - 2.0 ** -25, 2.0 ** -14), (0.1, 1638.0 / 16384.0)]
    x = np.array([c[0] for c in cases])
    assert np.array_equal(oracle.round_fp16(x), np.array([c[1] for c in cases]))


def pin_per_batch_slopes():
    """ALiBi slopes of shape (batch, nheads) [FA-overview §参数说明]: batch element (or packed
    sequence) b uses row b.  Checked against the scalar brute force, which reads the table
    on its own, and through every oracle entry that takes slopes; a table whose rows are
    all equal is the (nheads,) form."""
    rng = np.random.default_rng(80)
    B, Sq, Sk, H, D = 3, 5, 7, 2, 4
    q, k, v = rand((B, Sq, H, D), 81), rand((B, Sk, H, D), 82), rand((B, Sk, H, D), 83)
    sl = rng.uniform(0.05, 1.0, (B, H))

    def close(a, b, la, lb):
        assert np.allclose(a, b, atol=1e-12)
        assert np.array_equal(np.isneginf(la), np.isneginf(lb))
        fin = np.isfinite(lb)
        assert np.allclose(la[fin], lb[fin], atol=1e-12)

    for causal, wl in [(False, -1), (True, 2)]:
        o, l = oracle.attention_forward(q, k, v, 0.7, causal, wl, -1, sl)
        ob, lb = oracle.brute_force(q, k, v, 0.7, causal, wl, -1, sl)
        close(o, ob, l, lb)
        # split + combine, and sampled rows, with the same table
        oc, lc = oracle.combine(*oracle.splitkv_partials(q, k, v, 0.7, 3, causal, wl, -1, sl))
        close(oc, ob, lc, lb)
        samples = [(2, 1, 4), (0, 0, 0), (1, 1, 3)]
        os_, ls_ = oracle.attention_sampled(q, k, v, samples, 0.7, causal, wl, -1, sl)
        for n, (b, h, i) in enumerate(samples):
            close(os_[n], ob[b, i, h], ls_[n:n + 1], lb[b, h, i:i + 1])
    o_eq, _ = oracle.attention_forward(q, k, v, 0.7, True, -1, -1, np.tile(sl[1], (B, 1)))
    o_1d, _ = oracle.attention_forward(q, k, v, 0.7, True, -1, -1, sl[1])
    assert np.array_equal(o_eq, o_1d)

    # packed sequences: sequence b, of its own lengths, uses row b
    sq_b, sk_b = [5, 3, 0], [7, 2, 4]
    cu_q, cu_k = np.concatenate([[0], np.cumsum(sq_b)]), np.concatenate([[0], np.cumsum(sk_b)])
    qp = np.concatenate([q[b, :sq_b[b]] for b in range(B)])
    kp = np.concatenate([k[b, :sk_b[b]] for b in range(B)])
    vp = np.concatenate([v[b, :sk_b[b]] for b in range(B)])
    ov, lv = oracle.attention_varlen(qp, kp, vp, cu_q, cu_k, 0.7, True, -1, -1, sl)
    for b in range(B):
        if sq_b[b] == 0:
            continue
        ob, lb = oracle.brute_force(q[b:b + 1, :sq_b[b]], k[b:b + 1, :sk_b[b]], v[b:b + 1, :sk_b[b]], 0.7, True, -1,
                                    -1, sl[b])
        close(ov[cu_q[b]:cu_q[b + 1]], ob[0], lv[:, cu_q[b]:cu_q[b + 1]], lb[0])

    # backward: element b of the batch equals the (nheads,) form with row b alone
    g = rand((B, Sq, H, D), 84)
    dq, dk, dv = oracle.attention_backward(q, k, v, g, 0.7, True, -1, -1, sl)
    for b in range(B):
        ref = oracle.attention_backward(q[b:b + 1], k[b:b + 1], v[b:b + 1], g[b:b + 1], 0.7, True, -1, -1, sl[b])
        for x, r in zip((dq, dk, dv), ref):
            assert np.allclose(x[b], r[0], atol=1e-13)

    # KV cache (contiguous, grouped heads): brute force on each sequence's keys
    lens = [4, 0, 6]
    kc, vc = rand((B, 8, 1, D), 85), rand((B, 8, 1, D), 86)
    o, l, _, _ = oracle.attention_kvcache(q[:, :2], kc, vc, lens, 0.7, causal=True, alibi_slopes=sl)
    for b in range(B):
        ob, lb = oracle.brute_force(q[b:b + 1, :2], kc[b:b + 1, :lens[b], [0, 0]], vc[b:b + 1, :lens[b], [0, 0]], 0.7,
                                    True, -1, -1, sl[b])
        close(o[b], ob[0], l[b], lb[0])


def pin_bf16_widening():
    """bf16 inputs widen exactly: the oracle sees the very values the GPU gets."""
    t = torch.tensor([1.0, -2.5, 3.140625, 1e-3, 65280.0]).to(torch.bfloat16)
    w = oracle.as_f64(t)
    bits = t.view(torch.int16).numpy().astype(np.uint16).astype(np.uint32) << 16
    assert np.array_equal(w, bits.view(np.float32).astype(np.float64))


# --------------------------------------------------------------------------- tests


def test_causal_2x5_page_example():
    pin_causal_2x5()


def test_causal_5x2_zero_rows():
    pin_causal_5x2_zero_rows()


@pytest.mark.parametrize("causal,wl,wr,slopes", [
    (False, -1, -1, None), (True, -1, -1, None), (False, 2, 3, None), (True, 4, 0, np.array([0.3])),
    (False, -1, 1, np.array([1.5])),
])
def test_rows_sum_to_one(causal, wl, wr, slopes):
    pin_rows_sum_to_one(causal, wl, wr, slopes)


def test_constant_v():
    pin_constant_v()


def test_scale_zero():
    pin_scale_zero()


def test_window_zero():
    pin_window_zero()


def test_alibi_closed_form():
    pin_alibi_closed_form()


def test_sdpa_library():
    pin_sdpa_library()


@pytest.mark.parametrize("case", BRUTE_CASES)
def test_brute_force(case):
    pin_brute_force(case)


def test_invariants():
    pin_invariants()


def test_split_combine():
    pin_split_combine()


def test_sampled_rows():
    pin_sampled_rows()


def test_varlen_gqa():
    pin_varlen_gqa()


def test_backward_finite_differences():
    pin_backward_finite_differences()


def test_backward_autograd():
    pin_backward_autograd()


def test_backward_varlen_gqa():
    pin_backward_varlen_gqa()


def test_backward_closed_forms():
    pin_backward_closed_forms()


def test_kvcache():
    pin_kvcache()


def test_kvcache_fp16_storage():
    pin_kvcache("fp16")


def test_round_fp16():
    pin_round_fp16()


def test_round_bf16():
    pin_round_bf16()


def test_per_batch_slopes():
    pin_per_batch_slopes()


def test_bf16_widening():
    pin_bf16_widening()


def _torch_varlen_gqa_grads(q, k, v, dout, cq, ck, scale, causal, wl, wr, slopes):
    """Independent fp64 formulation: per sequence, each K/V head repeated for the query
    heads of its group, visibility written as index comparisons on the bottom-right
    aligned positions, softmax over the visible keys (rows without one give 0), and
    torch autograd for the gradients of sum(dout * out)."""
    qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    gt = torch.tensor(dout)
    group = q.shape[1] // k.shape[1]
    total = torch.zeros((), dtype=torch.float64)
    for b in range(len(cq) - 1):
        qs, gs = qt[cq[b]:cq[b + 1]], gt[cq[b]:cq[b + 1]]
        ks = kt[ck[b]:ck[b + 1]].repeat_interleave(group, dim=1)
        vs = vt[ck[b]:ck[b + 1]].repeat_interleave(group, dim=1)
        sq, sk = qs.shape[0], ks.shape[0]
        if sq == 0 or sk == 0:
            continue
        pos = torch.arange(sq)[:, None] + (sk - sq)
        key = torch.arange(sk)[None, :]
        vis = torch.ones(sq, sk, dtype=torch.bool)
        if wl >= 0:
            vis &= key >= pos - wl
        right = 0 if causal else wr
        if right >= 0:
            vis &= key <= pos + right
        s = torch.einsum("ihd,jhd->hij", qs, ks) * scale
        if slopes is not None:
            sl = torch.tensor(np.asarray(slopes, dtype=np.float64))
            sl = sl[b] if sl.dim() == 2 else sl
            s = s - sl[:, None, None] * (pos - key).abs().to(torch.float64)
        empty = ~vis.any(dim=1)
        s = s.masked_fill(~vis, float("-inf")).masked_fill(empty[:, None], 0.0)
        pr = torch.softmax(s, dim=-1) * vis
        out = torch.einsum("hij,jhd->ihd", pr, vs)
        total = total + (out * gs).sum()
    total.backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


def pin_backward_varlen_gqa():
    """Packed batch with grouped K/V heads (an empty query sequence, an empty key
    sequence, Sq > Sk and Sq < Sk sequences): the oracle's gradients equal torch
    autograd of an independent dense formulation, in every mask mode, with per-head
    and per-sequence ALiBi slopes; one tiny case also against central differences of
    the (separately pinned) packed forward."""
    nheads, nheads_k, headdim = 4, 2, 3
    lens_q, lens_k = [3, 0, 5, 2, 4], [5, 2, 3, 0, 4]
    cq, ck = np.concatenate([[0], np.cumsum(lens_q)]), np.concatenate([[0], np.cumsum(lens_k)])
    q, dout = rand((cq[-1], nheads, headdim), 62), rand((cq[-1], nheads, headdim), 63)
    k, v = rand((ck[-1], nheads_k, headdim), 64), rand((ck[-1], nheads_k, headdim), 65)
    per_head = np.array([0.3, 0.1, 0.0, 0.2])
    per_seq = np.array([[0.3, 0.1, 0.2, 0.05]] * 5) * np.arange(1, 6)[:, None] / 3
    for causal, wl, wr, al in [(False, -1, -1, None), (True, -1, -1, None), (True, 2, 0, per_head),
                               (False, 1, 2, per_seq), (False, -1, -1, per_head)]:
        got = oracle.attention_backward_varlen(q, k, v, dout, cq, ck, 0.8, causal, wl, wr, al)
        ref = _torch_varlen_gqa_grads(q, k, v, dout, cq, ck, 0.8, causal, wl, wr, al)
        for g, r in zip(got, ref):
            assert g.shape == r.shape
            assert np.allclose(g, r, atol=1e-12), float(np.abs(g - r).max())

    eps = 1e-6
    lq, lk = [2, 3], [3, 2]
    cq2, ck2 = np.concatenate([[0], np.cumsum(lq)]), np.concatenate([[0], np.cumsum(lk)])
    q2, g2 = rand((5, 2, 2), 66), rand((5, 2, 2), 67)
    k2, v2 = rand((5, 1, 2), 68), rand((5, 1, 2), 69)
    grads = oracle.attention_backward_varlen(q2, k2, v2, g2, cq2, ck2, 0.7, True, -1, -1, per_head[:2])
    loss = lambda: float(np.sum(oracle.attention_varlen(q2, k2, v2, cq2, ck2, 0.7, True, -1, -1, per_head[:2])[0]
                                * g2))
    for x, g in ((q2, grads[0]), (k2, grads[1]), (v2, grads[2])):
        for idx in np.ndindex(*x.shape):
            old = x[idx]
            x[idx] = old + eps
            up = loss()
            x[idx] = old - eps
            dn = loss()
            x[idx] = old
            fd = (up - dn) / (2 * eps)
            assert abs(fd - g[idx]) <= 1e-7 * (1 + abs(fd)), (idx, fd, g[idx])


# --------------------------------------------------------------------------- planted mistakes


def _all_pins():
    pin_causal_2x5()
    pin_causal_5x2_zero_rows()
    pin_rows_sum_to_one(True, 4, 0, np.array([0.3]))
    pin_constant_v()
    pin_scale_zero()
    pin_window_zero()
    pin_alibi_closed_form()
    pin_sdpa_library()
    for case in BRUTE_CASES:
        pin_brute_force(case)
    pin_invariants()
    pin_split_combine()
    pin_varlen_gqa()
    pin_backward_autograd()
    pin_backward_closed_forms()
    pin_backward_varlen_gqa()
    pin_kvcache()
    pin_kvcache("fp16")
    pin_round_fp16()
    pin_round_bf16()
    pin_per_batch_slopes()


def _top_left(i, seqlen_q, seqlen_k):
    return i


def _alibi_wrong_sign(slope, seqlen_q, seqlen_k, rows=None):
    return -_ORIG_ALIBI(slope, seqlen_q, seqlen_k, rows)


def _softmax_log2_lse(scores, keep):
    p, lse = _ORIG_SOFTMAX(scores, keep)
    return p, lse / math.log(2)


def _softmax_unmasked_max(scores, keep):
    # max taken over all keys, masked ones included: a plausible slip
    s = np.where(keep, scores, -np.inf)
    m = scores.max(axis=1)
    e = np.where(keep, np.exp(s - m[:, None]), 0.0)
    l = e.sum(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        p = np.nan_to_num(e / l[:, None])
        lse = np.where(l > 0, m + np.log(l), -np.inf)
    return p, lse


def _visible_exclusive_window(seqlen_q, seqlen_k, causal, window_left=-1, window_right=-1, rows=None):
    keep = _ORIG_VISIBLE(seqlen_q, seqlen_k, causal, window_left, window_right, rows)
    if window_left >= 0:
        i = np.arange(seqlen_q) if rows is None else np.asarray(rows)
        c = i + seqlen_k - seqlen_q
        j = np.arange(seqlen_k)
        keep &= ~(j[None, :] == (c - window_left)[:, None])
    return keep


def _combine_no_weights(out_partial, lse_partial):
    out, lse = _ORIG_COMBINE(out_partial, lse_partial)
    op = oa.as_f64(out_partial)
    return op.mean(axis=0).transpose(0, 2, 1, 3), lse


def _head_rows_bias_scaled(q_rows, k_head, v_head, rows, seqlen_q, softmax_scale, causal, window_left,
                           window_right, slope, key_range=None):
    # bias added before the scale instead of after it
    seqlen_k = k_head.shape[0]
    keep = oa.visible_mask(seqlen_q, seqlen_k, causal, window_left, window_right, rows)
    if key_range is not None:
        j = np.arange(seqlen_k)
        keep &= ((j >= key_range[0]) & (j < key_range[1]))[None, :]
    raw = q_rows @ k_head.T
    if slope is not None:
        raw = raw + oa.alibi_bias(slope, seqlen_q, seqlen_k, rows)
    p, lse = oa.softmax_rows(softmax_scale * raw, keep)
    return p @ v_head, lse


def _head_rows_k_for_v(q_rows, k_head, v_head, *args, **kwargs):
    # operands mixed up: keys used as values
    return _ORIG_HEAD_ROWS(q_rows, k_head, k_head, *args, **kwargs)


def _varlen_heads_modulo(q, k, v, cu_q, cu_k, *args, **kwargs):
    # query head h paired with K/V head h % H_k instead of h // (H / H_k)
    nheads, nheads_k = q.shape[1], k.shape[1]
    idx = [h % nheads_k for h in range(nheads)]
    return _ORIG_VARLEN(q, oa.as_f64(k)[:, idx], oa.as_f64(v)[:, idx], cu_q, cu_k, *args, **kwargs)


def _varlen_global_alignment(q, k, v, cu_q, cu_k, softmax_scale, causal=False, window_left=-1, window_right=-1,
                             alibi_slopes=None, row_chunk=512):
    # bottom-right alignment taken from the longest sequences instead of each sequence's own lengths
    cq, ck = np.asarray(cu_q), np.asarray(cu_k)
    sq_max, sk_max = int(np.diff(cq).max()), int(np.diff(ck).max())
    qd, kd, vd = oa.as_f64(q), oa.as_f64(k), oa.as_f64(v)
    out = np.zeros(qd.shape)
    lse = np.full((qd.shape[1], qd.shape[0]), -np.inf)
    group = qd.shape[1] // kd.shape[1]
    for b in range(len(cq) - 1):
        sq, sk = cq[b + 1] - cq[b], ck[b + 1] - ck[b]
        for h in range(qd.shape[1]):
            slope = None if alibi_slopes is None else float(alibi_slopes[h])
            rows = np.arange(sq) + (sq_max - sq)
            kh = np.concatenate([np.zeros((sk_max - sk, qd.shape[2])), kd[ck[b]:ck[b + 1], h // group]])
            vh = np.concatenate([np.zeros((sk_max - sk, qd.shape[2])), vd[ck[b]:ck[b + 1], h // group]])
            if sq == 0:
                continue
            o, l = oa.head_rows(qd[cq[b]:cq[b + 1], h], kh, vh, rows, sq_max, softmax_scale, causal, window_left,
                                window_right, slope)
            out[cq[b]:cq[b + 1], h] = o
            lse[h, cq[b]:cq[b + 1]] = l
    return out, lse


def _bwd_variant(drop_delta=False, unscaled_dk=False, dv_from_dp=False):
    def bwd(q, k, v, dout, softmax_scale, causal=False, window_left=-1, window_right=-1, alibi_slopes=None):
        qd, kd, vd, gd = oa.as_f64(q), oa.as_f64(k), oa.as_f64(v), oa.as_f64(dout)
        dq, dk, dv = np.zeros(qd.shape), np.zeros(kd.shape), np.zeros(vd.shape)
        sq, sk = qd.shape[1], kd.shape[1]
        keep = oa.visible_mask(sq, sk, causal, window_left, window_right)
        for b in range(qd.shape[0]):
            for h in range(qd.shape[2]):
                sc = softmax_scale * (qd[b, :, h] @ kd[b, :, h].T)
                if alibi_slopes is not None:
                    sc = sc + oa.alibi_bias(float(alibi_slopes[h]), sq, sk)
                p, _ = oa.softmax_rows(sc, keep)
                dp = gd[b, :, h] @ vd[b, :, h].T
                dv[b, :, h] = (dp if dv_from_dp else p).T @ gd[b, :, h]
                ds = p * dp if drop_delta else p * (dp - np.sum(p * dp, axis=1)[:, None])
                dq[b, :, h] = softmax_scale * (ds @ kd[b, :, h])
                dk[b, :, h] = (1.0 if unscaled_dk else softmax_scale) * (ds.T @ qd[b, :, h])
        return dq, dk, dv
    return bwd


def _bwd_varlen_variant(overwrite_kv=False, heads_modulo=False):
    def bwd(q, k, v, dout, cu_q, cu_k, softmax_scale, causal=False, window_left=-1, window_right=-1,
            alibi_slopes=None):
        qd, kd, vd, gd = oa.as_f64(q), oa.as_f64(k), oa.as_f64(v), oa.as_f64(dout)
        nheads, nk = qd.shape[1], kd.shape[1]
        slopes = oa.slope_table(alibi_slopes, len(cu_q) - 1, nheads)
        dq, dk, dv = np.zeros(qd.shape), np.zeros(kd.shape), np.zeros(vd.shape)
        for b in range(len(cu_q) - 1):
            q0, sq, k0, sk = cu_q[b], cu_q[b + 1] - cu_q[b], cu_k[b], cu_k[b + 1] - cu_k[b]
            if sq == 0 or sk == 0:
                continue
            rows = np.arange(sq)
            keep = oa.visible_mask(sq, sk, causal, window_left, window_right, rows)
            for h in range(nheads):
                hk = h % nk if heads_modulo else h // (nheads // nk)
                qh, gh, kh, vh = qd[q0:q0 + sq, h], gd[q0:q0 + sq, h], kd[k0:k0 + sk, hk], vd[k0:k0 + sk, hk]
                sc = softmax_scale * (qh @ kh.T)
                if slopes is not None:
                    sc = sc + oa.alibi_bias(float(slopes[b, h]), sq, sk, rows)
                p, _ = oa.softmax_rows(sc, keep)
                dp = gh @ vh.T
                ds = p * (dp - np.sum(p * dp, axis=1)[:, None])
                dq[q0:q0 + sq, h] = softmax_scale * (ds @ kh)
                if overwrite_kv:
                    dk[k0:k0 + sk, hk] = softmax_scale * (ds.T @ qh)
                    dv[k0:k0 + sk, hk] = p.T @ gh
                else:
                    dk[k0:k0 + sk, hk] += softmax_scale * (ds.T @ qh)
                    dv[k0:k0 + sk, hk] += p.T @ gh
        return dq, dk, dv
    return bwd


def _rotary_wrong_sign(x, positions, cos, sin, rotary_dim):
    return _ORIG_ROTARY(x, positions, cos, -sin, rotary_dim)


def _slopes_first_row(alibi_slopes, batch, nheads):
    # a (batch, nheads) table read as if every batch element had row 0
    t = _ORIG_SLOPES(alibi_slopes, batch, nheads)
    return None if t is None else np.tile(t[0], (batch, 1))


def _round_bf16_truncate(x):
    # toward zero: keep the top 16 bits of the fp32 pattern
    b = np.asarray(x, dtype=np.float64).astype(np.float32).view(np.uint32) & np.uint32(0xFFFF0000)
    return b.view(np.float32).astype(np.float64)


def _round_bf16_half_away(x):
    # ties away from zero instead of to even
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0)
    _, e2 = np.frexp(x[fin])
    sp = np.ldexp(1.0, (np.maximum(e2 - 1, -126) - 7).astype(np.int32))
    q = x[fin] / sp
    r = np.sign(q) * np.floor(np.abs(q) + 0.5) * sp
    out[fin] = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, x[fin]), r)
    return out


def _round_bf16_via_fp16(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def _round_bf16_via_fp32(x):
    # two roundings (fp64 -> fp32 -> bf16) instead of one
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()


def _round_fp16_via_bf16(x):
    return oa.round_bf16(x)


def _round_fp16_truncate(x):
    # toward zero instead of to nearest
    y = np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)
    over = np.abs(y) > np.abs(x)
    return np.where(over, np.nextafter(y.astype(np.float16), np.float16(0)).astype(np.float64), y)


_ORIG_HEAD_ROWS = oa.head_rows
_ORIG_ROTARY = oa.rotary
_ORIG_VARLEN = oa.attention_varlen
_ORIG_ALIBI = oa.alibi_bias
_ORIG_SOFTMAX = oa.softmax_rows
_ORIG_VISIBLE = oa.visible_mask
_ORIG_COMBINE = oa.combine
_ORIG_SLOPES = oa.slope_table


@pytest.mark.parametrize("target,replacement", [
    ("aligned_key_position", _top_left),
    ("alibi_bias", _alibi_wrong_sign),
    ("softmax_rows", _softmax_log2_lse),
    ("softmax_rows", _softmax_unmasked_max),
    ("visible_mask", _visible_exclusive_window),
    ("combine", _combine_no_weights),
    ("head_rows", _head_rows_bias_scaled),
    ("head_rows", _head_rows_k_for_v),
    ("attention_varlen", _varlen_heads_modulo),
    ("attention_varlen", _varlen_global_alignment),
    ("attention_backward", _bwd_variant(drop_delta=True)),
    ("attention_backward", _bwd_variant(unscaled_dk=True)),
    ("attention_backward", _bwd_variant(dv_from_dp=True)),
    ("attention_backward_varlen", _bwd_varlen_variant(overwrite_kv=True)),
    ("attention_backward_varlen", _bwd_varlen_variant(heads_modulo=True)),
    ("rotary", _rotary_wrong_sign),
    ("slope_table", _slopes_first_row),
    ("round_fp16", _round_fp16_via_bf16),
    ("round_fp16", _round_fp16_truncate),
    ("round_bf16", _round_bf16_truncate),
    ("round_bf16", _round_bf16_half_away),
    ("round_bf16", _round_bf16_via_fp16),
    ("round_bf16", _round_bf16_via_fp32),
])
def test_planted_mistake_is_caught(monkeypatch, target, replacement):
    """Each planted oracle mistake must make at least one pin fail."""
    _all_pins()  # unmodified oracle passes
    monkeypatch.setattr(oa, target, replacement)
    monkeypatch.setattr(oracle, target, replacement, raising=False)
    with pytest.raises(AssertionError):
        with np.errstate(all="ignore"):
            _all_pins()
