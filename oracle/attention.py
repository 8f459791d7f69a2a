"""fp64 CPU oracle for exact scaled-dot-product attention (forward), TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module.  The GPU library never calls it and shares no code with it: this
file is the plain definition written out, row by row, with a full-row softmax
(no tiling, no online rescaling), so that it can be checked against the pages
by eye.

Sources (the pages are web articles; each is cited by title and section):
  [FA-overview] "FlashAttention：快速且内存高效的准确注意力机制"
                (cloud.tencent.com.cn/developer/article/2433927)
    - section "使用示例": the method computes softmax(Q @ K^T * softmax_scale) @ V
      exactly (the title says "准确", exact).
    - section "参数说明": softmax_scale defaults to 1/sqrt(headdim); window_size
      (left, right), (-1, -1) = no window; alibi_slopes fp32 (nheads,) or
      (batch, nheads) add -slope * |i - j| to the score of query i and key j.
    - section "算法 / 前向传播": the forward also writes the row-wise
      logsumexp L, which the backward uses.
    - section "算法 / 反向传播": the backward recomputes P from L alone.
    - section "2.1：更改causal标志的行为": when seqlen_q != seqlen_k the causal
      mask is aligned to the bottom-right corner of the score matrix (2x5 example).
      A mask row with no kept entry gives a zero output row.
    - section "2.2：针对推理进行优化": for very short queries the keys are split
      across thread blocks and a separate kernel merges the partial results.
    - section "2.3：局部（即滑动窗口）注意力": sliding-window local attention.
    - section "2.5：分页KV缓存": the KV cache may be paged (a block table maps each
      sequence's logical blocks to physical ones); section "2.2" also names the
      KV-cache entry that rotates q and the new keys and appends to the cache in place.

Readings where the pages are silent (each one is a documented convention,
shared with the GPU library by specification only):
  * window bounds are inclusive, measured from the bottom-right-aligned key
    position c_i = i + seqlen_k - seqlen_q of query i: key j is visible iff
    (left < 0 or j >= c_i - left) and (right < 0 or j <= c_i + right);
    causal forces right = 0 (causal wins over a positive right window);
  * ALiBi uses the same aligned position, bias = -slope * |c_i - j|, and is
    added after the scores are multiplied by softmax_scale;
  * an empty row gives out = 0 and lse = -inf (log of an empty sum);
  * lse is the natural logarithm of sum_j exp(scale * q_i.k_j + bias_ij);
  * split s of num_splits covers keys [s*C, min(Sk, (s+1)*C)), C = ceil(Sk / num_splits),
    and its partial output is normalised within the split.

Every array here is float64; bf16 inputs are widened exactly before use.
"""

from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np


def as_f64(x) -> np.ndarray:
    """Exact widening of a torch/numpy array (bf16, fp16, fp32, fp64) to float64."""
    if hasattr(x, "detach"):  # torch tensor: widen inside torch, bf16 -> fp64 is exact
        import torch  # local import: the oracle itself is NumPy

        return x.detach().to(device="cpu", dtype=torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def slope_table(alibi_slopes, batch: int, nheads: int) -> Optional[np.ndarray]:
    """ALiBi slopes as a [batch, nheads] fp64 table [FA-overview §参数说明: the slopes are
    (nheads,), shared by every batch element, or (batch, nheads)], or None."""
    if alibi_slopes is None:
        return None
    sl = as_f64(alibi_slopes)
    if sl.ndim == 1:
        return np.tile(sl.reshape(1, nheads), (batch, 1))
    return sl.reshape(batch, nheads)


def aligned_key_position(i, seqlen_q: int, seqlen_k: int):
    """Bottom-right alignment [FA-overview §2.1]: query i sits at key position i + Sk - Sq."""
    return i + (seqlen_k - seqlen_q)


def visible_mask(seqlen_q: int, seqlen_k: int, causal: bool, window_left: int = -1,
                 window_right: int = -1, rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Boolean [len(rows), Sk]: True where query i may attend to key j.

    [FA-overview §2.1] bottom-right causal alignment; [§参数说明, §2.3] window
    (left, right) with -1 meaning unbounded on that side.  Causal sets the right
    side to 0.
    """
    if rows is None:
        rows = np.arange(seqlen_q)
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.arange(seqlen_k, dtype=np.int64)[None, :]
    c = aligned_key_position(i, seqlen_q, seqlen_k)
    right = 0 if causal else window_right
    keep = np.ones((i.shape[0], seqlen_k), dtype=bool)
    if window_left >= 0:
        keep &= j >= c - window_left
    if right >= 0:
        keep &= j <= c + right
    return keep


def alibi_bias(slope: float, seqlen_q: int, seqlen_k: int, rows: Optional[np.ndarray] = None) -> np.ndarray:
    """[len(rows), Sk] bias -slope * |c_i - j| [FA-overview §参数说明 (alibi_slopes), §2.4]."""
    if rows is None:
        rows = np.arange(seqlen_q)
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.arange(seqlen_k, dtype=np.int64)[None, :]
    c = aligned_key_position(i, seqlen_q, seqlen_k)
    return -float(slope) * np.abs(c - j).astype(np.float64)


def softmax_rows(scores: np.ndarray, keep: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Full-row softmax over the kept entries of each row.

    Returns (P, lse): P[r, j] = exp(s_rj - m_r) / l_r on kept entries and 0
    elsewhere, lse_r = m_r + ln l_r with m_r the row max over kept entries.
    A row with no kept entry has P = 0 and lse = -inf [FA-overview §2.1].
    """
    s = np.where(keep, scores, -np.inf)
    m = s.max(axis=1) if s.shape[1] > 0 else np.full(s.shape[0], -np.inf)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.where(keep, np.exp(s - m_safe[:, None]), 0.0)
    l = e.sum(axis=1)
    p = np.where(empty[:, None], 0.0, e / np.where(empty, 1.0, l)[:, None])
    lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, l)))
    return p, lse


def head_rows(q_rows: np.ndarray, k_head: np.ndarray, v_head: np.ndarray, rows: np.ndarray,
              seqlen_q: int, softmax_scale: float, causal: bool, window_left: int,
              window_right: int, slope: Optional[float],
              key_range: Optional[Tuple[int, int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Attention for some query rows of one (batch, head).

    q_rows [R, D] (the rows listed in ``rows``), k_head/v_head [Sk, D], all fp64.
    s_ij = softmax_scale * q_i . k_j + bias_ij [FA-overview §使用示例, §参数说明];
    out_i = sum_j P_ij v_j; lse_i = ln sum_j exp(s_ij).  ``key_range`` = (lo, hi)
    further restricts the visible keys to lo <= j < hi (one split of the keys).
    """
    seqlen_k = k_head.shape[0]
    keep = visible_mask(seqlen_q, seqlen_k, causal, window_left, window_right, rows)
    if key_range is not None:
        lo, hi = key_range
        j = np.arange(seqlen_k)
        keep &= ((j >= lo) & (j < hi))[None, :]
    scores = softmax_scale * (q_rows @ k_head.T)
    if slope is not None:
        scores = scores + alibi_bias(slope, seqlen_q, seqlen_k, rows)
    p, lse = softmax_rows(scores, keep)
    return p @ v_head, lse


def attention_forward(q, k, v, softmax_scale: float, causal: bool = False, window_left: int = -1,
                      window_right: int = -1, alibi_slopes=None,
                      row_chunk: int = 512) -> Tuple[np.ndarray, np.ndarray]:
    """Full forward: q [B,Sq,H,D], k/v [B,Sk,H,D] -> out [B,Sq,H,D], lse [B,H,Sq] (fp64).

    Rows are independent, so they are processed in chunks of ``row_chunk``; no
    arithmetic changes with the chunking.
    """
    qd, kd, vd = as_f64(q), as_f64(k), as_f64(v)
    batch, seqlen_q, nheads, headdim = qd.shape
    slopes = slope_table(alibi_slopes, batch, nheads)
    out = np.zeros((batch, seqlen_q, nheads, headdim))
    lse = np.zeros((batch, nheads, seqlen_q))
    for b in range(batch):
        for h in range(nheads):
            kh, vh = kd[b, :, h, :], vd[b, :, h, :]
            slope = None if slopes is None else float(slopes[b, h])
            for r0 in range(0, seqlen_q, row_chunk):
                rows = np.arange(r0, min(seqlen_q, r0 + row_chunk))
                o, l = head_rows(qd[b, rows, h, :], kh, vh, rows, seqlen_q, softmax_scale, causal,
                                 window_left, window_right, slope)
                out[b, rows, h, :] = o
                lse[b, h, rows] = l
    return out, lse


def attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, softmax_scale: float, causal: bool = False,
                     window_left: int = -1, window_right: int = -1, alibi_slopes=None,
                     row_chunk: int = 512) -> Tuple[np.ndarray, np.ndarray]:
    """Packed batch of sequences with grouped K/V heads, fp64.

    [FA-overview §代码解读：FlashSelfAttention, §代码解读博客：FlashCrossAttention,
    §函数重命名]: sequence b is rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 of q and
    rows cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1 of k and v, and is an attention
    problem of its own (its own lengths for the causal alignment, windows and ALiBi).
    K/V carry H_k heads (H_k divides H); query head h reads K/V head h // (H // H_k).
    q [total_q, H, D], k/v [total_k, H_k, D] -> out [total_q, H, D], lse [H, total_q].
    """
    qd, kd, vd = as_f64(q), as_f64(k), as_f64(v)
    cq = [int(x) for x in np.asarray(cu_seqlens_q).reshape(-1)]
    ck = [int(x) for x in np.asarray(cu_seqlens_k).reshape(-1)]
    total_q, nheads, headdim = qd.shape
    group = nheads // kd.shape[1]
    slopes = slope_table(alibi_slopes, len(cq) - 1, nheads)  # one row per sequence when (batch, nheads)
    out = np.zeros((total_q, nheads, headdim))
    lse = np.full((nheads, total_q), -np.inf)
    for b in range(len(cq) - 1):
        q0, sq = cq[b], cq[b + 1] - cq[b]
        k0, sk = ck[b], ck[b + 1] - ck[b]
        for h in range(nheads):
            kh, vh = kd[k0:k0 + sk, h // group, :], vd[k0:k0 + sk, h // group, :]
            slope = None if slopes is None else float(slopes[b, h])
            for r0 in range(0, sq, row_chunk):
                rows = np.arange(r0, min(sq, r0 + row_chunk))
                o, l = head_rows(qd[q0 + rows, h, :], kh, vh, rows, sq, softmax_scale, causal, window_left,
                                 window_right, slope)
                out[q0 + rows, h, :] = o
                lse[h, q0 + rows] = l
    return out, lse


def attention_backward(q, k, v, dout, softmax_scale: float, causal: bool = False, window_left: int = -1,
                       window_right: int = -1, alibi_slopes=None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Exact gradients of out = attention(q, k, v) for an upstream gradient dout, fp64.

    [FA-overview §算法 / 反向传播]: the backward needs only the row-wise logsumexp L of
    the forward; P is recomputed as exp(S - L).  Per (batch, head), with S the scaled
    and biased scores and P = exp(S - L) on the visible pairs (0 elsewhere):
      dV = P^T dO,   dP = dO V^T,   D_i = sum_j P_ij dP_ij (= dO_i . O_i),
      dS = P o (dP - D),   dQ = scale * dS K,   dK = scale * dS^T Q.
    The bias (mask, ALiBi) is a constant: it has no gradient here.
    q [B,Sq,H,D], k/v [B,Sk,H,D], dout [B,Sq,H,D] -> dq, dk, dv with the shapes of q, k, v.
    """
    qd, kd, vd, gd = as_f64(q), as_f64(k), as_f64(v), as_f64(dout)
    batch, seqlen_q, nheads, headdim = qd.shape
    seqlen_k = kd.shape[1]
    slopes = slope_table(alibi_slopes, batch, nheads)
    dq, dk, dv = np.zeros(qd.shape), np.zeros(kd.shape), np.zeros(vd.shape)
    rows = np.arange(seqlen_q)
    keep = visible_mask(seqlen_q, seqlen_k, causal, window_left, window_right, rows)
    for b in range(batch):
        for h in range(nheads):
            qh, kh, vh, gh = qd[b, :, h], kd[b, :, h], vd[b, :, h], gd[b, :, h]
            scores = softmax_scale * (qh @ kh.T)
            if slopes is not None:
                scores = scores + alibi_bias(float(slopes[b, h]), seqlen_q, seqlen_k, rows)
            p, _ = softmax_rows(scores, keep)
            dv[b, :, h] = p.T @ gh
            dp = gh @ vh.T
            d_row = np.sum(p * dp, axis=1)
            ds = p * (dp - d_row[:, None])
            dq[b, :, h] = softmax_scale * (ds @ kh)
            dk[b, :, h] = softmax_scale * (ds.T @ qh)
    return dq, dk, dv


def attention_backward_varlen(q, k, v, dout, cu_seqlens_q, cu_seqlens_k, softmax_scale: float,
                              causal: bool = False, window_left: int = -1, window_right: int = -1,
                              alibi_slopes=None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Exact gradients for a packed batch of sequences with grouped K/V heads, fp64.

    [FA-overview §算法 / 反向传播] on each sequence's own rows ([FA-overview
    §代码解读：FlashSelfAttention, §代码解读博客：FlashCrossAttention]: sequence b is rows
    cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 of q and dout and rows cu_seqlens_k[b] ..
    cu_seqlens_k[b+1]-1 of k and v, with its own lengths for the masks).  Per sequence and
    query head h the formulas of attention_backward apply with K/V head h // (H / H_k); the
    forward reads that K/V head once for every query head of its group, so its dk and dv are
    the sums over the group.
    q, dout [total_q, H, D], k/v [total_k, H_k, D] -> dq, dk, dv with the shapes of q, k, v.
    """
    qd, kd, vd, gd = as_f64(q), as_f64(k), as_f64(v), as_f64(dout)
    cq = [int(x) for x in np.asarray(cu_seqlens_q).reshape(-1)]
    ck = [int(x) for x in np.asarray(cu_seqlens_k).reshape(-1)]
    nheads = qd.shape[1]
    group = nheads // kd.shape[1]
    slopes = slope_table(alibi_slopes, len(cq) - 1, nheads)
    dq, dk, dv = np.zeros(qd.shape), np.zeros(kd.shape), np.zeros(vd.shape)
    for b in range(len(cq) - 1):
        q0, sq = cq[b], cq[b + 1] - cq[b]
        k0, sk = ck[b], ck[b + 1] - ck[b]
        if sq == 0 or sk == 0:  # no (query, key) pair: every gradient of the sequence stays 0
            continue
        rows = np.arange(sq)
        keep = visible_mask(sq, sk, causal, window_left, window_right, rows)
        for h in range(nheads):
            hk = h // group
            qh, gh = qd[q0:q0 + sq, h], gd[q0:q0 + sq, h]
            kh, vh = kd[k0:k0 + sk, hk], vd[k0:k0 + sk, hk]
            scores = softmax_scale * (qh @ kh.T)
            if slopes is not None:
                scores = scores + alibi_bias(float(slopes[b, h]), sq, sk, rows)
            p, _ = softmax_rows(scores, keep)
            dp = gh @ vh.T
            ds = p * (dp - np.sum(p * dp, axis=1)[:, None])
            dq[q0:q0 + sq, h] = softmax_scale * (ds @ kh)
            dk[k0:k0 + sk, hk] += softmax_scale * (ds.T @ qh)
            dv[k0:k0 + sk, hk] += p.T @ gh
    return dq, dk, dv


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to bf16 in one step (round to nearest, ties to even), returned
    as fp64: the precision of the cache and of the operands the kernels multiply.

    bf16 keeps fp32's 8 exponent bits and 7 stored mantissa bits.  A value of binary
    exponent e (2^e <= |x| < 2^(e+1)) therefore sits on a grid of spacing 2^(e-7),
    and below the smallest normal 2^-126 on the subnormal grid 2^-133.  The quotient
    x / spacing is exact in fp64 (a power-of-two scaling), numpy's rint rounds it to
    the nearest integer with ties to even, and the product is exact again.  A result
    of magnitude 2^128 or more lies past the largest finite bf16 (2 - 2^-7) * 2^127,
    so it becomes infinity; zeros, infinities and NaN pass through.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0)
    xf = x[fin]
    _, e2 = np.frexp(xf)  # xf = m * 2^e2 with 0.5 <= |m| < 1, so e = e2 - 1
    e = np.maximum(e2.astype(np.int64) - 1, -126)
    spacing = np.ldexp(1.0, (e - 7).astype(np.int32))
    r = np.rint(xf / spacing) * spacing
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, xf), r)
    out[fin] = r
    return out


def round_fp16(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to IEEE binary16 (round to nearest, ties to even; overflow to
    inf, gradual underflow), returned as fp64: the fp16 counterpart of round_bf16."""
    with np.errstate(over="ignore"):  # overflow to inf is the IEEE result
        return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)



def rotary(x: np.ndarray, positions: np.ndarray, cos: np.ndarray, sin: np.ndarray, rotary_dim: int) -> np.ndarray:
    """Rotary position embedding, half-split layout, fp64: for d < rotary_dim / 2 the pair
    (x_d, x_{d + rotary_dim/2}) of the row at position p is rotated by the angle whose
    cosine and sine are cos[p, d], sin[p, d]; columns from rotary_dim on are unchanged.
    x [..., S, H, D] with positions [S]."""
    half = rotary_dim // 2
    c = cos[positions][:, None, :]  # [S, 1, half]
    s = sin[positions][:, None, :]
    y = np.array(x, dtype=np.float64, copy=True)
    x1, x2 = x[..., :half], x[..., half:rotary_dim]
    y[..., :half] = x1 * c - x2 * s
    y[..., half:rotary_dim] = x2 * c + x1 * s
    return y


def attention_kvcache(q, k_cache, v_cache, cache_seqlens, softmax_scale: float, block_table=None, k_new=None,
                      v_new=None, rotary_cos=None, rotary_sin=None, rotary_dim: int = 0, causal: bool = False,
                      window_left: int = -1, window_right: int = -1, alibi_slopes=None, storage: str = "bf16"):
    """Decode against a KV cache, fp64 [FA-overview §2.2 (KV-cache decoding: rotary embedding,
    in-place cache update), §2.5 (paged KV cache)].

    q [B, Sq, H, D]; k_cache, v_cache [num_blocks, page, H_k, D] with block_table [B, blocks]
    (logical block n of sequence b is physical block block_table[b, n]), or [B, capacity, H_k, D]
    with block_table None.  Sequence b holds cache_seqlens[b] keys; the new rows k_new, v_new
    [B, S_new, H_k, D] are appended at positions cache_seqlens[b] .. + S_new - 1.  With rotary
    tables, q row i and new key row i are rotated at position cache_seqlens[b] + i and rounded
    to the storage type `storage` ("bf16" or "fp16": the cache stores it and the kernels
    multiply operands of that type).  Query head h reads
    K/V head h // (H / H_k).  Returns out [B, Sq, H, D], lse [B, H, Sq], and the appended key
    and value rows as stored [B, S_new, H_k, D] (None without new rows).
    """
    qd, kc, vc = as_f64(q), as_f64(k_cache), as_f64(v_cache)
    lens = [int(x) for x in np.asarray(cache_seqlens).reshape(-1)]
    batch, seqlen_q, nheads, headdim = qd.shape
    nheads_k = kc.shape[2]
    group = nheads // nheads_k
    page = kc.shape[1]
    kn = None if k_new is None else as_f64(k_new)
    vn = None if v_new is None else as_f64(v_new)
    snew = 0 if kn is None else kn.shape[1]
    use_rot = rotary_cos is not None
    if use_rot:
        cos, sin = as_f64(rotary_cos), as_f64(rotary_sin)
    out = np.zeros(qd.shape)
    lse = np.zeros((batch, nheads, seqlen_q))
    k_app = None if kn is None else np.zeros(kn.shape)
    v_app = None if vn is None else np.zeros(vn.shape)
    heads = [h // group for h in range(nheads)]
    slopes = slope_table(alibi_slopes, batch, nheads)
    rnd = {"bf16": round_bf16, "fp16": round_fp16}[storage]  # looked up per call
    for b in range(batch):
        rows = []
        for j in range(lens[b]):  # the cached keys, through the block table
            if block_table is None:
                rows.append((b, j))
            else:
                rows.append((int(block_table[b][j // page]), j % page))
        kb = np.array([kc[blk, r] for blk, r in rows]).reshape(lens[b], nheads_k, headdim)
        vb = np.array([vc[blk, r] for blk, r in rows]).reshape(lens[b], nheads_k, headdim)
        if snew:
            knb, vnb = kn[b], vn[b]
            if use_rot:
                knb = rnd(rotary(knb, lens[b] + np.arange(snew), cos, sin, rotary_dim))
            k_app[b], v_app[b] = knb, vnb
            kb, vb = np.concatenate([kb, knb]), np.concatenate([vb, vnb])
        qb = qd[b]
        if use_rot:
            qb = rnd(rotary(qb, lens[b] + np.arange(seqlen_q), cos, sin, rotary_dim))
        o, l = attention_forward(qb[None], kb[:, heads][None], vb[:, heads][None], softmax_scale, causal,
                                 window_left, window_right, None if slopes is None else slopes[b:b + 1])
        out[b], lse[b] = o[0], l[0]
    return out, lse, k_app, v_app


def attention_sampled(q, k, v, samples: Iterable[Tuple[int, int, int]], softmax_scale: float,
                      causal: bool = False, window_left: int = -1, window_right: int = -1,
                      alibi_slopes=None) -> Tuple[np.ndarray, np.ndarray]:
    """Oracle for a list of (b, h, i) output rows only: out [n, D], lse [n].

    Same definition as attention_forward, evaluated for the sampled rows; used
    where the full problem is too large for the CPU.  Each (b, h) slice of K/V
    is widened to fp64 once.
    """
    samples = list(samples)
    seqlen_q, headdim = q.shape[1], q.shape[3]
    slopes = slope_table(alibi_slopes, q.shape[0], q.shape[2])
    out = np.zeros((len(samples), headdim))
    lse = np.zeros(len(samples))
    groups = {}
    for n, (b, h, i) in enumerate(samples):
        groups.setdefault((b, h), []).append((n, i))
    for (b, h), items in groups.items():
        kh, vh = as_f64(k[b, :, h, :]), as_f64(v[b, :, h, :])
        rows = np.array([i for _, i in items], dtype=np.int64)
        qr = as_f64(q[b, :, h, :])[rows]
        slope = None if slopes is None else float(slopes[b, h])
        o, l = head_rows(qr, kh, vh, rows, seqlen_q, softmax_scale, causal, window_left, window_right, slope)
        for r, (n, _) in enumerate(items):
            out[n] = o[r]
            lse[n] = l[r]
    return out, lse


def split_bounds(seqlen_k: int, num_splits: int) -> Sequence[Tuple[int, int]]:
    """Key range of each split: [s*C, min(Sk, (s+1)*C)), C = ceil(Sk / num_splits)."""
    chunk = -(-seqlen_k // num_splits)
    return [(min(seqlen_k, s * chunk), min(seqlen_k, (s + 1) * chunk)) for s in range(num_splits)]


def splitkv_partials(q, k, v, softmax_scale: float, num_splits: int, causal: bool = False,
                     window_left: int = -1, window_right: int = -1,
                     alibi_slopes=None) -> Tuple[np.ndarray, np.ndarray]:
    """Per-split partial results [FA-overview §2.2]: each split attends only to its own keys.

    Returns out_partial [S,B,H,Sq,D] (normalised within the split) and
    lse_partial [S,B,H,Sq]; a split with no visible key gives 0 and -inf.
    """
    qd, kd, vd = as_f64(q), as_f64(k), as_f64(v)
    batch, seqlen_q, nheads, headdim = qd.shape
    seqlen_k = kd.shape[1]
    slopes = slope_table(alibi_slopes, batch, nheads)
    out_p = np.zeros((num_splits, batch, nheads, seqlen_q, headdim))
    lse_p = np.zeros((num_splits, batch, nheads, seqlen_q))
    rows = np.arange(seqlen_q)
    for s, key_range in enumerate(split_bounds(seqlen_k, num_splits)):
        for b in range(batch):
            for h in range(nheads):
                slope = None if slopes is None else float(slopes[b, h])
                o, l = head_rows(qd[b, :, h, :], kd[b, :, h, :], vd[b, :, h, :], rows, seqlen_q,
                                 softmax_scale, causal, window_left, window_right, slope, key_range)
                out_p[s, b, h] = o
                lse_p[s, b, h] = l
    return out_p, lse_p


def combine(out_partial, lse_partial) -> Tuple[np.ndarray, np.ndarray]:
    """Merge split results [FA-overview §2.2].

    With L = ln sum_s exp(lse_s): out = sum_s exp(lse_s - L) * out_s, lse = L.
    If every split is empty (all lse_s = -inf) the row gives out = 0, lse = -inf.
    Input out_partial [S,B,H,Sq,D], lse_partial [S,B,H,Sq]; returns
    out [B,Sq,H,D] and lse [B,H,Sq].
    """
    op = as_f64(out_partial)
    lp = as_f64(lse_partial)
    m = lp.max(axis=0)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.exp(lp - m_safe[None])  # exp(-inf) = 0 for empty splits
    total = w.sum(axis=0)
    lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, total)))
    wn = np.where(empty[None], 0.0, w / np.where(empty, 1.0, total)[None])
    out = (wn[..., None] * op).sum(axis=0)  # [B,H,Sq,D]
    return out.transpose(0, 2, 1, 3).copy(), lse


def brute_force(q, k, v, softmax_scale: float, causal: bool = False, window_left: int = -1,
                window_right: int = -1, alibi_slopes=None):
    """Scalar pure-Python loops (math.exp, math.fsum) for tiny shapes.

    Written independently of the NumPy path above: the visibility test and the
    bias are spelled out per (i, j) from the same stated conventions.
    """
    qd, kd, vd = as_f64(q), as_f64(k), as_f64(v)
    batch, seqlen_q, nheads, headdim = qd.shape
    seqlen_k = kd.shape[1]
    slopes = None
    if alibi_slopes is not None:
        arr = as_f64(alibi_slopes)
        # (nheads,): every batch element uses the same slopes; (batch, nheads): row b
        slopes = [[float(x) for x in (arr if arr.ndim == 1 else arr[b])] for b in range(batch)]
    out = [[[[0.0] * headdim for _ in range(nheads)] for _ in range(seqlen_q)] for _ in range(batch)]
    lse = [[[0.0] * seqlen_q for _ in range(nheads)] for _ in range(batch)]
    for b in range(batch):
        for h in range(nheads):
            for i in range(seqlen_q):
                pos = i + seqlen_k - seqlen_q
                scores = {}
                for j in range(seqlen_k):
                    if window_left >= 0 and j < pos - window_left:
                        continue
                    if causal and j > pos:
                        continue
                    if (not causal) and window_right >= 0 and j > pos + window_right:
                        continue
                    dot = math.fsum(qd[b, i, h, d] * kd[b, j, h, d] for d in range(headdim))
                    s = softmax_scale * dot
                    if slopes is not None:
                        s -= slopes[b][h] * abs(pos - j)
                    scores[j] = s
                if not scores:
                    lse[b][h][i] = -math.inf
                    continue
                mx = max(scores.values())
                weights = {j: math.exp(s - mx) for j, s in scores.items()}
                total = math.fsum(weights.values())
                lse[b][h][i] = mx + math.log(total)
                for d in range(headdim):
                    out[b][i][h][d] = math.fsum(w * vd[b, j, h, d] for j, w in weights.items()) / total
    return np.array(out), np.array(lse)
