"""MI355X (gfx950) exact attention: thin Python binding over libfa_mi355x.so.

The binding only marshals arguments: it checks dtypes, devices, shapes and
contiguity, allocates outputs with torch when asked to, and passes raw device
pointers and torch's current HIP stream to the C ABI declared in include/fa.h.
Every step of the computation runs in the library's HIP kernels; there is no
other implementation to fall back to.  A missing library raises at the first call.
q/k/v (and out, the gradients and the KV cache) are torch.bfloat16 or torch.float16,
all of one type; alibi_slopes are fp32 of shape (nheads,) or (batch, nheads).

Functions
  flash_attn_func(q, k, v, softmax_scale=None, causal=False, window_size=(-1, -1),
                  alibi_slopes=None) -> (out, lse)
  fwd(q, k, v, out, lse, ...)                      preallocated outputs
  flash_attn_varlen_func(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, ...)
                                                   packed sequences, grouped K/V heads
  fwd_varlen(q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k, ...)
  fwd_splitkv(q, k, v, out_partial, lse_partial, num_splits, ...)
  combine(out_partial, lse_partial, out, lse)
  decode(q, k_cache, v_cache, num_splits=16, ...) -> (out, lse)
  kvcache_decode(q, k_cache, v_cache, cache_seqlens, ...) -> (out, lse)   KV-cache decode step
  fwd_kvcache_noalloc(q, k_cache, v_cache, cache_seqlens, out, lse, ...)  the same step, no allocation
  bwd(q, k, v, out, lse, dout, dq, dk, dv, delta, ...)   gradients into preallocated tensors
  attention_backward(q, k, v, out, lse, dout, ...) -> (dq, dk, dv)
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

_LIB = None
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa_mi355x.so")

FA_OK = 0
FA_BF16 = 0
FA_FP16 = 1
_DTYPES = {torch.bfloat16: FA_BF16, torch.float16: FA_FP16}


class FAError(RuntimeError):
    """A non-zero status returned by the C library."""


def load_library() -> ctypes.CDLL:
    """Load libfa_mi355x.so (built in-tree) and declare its C signatures."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                           "(python -m exact_attention_56_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    # every alibi_slopes pointer is followed by alibi_per_batch and dtype
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, vp, i, i, vp]
    lib.fa_fwd.restype = i
    lib.fa_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, vp, i, i, i, vp]
    lib.fa_fwd_splitkv.restype = i
    lib.fa_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, i, i, vp, i, i, vp]
    lib.fa_fwd_varlen.restype = i
    lib.fa_fwd_kvcache.argtypes = [vp, vp, vp, vp, vp, i, i, vp, vp, i, vp, vp, i, vp, vp, vp, vp, i, i, i, i, i,
                                   i, f, i, i, i, vp, i, i, i, vp]
    lib.fa_fwd_kvcache.restype = i
    lib.fa_fwd_kvcache_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, vp, vp, i, vp, vp, i, vp, vp, i, i, i, i, i, f,
                                           i, i, i, vp, i, i, i, vp]
    lib.fa_fwd_kvcache_noalloc.restype = i
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, vp, i, i, vp]
    lib.fa_bwd.restype = i
    lib.fa_bwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, i, i,
                                  i, vp, i, i, vp]
    lib.fa_bwd_varlen.restype = i
    lib.fa_combine.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, vp]
    lib.fa_combine.restype = i
    lib.fa_status_str.argtypes = [i]
    lib.fa_status_str.restype = ctypes.c_char_p
    _LIB = lib
    return lib


def _check(status: int) -> None:
    if status != FA_OK:
        msg = load_library().fa_status_str(status).decode()
        raise FAError(f"libfa_mi355x returned {status}: {msg}")


def _stream_handle(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _require(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: int, device=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _dtype_code(t: torch.Tensor, name: str) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in _DTYPES:
        raise TypeError(f"{name} must be torch.bfloat16 or torch.float16, got {t.dtype}")
    return _DTYPES[t.dtype]


def _check_qkv(q, k, v):
    _dtype_code(q, "q")
    for t, name in ((k, "k"), (v, "v")):
        if isinstance(t, torch.Tensor) and t.dtype != q.dtype:
            raise TypeError(f"{name} must have q's dtype {q.dtype}, got {t.dtype}")
    _require(q, "q", q.dtype, 4)
    _require(k, "k", q.dtype, 4, q.device)
    _require(v, "v", q.dtype, 4, q.device)
    b, sq, h, d = q.shape
    if k.shape != v.shape:
        raise ValueError(f"k {tuple(k.shape)} and v {tuple(v.shape)} differ")
    if k.shape[0] != b or k.shape[2] != h or k.shape[3] != d:
        raise ValueError(f"k/v shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    return b, sq, k.shape[1], h, d


def _alibi(alibi_slopes, batch, nheads, device):
    """(slopes, alibi_per_batch) for slopes of shape (nheads,) or (batch, nheads)."""
    if alibi_slopes is None:
        return None, 0
    _require(alibi_slopes, "alibi_slopes", torch.float32, alibi_slopes.dim(), device)
    if tuple(alibi_slopes.shape) == (nheads,):
        return alibi_slopes, 0
    if tuple(alibi_slopes.shape) == (batch, nheads):
        return alibi_slopes, 1
    raise ValueError(f"alibi_slopes must have shape ({nheads},) or ({batch}, {nheads})")


def _scale(softmax_scale, headdim) -> float:
    return 1.0 / math.sqrt(headdim) if softmax_scale is None else float(softmax_scale)


def fwd(q, k, v, out, lse, softmax_scale=None, causal=False, window_size=(-1, -1),
        alibi_slopes=None) -> None:
    """fa_fwd on preallocated out [B,Sq,H,D] (q's dtype) and lse [B,H,Sq] fp32."""
    b, sq, sk, h, d = _check_qkv(q, k, v)
    _require(out, "out", q.dtype, 4, q.device)
    _require(lse, "lse", torch.float32, 3, q.device)
    if out.shape != q.shape or tuple(lse.shape) != (b, h, sq):
        raise ValueError("out must match q and lse must be [batch, nheads, seqlen_q]")
    slopes, per_batch = _alibi(alibi_slopes, b, h, q.device)
    _check(load_library().fa_fwd(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), b, sq, sk, h, d,
        _scale(softmax_scale, d), int(bool(causal)), int(window_size[0]), int(window_size[1]),
        _ptr(slopes), per_batch, _DTYPES[q.dtype], _stream_handle(q)))


def flash_attn_func(q, k, v, softmax_scale=None, causal=False, window_size=(-1, -1),
                    alibi_slopes=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Attention forward; returns (out [B,Sq,H,D] in q's dtype, lse [B,H,Sq] fp32)."""
    b, sq, sk, h, d = _check_qkv(q, k, v)
    out = torch.empty_like(q)
    lse = torch.empty(b, h, sq, dtype=torch.float32, device=q.device)
    fwd(q, k, v, out, lse, softmax_scale, causal, window_size, alibi_slopes)
    return out, lse


def fwd_varlen(q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
               softmax_scale=None, causal=False, window_size=(-1, -1), alibi_slopes=None) -> None:
    """fa_fwd_varlen on preallocated out [total_q,H,D] (q's dtype) and lse [H,total_q] fp32.

    q [total_q, H, D], k/v [total_k, H_k, D] (H_k divides H), cu_seqlens_* int32 [batch+1]
    on the same device.  The cumulative lengths are read by the kernel only: they must
    lie inside the tensors (see fa_fwd_varlen in include/fa.h).
    """
    _dtype_code(q, "q")
    _require(q, "q", q.dtype, 3)
    _require(k, "k", q.dtype, 3, q.device)
    _require(v, "v", q.dtype, 3, q.device)
    _require(out, "out", q.dtype, 3, q.device)
    _require(lse, "lse", torch.float32, 2, q.device)
    _require(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1, q.device)
    _require(cu_seqlens_k, "cu_seqlens_k", torch.int32, 1, q.device)
    total_q, h, d = q.shape
    hk = k.shape[1]
    if k.shape != v.shape or k.shape[2] != d:
        raise ValueError(f"k {tuple(k.shape)} and v {tuple(v.shape)} must be [total_k, H_k, {d}]")
    if hk < 1 or h % hk != 0:
        raise ValueError(f"K/V heads ({hk}) must divide query heads ({h})")
    if out.shape != q.shape or tuple(lse.shape) != (h, total_q):
        raise ValueError("out must match q and lse must be [nheads, total_q]")
    if cu_seqlens_q.shape != cu_seqlens_k.shape or cu_seqlens_q.shape[0] < 2:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both be [batch + 1]")
    batch = cu_seqlens_q.shape[0] - 1
    slopes, per_batch = _alibi(alibi_slopes, batch, h, q.device)
    _check(load_library().fa_fwd_varlen(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), cu_seqlens_q.data_ptr(),
        cu_seqlens_k.data_ptr(), batch, int(max_seqlen_q), int(max_seqlen_k), total_q, h, hk, d,
        _scale(softmax_scale, d), int(bool(causal)), int(window_size[0]), int(window_size[1]), _ptr(slopes),
        per_batch, _DTYPES[q.dtype], _stream_handle(q)))


def flash_attn_varlen_func(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, softmax_scale=None,
                           causal=False, window_size=(-1, -1), alibi_slopes=None):
    """Packed-sequence forward; returns (out [total_q,H,D] in q's dtype, lse [H,total_q] fp32)."""
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[1], q.shape[0], dtype=torch.float32, device=q.device)
    fwd_varlen(q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, softmax_scale, causal,
               window_size, alibi_slopes)
    return out, lse


def fwd_splitkv(q, k, v, out_partial, lse_partial, num_splits, softmax_scale=None, causal=False,
                window_size=(-1, -1), alibi_slopes=None) -> None:
    """fa_fwd_splitkv: out_partial [S,B,H,Sq,D] fp32, lse_partial [S,B,H,Sq] fp32."""
    b, sq, sk, h, d = _check_qkv(q, k, v)
    _require(out_partial, "out_partial", torch.float32, 5, q.device)
    _require(lse_partial, "lse_partial", torch.float32, 4, q.device)
    if tuple(out_partial.shape) != (num_splits, b, h, sq, d) or tuple(lse_partial.shape) != (num_splits, b, h, sq):
        raise ValueError("partials must be [num_splits, B, H, Sq, D] and [num_splits, B, H, Sq]")
    slopes, per_batch = _alibi(alibi_slopes, b, h, q.device)
    _check(load_library().fa_fwd_splitkv(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out_partial.data_ptr(), lse_partial.data_ptr(),
        b, sq, sk, h, d, _scale(softmax_scale, d), int(bool(causal)), int(window_size[0]),
        int(window_size[1]), _ptr(slopes), per_batch, _DTYPES[q.dtype], int(num_splits), _stream_handle(q)))


def combine(out_partial, lse_partial, out, lse) -> None:
    """fa_combine: merge [S,B,H,Sq,D] / [S,B,H,Sq] partials into out [B,Sq,H,D] (bf16 or fp16),
    lse [B,H,Sq]."""
    _require(out_partial, "out_partial", torch.float32, 5)
    _require(lse_partial, "lse_partial", torch.float32, 4, out_partial.device)
    _dtype_code(out, "out")
    _require(out, "out", out.dtype, 4, out_partial.device)
    _require(lse, "lse", torch.float32, 3, out_partial.device)
    s, b, h, sq, d = out_partial.shape
    if tuple(lse_partial.shape) != (s, b, h, sq) or tuple(out.shape) != (b, sq, h, d) or tuple(lse.shape) != (b, h, sq):
        raise ValueError("inconsistent shapes for combine")
    _check(load_library().fa_combine(out_partial.data_ptr(), lse_partial.data_ptr(), out.data_ptr(),
                                     lse.data_ptr(), b, sq, h, d, s, _DTYPES[out.dtype], _stream_handle(out)))


def decode(q, k_cache, v_cache, num_splits=16, softmax_scale=None, causal=False, window_size=(-1, -1),
           alibi_slopes=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Split-KV forward (partials + combine on the current stream); returns (out, lse)."""
    b, sq, sk, h, d = _check_qkv(q, k_cache, v_cache)
    op = torch.empty(num_splits, b, h, sq, d, dtype=torch.float32, device=q.device)
    lp = torch.empty(num_splits, b, h, sq, dtype=torch.float32, device=q.device)
    fwd_splitkv(q, k_cache, v_cache, op, lp, num_splits, softmax_scale, causal, window_size, alibi_slopes)
    out = torch.empty_like(q)
    lse = torch.empty(b, h, sq, dtype=torch.float32, device=q.device)
    combine(op, lp, out, lse)
    return out, lse


def bwd(q, k, v, out, lse, dout, dq, dk, dv, delta, softmax_scale=None, causal=False, window_size=(-1, -1),
        alibi_slopes=None) -> None:
    """fa_bwd: gradients into preallocated dq/dk/dv (q's dtype, shapes of q/k/v); delta [B,H,Sq]
    fp32 is scratch.  out and lse must be the forward's outputs for the same arguments."""
    b, sq, sk, h, d = _check_qkv(q, k, v)
    for t, name, like in ((out, "out", q), (dout, "dout", q), (dq, "dq", q), (dk, "dk", k), (dv, "dv", v)):
        _require(t, name, q.dtype, 4, q.device)
        if t.shape != like.shape:
            raise ValueError(f"{name} must have shape {tuple(like.shape)}")
    _require(lse, "lse", torch.float32, 3, q.device)
    _require(delta, "delta", torch.float32, 3, q.device)
    if tuple(lse.shape) != (b, h, sq) or tuple(delta.shape) != (b, h, sq):
        raise ValueError("lse and delta must be [batch, nheads, seqlen_q]")
    slopes, per_batch = _alibi(alibi_slopes, b, h, q.device)
    _check(load_library().fa_bwd(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), dout.data_ptr(), dq.data_ptr(),
        dk.data_ptr(), dv.data_ptr(), delta.data_ptr(), b, sq, sk, h, d, _scale(softmax_scale, d),
        int(bool(causal)), int(window_size[0]), int(window_size[1]), _ptr(slopes), per_batch, _DTYPES[q.dtype],
        _stream_handle(q)))


def attention_backward(q, k, v, out, lse, dout, softmax_scale=None, causal=False, window_size=(-1, -1),
                       alibi_slopes=None):
    """Gradients (dq, dk, dv) of flash_attn_func's out for the upstream gradient dout."""
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty(q.shape[0], q.shape[2], q.shape[1], dtype=torch.float32, device=q.device)
    bwd(q, k, v, out, lse, dout, dq, dk, dv, delta, softmax_scale, causal, window_size, alibi_slopes)
    return dq, dk, dv


def bwd_varlen(q, k, v, out, lse, dout, dq, dk, dv, delta, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
               softmax_scale=None, causal=False, window_size=(-1, -1), alibi_slopes=None) -> None:
    """fa_bwd_varlen: gradients of fwd_varlen into preallocated dq [total_q,H,D] and dk/dv
    [total_k,H_k,D] (q's dtype); delta [H,total_q] fp32 is scratch.  out and lse must be the
    forward's outputs for the same arguments; the cumulative lengths are read by the kernels
    only (see fa_bwd_varlen in include/fa.h)."""
    _dtype_code(q, "q")
    _require(q, "q", q.dtype, 3)
    for t, name, like in ((k, "k", k), (v, "v", k), (out, "out", q), (dout, "dout", q), (dq, "dq", q),
                          (dk, "dk", k), (dv, "dv", k)):
        _require(t, name, q.dtype, 3, q.device)
        if t.shape != like.shape:
            raise ValueError(f"{name} must have shape {tuple(like.shape)}")
    total_q, h, d = q.shape
    total_k, hk = k.shape[0], k.shape[1]
    if k.shape[2] != d:
        raise ValueError(f"k and v must be [total_k, H_k, {d}]")
    if hk < 1 or h % hk != 0:
        raise ValueError(f"K/V heads ({hk}) must divide query heads ({h})")
    _require(lse, "lse", torch.float32, 2, q.device)
    _require(delta, "delta", torch.float32, 2, q.device)
    if tuple(lse.shape) != (h, total_q) or tuple(delta.shape) != (h, total_q):
        raise ValueError("lse and delta must be [nheads, total_q]")
    _require(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1, q.device)
    _require(cu_seqlens_k, "cu_seqlens_k", torch.int32, 1, q.device)
    if cu_seqlens_q.shape != cu_seqlens_k.shape or cu_seqlens_q.shape[0] < 2:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both be [batch + 1]")
    batch = cu_seqlens_q.shape[0] - 1
    slopes, per_batch = _alibi(alibi_slopes, batch, h, q.device)
    _check(load_library().fa_bwd_varlen(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), dout.data_ptr(), dq.data_ptr(),
        dk.data_ptr(), dv.data_ptr(), delta.data_ptr(), cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), batch,
        int(max_seqlen_q), int(max_seqlen_k), total_q, total_k, h, hk, d, _scale(softmax_scale, d),
        int(bool(causal)), int(window_size[0]), int(window_size[1]), _ptr(slopes), per_batch, _DTYPES[q.dtype],
        _stream_handle(q)))


def attention_varlen_backward(q, k, v, out, lse, dout, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                              softmax_scale=None, causal=False, window_size=(-1, -1), alibi_slopes=None):
    """Gradients (dq, dk, dv) of flash_attn_varlen_func's out for the upstream gradient dout."""
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty(q.shape[1], q.shape[0], dtype=torch.float32, device=q.device)
    bwd_varlen(q, k, v, out, lse, dout, dq, dk, dv, delta, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
               softmax_scale, causal, window_size, alibi_slopes)
    return dq, dk, dv


def kvcache_decode(q, k_cache, v_cache, cache_seqlens, block_table=None, k_new=None, v_new=None, rotary_cos=None,
                   rotary_sin=None, softmax_scale=None, causal=False, window_size=(-1, -1), alibi_slopes=None,
                   num_splits=0, max_splits=64):
    """fa_fwd_kvcache: appends k_new/v_new (rotated with the rotary tables if given) to the
    cache in place, then attends.  q [B,Sq,H,D]; k_cache/v_cache [num_blocks, page, H_k, D]
    with block_table [B, max_blocks] int32, or [B, capacity, H_k, D] without; cache_seqlens
    [B] int32.  Returns (out [B,Sq,H,D] in q's dtype, lse [B,H,Sq] fp32)."""
    b, sq, h, d = q.shape
    out = torch.empty_like(q)
    lse = torch.empty(b, h, sq, dtype=torch.float32, device=q.device)
    op = torch.empty(max_splits, b, h, sq, d, dtype=torch.float32, device=q.device)
    lp = torch.empty(max_splits, b, h, sq, dtype=torch.float32, device=q.device)
    fwd_kvcache(q, k_cache, v_cache, cache_seqlens, out, lse, op, lp, block_table, k_new, v_new, rotary_cos,
                rotary_sin, softmax_scale, causal, window_size, alibi_slopes, num_splits)
    return out, lse


def _kvcache_common(q, k_cache, v_cache, cache_seqlens, out, lse, block_table, k_new, v_new, rotary_cos,
                    rotary_sin, alibi_slopes):
    """Checks shared by the KV-cache entry points; returns (b, sq, h, d, hk, page,
    max_blocks, snew, rd, slopes, per_batch)."""
    _dtype_code(q, "q")
    _require(q, "q", q.dtype, 4)
    _require(k_cache, "k_cache", q.dtype, 4, q.device)
    _require(v_cache, "v_cache", q.dtype, 4, q.device)
    _require(cache_seqlens, "cache_seqlens", torch.int32, 1, q.device)
    b, sq, h, d = q.shape
    if k_cache.shape != v_cache.shape or k_cache.shape[3] != d:
        raise ValueError("k_cache and v_cache must match and end in headdim")
    hk, page = k_cache.shape[2], k_cache.shape[1]
    if cache_seqlens.shape[0] != b:
        raise ValueError("cache_seqlens must be [batch]")
    max_blocks = 1
    if block_table is not None:
        _require(block_table, "block_table", torch.int32, 2, q.device)
        if block_table.shape[0] != b:
            raise ValueError("block_table must be [batch, max_blocks]")
        max_blocks = block_table.shape[1]
    elif k_cache.shape[0] != b:
        raise ValueError("a contiguous cache must be [batch, capacity, H_k, D]")
    snew = 0
    if k_new is not None:
        _require(k_new, "k_new", q.dtype, 4, q.device)
        _require(v_new, "v_new", q.dtype, 4, q.device)
        if k_new.shape != v_new.shape or k_new.shape[0] != b or k_new.shape[2] != hk or k_new.shape[3] != d:
            raise ValueError("k_new and v_new must be [batch, seqlen_new, H_k, D]")
        snew = k_new.shape[1]
    rd = 0
    if rotary_cos is not None:
        _require(rotary_cos, "rotary_cos", torch.float32, 2, q.device)
        _require(rotary_sin, "rotary_sin", torch.float32, 2, q.device)
        if rotary_sin.shape != rotary_cos.shape:
            raise ValueError("rotary_cos and rotary_sin must have the same shape [positions, rotary_dim / 2]")
        # one row per cache position: rows cache_seqlens[b] + i are read for every
        # appended key and query, and the positions reach the capacity at most
        capacity = page * max_blocks
        if rotary_cos.shape[0] < capacity:
            raise ValueError(f"rotary tables need a row for every cache position ({capacity}), "
                             f"got {rotary_cos.shape[0]}")
        rd = 2 * rotary_cos.shape[1]
    slopes, per_batch = _alibi(alibi_slopes, b, h, q.device)
    _require(out, "out", q.dtype, 4, q.device)
    _require(lse, "lse", torch.float32, 3, q.device)
    if out.shape != q.shape or tuple(lse.shape) != (b, h, sq):
        raise ValueError("out/lse do not match q")
    return b, sq, h, d, hk, page, max_blocks, snew, rd, slopes, per_batch


def fwd_kvcache(q, k_cache, v_cache, cache_seqlens, out, lse, out_partial, lse_partial, block_table=None, k_new=None,
                v_new=None, rotary_cos=None, rotary_sin=None, softmax_scale=None, causal=False, window_size=(-1, -1),
                alibi_slopes=None, num_splits=0) -> None:
    """fa_fwd_kvcache with preallocated out [B,Sq,H,D], lse [B,H,Sq] and split scratch
    out_partial [S,B,H,Sq,D] / lse_partial [S,B,H,Sq] (fp32; S = max_splits)."""
    b, sq, h, d, hk, page, max_blocks, snew, rd, slopes, per_batch = _kvcache_common(
        q, k_cache, v_cache, cache_seqlens, out, lse, block_table, k_new, v_new, rotary_cos, rotary_sin, alibi_slopes)
    _require(out_partial, "out_partial", torch.float32, 5, q.device)
    _require(lse_partial, "lse_partial", torch.float32, 4, q.device)
    max_splits = out_partial.shape[0]
    if tuple(out_partial.shape[1:]) != (b, h, sq, d) or tuple(lse_partial.shape) != (max_splits, b, h, sq):
        raise ValueError("the partials do not match q")
    _check(load_library().fa_fwd_kvcache(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), cache_seqlens.data_ptr(), _ptr(block_table), page,
        max_blocks, _ptr(k_new), _ptr(v_new), snew, _ptr(rotary_cos), _ptr(rotary_sin), rd, out.data_ptr(),
        lse.data_ptr(), out_partial.data_ptr(), lse_partial.data_ptr(), int(max_splits), b, sq, h, hk, d,
        _scale(softmax_scale, d), int(bool(causal)), int(window_size[0]), int(window_size[1]), _ptr(slopes), per_batch,
        _DTYPES[q.dtype], int(num_splits), _stream_handle(q)))


def fwd_kvcache_noalloc(q, k_cache, v_cache, cache_seqlens, out, lse, block_table=None, k_new=None, v_new=None,
                        rotary_cos=None, rotary_sin=None, softmax_scale=None, causal=False, window_size=(-1, -1),
                        alibi_slopes=None, num_splits=0) -> None:
    """fa_fwd_kvcache_noalloc: fwd_kvcache with the split partials in the library's own
    device buffer (no allocation by the call; overlapping calls on one GPU race)."""
    b, sq, h, d, hk, page, max_blocks, snew, rd, slopes, per_batch = _kvcache_common(
        q, k_cache, v_cache, cache_seqlens, out, lse, block_table, k_new, v_new, rotary_cos, rotary_sin, alibi_slopes)
    _check(load_library().fa_fwd_kvcache_noalloc(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), cache_seqlens.data_ptr(), _ptr(block_table), page,
        max_blocks, _ptr(k_new), _ptr(v_new), snew, _ptr(rotary_cos), _ptr(rotary_sin), rd, out.data_ptr(),
        lse.data_ptr(), b, sq, h, hk, d, _scale(softmax_scale, d), int(bool(causal)), int(window_size[0]),
        int(window_size[1]), _ptr(slopes), per_batch, _DTYPES[q.dtype], int(num_splits), _stream_handle(q)))
