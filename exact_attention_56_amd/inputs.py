"""Seeded synthetic inputs for the attention forward workloads.

This module only draws random tensors and describes workload shapes; it holds
none of the attention arithmetic.  Both the GPU path and the fp64 CPU oracle are
fed from here, so the two sides always see bit-identical bf16 inputs.

Recipe (the pages give shapes, not data): Q, K, V are iid N(0, 1) drawn in fp32
from ``torch.Generator('cpu').manual_seed(seed)`` in the order q, k, v, then
rounded to bf16 with round-to-nearest-even.  Layout is contiguous
[batch, seqlen, nheads, headdim] (the page "FlashAttention：快速且内存高效的准确注意力机制",
section "参数说明", gives q/k/v as (batch_size, seqlen, nheads, headdim)).
ALiBi slopes follow the geometric recipe 2^(-8 (i+1) / nheads), fp32, one per head.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention forward workload (shapes and mask options, no data)."""

    name: str
    batch: int
    nheads: int
    seqlen_q: int
    seqlen_k: int
    headdim: int
    causal: bool = False
    window_left: int = -1
    window_right: int = -1
    alibi: bool = False
    num_splits: int = 0  # >0: split-KV decode pair (partial kernel + combine)
    seed: int = 0

    @property
    def softmax_scale(self) -> float:
        """Default scale 1/sqrt(headdim), rounded to the fp32 value the kernels receive."""
        return float(torch.tensor(1.0 / math.sqrt(self.headdim), dtype=torch.float32))


# The five workloads the method is checked and timed on.  Seeds 0..4 follow the
# list order; the causal and non-causal variants of the benchmark shape share
# one seed (same tensors).
WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 128, 128, 64, seed=0),
    "bench_s2048": Workload("bench_s2048", 8, 16, 2048, 2048, 128, seed=1),
    "bench_s2048_causal": Workload("bench_s2048_causal", 8, 16, 2048, 2048, 128, causal=True, seed=1),
    "local_alibi_s8192": Workload("local_alibi_s8192", 2, 32, 8192, 8192, 64, causal=True,
                                  window_left=1024, window_right=0, alibi=True, seed=2),
    "hd256_s16384": Workload("hd256_s16384", 1, 8, 16384, 16384, 256, seed=3),
    "decode_s32768": Workload("decode_s32768", 8, 16, 1, 32768, 128, causal=True, num_splits=16, seed=4),
}


def sweep_workload(seqlen: int, causal: bool = False) -> Workload:
    """The pages' benchmark recipe: hidden 2048 = 16 heads x 128, batch = 16384 / seqlen."""
    return Workload(f"sweep_s{seqlen}{'_causal' if causal else ''}", 16384 // seqlen, 16,
                    seqlen, seqlen, 128, causal=causal, seed=1)


def make_qkv(batch: int, seqlen_q: int, seqlen_k: int, nheads: int, headdim: int, seed: int,
             nheads_k: Optional[int] = None, device: str = "cpu", dtype: torch.dtype = torch.bfloat16):
    """Draw q [B,Sq,H,D], k and v [B,Sk,H,D] from one seeded generator: N(0, 1) in fp32,
    rounded to `dtype` (bf16 or fp16, nearest even).

    device="cpu" (the default) gives the tensors the oracle and the parity tests
    use.  A GPU device draws from that device's generator instead: same
    distribution and seed, different values; it only serves timing runs.
    """
    hk = nheads if nheads_k is None else nheads_k
    g = torch.Generator(device=device).manual_seed(seed)

    def draw(*shape):
        return torch.randn(*shape, generator=g, dtype=torch.float32, device=device).to(dtype)

    q = draw(batch, seqlen_q, nheads, headdim)
    k = draw(batch, seqlen_k, hk, headdim)
    v = draw(batch, seqlen_k, hk, headdim)
    return q, k, v


def make_alibi_slopes(nheads: int, batch: Optional[int] = None) -> torch.Tensor:
    """fp32 slopes 2^(-8 (i+1) / nheads), i = 0..nheads-1, shape (nheads,); with `batch`,
    a (batch, nheads) table whose row b is that row times 2^(-b/4)."""
    row = [2.0 ** (-8.0 * (i + 1) / nheads) for i in range(nheads)]
    if batch is None:
        return torch.tensor(row, dtype=torch.float32)
    return torch.tensor([[x * 2.0 ** (-b / 4.0) for x in row] for b in range(batch)], dtype=torch.float32)


def workload_inputs(w: Workload):
    """(q, k, v, alibi_slopes or None) for a workload, all on the CPU."""
    q, k, v = make_qkv(w.batch, w.seqlen_q, w.seqlen_k, w.nheads, w.headdim, w.seed)
    slopes = make_alibi_slopes(w.nheads) if w.alibi else None
    return q, k, v, slopes


@dataclasses.dataclass(frozen=True)
class VarlenWorkload:
    """A packed batch of sequences (self-attention, q and k share the lengths) with
    grouped K/V heads."""

    name: str
    lengths: tuple
    nheads: int
    nheads_k: int
    headdim: int
    causal: bool = True
    seed: int = 6

    @property
    def softmax_scale(self) -> float:
        return float(torch.tensor(1.0 / math.sqrt(self.headdim), dtype=torch.float32))


def varlen_lengths(count: int, lo: int, hi: int, seed: int) -> tuple:
    """`count` sequence lengths drawn uniformly from [lo, hi] by a seeded generator."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    return tuple(int(x) for x in torch.randint(lo, hi + 1, (count,), generator=g))


# 16 sequences of 256..4096 tokens, 32 query heads sharing 8 K/V heads, headdim 128, causal.
VARLEN_GQA = VarlenWorkload("varlen_gqa_causal", varlen_lengths(16, 256, 4096, seed=6), 32, 8, 128)


def make_varlen_qkv(w: VarlenWorkload, device: str = "cpu"):
    """q [total, H, D], k and v [total, H_k, D] bf16 (same recipe as make_qkv, drawn
    as one long sequence) and cu_seqlens int32 [len(lengths) + 1]."""
    total = sum(w.lengths)
    q, k, v = make_qkv(1, total, total, w.nheads, w.headdim, w.seed, nheads_k=w.nheads_k, device=device)
    cu = torch.tensor([0] + list(_cumsum(w.lengths)), dtype=torch.int32, device=device)
    return q[0], k[0], v[0], cu


def _cumsum(xs):
    s = 0
    for x in xs:
        s += x
        yield s
