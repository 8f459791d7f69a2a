"""The library's launches under HIP graph capture: a decode step against a paged KV
cache (append + rotary, split partials, combine) and a forward are captured once and
replayed several times, with eager work and synchronisations between the replays;
every replay must reproduce the eager result bit for bit (the kernels are
deterministic and the cache append rewrites the same rows)."""

import math
import sys

import numpy as np
import pytest
import torch

import exact_attention_56_amd as fa
from exact_attention_56_amd.inputs import make_qkv

pytestmark = pytest.mark.gpu
DEV = "cuda"


def bits(t):
    return t.view(torch.int16) if t.dtype in (torch.bfloat16, torch.float16) else t.view(torch.int32)


def replay_matches(capture, outputs, expected, replays=3):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture
        capture()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        capture()
    for r in range(replays):
        for o in outputs:
            o.fill_(float("nan"))  # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for o, e in zip(outputs, expected):
            assert torch.equal(bits(o), bits(e)), f"replay {r} differs from the eager result"


def test_kvcache_decode_step_in_graph():
    print("[case] graph: paged kvcache decode step b2 h8/2 d128", file=sys.stderr, flush=True)
    g = torch.Generator(device="cpu").manual_seed(5)
    b, h, hk, d, page, blocks = 2, 8, 2, 128, 64, 8
    mk = lambda *shape: torch.randn(*shape, generator=g).to(torch.bfloat16).to(DEV)
    kc, vc = mk(b * blocks, page, hk, d), mk(b * blocks, page, hk, d)
    table = torch.randperm(b * blocks, generator=g).to(torch.int32).view(b, blocks).contiguous().to(DEV)
    lens = torch.tensor([300, 77], dtype=torch.int32, device=DEV)
    q, knew, vnew = mk(b, 1, h, d), mk(b, 1, hk, d), mk(b, 1, hk, d)
    theta = torch.rand(1024, d // 2, generator=g) * 2 * math.pi
    cos, sin = torch.cos(theta).to(DEV), torch.sin(theta).to(DEV)
    out = torch.empty_like(q)
    lse = torch.empty(b, h, 1, dtype=torch.float32, device=DEV)
    op = torch.empty(16, b, h, 1, d, dtype=torch.float32, device=DEV)
    lp = torch.empty(16, b, h, 1, dtype=torch.float32, device=DEV)
    scale = float(np.float32(1 / math.sqrt(d)))

    def step():
        fa.fwd_kvcache(q, kc, vc, lens, out, lse, op, lp, table, knew, vnew, cos, sin, scale, True)

    step()
    torch.cuda.synchronize()
    expected = (out.clone(), lse.clone())
    replay_matches(step, (out, lse), expected)


def test_forward_in_graph():
    print("[case] graph: forward b2 h4 s1000 d128 causal", file=sys.stderr, flush=True)
    q, k, v = (t.to(DEV) for t in make_qkv(2, 1000, 1000, 4, 128, seed=8))
    out = torch.empty_like(q)
    lse = torch.empty(2, 4, 1000, dtype=torch.float32, device=DEV)

    def fwd():
        fa.fwd(q, k, v, out, lse, None, True)

    fwd()
    torch.cuda.synchronize()
    expected = (out.clone(), lse.clone())
    replay_matches(fwd, (out, lse), expected)
