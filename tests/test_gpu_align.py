"""Planner parity on the GPU: moe_align through the C ABI must equal the
oracle's alignment bit for bit (all three outputs, over the whole capacity)."""

import numpy as np
import pytest
import torch

import datagen
import mixture_experts_ffn_moe_amd as moe
from oracle.align import align_ref

from .gpu_helpers import say

pytestmark = pytest.mark.gpu


def _routing(kind, T, E, k, seed):
    g = torch.Generator().manual_seed(seed)
    if kind == "uniform":
        ids, _ = datagen.make_routing(T, E, k, "uniform", tag=f"al{seed}")
    elif kind == "zipf":
        ids, _ = datagen.make_routing(T, E, k, "zipf", tag=f"al{seed}")
    elif kind == "masked":
        ids, _ = datagen.make_routing(T, E, k, "normal_masked", tag=f"al{seed}", n_masked=8)
    elif kind == "one":
        ids = torch.randint(0, E, (T, k), generator=g, dtype=torch.int32)
        ids[:, 0] = 3
    elif kind == "oor":
        ids = torch.randint(-3, E + 3, (T, k), generator=g, dtype=torch.int32)
    else:
        raise ValueError(kind)
    return ids.to(torch.int32)


CASES = [
    ("uniform", 0, 8, 2), ("uniform", 1, 8, 2), ("uniform", 37, 8, 2),
    ("uniform", 8, 256, 6), ("uniform", 256, 256, 6), ("masked", 1024, 288, 8),
    ("zipf", 4096, 384, 6), ("one", 300, 16, 4), ("oor", 500, 10, 3),
    ("uniform", 8192, 288, 8), ("uniform", 512, 32, 8), ("uniform", 50, 1024, 4),
]


SENTINEL = 0x7F7F7F7F


def _outputs(T, k, E, bm, S=0):
    """Planner outputs pre-filled with a sentinel: the planner must write
    every element of the capacity (ids, -1 padding and the count)."""
    rows, blocks = moe.moe_align_capacity(T, k + S, E + S, bm)
    return (torch.full((max(rows, 1),), SENTINEL, dtype=torch.int32, device="cuda")[:rows],
            torch.full((max(blocks, 1),), SENTINEL, dtype=torch.int32, device="cuda")[:blocks],
            torch.full((1,), SENTINEL, dtype=torch.int32, device="cuda"))


@pytest.mark.parametrize("bm", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("kind,T,E,k", CASES)
def test_align_bit_exact(kind, T, E, k, bm):
    say(f"[gpu] align kind={kind} T={T} E={E} k={k} bm={bm}")
    ids = _routing(kind, T, E, k, T * 7 + E)
    s_ref, e_ref, n_ref = align_ref(ids.numpy(), E, bm)
    s, e, n = moe.moe_align(ids.cuda(), E, bm, out=_outputs(T, k, E, bm), workspace=None)
    torch.cuda.synchronize()
    assert int(n.item()) == n_ref
    assert np.array_equal(s.cpu().numpy(), s_ref)
    assert np.array_equal(e.cpu().numpy(), e_ref)


def test_align_repeatable():
    ids = _routing("uniform", 2048, 256, 6, 3).cuda()
    a = moe.moe_align(ids, 256, 64)
    b = moe.moe_align(ids, 256, 64)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


# moe_align_ws: chunked planning past 16,384 routes (three launches over
# chunks of 512 route ids), bit for bit the one-workgroup plan
CHUNKED = [
    ("uniform", 2049, 288, 8),      # 16,392 routes: just past the switch
    ("masked", 8192, 288, 8),       # 65,536 routes
    ("zipf", 4096, 384, 6),         # 24,576 routes, a few huge experts
    ("oor", 9000, 10, 2),           # ids outside [0, E): not routes
    ("uniform", 5000, 1024, 4),     # E = 1024, last chunk partial
    ("one", 20000, 8, 1),           # one expert per token, 8 experts
]


@pytest.mark.parametrize("bm", [16, 64, 128, 256])
@pytest.mark.parametrize("kind,T,E,k", CHUNKED)
def test_align_chunked_bit_exact(kind, T, E, k, bm):
    say(f"[gpu] align chunked kind={kind} T={T} E={E} k={k} bm={bm}")
    assert moe.moe_align_ws_size(T, k, E) > 0
    ids = _routing(kind, T, E, k, T * 7 + E)
    s_ref, e_ref, n_ref = align_ref(ids.numpy(), E, bm)
    # a workspace full of garbage: the chunk counts must not depend on it
    ws = torch.full((moe.moe_align_ws_size(T, k, E),), 0x5A, dtype=torch.uint8, device="cuda")
    s, e, n = moe.moe_align_ws(ids.cuda(), E, bm, workspace=ws, out=_outputs(T, k, E, bm))
    torch.cuda.synchronize()
    assert int(n.item()) == n_ref
    assert np.array_equal(s.cpu().numpy(), s_ref)
    assert np.array_equal(e.cpu().numpy(), e_ref)
    # moe_align with its workspace runs the same chunked plan
    assert moe.moe_align_workspace_size(T, k, E) == ws.numel()
    s2, e2, n2 = moe.moe_align(ids.cuda(), E, bm, workspace=ws, out=_outputs(T, k, E, bm))
    torch.cuda.synchronize()
    assert torch.equal(s2, s) and torch.equal(e2, e) and torch.equal(n2, n)


@pytest.mark.parametrize("S", [1, 2])
def test_align_chunked_shared(S):
    """Shared experts through the chunked planner equal moe_align_shared."""
    T, E, k = 3000, 64, 6
    ids = _routing("uniform", T, E, k, 91).cuda()
    assert moe.moe_align_ws_size(T, k, E, S) > 0
    a = moe.moe_align_ws(ids, E, 64, n_shared=S)
    b = moe.moe_align_shared(ids, E, S, 64)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_align_ws_small_is_moe_align():
    """At or below 16,384 routes moe_align_ws needs no workspace and is moe_align."""
    ids = _routing("uniform", 256, 256, 6, 5).cuda()
    assert moe.moe_align_ws_size(256, 6, 256) == 0
    a = moe.moe_align_ws(ids, 256, 16)
    b = moe.moe_align(ids, 256, 16)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("T,E,k,bm", [(4096, 288, 8, 128), (8192, 288, 8, 256), (3000, 64, 6, 64)])
def test_route_align_chunked_planner(T, E, k, bm):
    """Past 16,384 routes with room for the chunk counts, moe_route_align
    routes in one launch and plans with the chunked planner: the outputs
    equal the router oracle's ids and moe_align's plan of them."""
    from oracle.router import route_ref
    g = torch.Generator().manual_seed(T + E)
    logits = torch.randn(T, E, generator=g)
    need = moe.moe_route_align_workspace_size() + moe.moe_align_workspace_size(T, k, E)
    assert need > 256 or T * k <= 16384
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    ids, w, s, e, n = moe.moe_route_align(logits.cuda(), k, bm, workspace=ws)
    torch.cuda.synchronize()
    ids_ref, _ = route_ref(logits.numpy(), k)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    s_ref, e_ref, n_ref = align_ref(ids_ref, E, bm)
    assert int(n.item()) == n_ref
    assert np.array_equal(s.cpu().numpy(), s_ref) and np.array_equal(e.cpu().numpy(), e_ref)
    assert not bool(ws[:256].any())      # the ticket is back at zero
