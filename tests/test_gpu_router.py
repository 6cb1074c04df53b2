"""Router + planner in one launch (moe_route_align) against the oracle:
topk_ids bit-exact (the selection compares the given fp32 logits, so both
sides decide exactly), topk_weights within a few fp32 ulp of the fp64
value, and the planner outputs bit-exact against the planner oracle run on
the oracle's ids.

Weight tolerance: the kernel computes exp(l_j - l_max) with the library expf
(within 2 ulp), sums at most 16 terms in fp32 (each addition rounds once) and
divides once, so the relative error stays below about (2 + 16 + 1) ulp of
fp32 = 2.3e-6; the test allows 4e-6."""

import numpy as np
import pytest
import torch

import datagen
import mixture_experts_ffn_moe_amd as moe
from oracle.align import align_ref
from oracle.router import route_ref

from .gpu_helpers import say

pytestmark = pytest.mark.gpu

RTOL_W = 4e-6


def check(logits, k, bm, label, runs=1):
    T, E = logits.shape
    ref_ids, ref_w = route_ref(logits.cpu().numpy(), k)
    s_ref, e_ref, n_ref = align_ref(ref_ids, E, bm)
    say(f"[gpu] route_align {label} T={T} E={E} k={k} bm={bm}")
    for _ in range(runs):
        ids, w, sid, eid, ntp = moe.moe_route_align(logits.cuda(), k, bm)
        torch.cuda.synchronize()
        assert np.array_equal(ids.cpu().numpy(), ref_ids), label
        np.testing.assert_allclose(w.cpu().numpy(), ref_w, rtol=RTOL_W, atol=1e-30, err_msg=label)
        assert np.array_equal(sid.cpu().numpy(), s_ref), label
        assert np.array_equal(eid.cpu().numpy(), e_ref), label
        assert int(ntp.item()) == n_ref, label


@pytest.mark.parametrize("T,E,k,routing", [
    (50, 16, 4, "normal"), (1, 8, 2, "normal"), (200, 70, 8, "uniform"),
    (300, 256, 6, "uniform"), (129, 5, 5, "normal"), (64, 1024, 16, "normal"),
    (1000, 288, 8, "normal_masked"), (777, 384, 6, "zipf")])
@pytest.mark.parametrize("bm", [16, 64])
def test_route_align_parity(T, E, k, routing, bm):
    logits = datagen.make_router_logits(T, E, k, routing, tag="router")
    check(logits, k, bm, f"{routing}")


def test_ties_go_to_lower_ids():
    g = torch.Generator().manual_seed(11)
    # logits on a coarse grid: many exact ties per token
    logits = (torch.randint(-4, 5, (300, 40), generator=g).float() / 2).contiguous()
    check(logits, 6, 16, "ties")


def test_masked_experts_and_all_selected():
    g = torch.Generator().manual_seed(12)
    logits = torch.randn(100, 12, generator=g)
    logits[:, [1, 5, 6]] = float("-inf")
    check(logits, 9, 16, "masked, k = unmasked count")
    check(torch.randn(40, 7, generator=g), 7, 32, "k = E")


def test_workspace_left_zero_and_reused():
    """Back-to-back calls on one workspace (the ticket must come back to 0),
    with different grid sizes in between."""
    ws = torch.zeros(moe.moe_route_align_workspace_size(), dtype=torch.uint8, device="cuda")
    for T in (8, 3000, 1, 256, 3000):
        logits = datagen.make_router_logits(T, 64, 4, "normal", tag="router-ws").cuda()
        ids, w, sid, eid, ntp = moe.moe_route_align(logits, 4, 16, workspace=ws)
        torch.cuda.synchronize()
        ref_ids, _ = route_ref(logits.cpu().numpy(), 4)
        assert np.array_equal(ids.cpu().numpy(), ref_ids)
        assert int(ws.sum().item()) == 0


def test_empty_batch():
    logits = torch.empty(0, 32, device="cuda")
    ids, w, sid, eid, ntp = moe.moe_route_align(logits, 4, 16)
    torch.cuda.synchronize()
    assert ids.shape == (0, 4) and int(ntp.item()) == 0


def test_full_size_many_tokens():
    """8192 tokens, 288 experts (8 masked), top-8: 128 workgroups route, the
    last plans 65,536 routes."""
    logits = datagen.make_router_logits(8192, 288, 8, "normal_masked", tag="router-big")
    check(logits, 8, 128, "full size", runs=2)


def test_matches_separate_planner():
    """The fused call's planner outputs equal moe_align's on the ids it
    produced (same kernel body, same routing)."""
    logits = datagen.make_router_logits(500, 256, 6, "uniform", tag="router-sep").cuda()
    ids, w, sid, eid, ntp = moe.moe_route_align(logits, 6, 16)
    s2, e2, n2 = moe.moe_align(ids, 256, 16)
    torch.cuda.synchronize()
    assert torch.equal(sid, s2) and torch.equal(eid, e2) and torch.equal(ntp, n2)
