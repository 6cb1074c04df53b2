"""Shared experts (fused_moe_shared, moe_align_shared) on the GPU against the
oracle: the planner bit-exact against the planner oracle run on the whole
route list (routed routes t*top_k + j, then shared routes T*top_k + t*S + s),
and the forward within the dtype's tolerance against moe_ref(n_shared=S), in
both modes and at several block sizes (streaming and LDS-tiled kernels)."""

import numpy as np
import pytest
import torch

import datagen
import mixture_experts_ffn_moe_amd as moe
from oracle.align import align_ref

from .gpu_helpers import check, say
from .test_gpu_moe import SHAPES, to_gpu

pytestmark = pytest.mark.gpu


def shared_case(kind, T=40, E=6, k=2, S=1, routing="normal", tag="gpu-shared", **kw):
    shp = dict(SHAPES[kind])
    shp.update(kw)
    return to_gpu(datagen.make_case(kind, T, shp["K"], shp["I"], E, k, routing=routing, tag=tag,
                                    n_shared=S))


def expected_plan(ids, E, S, bm):
    T, k = ids.shape
    routed = np.where((ids >= 0) & (ids < E), ids, -1).reshape(-1)
    shared = np.tile(np.arange(E, E + S), T)
    return align_ref(np.concatenate([routed, shared])[None, :], E + S, bm)


@pytest.mark.parametrize("S", [1, 3])
@pytest.mark.parametrize("bm", [16, 64, 128])
def test_planner_with_shared(S, bm):
    ids = datagen.make_routing(77, 10, 3, "normal", tag="plan-shared")[0]
    ids[5, 1] = 11            # outside the routed experts: not a route
    ids[9, 0] = -1
    s_ref, e_ref, n_ref = expected_plan(ids.numpy(), 10, S, bm)
    sid, eid, ntp = moe.moe_align_shared(ids.cuda(), 10, S, bm)
    torch.cuda.synchronize()
    assert np.array_equal(sid.cpu().numpy(), s_ref)
    assert np.array_equal(eid.cpu().numpy(), e_ref)
    assert int(ntp.item()) == n_ref


@pytest.mark.parametrize("split", [1, 0])
@pytest.mark.parametrize("bm", [16, 64, 128])
@pytest.mark.parametrize("kind", ["bf16", "fp8_blockwise", "mxfp8", "mxfp4"])
def test_shared_parity(kind, bm, split):
    c = shared_case(kind, S=2 if kind == "fp8_blockwise" else 1)
    check(c, bm, split, label="shared")


@pytest.mark.parametrize("kind", ["fp8_blockwise", "mxfp4"])
def test_shared_only_and_single_token(kind):
    c = shared_case(kind, T=30)
    c.topk_ids = torch.full_like(c.topk_ids, -1)        # no routed expert is local
    check(c, 16, 1, label="shared only")
    c1 = shared_case(kind, T=1, tag="gpu-shared-1")
    for split in (1, 0):
        check(c1, 16, split, label="shared, T=1")


def test_shared_split_deterministic():
    c = shared_case("mxfp8", T=120, E=8, k=2, S=2)
    a, _ = moe.run_case(c, block_m=16, split=1)
    b, _ = moe.run_case(c, block_m=16, split=1)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_no_shared_matches_plain_entry_point():
    """n_shared = 0 through fused_moe_shared is the plain call, bit for bit."""
    c = shared_case("fp8_blockwise", S=0)
    sid, eid, ntp = moe.moe_align(c.topk_ids, c.E, 16)
    a = moe.fused_moe_fp8_blockwise(c.x, c.x_scale, c.w1, c.w1_scale, c.w2, c.w2_scale, sid, eid,
                                    ntp, c.topk_weights, c.top_k, 16, split=1)
    s2, e2, n2 = moe.moe_align_shared(c.topk_ids, c.E, 0, 16)
    b = moe.fused_moe_shared("fp8_blockwise", c.x, c.x_scale, c.w1, c.w1_scale, c.w2, c.w2_scale,
                             0, s2, e2, n2, c.topk_weights, c.top_k, 16, split=1)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_full_size_shared_sampled():
    """K=4096, I=2048, 256 routed experts top-6 plus one shared expert, T=64:
    sampled tokens against the oracle."""
    from oracle.moe import tolerance_check
    from .gpu_helpers import TOL, oracle, oracle_threads, out_bits
    from .test_gpu_fullsize import sample_tokens
    c = datagen.make_case("fp8_blockwise", 64, 4096, 2048, 256, 6, routing="uniform",
                          device="cuda", tag="fp8-shared-full", n_shared=1)
    bm = moe.moe_select_block_m(64, 7, 257, "fp8_blockwise", 4096)
    say(f"[gpu] full size shared T=64 block_m={bm}")
    out, _ = moe.run_case(c, block_m=bm, split=1)
    torch.cuda.synchronize()
    toks = sample_tokens(c, 32)
    ref = oracle(c, tokens=toks, threads=oracle_threads())
    ok, stats = tolerance_check(out_bits(out)[toks], ref["out64"], TOL["fp8_blockwise"],
                                ref["allowance"])
    say(f"      stats {stats}")
    assert ok, stats
