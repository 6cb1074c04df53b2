"""fused_moe_fp8_blockwise_noalloc (the library's static workspace, nothing
allocated) against fused_moe_fp8_blockwise with a workspace: two calls in a
row on one GPU, the second smaller, both through the C ABI; the split mode
is deterministic, so the outputs must be the same bits.  A call too large
for the static workspace fails before anything is launched."""

import ctypes

import numpy as np
import pytest
import torch

import datagen
import mixture_experts_ffn_moe_amd as moe

pytestmark = pytest.mark.gpu


def _case(T, tag):
    c = datagen.make_case("fp8_blockwise", T, 512, 384, 8, 2, routing="normal", tag=tag)
    for f in ("x", "x_scale", "w1", "w1_scale", "w2", "w2_scale", "topk_ids", "topk_weights"):
        setattr(c, f, getattr(c, f).cuda())
    return c


def _bits(t):
    return t.view(torch.int16).cpu().numpy()


@pytest.mark.parametrize("split", [1, -1])
def test_noalloc_matches_workspace_call(split):
    for T, tag in ((64, "noalloc-a"), (9, "noalloc-b")):       # the second call is smaller
        c = _case(T, tag)
        sid, eid, ntp = moe.moe_align(c.topk_ids, c.E, 16)
        args = (c.x, c.x_scale, c.w1, c.w1_scale, c.w2, c.w2_scale, sid, eid, ntp,
                c.topk_weights, c.top_k, 16)
        ref = moe.fused_moe_fp8_blockwise(*args, split=split)
        out = torch.full_like(ref, float("nan"))
        moe.fused_moe_fp8_blockwise_noalloc(*args, split=split, out=out)
        torch.cuda.synchronize()
        if moe.moe_select_split("fp8_blockwise", T, 512, 768, 8, 2, 16) == 1 or split == 1:
            assert np.array_equal(_bits(out), _bits(ref)), (T, split)
        else:   # the fused mode adds with atomics: equal up to summation order
            d = (out.float() - ref.float()).abs().max().item()
            assert d <= 1e-2 * ref.float().std().item(), (T, split, d)


def test_noalloc_rejects_sizes_beyond_its_workspace():
    L = moe.lib()
    P = ctypes.c_void_p
    fake = P(1 << 20)
    # T = 4096, K = 4096, I = 2048, 256 experts top-6, 64-row blocks, split mode: 274 MiB
    rc = L.fused_moe_fp8_blockwise_noalloc(*([fake] * 11), 4096, 4096, 4096, 256, 6, 64, 1, None)
    assert rc == -5
    assert b"static scratch" in L.moe_last_error()
