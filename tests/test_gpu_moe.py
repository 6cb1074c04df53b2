"""Fused MoE forward parity on the GPU (through the C ABI) against the fp64
oracle: every dtype x mode x block_m on shapes that span several tiles and
ragged blocks, the tiny bf16 workload, the split-mode intermediate against
the oracle's requantized intermediate, determinism, empty experts, routes
outside [0, E), and T = 1."""

import numpy as np
import pytest
import torch

import datagen
import mixture_experts_ffn_moe_amd as moe
from oracle import codecs

from .gpu_helpers import TOL, check, oracle, out_bits, say

pytestmark = pytest.mark.gpu

SHAPES = {
    "bf16": dict(K=512, I=256),
    "fp8_blockwise": dict(K=512, I=384),
    "mxfp8": dict(K=384, I=256),
    "mxfp4": dict(K=384, I=256),
}


def small_case(kind, T=50, E=8, k=2, routing="normal", tag="gpu", **kw):
    shp = dict(SHAPES[kind])
    shp.update(kw)
    c = datagen.make_case(kind, T, shp["K"], shp["I"], E, k, routing=routing, tag=tag)
    return to_gpu(c)


def to_gpu(c):
    for f in ("x", "x_scale", "w1", "w1_scale", "w2", "w2_scale", "topk_ids", "topk_weights"):
        v = getattr(c, f)
        if v is not None:
            setattr(c, f, v.cuda())
    return c


@pytest.mark.parametrize("split", [1, 0])
@pytest.mark.parametrize("bm", [16, 32, 64, 128])
@pytest.mark.parametrize("kind", ["bf16", "fp8_blockwise", "mxfp8", "mxfp4"])
def test_small_parity(kind, bm, split):
    c = small_case(kind)
    check(c, bm, split, label="small")


def test_bf16_tiny_workload():
    c = to_gpu(datagen.make_workload_case("bf16-k512-i256-e8-top2", 32))
    for split in (1, 0):
        check(c, 16, split, label="bf16 workload")


@pytest.mark.parametrize("kind", ["bf16", "fp8_blockwise", "mxfp8", "mxfp4"])
def test_split_mode_deterministic(kind):
    c = small_case(kind, T=200, E=16, k=4)
    a, _ = moe.run_case(c, block_m=32, split=1)
    b, _ = moe.run_case(c, block_m=32, split=1)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("kind", ["bf16", "fp8_blockwise", "mxfp8", "mxfp4"])
def test_fused_matches_split(kind):
    c = small_case(kind, T=100, E=8, k=2)
    a, _ = moe.run_case(c, block_m=16, split=1)
    b, _ = moe.run_case(c, block_m=16, split=0)
    torch.cuda.synchronize()
    fa, fb = a.float(), b.float()
    rms = fa.pow(2).mean().sqrt().item()
    assert (fa - fb).abs().max().item() <= TOL[kind] * rms + 2 ** -7 * fa.abs().max().item()


def _adjacent(a, b, sign):
    """Codes equal, or one rounding step apart (e4m3 and bf16 order their
    magnitudes like the integers below the sign bit ``sign``)."""
    a = a.astype(np.int64)
    b = b.astype(np.int64)
    same_sign = (a & sign) == (b & sign)
    step = np.abs((a & (sign - 1)) - (b & (sign - 1)))
    return (a == b) | (same_sign & (step == 1)) | ((a & (sign - 1)) + (b & (sign - 1)) <= 1)


@pytest.mark.parametrize("kind", ["bf16", "fp8_blockwise", "mxfp8", "mxfp4"])
def test_split_intermediate_matches_oracle(kind):
    """The requantized intermediate the split mode writes (values and scales)
    against the oracle's.  Every code equals the oracle's, except where the
    oracle flags the decision as a near-tie (alt > 0: the GPU's fp32 h, with
    its own summation order, may lie on the other side of the rounding
    boundary), and then it is the neighbouring code.  Blockwise scales lie
    within the oracle's bound on their deviation; an MX shared exponent
    differs only in a group the oracle flags, whose codes are then the other
    exponent's.  The number of flipped decisions stays within what the
    oracle's model expects (the sum of its flip probabilities)."""
    c = small_case(kind, T=40, E=4, k=2)
    bm = 16
    K, I, E, k = c.K, c.I, c.E, c.top_k
    N = 2 * I
    need = moe.moe_workspace_size(kind, c.T, K, N, E, k, bm, split=1)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    out, (sorted_ids, _, ntp) = moe.run_case(c, block_m=bm, split=1, workspace=ws)
    torch.cuda.synchronize()
    h_off, hs_off = moe.moe_workspace_layout(kind, c.T, K, N, E, k, bm)
    ref = oracle(c, keep_h=True)["h"]
    sid = sorted_ids.cpu().numpy()
    n = int(ntp.item())
    wsn = ws.cpu().numpy()
    es = 2 if kind == "bf16" else 1
    sign = 0x8000 if es == 2 else 0x80
    flips = total = scale_flips = 0
    expected = 0.0
    for pos in range(n):
        rid = int(sid[pos])
        if rid < 0:
            continue
        q_ref, s_ref, _, alt, info = ref[rid]
        row = wsn[h_off + pos * I * es: h_off + (pos + 1) * I * es]
        if kind == "bf16":
            row = row.view(np.uint16)
        keep = np.ones(I, bool)
        if kind == "fp8_blockwise":
            srow = wsn[hs_off + pos * (I // 128) * 4: hs_off + (pos + 1) * (I // 128) * 4]
            rel = np.abs(srow.view(np.float32).astype(np.float64) / s_ref - 1.0)
            assert np.all(rel <= info["scale_rel"] + 2.0 ** -23), (pos, rel, info["scale_rel"])
        if kind in ("mxfp8", "mxfp4"):
            srow = wsn[hs_off + pos * (I // 32): hs_off + (pos + 1) * (I // 32)]
            moved = srow != s_ref          # power-of-two scale decided the other way
            assert np.all(info["moved"][moved]), (pos, np.nonzero(moved))
            scale_flips += int(moved.sum())
            for gi in np.nonzero(moved)[0]:
                sl = slice(32 * gi, 32 * gi + 32)
                s_alt = int(srow[gi]) - 127
                q_alt = codecs.e4m3_encode((codecs.e4m3_decode(q_ref[sl]) * 2.0 ** (int(s_ref[gi]) - 127)
                                            + info["dhd"][sl]) * 2.0 ** -s_alt)
                same = row[sl] == q_alt
                assert np.all(same | ((info["alt2"][sl] > 0) & _adjacent(row[sl], q_alt, sign))), pos
            keep = ~np.repeat(moved, 32)
        diff = row[keep] != q_ref[keep]
        assert np.all(alt[keep][diff] > 0), (pos, np.nonzero(diff))
        assert np.all(_adjacent(row[keep][diff], q_ref[keep][diff], sign)), pos
        flips += int(diff.sum())
        total += int(keep.sum())
        expected += float(np.sum(info["prob"]))
    say(f"      intermediate code flips {flips}/{total} (model expects {expected:.1f}), "
        f"scale flips {scale_flips}")
    assert flips <= expected + 5 * np.sqrt(expected) + 3


@pytest.mark.parametrize("kind", ["bf16", "fp8_blockwise", "mxfp8", "mxfp4"])
def test_empty_experts_never_read(kind):
    c = small_case(kind, T=6, E=32, k=2)
    base, _ = moe.run_case(c, block_m=16, split=1)
    used = set(c.topk_ids.flatten().tolist())
    empty = [e for e in range(c.E) if e not in used]
    assert empty
    idx = torch.tensor(empty, device="cuda")
    if kind == "mxfp4":
        # every e2m1 code is finite: poison the e8m0 scales (0xFF is NaN)
        s1 = c.w1_scale.clone()
        s2 = c.w2_scale.clone()
        s1[idx] = 0xFF
        s2[idx] = 0xFF
        c.w1_scale, c.w2_scale = s1, s2
    else:
        w1 = c.w1.view(torch.uint8).clone()
        w2 = c.w2.view(torch.uint8).clone()
        if kind == "bf16":
            w1.view(torch.int16)[idx] = 0x7FC0
            w2.view(torch.int16)[idx] = 0x7FC0
        else:
            w1[idx] = 0x7F
            w2[idx] = 0x7F
        c.w1 = w1.view(c.w1.dtype)
        c.w2 = w2.view(c.w2.dtype)
    for split in (1, 0):
        got, _ = moe.run_case(c, block_m=16, split=split)
        torch.cuda.synchronize()
        assert torch.isfinite(got.float()).all()
        if split == 1:
            assert torch.equal(got.view(torch.int16), base.view(torch.int16))


@pytest.mark.parametrize("split", [1, 0])
def test_routes_outside_local_experts(split):
    c = small_case("fp8_blockwise", T=30, E=8, k=2)
    ids = c.topk_ids.clone()
    ids[::3, 1] = -1          # non-local route
    ids[5, :] = -1            # a token with no local route -> zeros
    ids[7, 0] = 11            # beyond E
    c.topk_ids = ids
    out, _, _ = check(c, 16, split, label="oor")
    assert torch.all(out[5].float() == 0)


@pytest.mark.parametrize("kind", ["fp8_blockwise", "mxfp8"])
@pytest.mark.parametrize("bm,split", [(64, 1), (128, 1), (256, 1), (16, 2), (32, 2)])
def test_routes_outside_local_experts_tiled_and_ring(kind, bm, split):
    """The LDS-tiled kernels and the ring mode with non-local routes, ids
    beyond E and tokens with no local route at all (their rows must be
    zeros, written although no tile ever holds them)."""
    c = small_case(kind, T=300, E=4, k=2, K=512, tag="gpu-oor-tiled")
    ids = c.topk_ids.clone()
    ids[::3, 1] = -1
    ids[5, :] = -1
    ids[299, :] = -1          # the last token too
    ids[7, 0] = 9
    c.topk_ids = ids
    out, _, _ = check(c, bm, split, label="oor tiled/ring")
    assert torch.all(out[5].float() == 0) and torch.all(out[299].float() == 0)


@pytest.mark.parametrize("kind", ["bf16", "fp8_blockwise", "mxfp8", "mxfp4"])
def test_single_token(kind):
    c = small_case(kind, T=1, E=8, k=2)
    for split in (1, 0):
        check(c, 16, split, label="T=1")


def test_many_routes_fused_atomics():
    c = small_case("fp8_blockwise", T=600, E=8, k=4, routing="uniform")
    check(c, 64, 0, label="fused many routes")
    check(c, 64, 1, label="split many routes")


@pytest.mark.parametrize("split", [1, 0])
@pytest.mark.parametrize("bm", [16, 32])
@pytest.mark.parametrize("kind", ["bf16", "fp8_blockwise", "mxfp8", "mxfp4"])
def test_ksplit_parity(kind, bm, split):
    """Few (block, slice) tiles and at least 8 K steps: the up GEMM runs with
    two K groups per workgroup; 9 K steps give the groups an uneven share."""
    c = small_case(kind, T=20, E=8, k=2, K=1152, I=256)
    check(c, bm, split, label="ksplit")


@pytest.mark.parametrize("split", [1, 0])
@pytest.mark.parametrize("kind,K,I,T,E", [
    ("mxfp8", 1024, 512, 20, 8),     # two K groups of 4 steps: one chunk per row; down 4 steps
    ("mxfp4", 2048, 512, 60, 8),     # two K groups of 8 steps: two chunks per row
    ("mxfp4", 1536, 1536, 40, 32),   # one K group of 12 steps (3 chunks); down 12 steps
    ("mxfp8", 1536, 1536, 40, 32)])
def test_staged_scale_parity(kind, K, I, T, E, split):
    """MX walks whose step count is a multiple of 4 read their e8m0 scale
    runs from rows copied into LDS before the walk (block_m 16, ring depth 4),
    with the chunk rotation taken modulo the row's chunk count."""
    c = small_case(kind, T=T, E=E, k=2, K=K, I=I)
    check(c, 16, split, label="staged")


def test_ksplit_deterministic():
    c = small_case("mxfp8", T=20, E=8, k=2, K=1152, I=256)
    a, _ = moe.run_case(c, block_m=16, split=1)
    b, _ = moe.run_case(c, block_m=16, split=1)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("bm", [64, 128, 256])
@pytest.mark.parametrize("kind,K,I", [("fp8_blockwise", 768, 384), ("mxfp8", 512, 256),
                                      ("fp8_blockwise", 256, 128), ("fp8_blockwise", 512, 640),
                                      ("mxfp8", 256, 640)])
def test_tiled_split_parity(kind, K, I, bm):
    """The LDS-tiled split-mode kernels (block_m 64 / 128, K a multiple of
    256): several blocks per expert, several K steps and slices, ragged last
    blocks, skewed expert load."""
    c = datagen.make_case(kind, 700, K, I, 6, 2, routing="zipf", tag="tiled")
    c = to_gpu(c)
    check(c, bm, 1, label="tiled")


def test_tiled_deterministic():
    c = to_gpu(datagen.make_case("fp8_blockwise", 500, 512, 256, 4, 2, routing="normal",
                                 tag="tiled-det"))
    for bm in (128, 256):
        a, _ = moe.run_case(c, block_m=bm, split=1)
        b, _ = moe.run_case(c, block_m=bm, split=1)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("bm", [16, 32])
@pytest.mark.parametrize("kind", ["bf16", "fp8_blockwise", "mxfp8", "mxfp4"])
def test_k_split_over_workgroups_parity(kind, bm):
    """Few tiles (8 experts x 2 slices) and 16 K steps: the gate/up GEMM
    splits K over four workgroups per tile, the last adds the four sums in
    order; against the oracle, and bitwise repeatable."""
    c = small_case(kind, T=20, E=8, k=2, K=2048, I=256, tag="gpu-kw")
    out, _, _ = check(c, bm, 1, label="k split over workgroups")
    again, _ = moe.run_case(c, block_m=bm, split=1)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), again.view(torch.int16))


@pytest.mark.parametrize("kind", ["fp8_blockwise", "mxfp8"])
@pytest.mark.parametrize("T", [20, 300])
def test_tiled_k_split_parity(kind, T):
    """64-row LDS-tiled gate/up GEMM with few tiles (8 experts x 2 slices):
    K split over four workgroups per tile, the last adding the four sums in
    order; one block per expert (T = 20) and two, the second ragged (T =
    300).  Against the oracle, bitwise repeatable, and through the same
    kernels' K split = 1 within the gate."""
    c = small_case(kind, T=T, E=8, k=2, K=2048, I=256, tag="gpu-kw-tiled")
    assert moe.moe_workspace_size(kind, T, 2048, 512, 8, 2, 64, split=1) > \
        moe.moe_workspace_size(kind, T, 2048, 512, 8, 2, 64, split=1, tune={"k_split": 1})
    out, _, _ = check(c, 64, 1, label="tiled k split over workgroups")
    again, _ = moe.run_case(c, block_m=64, split=1)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), again.view(torch.int16))
    check(c, 64, 1, tune={"k_split": 1}, label="tiled, one workgroup per tile")


def test_tiled_k_split_reused_workspace():
    """The tiled K split's tickets are cleared by every call: one workspace
    for three calls in a row, the second smaller."""
    a = small_case("fp8_blockwise", T=300, E=8, k=2, K=2048, I=256, tag="gpu-kwt-a")
    b = small_case("fp8_blockwise", T=40, E=8, k=2, K=2048, I=256, tag="gpu-kwt-b")
    need = moe.moe_workspace_size("fp8_blockwise", 300, 2048, 512, 8, 2, 64, split=1)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    for c in (a, b, a):
        out, _ = moe.run_case(c, block_m=64, split=1, workspace=ws)
        torch.cuda.synchronize()
        ref, _ = moe.run_case(c, block_m=64, split=1)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    check(b, 64, 1, label="tiled k split, second call")


def test_k_split_over_workgroups_reused_workspace():
    """One workspace for two calls in a row, the second smaller: the tile
    tickets are cleared by each call."""
    a = small_case("mxfp8", T=24, E=8, k=2, K=2048, I=256, tag="gpu-kw-a")
    b = small_case("mxfp8", T=5, E=8, k=2, K=2048, I=256, tag="gpu-kw-b")
    need = moe.moe_workspace_size("mxfp8", 24, 2048, 512, 8, 2, 16, split=1)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    for c in (a, b, a):
        out, _ = moe.run_case(c, block_m=16, split=1, workspace=ws)
        torch.cuda.synchronize()
        ref, _ = moe.run_case(c, block_m=16, split=1)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    check(b, 16, 1, label="k split over workgroups, second call")
