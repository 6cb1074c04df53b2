"""LDS-tiled plans (64-, 128- and 256-row blocks) under skewed routing,
where one plan holds experts with a few routes beside experts with hundreds:
parity with the fp64 oracle, and for MXFP8 the same bits as the 16-row
streaming kernels (the block-scaled MFMA sums in one order in both).  A
plan whose rows are shuffled inside each block (routes behind -1 padding,
as a caller's planner may leave them) must give the plan's answer up to
summation order."""

import numpy as np
import pytest
import torch

import datagen
import mixture_experts_ffn_moe_amd as moe

from .gpu_helpers import check, oracle, out_bits, say
from .test_gpu_moe import to_gpu
from oracle import codecs
from oracle.moe import tolerance_check

pytestmark = pytest.mark.gpu

TOL = {"fp8_blockwise": 2e-2, "mxfp8": 2e-2}


def skewed_case(kind, T, E, k, K, I, tag):
    c = datagen.make_case(kind, T, K, I, E, k, routing="zipf", tag=tag, zipf_s=1.1)
    return to_gpu(c)


def block_rows(align, bm):
    ntp = int(align[2].item())
    return align[0].cpu().numpy()[: ntp // bm * bm].reshape(-1, bm)


@pytest.mark.parametrize("kind,bm", [("fp8_blockwise", 64), ("fp8_blockwise", 128),
                                     ("fp8_blockwise", 256), ("mxfp8", 64), ("mxfp8", 128)])
def test_skewed_plan(kind, bm):
    c = skewed_case(kind, 300, 24, 4, 512, 256, f"mixed-{kind}-{bm}")
    out, align, ref = check(c, bm, 1, label="skewed")
    rows = block_rows(align, bm)
    small = int(((rows[:, 16:] >= 0).sum(axis=1) == 0).sum())
    say(f"      blocks {len(rows)}, of them with every route in the first 16 rows: {small}")
    assert 0 < small < len(rows)  # nearly empty and full blocks in one plan
    if kind == "mxfp8":
        s16, _ = moe.run_case(c, block_m=16, split=1)
        torch.cuda.synchronize()
        assert np.array_equal(out_bits(out), out_bits(s16))


@pytest.mark.parametrize("bm", [64, 128])
def test_routes_behind_padding(bm):
    kind = "fp8_blockwise"
    c = skewed_case(kind, 300, 24, 4, 512, 256, f"mixed-{kind}-{bm}")
    plan_out, align = moe.run_case(c, block_m=bm, split=1)
    torch.cuda.synchronize()
    plan_bits = out_bits(plan_out).copy()
    ntp = int(align[2].item())
    s = align[0].cpu().numpy().copy()
    g = np.random.default_rng(7)
    nb = ntp // bm
    for b in range(nb):  # shuffle every block's rows, padding included
        s[b * bm:(b + 1) * bm] = g.permutation(s[b * bm:(b + 1) * bm])
    rows = s[: nb * bm].reshape(nb, bm)
    late = int(((rows[:, :16] < 0).any(axis=1) & (rows[:, 16:] >= 0).any(axis=1)).sum())
    say(f"[gpu] shuffled plan bm={bm}: {nb} blocks, {late} with routes behind padding")
    assert late > 0
    shuffled = (torch.from_numpy(s).to(align[0].device), align[1], align[2])
    out, _ = moe.run_case(c, block_m=bm, split=1, align_out=shuffled, skip_align=True)
    torch.cuda.synchronize()
    got = out_bits(out)
    ref = oracle(c)
    ok, stats = tolerance_check(got, ref["out64"], TOL[kind], ref["allowance"])
    say(f"      stats {stats}")
    assert ok, stats
    # the same routes in other rows of the tiles: equal up to summation order
    d = np.abs(codecs.bf16_decode(got) - codecs.bf16_decode(plan_bits))
    say(f"      against the unshuffled plan: {int((got != plan_bits).sum())} outputs differ, "
        f"max {d.max() / ref['out64'].std():.2e} rms")
    assert d.max() <= 1e-3 * ref["out64"].std()


def hot_expert_case(kind, bm, K):
    """Zipf routing over 24 experts with route 0 of every one of 9 * bm + 37
    tokens sent to expert 0 (each token's experts stay distinct)."""
    T = 9 * bm + 37
    c = datagen.make_case(kind, T, K, 256, 24, 4, routing="zipf", tag=f"hot-{kind}-{bm}",
                          zipf_s=1.1)
    ids = c.topk_ids.clone()
    for t in range(T):
        row = ids[t].tolist()
        if 0 in row:
            j = row.index(0)
            row[0], row[j] = row[j], row[0]
        else:
            row[0] = 0
        ids[t] = torch.tensor(row, dtype=ids.dtype)
    c.topk_ids = ids.contiguous()
    return to_gpu(c)


@pytest.mark.parametrize("kind,bm", [("fp8_blockwise", 64), ("fp8_blockwise", 128),
                                     ("fp8_blockwise", 256), ("mxfp8", 64), ("mxfp8", 128)])
def test_hot_expert_block_groups(kind, bm):
    """One expert in every token: its ten consecutive blocks (nine full, one
    ragged) make an aligned group of eight blocks of one expert, which the
    tiled kernels walk slice by slice (down GEMM: column tile by column
    tile), followed by a group that mixes experts and goes block by block.
    Parity with the oracle over every token; for MXFP8 also the same bits as
    the 16-row streaming kernels."""
    c = hot_expert_case(kind, bm, 512)
    out, align, ref = check(c, bm, 1, label="hot expert")
    eid = align[1].cpu().numpy()[: int(align[2].item()) // bm]
    say(f"      blocks {len(eid)}, of expert 0: {int((eid == 0).sum())}")
    assert (eid[:8] == 0).all() and (eid == 0).sum() == 10
    if kind == "mxfp8":
        s16, _ = moe.run_case(c, block_m=16, split=1)
        torch.cuda.synchronize()
        assert np.array_equal(out_bits(out), out_bits(s16))


@pytest.mark.parametrize("kind", ["fp8_blockwise", "mxfp8"])
def test_hot_expert_block_groups_k_split(kind):
    """The same plan at 64-row tiles with the gate/up K split over four
    workgroups per tile (K = 2048: 16 K steps), whose partial sums and
    tickets are indexed by the tile in walk order: parity with the oracle
    over every token."""
    c = hot_expert_case(kind, 64, 2048)
    out, align, _ = check(c, 64, 1, label="hot expert, K split", tune={"k_split": 4})
    eid = align[1].cpu().numpy()[: int(align[2].item()) // 64]
    assert (eid[:8] == 0).all() and (eid == 0).sum() == 10
