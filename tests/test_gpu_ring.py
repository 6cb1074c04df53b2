"""Ring mode (split=2: one persistent grid over the lag-ordered task stream,
the intermediate in a ring of block slots) on the GPU.  It runs the split
mode's tiles with the split mode's arithmetic, so wherever the split mode's
gate/up workgroups take the whole K range in one group, the two outputs are
compared bit for bit.  The oracle checks run on the inputs the split-mode
parity tests use (the same seeds) and on inputs of their own, every dtype.
Rings of 1, 2, 3 and 7 slots wrap many times.  After every call the ring's error word (byte
offset 4 of the workspace) must be zero."""

import numpy as np
import pytest
import torch

import datagen
import mixture_experts_ffn_moe_amd as moe
from oracle.moe import tolerance_check

from .gpu_helpers import TOL, oracle, oracle_threads, out_bits, say
from .test_gpu_fullsize import sample_tokens, weights
from .test_gpu_moe import small_case
from .test_gpu_shared import shared_case

pytestmark = pytest.mark.gpu


def one_k_group(c, bm):
    """True where the split mode's gate/up kernel runs one K group per
    workgroup (it splits K in two only for at most 256 (block, slice) tiles
    with 8 or more K steps)."""
    R = c.T * (c.top_k + c.n_shared)
    tiles = min(R, c.E + c.n_shared) * (c.I // 128)
    return bm > 32 or c.K // 128 < 8 or tiles > 256


def run_ring(c, bm, slots=None):
    E_all, k_all = c.E + c.n_shared, c.top_k + c.n_shared
    fixed, slot, default = moe.moe_ring_layout(c.kind, c.T, c.K, 2 * c.I, E_all, k_all, bm)
    n = default if slots is None else slots
    ws = torch.zeros(fixed + n * slot, dtype=torch.uint8, device="cuda")
    say(f"[gpu] ring kind={c.kind} T={c.T} K={c.K} I={c.I} E={c.E} k={c.top_k} "
        f"S={c.n_shared} block_m={bm} slots={n}")
    out, _ = moe.run_case(c, block_m=bm, split=2, workspace=ws)
    torch.cuda.synchronize()
    assert int(ws[4:8].view(torch.int32).item()) == 0, "a ring wait gave up"
    return out


def split_out(c, bm):
    out, _ = moe.run_case(c, block_m=bm, split=1)
    torch.cuda.synchronize()
    return out


def against_oracle(c, out, tokens=None):
    ref = oracle(c, tokens, threads=oracle_threads())
    got = out_bits(out)
    if tokens is not None:
        got = got[np.asarray(tokens)]
    ok, stats = tolerance_check(got, ref["out64"], TOL[c.kind], ref["allowance"])
    say(f"      stats {stats}")
    assert ok, stats


def same_bits(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("bm", [16, 32])
@pytest.mark.parametrize("kind", ["bf16", "fp8_blockwise", "mxfp8", "mxfp4"])
def test_ring_parity(kind, bm):
    c = small_case(kind)          # the split-mode parity test's inputs
    assert one_k_group(c, bm)
    out = run_ring(c, bm)
    against_oracle(c, out)
    assert same_bits(out, split_out(c, bm))


@pytest.mark.parametrize("slots", [1, 2, 3, 7])
@pytest.mark.parametrize("kind", ["fp8_blockwise", "mxfp8", "mxfp4", "bf16"])
def test_ring_wraps(kind, slots):
    """Many more blocks than slots: every slot is rewritten many times, the
    up tasks of a block wait for the down tasks of the block slots earlier."""
    c = small_case(kind, T=300, E=8, k=2, routing="zipf", tag="gpu-ring-wrap")
    bm = 16
    _, blocks = moe.moe_align_capacity(c.T, c.top_k, c.E, bm)
    assert blocks > 4 * slots
    out = run_ring(c, bm, slots)
    assert same_bits(out, split_out(c, bm))
    if slots == 3:
        against_oracle(c, out)


@pytest.mark.parametrize("kind", ["fp8_blockwise", "mxfp4"])
def test_ring_shared_experts(kind):
    c = shared_case(kind, S=2 if kind == "fp8_blockwise" else 1)   # the shared parity inputs
    out = run_ring(c, 16)
    against_oracle(c, out)
    assert same_bits(out, split_out(c, 16))


def test_ring_routes_outside_and_single_token():
    c = small_case("fp8_blockwise", T=40, tag="gpu-ring-edge")
    ids = c.topk_ids.clone()
    ids[3, 0] = -1
    ids[7, 1] = c.E + 5           # not a local expert: no route
    ids[11, :] = -1               # a token with no route: zeros
    c.topk_ids = ids
    out = run_ring(c, 16, slots=2)
    against_oracle(c, out)
    assert same_bits(out, split_out(c, 16))
    assert (out[11].float() == 0).all()
    for kind in ("mxfp8", "mxfp4"):
        c1 = small_case(kind, T=1, E=8, k=2)   # the split-mode single-token inputs
        out1 = run_ring(c1, 32)
        against_oracle(c1, out1)
        assert same_bits(out1, split_out(c1, 32))


def test_ring_reuses_workspace():
    """Two calls on one workspace, the second smaller: the control words are
    cleared by each call."""
    a = small_case("mxfp8", T=200, E=8, k=2, tag="gpu-ring-a")
    b = small_case("mxfp8", T=37, E=8, k=2, tag="gpu-ring-b")
    fixed, slot, _ = moe.moe_ring_layout("mxfp8", 200, a.K, 2 * a.I, a.E, a.top_k, 16)
    ws = torch.zeros(fixed + 4 * slot, dtype=torch.uint8, device="cuda")
    for c in (a, b, a):
        out, _ = moe.run_case(c, block_m=16, split=2, workspace=ws)
        torch.cuda.synchronize()
        assert int(ws[4:8].view(torch.int32).item()) == 0
        assert same_bits(out, split_out(c, 16))


def test_ring_two_k_groups_shape():
    """Few tiles and many K steps: the split mode splits K over two groups
    of waves, the ring does not; both stay within the oracle's tolerance."""
    c = small_case("fp8_blockwise", T=4, E=8, k=2, K=1152, I=256, tag="gpu-ring-ksplit")
    assert not one_k_group(c, 16)
    against_oracle(c, run_ring(c, 16))


@pytest.mark.parametrize("name,T", [("fp8-k4096-i2048-e256-top6", 8),
                                    ("fp8-k4096-i2048-e256-top6", 64),
                                    ("fp8-k4096-i2048-e256-top6", 256),
                                    ("mxfp4-k4096-i2048-e256-top6", 64)])
def test_ring_full_size(name, T):
    """At full size, block_m 16, the default ring and a 5-slot one: bit for
    bit the split mode's output, sampled tokens against the oracle."""
    c = datagen.make_workload_case(name, T, device="cuda", weights=weights(name))
    assert one_k_group(c, 16)
    ref = split_out(c, 16)
    out = run_ring(c, 16)
    assert same_bits(out, ref)
    assert same_bits(run_ring(c, 16, slots=5), ref)
    align = moe.moe_align(c.topk_ids, c.E, 16)
    against_oracle(c, out, tokens=sample_tokens(c, 32, align, 16))


def test_ring_full_size_narrow_intermediate():
    """The narrow-intermediate workload (I = 256: two slices, so the split
    mode runs two K groups): sampled tokens against the oracle."""
    c = datagen.make_workload_case("mx-k4096-i256-e32-top8", 128, device="cuda",
                                   weights=weights("mx-k4096-i256-e32-top8"))
    align = moe.moe_align(c.topk_ids, c.E, 16)
    against_oracle(c, run_ring(c, 16), tokens=sample_tokens(c, 32, align, 16))
