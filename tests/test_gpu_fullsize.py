"""Parity at the benchmark workloads' full sizes, in the launch configuration
bench.py times (block_m from moe_select_block_m, mode from moe_select_split),
on sampled tokens the oracle computes one by one, plus properties that hold
at any size (every output finite; the planner's padded count matches the
closed form)."""

import numpy as np
import pytest
import torch

import datagen
import mixture_experts_ffn_moe_amd as moe
from oracle import codecs
from oracle.moe import tolerance_check

from .gpu_helpers import TOL, oracle, out_bits, say

pytestmark = pytest.mark.gpu

_WEIGHTS = {}


def weights(name):
    if name not in _WEIGHTS:
        _WEIGHTS.clear()
        torch.cuda.empty_cache()
        spec = datagen.WORKLOADS[name]
        say(f"[gpu] generating {name} weights")
        _WEIGHTS[name] = datagen.make_weights(spec["kind"], spec["K"], spec["I"], spec["E"],
                                              device="cuda", tag=name, w_std=spec.get("w_std"))
    return _WEIGHTS[name]


CASES = [(name, T) for name in ("fp8-k4096-i2048-e256-top6", "fp8-k4096-i2048-e288-top8",
                                "fp8-k7168-i3072-e384-top6", "mx-k4096-i256-e32-top8",
                                "mxfp4-k4096-i2048-e256-top6")
         for T in datagen.WORKLOADS[name]["tokens"]]


def sample_tokens(case, n):
    T = case.T
    pick = sorted(set([0, T // 2, T - 1] + list(np.random.default_rng(T).integers(0, T, n))))
    return np.array(pick[:max(n, 3)])


@pytest.mark.parametrize("name,T", CASES)
def test_full_size_sampled(name, T):
    c = datagen.make_workload_case(name, T, device="cuda", weights=weights(name))
    K, I, E, k = c.K, c.I, c.E, c.top_k
    bm = moe.moe_select_block_m_routed(T, k, E, moe.active_experts(c.topk_ids, E), c.kind, K)
    split = moe.moe_select_split(c.kind, T, K, 2 * I, E, k, bm)
    say(f"[gpu] full size {name} T={T} block_m={bm} split={split}")
    out, (sid, eid, ntp) = moe.run_case(c, block_m=bm, split=split)
    torch.cuda.synchronize()
    # properties at full size
    assert torch.isfinite(out.float()).all()
    ids = c.topk_ids.cpu().numpy()
    counts = np.bincount(ids[(ids >= 0) & (ids < E)], minlength=E)
    assert int(ntp.item()) == int(np.sum(-(-counts // bm) * bm))
    # sampled tokens against the oracle
    n = 2 if name.startswith("fp8-k7168") else 3
    toks = sample_tokens(c, n)
    ref = oracle(c, tokens=toks)
    got = out_bits(out)[toks]
    ok, stats = tolerance_check(got, ref["out64"], TOL[c.kind], ref["flip_bound"])
    say(f"      tokens {toks.tolist()} stats {stats}")
    assert ok, stats


@pytest.mark.parametrize("name,T", [("fp8-k4096-i2048-e256-top6", 256),
                                    ("mx-k4096-i256-e32-top8", 512),
                                    ("mxfp4-k4096-i2048-e256-top6", 64)])
def test_full_size_modes_agree(name, T):
    """Both modes at full size on the same inputs agree on sampled tokens
    within the oracle gate."""
    c = datagen.make_workload_case(name, T, device="cuda", weights=weights(name))
    bm = moe.moe_select_block_m_routed(T, c.top_k, c.E, moe.active_experts(c.topk_ids, c.E),
                                       c.kind, c.K)
    toks = sample_tokens(c, 3)
    ref = oracle(c, tokens=toks)
    for split in (0, 1):
        out, _ = moe.run_case(c, block_m=bm, split=split)
        torch.cuda.synchronize()
        ok, stats = tolerance_check(out_bits(out)[toks], ref["out64"], TOL[c.kind],
                                    ref["flip_bound"])
        say(f"      split={split} stats {stats}")
        assert ok, stats
