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

from .gpu_helpers import TOL, oracle, oracle_threads, out_bits, say

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


def sample_tokens(case, n=32, align=None, bm=None):
    """At least min(n, T) sorted token ids: 0, T/2 and T - 1; with a plan
    (align, bm), the tokens of the last route of the first and last planner
    block of each XCD run of the tiled kernels' tile order (the valid tiles of
    each stage's grid split into 8 equal runs, run x on XCD x), then the last
    route of experts' ragged last blocks, preferring tokens whose routes
    reuse experts already sampled (each expert costs the oracle a pass over
    its weights); random tokens fill up to n."""
    T = case.T
    n = min(n, T)
    pick = [0, T // 2, T - 1]
    rng = np.random.default_rng(T)
    ids = case.topk_ids.cpu().numpy()
    k = case.top_k
    if align is not None:
        sid = align[0].cpu().numpy()
        nb = int(align[2].item()) // bm
        rows = sid[:nb * bm].reshape(nb, bm)

        def last_token(b):
            r = rows[b][rows[b] >= 0]
            return int(r[-1]) // k if r.size and int(r[-1]) < T * k else None

        for per_block in (case.I // 128, case.K // 256):   # gate/up and down tiles per block
            if nb == 0 or per_block == 0:
                continue
            per = -(-nb * per_block // 8)
            for x in range(8):
                lo, hi = x * per, min((x + 1) * per, nb * per_block) - 1
                if lo > hi:
                    continue
                for b in (lo // per_block, hi // per_block):
                    t = last_token(b)
                    if t is not None:
                        pick.append(t)
        pick = list(dict.fromkeys(pick))
        seen = set(int(e) for e in ids[pick].ravel())
        # ragged last blocks: the block's expert changes after it, and it has padding
        eid = align[1].cpu().numpy()[:nb]
        ragged = [b for b in range(nb) if (b + 1 == nb or eid[b + 1] != eid[b]) and
                  np.any(rows[b] < 0)]
        cand = [t for t in (last_token(b) for b in ragged) if t is not None and t not in pick]
        while len(pick) < n and cand:
            cost = [len(set(int(e) for e in ids[t]) - seen) for t in cand]
            t = cand.pop(int(np.argmin(cost)))
            pick.append(t)
            seen |= set(int(e) for e in ids[t])
    pick = list(dict.fromkeys(pick))
    while len(pick) < n:
        t = int(rng.integers(0, T))
        if t not in pick:
            pick.append(t)
    return np.array(sorted(pick))


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
    toks = sample_tokens(c, 32, (sid, eid, ntp), bm)
    assert toks.size >= min(32, T) and toks[-1] == T - 1
    ref = oracle(c, tokens=toks, threads=oracle_threads())
    got = out_bits(out)[toks]
    ok, stats = tolerance_check(got, ref["out64"], TOL[c.kind], ref["allowance"])
    say(f"      {toks.size} tokens {toks.tolist()} stats {stats}")
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
    toks = None
    for split in (1, 0):
        out, align = moe.run_case(c, block_m=bm, split=split)
        if toks is None:
            toks = sample_tokens(c, 32, align, bm)
            ref = oracle(c, tokens=toks, threads=oracle_threads())
        torch.cuda.synchronize()
        ok, stats = tolerance_check(out_bits(out)[toks], ref["out64"], TOL[c.kind],
                                    ref["allowance"])
        say(f"      split={split} stats {stats}")
        assert ok, stats
