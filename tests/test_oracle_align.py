"""Pins for the planner oracle (CPU only): hand-derived golden outputs,
brute-force grouping by Python's sort, and closed forms."""

import json
import os

import numpy as np
import pytest

from oracle.align import align_ref, capacity

GOLD = os.path.join(os.path.dirname(__file__), "golden", "align_small.json")


def brute(topk_ids, E, bm):
    flat = [int(v) for v in np.asarray(topk_ids).reshape(-1)]
    pairs = sorted((e, i) for i, e in enumerate(flat) if 0 <= e < E)
    rows, blocks = capacity(len(flat), E, bm)
    sorted_ids, expert_ids = [], []
    for e in sorted(set(p[0] for p in pairs)):
        members = [i for (ee, i) in pairs if ee == e]
        while members:
            chunk, members = members[:bm], members[bm:]
            sorted_ids += chunk + [-1] * (bm - len(chunk))
            expert_ids.append(e)
    ntp = len(sorted_ids)
    sorted_ids += [-1] * (rows - ntp)
    expert_ids += [-1] * (blocks - len(expert_ids))
    return sorted_ids, expert_ids, ntp


def test_golden():
    with open(GOLD) as f:
        g = json.load(f)
    for case in g["cases"]:
        s, e, n = align_ref(np.array(g["topk_ids"]), case["E"], case["block_m"])
        assert s.tolist() == case["sorted_token_ids"]
        assert e.tolist() == case["expert_ids"]
        assert n == case["num_tokens_post_padded"]


@pytest.mark.parametrize("bm", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("T,E,k,mode", [
    (0, 8, 2, "uniform"), (1, 8, 2, "uniform"), (37, 8, 2, "uniform"),
    (64, 256, 6, "uniform"), (200, 16, 4, "one"), (128, 4, 1, "multiple"),
    (50, 10, 3, "oor")])
def test_brute_force(T, E, k, mode, bm):
    rng = np.random.default_rng(T * 1000 + E + k)
    if mode == "one":
        ids = np.full((T, k), 3)
        ids[:, 1:] = rng.integers(0, E, (T, k - 1))
    elif mode == "multiple":
        ids = np.repeat(np.arange(4), T // 4)[:, None]   # c_e exact multiple
    elif mode == "oor":
        ids = rng.integers(-2, E + 3, (T, k))
    else:
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]) if T else \
            np.zeros((0, k), np.int64)
    s, e, n = align_ref(ids, E, bm)
    bs, be, bn = brute(ids, E, bm)
    assert s.tolist() == bs and e.tolist() == be and n == bn


def test_closed_forms():
    rng = np.random.default_rng(7)
    for _ in range(20):
        E = int(rng.integers(1, 300))
        T = int(rng.integers(0, 500))
        k = int(rng.integers(1, min(E, 8) + 1))
        bm = int(rng.choice([16, 32, 64, 128]))
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]) if T else \
            np.zeros((0, k), np.int64)
        s, e, n = align_ref(ids, E, bm)
        counts = np.bincount(ids.reshape(-1), minlength=E)
        assert n == int(np.sum(-(-counts // bm) * bm))
        valid = s[s >= 0]
        assert sorted(valid.tolist()) == list(range(T * k))
        assert int(np.sum(s == -1)) == s.size - T * k
        assert n % bm == 0
        assert np.all(s[n:] == -1) and np.all(e[n // bm:] == -1)
        # each block holds ids of its own expert only
        for b in range(n // bm):
            blk = s[b * bm:(b + 1) * bm]
            blk = blk[blk >= 0]
            assert blk.size > 0
            assert np.all(ids.reshape(-1)[blk] == e[b])
            assert np.all(np.diff(blk) > 0)
