"""Pins for the router oracle (CPU only): hand-derived golden cases, a
pure-Python brute force written differently (repeated maximum with an
explicit tie rule, weights from math.exp over all experts), invariants, and
planted mistakes that must fail a pin."""

import json
import math
import os

import numpy as np
import pytest

import oracle.router as router
from oracle.router import route_ref

GOLD = os.path.join(os.path.dirname(__file__), "golden", "router.json")


def _logits(rows):
    return np.array([[float(v) for v in r] for r in rows], dtype=np.float32)


def brute(logits, k):
    """Per token: pick the maximum k times (ties to the lower id, picked ids
    excluded), then exp(l - max_all) / sum over all experts, renormalized."""
    ids, ws = [], []
    for row in np.asarray(logits, dtype=np.float32).tolist():
        E = len(row)
        taken = []
        for _ in range(k):
            best = None
            for e in range(E):
                if e in taken:
                    continue
                if best is None or row[e] > row[best]:
                    best = e
            taken.append(best)
        m = max(row)
        p = [math.exp(v - m) for v in row]
        tot = sum(p)
        sel = [p[e] / tot for e in taken]
        s = sum(sel)
        ids.append(taken)
        ws.append([v / s for v in sel])
    return np.array(ids, dtype=np.int32), np.array(ws, dtype=np.float64)


def test_golden_cases():
    d = json.load(open(GOLD))
    for c in d["cases"]:
        ids, w = route_ref(_logits(c["logits"]), c["top_k"])
        assert ids.tolist() == c["topk_ids"], c["note"]
        np.testing.assert_allclose(w, np.array(c["topk_weights"]), rtol=5e-7, atol=0,
                                   err_msg=c["note"])


@pytest.mark.parametrize("T,E,k,seed", [(7, 5, 2, 0), (5, 16, 6, 1), (3, 9, 9, 2), (6, 70, 8, 3)])
def test_brute_force(T, E, k, seed):
    rng = np.random.default_rng(seed)
    # coarse values make ties common
    L = (np.round(rng.normal(size=(T, E)) * 2) / 2).astype(np.float32)
    ids, w = route_ref(L, k)
    bi, bw = brute(L, k)
    assert np.array_equal(ids, bi)
    np.testing.assert_allclose(w, bw, rtol=1e-13, atol=0)


def test_masked_experts_brute_force():
    rng = np.random.default_rng(4)
    L = rng.normal(size=(8, 12)).astype(np.float32)
    L[:, [2, 7, 9]] = -np.inf
    ids, w = route_ref(L, 4)
    bi, bw = brute(L, 4)
    assert np.array_equal(ids, bi)
    np.testing.assert_allclose(w, bw, rtol=1e-13)
    assert not np.isin(ids, [2, 7, 9]).any()


def test_invariants():
    rng = np.random.default_rng(5)
    T, E, k = 40, 64, 6
    L = rng.normal(size=(T, E)).astype(np.float32)
    ids, w = route_ref(L, k)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    assert all(len(set(r)) == k for r in ids.tolist())
    sel = np.take_along_axis(L, ids, axis=1)
    assert (np.diff(sel, axis=1) <= 0).all()            # descending logits
    # every unselected logit is at most the smallest selected one
    mask = np.ones_like(L, bool)
    np.put_along_axis(mask, ids, False, axis=1)
    assert (np.where(mask, L, -np.inf).max(axis=1) <= sel[:, -1]).all()
    # weight ratios are exp of logit differences
    np.testing.assert_allclose(w[:, 0] / w[:, 1], np.exp(sel[:, 0].astype(np.float64) - sel[:, 1]),
                               rtol=1e-13)


def test_shift_and_permutation():
    rng = np.random.default_rng(6)
    T, E, k = 20, 32, 4
    L = (rng.integers(-64, 64, size=(T, E)) / 8.0).astype(np.float32)   # exact in fp32
    ids, w = route_ref(L, k)
    ids2, w2 = route_ref(L + np.float32(4.0), k)                          # exact shift
    assert np.array_equal(ids, ids2)
    np.testing.assert_allclose(w, w2, rtol=1e-14)
    perm = rng.permutation(E)
    # relabel expert e as perm[e]; with ties, the tie order follows the new labels
    Lp = np.empty_like(L)
    Lp[:, perm] = L
    ids_p, w_p = route_ref(Lp, k)
    sel = np.sort(np.take_along_axis(L, ids, axis=1), axis=1)
    sel_p = np.sort(np.take_along_axis(Lp, ids_p, axis=1), axis=1)
    assert np.array_equal(sel, sel_p)
    np.testing.assert_allclose(np.sort(w, axis=1), np.sort(w_p, axis=1), rtol=1e-14)


def test_empty_batch():
    ids, w = route_ref(np.zeros((0, 8), np.float32), 3)
    assert ids.shape == (0, 3) and w.shape == (0, 3)


# planted mistakes: each must make a pin above fail

def _ties_high(L, top_k):
    return np.argsort(-L[:, ::-1], axis=1, kind="stable")[:, :top_k] * -1 + (L.shape[1] - 1)


def _ascending(L, top_k):
    return np.argsort(-L, axis=1, kind="stable")[:, :top_k][:, ::-1]


def _no_renorm(L, ids):
    return np.take_along_axis(router._softmax(L), ids, axis=1)


def _softmax_sign(L):
    m = np.min(L, axis=1, keepdims=True)
    e = np.exp(m - L)
    return e / np.sum(e, axis=1, keepdims=True)


MUTATIONS = {
    "ties_to_higher_id": ("_select", _ties_high),
    "ascending_order": ("_select", _ascending),
    "no_renormalization": ("_weights", _no_renorm),
    "softmax_sign_flipped": ("_softmax", _softmax_sign),
}

PINS = [test_golden_cases, lambda: test_brute_force(5, 16, 6, 1), test_masked_experts_brute_force,
        test_invariants]


def _pins_hold():
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            return False
    return True


def test_unmutated_pins_hold():
    assert _pins_hold()


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(router, attr, fn)
    assert not _pins_hold(), f"{name} passed every pin"
