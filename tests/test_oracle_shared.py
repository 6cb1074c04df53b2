"""Pins for the oracle's shared experts (CPU only).  A shared expert takes
every token with weight 1 and is computed like a routed expert; the pins:
shared experts alone (no valid route) reduce to a dense SwiGLU FFN written
with np.matmul; a per-token brute-force loop; additivity over shared
experts and independence from the routing weights; planted mistakes."""

import numpy as np
import pytest

import datagen
import oracle.moe as om
from oracle import codecs
from oracle.moe import moe_ref

from .test_oracle_moe import brute_force


def case(kind, T, K, I, E, k, S, seed="shared"):
    return datagen.to_numpy(datagen.make_case(kind, T, K, I, E, k, routing="normal", tag=seed,
                                              n_shared=S))


def run(d, **kw):
    kw.setdefault("n_shared", d["n_shared"])
    return moe_ref(d["kind"], d["x"], d["x_scale"], d["w1"], d["w1_scale"], d["w2"],
                   d["w2_scale"], d["topk_ids"], d["topk_weights"], **kw)


def test_shared_only_is_a_dense_ffn():
    """No valid route (every id outside the routed experts) and one shared
    expert, h not rounded: the output is the dense SwiGLU FFN of the shared
    weights."""
    d = case("bf16", 12, 128, 64, 3, 2, 1)
    d["topk_ids"] = np.full_like(d["topk_ids"], -1)
    out = run(d, exact_h=True)["out64"]
    X = codecs.bf16_decode(d["x"])
    W1 = codecs.bf16_decode(d["w1"][3])
    W2 = codecs.bf16_decode(d["w2"][3])
    gate, up = X @ W1[:64].T, X @ W1[64:].T
    dense = (gate / (1.0 + np.exp(-gate)) * up) @ W2.T
    np.testing.assert_allclose(out, dense, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("kind,K,I", [("fp8_blockwise", 256, 128), ("mxfp8", 64, 64),
                                      ("mxfp4", 64, 64), ("bf16", 64, 32)])
def test_brute_force_with_shared(kind, K, I):
    """Per-token brute force: the routed routes, then each shared expert with
    weight 1 (ids of the shared experts in the routing are not routes)."""
    d = case(kind, 3, K, I, 3, 2, 2)
    d["topk_ids"] = d["topk_ids"].copy()
    d["topk_ids"][1, 0] = 3                  # a shared expert's index: not a route
    ref = run(d)["out64"]
    bd = dict(d)
    ids = np.where(d["topk_ids"] < 3, d["topk_ids"], -1)
    bd["topk_ids"] = np.concatenate([ids, np.tile([[3, 4]], (3, 1))], axis=1)
    bd["topk_weights"] = np.concatenate([d["topk_weights"], np.ones((3, 2), np.float32)], axis=1)
    for t in range(3):
        bf = brute_force(kind, bd, t)
        np.testing.assert_allclose(ref[t], bf, rtol=1e-10, atol=1e-12 * np.abs(bf).max())


def test_additive_and_independent_of_routing_weights():
    d = case("fp8_blockwise", 10, 256, 128, 4, 2, 2)
    full = run(d)["out64"]
    routed = dict(d, w1=d["w1"][:4], w2=d["w2"][:4], w1_scale=d["w1_scale"][:4],
                  w2_scale=d["w2_scale"][:4])
    part = [run(routed, n_shared=0)["out64"]]
    for s in range(2):
        one = dict(d, w1=d["w1"][[4 + s]], w2=d["w2"][[4 + s]], w1_scale=d["w1_scale"][[4 + s]],
                   w2_scale=d["w2_scale"][[4 + s]], topk_ids=np.full_like(d["topk_ids"], -1))
        part.append(run(one, n_shared=1)["out64"])
    np.testing.assert_allclose(full, sum(part), rtol=1e-12, atol=1e-12 * np.abs(full).max())
    zero = dict(d, topk_weights=np.zeros_like(d["topk_weights"]))
    np.testing.assert_allclose(run(zero)["out64"], part[1] + part[2], rtol=1e-12,
                               atol=1e-12 * np.abs(full).max())


def test_keep_h_keys_shared_routes():
    d = case("mxfp8", 5, 64, 64, 3, 2, 2)
    h = run(d, keep_h=True)["h"]
    T, k, S = 5, 2, 2
    assert all(T * k + t * S + s in h for t in range(T) for s in range(S))


def test_no_shared_is_unchanged():
    d = case("fp8_blockwise", 6, 256, 128, 4, 2, 0)
    a = run(d)["out64"]
    b = moe_ref(d["kind"], d["x"], d["x_scale"], d["w1"], d["w1_scale"], d["w2"], d["w2_scale"],
                d["topk_ids"], d["topk_weights"])["out64"]
    assert np.array_equal(a, b)


MUTATIONS = {
    "shared_index_off_by_one": ("_shared_expert", lambda e, s: e - 1 + s),
    "shared_weight_half": ("_shared_weight", lambda: 0.5),
}


def _pins_hold():
    try:
        test_shared_only_is_a_dense_ffn()
        test_brute_force_with_shared("fp8_blockwise", 256, 128)
        test_additive_and_independent_of_routing_weights()
    except AssertionError:
        return False
    return True


def test_unmutated_pins_hold():
    assert _pins_hold()


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(om, attr, fn)
    assert not _pins_hold(), f"{name} passed every pin"
