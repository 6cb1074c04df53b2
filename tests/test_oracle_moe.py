"""Pins for the expert-FFN oracle (CPU only).

* hand-derived requantization goldens (tests/golden/requant_*.json);
* a special case that reduces to a dense FFN written with np.matmul;
* per-token brute-force loops in plain Python, with requantization done by
  exhaustive nearest-code search (a different method from the oracle's);
* invariants: linearity in the routing weights, empty experts contribute
  nothing (their weights are NaN-poisoned), relabelling experts together with
  their weights changes nothing, routing weights sum to 1.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import datagen
from oracle import codecs
from oracle.moe import (LAMBDA, _flip_prob, _requant_blockwise, _requant_mx, _silu, gemm_sigma,
                        moe_ref, requant_blockwise, requant_bf16, requant_mx, route_flip_bound,
                        swiglu_band, tolerance_check)

HERE = os.path.dirname(__file__)


def _int(s):
    return int(s, 16)


# ---------------------------------------------------------------------------
# requantization goldens and properties
# ---------------------------------------------------------------------------

def test_requant_blockwise_golden():
    with open(os.path.join(HERE, "golden", "requant_blockwise.json")) as f:
        g = json.load(f)
    h = np.zeros((1, 256))
    for i, v in g["row_values"].items():
        h[0, int(i)] = v
    q, s, hd, alt = requant_blockwise(h)
    for i, c in g["expected_codes"].items():
        assert q[0, int(i)] == _int(c), (i, hex(q[0, int(i)]), c)
    assert np.all(q[0, 9:128] == 0)
    assert s[0, 0] == np.float32(eval(g["expected_scale"]))
    z = np.float32(np.float32(1e-10) * np.float32(9586981 * 2.0 ** -32))
    assert s[0, 1] == z and np.all(q[0, 128:] == 0)
    assert np.all(hd[0] == codecs.e4m3_decode(q[0]) * np.repeat(s[0].astype(np.float64), 128))


def test_requant_mx_golden():
    with open(os.path.join(HERE, "golden", "requant_mx.json")) as f:
        g = json.load(f)
    n = len(g["groups"])
    h = np.zeros((1, 32 * n))
    for gi, grp in enumerate(g["groups"]):
        for i, v in grp["values"].items():
            h[0, 32 * gi + int(i)] = v
    q, s, hd, alt = requant_mx(h)
    for gi, grp in enumerate(g["groups"]):
        assert s[0, gi] == grp["expected_e8m0"]
        for i, c in grp["expected_codes"].items():
            assert q[0, 32 * gi + int(i)] == _int(c)
        rest = [j for j in range(32) if str(j) not in grp["expected_codes"]]
        assert np.all(q[0, [32 * gi + j for j in rest]] == 0)


def test_requant_blockwise_properties():
    rng = np.random.default_rng(11)
    h = rng.normal(0, 3, (64, 512)) * np.exp2(rng.integers(-20, 20, (64, 1)))
    q, s, hd, _ = requant_blockwise(h)
    mag = q & 0x7F
    assert np.all(mag <= 0x7E)                                # |q| <= 448
    # the amax element of each group lands on +-448
    grp = np.abs(codecs.fp32(h)).reshape(64, 4, 128)
    arg = np.argmax(grp, axis=2)
    qg = q.reshape(64, 4, 128)
    top = np.take_along_axis(qg, arg[:, :, None], axis=2)[:, :, 0]
    assert np.all((top & 0x7F) == 0x7E)
    # relative quantization error within e4m3's half-spacing (2^-4) of amax*...
    rel = np.abs(hd - h) / np.repeat(grp.max(axis=2), 128, axis=1).reshape(64, 512)
    assert rel.max() <= 2.0 ** -4 * 1.0001


def test_requant_mx_properties():
    rng = np.random.default_rng(12)
    h = rng.normal(0, 1, (32, 256)) * np.exp2(rng.integers(-30, 30, (32, 1)))
    q, s, hd, _ = requant_mx(h)
    amax = np.abs(codecs.fp32(h)).reshape(32, 8, 32).max(axis=2)
    assert np.all(s.astype(int) - 127 == np.floor(np.log2(amax)) - 8)
    # values already on the scaled grid round-trip exactly
    q2, s2, hd2, _ = requant_mx(hd)
    assert np.array_equal(hd2, hd) and np.array_equal(q2, q)


# ---------------------------------------------------------------------------
# brute force
# ---------------------------------------------------------------------------

TABLE = codecs.e4m3_decode(np.arange(256, dtype=np.uint8))
FIN = [c for c in range(256) if not math.isnan(TABLE[c])]


def nearest_e4m3(v):
    v = min(max(v, -448.0), 448.0)
    best = min(abs(TABLE[c] - v) for c in FIN)
    cands = [c for c in FIN if abs(TABLE[c] - v) == best]
    if len(cands) > 1:
        cands = [c for c in cands if c % 2 == 0]
    return TABLE[cands[0]]


def brute_requant(kind, h):
    f32 = np.float32
    h32 = [f32(v) for v in h]
    if kind == "bf16":
        return [float(torch.tensor(float(v), dtype=torch.float32).to(torch.bfloat16))
                for v in h32]
    out = []
    G = 128 if kind == "fp8_blockwise" else 32
    for g0 in range(0, len(h32), G):
        grp = h32[g0:g0 + G]
        amax = max(abs(v) for v in grp)
        if kind == "fp8_blockwise":
            amax = max(amax, f32(1e-10))
            sf = f32(amax * f32(1.0 / 448.0))
            inv = f32(f32(1.0) / sf)
            out += [nearest_e4m3(float(f32(v * inv))) * float(sf) for v in grp]
        else:
            if amax == 0:
                s = -127
            else:
                _, ex = math.frexp(float(amax))
                s = max(-127, min(127, ex - 1 - 8))
            out += [nearest_e4m3(float(f32(float(v) * 2.0 ** -s))) * 2.0 ** s
                    for v in grp]
    return out


def brute_force(kind, d, t):
    x, xs, w1, s1, w2, s2 = d["x"], d["x_scale"], d["w1"], d["w1_scale"], d["w2"], d["w2_scale"]
    ids, wts = d["topk_ids"], d["topk_weights"]
    E, N, K = w1.shape
    if kind == "mxfp4":
        K *= 2
    I = N // 2

    def fp4(byte, c):  # element c of a packed row: low nibble holds the even index
        code = (byte >> 4) if c % 2 else (byte & 15)
        mag = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0][code & 7]
        return -mag if code & 8 else mag

    def deq(arr, scale, e, r, c, rowwise):
        if kind == "bf16":
            return float(codecs.bf16_decode(np.array([arr[e][r, c] if e is not None else arr[r, c]]))[0])
        if kind == "mxfp4" and e is not None:
            return fp4(int(arr[e][r, c // 2]), c) * 2.0 ** (int(scale[e][r, c // 32]) - 127)
        v = TABLE[arr[e][r, c] if e is not None else arr[r, c]]
        if kind == "fp8_blockwise":
            if rowwise:
                return v * float(scale[r, c // 128])
            return v * float(scale[e][r // 128, c // 128])
        sc = scale[e][r, c // 32] if e is not None else scale[r, c // 32]
        return v * 2.0 ** (int(sc) - 127)

    out = [0.0] * K
    xv = [deq(x, xs, None, t, c, True) for c in range(K)]
    for j in range(ids.shape[1]):
        e = int(ids[t, j])
        if not 0 <= e < E:
            continue
        g = [sum(xv[c] * deq(w1, s1, e, n, c, False) for c in range(K)) for n in range(I)]
        u = [sum(xv[c] * deq(w1, s1, e, I + n, c, False) for c in range(K)) for n in range(I)]
        h = [g[n] / (1.0 + math.exp(-g[n])) * u[n] for n in range(I)]
        hq = brute_requant(kind, h)
        for c in range(K):
            y = sum(hq[n] * deq(w2, s2, e, c, n, False) for n in range(I))
            out[c] += float(wts[t, j]) * y
    return np.array(out)


def small_case(kind, T, K, I, E, k, routing="normal", seed="pin"):
    c = datagen.make_case(kind, T, K, I, E, k, routing=routing, tag=seed)
    return datagen.to_numpy(c)


def run(d, **kw):
    return moe_ref(d["kind"], d["x"], d["x_scale"], d["w1"], d["w1_scale"], d["w2"],
                   d["w2_scale"], d["topk_ids"], d["topk_weights"], **kw)


@pytest.mark.parametrize("kind,K,I", [("bf16", 64, 32), ("fp8_blockwise", 256, 128),
                                      ("mxfp8", 64, 64), ("mxfp4", 64, 64)])
def test_brute_force_per_token(kind, K, I):
    d = small_case(kind, 4, K, I, 4, 2)
    ref = run(d)["out64"]
    for t in range(4):
        bf = brute_force(kind, d, t)
        np.testing.assert_allclose(ref[t], bf, rtol=1e-10, atol=1e-12 * np.abs(bf).max())


def test_brute_force_out_of_range_ids_skipped():
    d = small_case("fp8_blockwise", 3, 128, 128, 4, 2)
    d["topk_ids"] = d["topk_ids"].copy()
    d["topk_ids"][0, 1] = -1
    d["topk_ids"][2, 0] = 7
    ref = run(d)["out64"]
    for t in range(3):
        np.testing.assert_allclose(ref[t], brute_force("fp8_blockwise", d, t), rtol=1e-10,
                                   atol=1e-14)


def test_dense_ffn_special_case():
    """E=1, top-1 with weight 1 and no rounding of h is a dense SwiGLU FFN."""
    d = small_case("bf16", 16, 128, 64, 1, 1)
    d["topk_weights"] = np.ones_like(d["topk_weights"])
    out = run(d, exact_h=True)["out64"]
    X = codecs.bf16_decode(d["x"])
    W1 = codecs.bf16_decode(d["w1"][0])
    W2 = codecs.bf16_decode(d["w2"][0])
    gate = X @ W1[:64].T
    up = X @ W1[64:].T
    dense = (gate * (1.0 / (1.0 + np.exp(-gate))) * up) @ W2.T
    np.testing.assert_allclose(out, dense, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("kind,K,I", [("bf16", 128, 64), ("fp8_blockwise", 256, 256),
                                      ("mxfp8", 128, 64), ("mxfp4", 128, 64)])
def test_linearity_in_routing_weights(kind, K, I):
    d = small_case(kind, 8, K, I, 6, 3)
    full = run(d)["out64"]
    acc = np.zeros_like(full)
    for j in range(3):
        dj = dict(d)
        w = np.zeros_like(d["topk_weights"])
        w[:, j] = 1.0
        dj["topk_weights"] = w
        acc += d["topk_weights"][:, j:j + 1].astype(np.float64) * run(dj)["out64"]
    np.testing.assert_allclose(full, acc, rtol=1e-12, atol=1e-14 * np.abs(full).max())


@pytest.mark.parametrize("kind", ["bf16", "fp8_blockwise", "mxfp8", "mxfp4"])
def test_empty_experts_contribute_nothing(kind):
    d = small_case(kind, 4, 256, 128, 16, 2)
    base = run(d)["out64"]
    used = set(np.unique(d["topk_ids"]).tolist())
    empty = [e for e in range(16) if e not in used]
    assert empty
    p = {n: (v.copy() if isinstance(v, np.ndarray) else v) for n, v in d.items()}
    for e in empty:
        if kind == "bf16":
            p["w1"][e] = 0x7FC0
            p["w2"][e] = 0x7FC0
        else:
            p["w1"][e] = 0x7F
            p["w2"][e] = 0x7F
            if kind == "fp8_blockwise":
                p["w1_scale"][e] = np.nan
                p["w2_scale"][e] = np.nan
            else:
                p["w1_scale"][e] = 255
                p["w2_scale"][e] = 255
    out = run(p)["out64"]
    assert np.all(np.isfinite(out))
    assert np.array_equal(out, base)


def test_expert_relabelling_invariance():
    d = small_case("fp8_blockwise", 6, 256, 128, 8, 3)
    base = run(d)["out64"]
    perm = np.random.default_rng(5).permutation(8)
    p = dict(d)
    p["topk_ids"] = perm[d["topk_ids"]].astype(np.int32)
    for n in ("w1", "w1_scale", "w2", "w2_scale"):
        arr = np.empty_like(d[n])
        arr[perm] = d[n]
        p[n] = arr
    np.testing.assert_allclose(run(p)["out64"], base, rtol=1e-12, atol=1e-15)


def test_routing_weights_sum_to_one():
    for routing in ("uniform", "normal", "normal_masked", "zipf"):
        ids, w = datagen.make_routing(500, 64, 6, routing)
        s = w.double().sum(dim=1)
        assert torch.all((s - 1).abs() < 1e-6)
        assert torch.all(w > 0)
        # ids distinct per token
        assert all(len(set(r)) == 6 for r in ids.tolist())


def test_token_subset_matches_full():
    d = small_case("fp8_blockwise", 10, 256, 128, 8, 2)
    full = run(d)["out64"]
    sub = run(d, tokens=np.array([1, 4, 9]))["out64"]
    np.testing.assert_allclose(sub, full[[1, 4, 9]], rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------------------
# arithmetic model and near-tie allowance
# ---------------------------------------------------------------------------

def test_gemm_sigma_closed_form():
    """sigma_G = sqrt(KAPPA^2 Q + (u sqrt(steps + 2) (|G| + 3 sqrt Q))^2),
    worked by hand for all-ones operands: Q = K, G = K."""
    u = 2.0 ** -24
    for kind, K, kappa, block in (("fp8_blockwise", 256, 2.0 ** -15, 128),
                                  ("mxfp8", 4096, 2.0 ** -15, 128),
                                  ("bf16", 512, 2.0 ** -24, 32)):
        a = np.ones((1, K))
        b = np.ones((1, K))
        got = gemm_sigma(kind, a, b, a @ b.T)[0, 0]
        chain = u * math.sqrt(K / block + 2) * (K + 3 * math.sqrt(K))
        want = math.sqrt((kappa * math.sqrt(K)) ** 2 + chain ** 2)
        assert got == pytest.approx(want, rel=1e-12), kind


def test_gemm_sigma_grows_like_sqrt_k():
    """Random operands: the instruction term scales with sqrt(K) (the 2-norm
    of the K products), so quadrupling K doubles it."""
    rng = np.random.default_rng(3)
    a = rng.normal(size=(4, 4096))
    b = rng.normal(size=(3, 4096))
    s1 = gemm_sigma("fp8_blockwise", a[:, :1024], b[:, :1024], a[:, :1024] @ b[:, :1024].T)
    s4 = gemm_sigma("fp8_blockwise", a, b, a @ b.T)
    assert 1.7 < np.median(s4 / s1) < 2.3


def test_swiglu_band_first_order():
    """With a tiny GEMM deviation the band is LAMBDA times the propagated
    standard deviation: silu'(g) |up| sigma_g and silu(g) sigma_u add in
    quadrature (silu' checked against a centred difference of silu), plus
    the fp32 evaluation term (|g| + 6) u |h|."""
    g = np.array([[-6.0, -1.3, 0.0, 0.7, 2.4, 9.0]])
    v = np.array([[1.5, -2.0, 0.5, 3.0, -0.25, 1.0]])
    G = np.concatenate([g, v], axis=1)
    eps = 1e-9
    sG = np.full(G.shape, eps)
    h, band = swiglu_band(G, sG, g.shape[1])
    d = 1e-6
    dsilu = (_silu(g + d) - _silu(g - d)) / (2 * d)
    want = LAMBDA * np.sqrt((dsilu * v * eps) ** 2 + (_silu(g) * eps) ** 2) + \
        (np.abs(g) + 6) * 2.0 ** -24 * np.abs(h)
    np.testing.assert_allclose(h, _silu(g) * v, rtol=1e-15)
    np.testing.assert_allclose(band, want, rtol=1e-6)


def test_flip_prob_closed_forms():
    """A boundary at the kernel value's own position is crossed half the
    time; one at LAMBDA standard deviations with the Gaussian tail
    Phi(-LAMBDA) = erfc(LAMBDA / sqrt 2) / 2."""
    assert _flip_prob(0.0, 1.0) == pytest.approx(0.5)
    assert _flip_prob(1.0, 1.0) == pytest.approx(0.5 * math.erfc(LAMBDA / math.sqrt(2)), rel=1e-9)
    assert _flip_prob(0.5, 1.0) == pytest.approx(0.5 * math.erfc(LAMBDA / 2 / math.sqrt(2)), rel=1e-9)


def test_near_tie_alt_blockwise():
    """h = 2 sets sf_inv = 224 - 2^-16 (see the blockwise golden); an element
    whose scaled value sits on the 352/384 midpoint (368) is a near-tie with
    alternative distance one step (32 * sf); one 0.3 step away is not."""
    sf_inv = 224.0 - 2.0 ** -16
    h = np.zeros((1, 128))
    h[0, 0] = 2.0
    h[0, 1] = 368.0 / sf_inv * (1 + 1e-7)       # a hair above the midpoint
    h[0, 2] = (352.0 + 0.3 * 32) / sf_inv       # 30% into the step: clear
    band = np.full(h.shape, 1e-6)
    q, s, hd, alt = requant_blockwise(h, band)
    sf = float(s[0, 0])
    assert q[0, 1] == 0x7C                      # 384: rounds up
    assert alt[0, 1] == pytest.approx(32 * sf)
    assert alt[0, 2] == 0.0
    assert alt[0, 0] == 0.0                     # the amax element is 448, exact
    # with no GEMM deviation the fp32 roundings of sf, 1/sf and the product
    # (4 u relative) still reach a boundary 1e-7 away, but not 0.3 steps
    alt0 = requant_blockwise(h)[3]
    assert alt0[0, 1] == pytest.approx(32 * sf) and alt0[0, 2] == 0.0
    # the probability of the near-tie element is close to one half (the
    # boundary lies a small fraction of the band away)
    *_, prob, _, _ = _requant_blockwise(h, band)
    assert 0.3 < prob[0, 1] < 0.5 and prob[0, 2] == 0.0


def test_near_tie_alt_mx_scale():
    """amax a hair below a power of two, band reaching past it: the shared
    exponent is a near-tie; the group's move under the other exponent is the
    exact difference of the two dequantized groups."""
    h = np.zeros((1, 64))
    h[0, 0] = 4.0 * (1 - 1e-7)
    h[0, 1] = 1.3
    h[0, 33] = 3.0                              # second group: exponent clear
    band = np.full(h.shape, 1e-5)
    q, s, hd, alt, prob, _, (moved, dhd, alt2, gprob) = _requant_mx(h, band)
    assert s[0, 0] == 127 + 1 - 8               # floor(log2 3.9999996) = 1
    assert moved[0, 0] and not moved[0, 1]
    # exponent -6 (amax 4 reaches 2^2): 3.9999996 * 64 -> 256, 1.3 * 64 = 83.2 -> 80
    assert dhd[0, 0] == pytest.approx(4.0 - 448.0 / 128.0)  # 4 against 3.5 (saturated)
    assert dhd[0, 1] == pytest.approx(80.0 / 64.0 - 1.25)   # 1.25 under both
    assert np.all(dhd[0, 32:] == 0)
    assert 0.0 < gprob[0, 0] <= 0.5 and gprob[0, 1] == 0.0
    # public wrapper: the move is part of alt
    assert requant_mx(h, band)[3][0, 0] == pytest.approx(0.5)


def test_near_tie_alt_bf16():
    h = np.zeros((1, 128))
    h[0, 0] = 1.0
    h[0, 1] = 0.5 + 2.0 ** -9                   # midpoint (bf16 spacing at 0.5 is 2^-8)
    h[0, 2] = 0.5 + 2.0 ** -10                  # 2^-10 from the midpoint, band 2^-14
    band = np.full(h.shape, 2.0 ** -14)
    _, _, hd, alt = requant_bf16(h, band)
    assert alt[0, 1] == pytest.approx(2.0 ** -8)
    assert alt[0, 2] == 0.0


def test_route_flip_bound_closed_forms():
    """One near-tie: its effect alt |w2_ci| exactly.  Two: min(sum, max + 3
    sqrt(p1 e1^2 + p2 e2^2)), worked by hand.  400 equal decisions taken with
    certainty: max + 3 * sqrt(400) = 61 times one effect (a random walk), below
    their sum (400)."""
    w2 = np.array([[1.0, -2.0, 0.5], [0.25, 4.0, -1.0]])   # K = 2, I = 3
    alt = np.array([[0.0, 0.1, 0.0]])
    prob = np.array([[0.0, 0.4, 0.0]])
    np.testing.assert_allclose(route_flip_bound(alt, prob, w2)[0], [0.2, 0.4])
    alt = np.array([[0.3, 0.1, 0.0]])
    prob = np.array([[0.5, 0.02, 0.0]])
    e = np.array([[0.3 * 1.0, 0.1 * 2.0], [0.3 * 0.25, 0.1 * 4.0]])  # [col][decision]
    want = [min(e[c].sum(), e[c].max() + 3 * math.sqrt(0.5 * e[c, 0] ** 2 + 0.02 * e[c, 1] ** 2))
            for c in range(2)]
    np.testing.assert_allclose(route_flip_bound(alt, prob, w2)[0], want)
    w2 = np.ones((1, 400))
    alt = np.full((1, 400), 0.01)
    got = route_flip_bound(alt, np.ones((1, 400)), w2)[0, 0]
    assert got == pytest.approx(0.61)


def test_route_flip_bound_mx_group_exact():
    """An MX group whose exponent is a near-tie is one decision: the kernel
    taking the other exponent (its amax nudged across the power of two,
    within the band) changes the down GEMM's outputs by at most the bound;
    the group term is what covers it (the element near-ties alone do not)."""
    rng = np.random.default_rng(8)
    h = rng.normal(0, 0.6, (1, 64))
    h[0, 5] = 4.0 * (1 - 1e-7)                  # group 0: amax just below 4
    band = np.full(h.shape, 1e-6)
    w2 = rng.normal(0, 1, (48, 64))
    q, s, hd, alt, prob, _, groups = _requant_mx(h, band)
    assert groups[0][0, 0]
    bound = route_flip_bound(alt, prob, w2, groups)[0]
    hk = h.copy()
    hk[0, 5] = 4.0 * (1 + 1e-7)                 # the kernel's h: across 4
    hd_k = requant_mx(hk)[2]
    moved = np.abs((hd_k - hd) @ w2.T)[0]
    assert np.max(moved) > 0.05
    assert np.all(moved <= bound + 1e-12)
    no_group = route_flip_bound(alt, prob, w2, None)[0]
    assert np.any(moved > no_group)


@pytest.mark.parametrize("kind,K,I,T", [("fp8_blockwise", 512, 384, 600), ("mxfp8", 256, 256, 300),
                                        ("bf16", 256, 256, 300)])
def test_allowance_covers_model_deviation(kind, K, I, T):
    """Soundness of the allowance: move h by a deviation of the model's size
    (normal, standard deviation band / LAMBDA) and requantize.  The moved
    outputs pass the gate with the allowance; for the blockwise case some
    codes flip and the strict bound alone fails (so the near-ties are real
    and the allowance is what covers them)."""
    d = small_case(kind, T, K, I, 8, 4, routing="uniform", seed="tie")
    base = run(d)
    rng = np.random.default_rng(1)

    def perturb(h, band):
        return h + rng.normal(size=h.shape) * band / LAMBDA

    moved = run(d, h_perturb=perturb)
    tol = 2e-2 if kind != "bf16" else 5e-3
    got = codecs.bf16_encode(moved["out64"])
    ok, stats = tolerance_check(got, base["out64"], tol, base["allowance"])
    assert ok, stats
    if kind == "fp8_blockwise":
        _, strict = tolerance_check(got, base["out64"], tol, None)
        assert strict["n_over_bound"] > 0


def test_allowance_covers_band_edge_deviation():
    """Harder than the model: every element of h moved by up to its whole
    band (uniform in [-band, band]), so a large share of the flagged
    decisions flip; the gate still accepts."""
    for kind in ("fp8_blockwise", "mxfp8"):
        d = small_case(kind, 200, 512, 256, 8, 4, routing="uniform", seed="edge")
        base = run(d)
        rng = np.random.default_rng(2)
        moved = run(d, h_perturb=lambda h, band: h + rng.uniform(-1, 1, h.shape) * band)
        ok, stats = tolerance_check(codecs.bf16_encode(moved["out64"]), base["out64"], 2e-2,
                                    base["allowance"])
        assert ok, (kind, stats)


def test_mxfp4_equals_mxfp8_on_exact_reencoding():
    """Every E2M1 value is exact in e4m3: MXFP4 weights re-encoded as MX FP8
    codes with the same e8m0 exponents describe the same numbers, so both
    paths must give bit-identical results (pins the MXFP4 weight decode to the
    pinned MX FP8 path)."""
    d = small_case("mxfp4", 5, 128, 64, 3, 2)
    out4 = run(d)
    d8 = dict(d)
    d8["kind"] = "mxfp8"
    for wk in ("w1", "w2"):
        d8[wk] = codecs.e4m3_encode(codecs.e2m1_decode(codecs.fp4_unpack(d[wk])))
    assert np.array_equal(codecs.e4m3_decode(d8["w1"]),
                          codecs.e2m1_decode(codecs.fp4_unpack(d["w1"])))
    out8 = run(d8)
    assert np.array_equal(out4["out64"], out8["out64"])
    assert np.array_equal(out4["out_bf16"], out8["out_bf16"])
