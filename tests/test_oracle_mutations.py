"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch each one: every mutation below must make at least one pin fail."""

import numpy as np
import pytest

import oracle.codecs as codecs
import oracle.moe as moe
from tests import test_oracle_codecs as tc
from tests import test_oracle_moe as tm


def _square_brute():
    """brute force on a shape with K == I so that a transposed w2 still fits."""
    d = tm.small_case("fp8_blockwise", 3, 128, 128, 3, 2, seed="mut")
    ref = tm.run(d)["out64"]
    for t in range(3):
        np.testing.assert_allclose(ref[t], tm.brute_force("fp8_blockwise", d, t),
                                   rtol=1e-10, atol=1e-14)


def _pins():
    checks = [
        lambda: tc.test_e4m3_decode_golden(tc.gold.__wrapped__()),
        tm.test_requant_blockwise_golden,
        tm.test_requant_mx_golden,
        tm.test_dense_ffn_special_case,
        lambda: tm.test_brute_force_per_token("fp8_blockwise", 128, 128),
        lambda: tm.test_brute_force_per_token("mxfp8", 64, 32),
        lambda: tm.test_brute_force_per_token("mxfp4", 64, 64),
        lambda: tc.test_e2m1_decode_golden(tc.gold.__wrapped__()),
        tc.test_fp4_unpack_nibble_order,
        _square_brute,
    ]
    failed = 0
    for c in checks:
        try:
            c()
        except AssertionError:
            failed += 1
    return failed


def _swap_gate_up(G, I):
    return moe._silu(G[:, I:]) * G[:, :I]


def _silu_sign(g):
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(g))


def _requant_256(h, band):
    out = list(ORIG["_requant_blockwise"](h * (448.0 / 256.0), band))
    out[2] = out[2] * (256.0 / 448.0)
    return tuple(out)


def _mx_shift(h, band):
    """MX requant with the shared exponent off by one (floor(log2 amax) - 7)."""
    rows, I = h.shape
    h32 = codecs.fp32(h).reshape(rows, I // 32, 32)
    amax = np.max(np.abs(h32), axis=2).astype(np.float64)
    lg = np.floor(np.log2(np.where(amax > 0, amax, 1.0)))
    s = np.where(amax > 0, np.clip(lg - 7, -127, 127), -127).astype(np.int64)
    p = codecs.fp32(h32.astype(np.float64) * np.ldexp(1.0, -s)[:, :, None])
    q = codecs.e4m3_encode(p.astype(np.float64))
    hd = codecs.e4m3_decode(q) * np.ldexp(1.0, s)[:, :, None]
    z = np.zeros((rows, I))
    groups = (np.zeros((rows, I // 32), dtype=bool), z, z, np.zeros((rows, I // 32)))
    return (q.reshape(rows, I), (s + 127).astype(np.uint8), hd.reshape(rows, I), z, z, None,
            groups)


def _dequant_w_T(kind, w, w_scale, e):
    m = ORIG["dequant_w"](kind, w, w_scale, e)
    return m.T if m.shape[0] == m.shape[1] else m


def _dequant_x_wrong_block(kind, x, x_scale, rows):
    v = ORIG["dequant_x"](kind, x, x_scale, rows)
    return v[:, ::-1] if kind != "bf16" else v


def _decode_bias8(codes):
    return ORIG["e4m3_decode"](codes) * 0.5


def _fp4_nibbles_swapped(packed):
    out = ORIG["fp4_unpack"](packed)
    return out.reshape(out.shape[:-1] + (-1, 2))[..., ::-1].reshape(out.shape)


def _e2m1_bias2(codes):
    # exponent bias 2 instead of 1: every normal value halves
    v = ORIG["e2m1_decode"](codes)
    return np.where(np.abs(v) >= 1.0, v * 0.5, v)


def _mxfp4_scale_per_16(kind, w, w_scale, e):
    if kind != "mxfp4":
        return ORIG["dequant_w"](kind, w, w_scale, e)
    v = codecs.e2m1_decode(codecs.fp4_unpack(w[e]))
    sc = np.repeat(codecs.e8m0_decode(w_scale[e]), 16, axis=1)
    return v * np.concatenate([sc, sc], axis=1)[:, :v.shape[1]]


ORIG = {"_requant_blockwise": moe._requant_blockwise, "_requant_mx": moe._requant_mx,
        "dequant_w": moe.dequant_w, "dequant_x": moe.dequant_x,
        "e4m3_decode": codecs.e4m3_decode, "fp4_unpack": codecs.fp4_unpack,
        "e2m1_decode": codecs.e2m1_decode}

MUTATIONS = {
    "gate_up_swapped": (moe, "_swiglu", _swap_gate_up),
    "silu_sign": (moe, "_silu", _silu_sign),
    "requant_1_over_256": (moe, "_requant_blockwise", _requant_256),
    "mx_exponent_off_by_one": (moe, "_requant_mx", _mx_shift),
    "w2_transposed": (moe, "dequant_w", _dequant_w_T),
    "x_columns_permuted": (moe, "dequant_x", _dequant_x_wrong_block),
    "e4m3_bias_8": (codecs, "e4m3_decode", _decode_bias8),
    "fp4_nibbles_swapped": (codecs, "fp4_unpack", _fp4_nibbles_swapped),
    "e2m1_bias_2": (codecs, "e2m1_decode", _e2m1_bias2),
    "mxfp4_scale_block_16": (moe, "dequant_w", _mxfp4_scale_per_16),
}


def test_unmutated_pins_pass():
    assert _pins() == 0


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    mod, attr, fn = MUTATIONS[name]
    monkeypatch.setattr(mod, attr, fn)
    assert _pins() > 0, name


# ---------------------------------------------------------------------------
# mistakes planted in the gate and in its arithmetic model
# ---------------------------------------------------------------------------

from tests import test_oracle_gate as tg  # noqa: E402

GATE_ORIG = {"bf16_half_ulp": codecs.bf16_half_ulp, "route_flip_bound": moe.route_flip_bound,
             "gemm_sigma": moe.gemm_sigma, "swiglu_band": moe.swiglu_band,
             "tolerance_check": moe.tolerance_check, "_alt_e4m3": moe._alt_e4m3}


def _gate_pins():
    checks = [
        tg.test_bf16_half_ulp_golden,
        tg.test_gate_next_code_rejected_midpoint_accepted,
        tg.test_gate_half_spacing_at_the_binade_the_kernel_reaches,
        tg.test_gate_rejects_nan_and_large_mean_error,
        tm.test_gemm_sigma_closed_form,
        tm.test_swiglu_band_first_order,
        tm.test_route_flip_bound_closed_forms,
        tm.test_route_flip_bound_mx_group_exact,
        tm.test_near_tie_alt_blockwise,
        lambda: tm.test_allowance_covers_model_deviation("fp8_blockwise", 512, 384, 600),
        lambda: tg.test_gate_rejects_weight_applied_twice("fp8_blockwise", 1024, 256),
    ]
    failed = 0
    for c in checks:
        try:
            c()
        except AssertionError:
            failed += 1
    return failed


def _half_ulp_doubled(values):
    return 2.0 * GATE_ORIG["bf16_half_ulp"](values)


def _half_ulp_at_ref(out_bits, out64, tol, allowance=None):
    """The half spacing taken at |out64| rather than at the largest value
    the kernel's fp32 result can reach."""
    got = codecs.bf16_decode(out_bits)
    ref = np.asarray(out64, dtype=np.float64)
    err = np.abs(got - ref)
    rms = float(np.sqrt(np.mean(ref * ref)))
    dev = tol * rms + (0.0 if allowance is None else allowance)
    ok = bool(np.all(err <= dev + codecs.bf16_half_ulp(ref))) and \
        float(np.sum(err) / np.sum(np.abs(ref))) <= 5e-3 and bool(np.all(np.isfinite(got)))
    return ok, {"n_over_bound": int(np.sum(err > dev + codecs.bf16_half_ulp(ref)))}


def _allowance_ignored(out_bits, out64, tol, allowance=None):
    return GATE_ORIG["tolerance_check"](out_bits, out64, tol, None)


def _flip_no_groups(alt, prob, w2d, groups=None):
    return GATE_ORIG["route_flip_bound"](alt, prob, w2d, None)


def _flip_max_only(alt, prob, w2d, groups=None):
    """Only the largest decision's effect (no random walk of the others)."""
    return GATE_ORIG["route_flip_bound"](alt, np.zeros_like(prob), w2d, groups)


def _sigma_linear_in_k(kind, a, b, G):
    return GATE_ORIG["gemm_sigma"](kind, a, b, G) * np.sqrt(a.shape[1])


def _band_no_derivative(G, sigma_G, I):
    """The gate deviation propagated with silu(g) in place of silu'(g)."""
    h, _ = GATE_ORIG["swiglu_band"](G, sigma_G, I)
    g, v = G[:, :I], G[:, I:]
    sg, sv = sigma_G[:, :I], sigma_G[:, I:]
    silu = moe._silu(g)
    band = moe.LAMBDA * np.sqrt((silu * v * sg) ** 2 + (silu * sv) ** 2) + \
        (np.abs(g) + 6.0) * moe.U32 * np.abs(h)
    return h, band


def _alt_no_band(p, band):
    return GATE_ORIG["_alt_e4m3"](p, np.zeros_like(p))


GATE_MUTATIONS = {
    "bf16_half_ulp_doubled": (codecs, "bf16_half_ulp", _half_ulp_doubled),
    "half_ulp_at_ref_binade": (moe, "tolerance_check", _half_ulp_at_ref),
    "allowance_ignored": (moe, "tolerance_check", _allowance_ignored),
    "mx_group_term_dropped": (moe, "route_flip_bound", _flip_no_groups),
    "random_walk_dropped": (moe, "route_flip_bound", _flip_max_only),
    "sigma_grows_like_k": (moe, "gemm_sigma", _sigma_linear_in_k),
    "silu_derivative_wrong": (moe, "swiglu_band", _band_no_derivative),
    "near_tie_band_ignored": (moe, "_alt_e4m3", _alt_no_band),
}


def test_unmutated_gate_pins_pass():
    assert _gate_pins() == 0


@pytest.mark.parametrize("name", sorted(GATE_MUTATIONS))
def test_gate_mutation_is_caught(name, monkeypatch):
    mod, attr, fn = GATE_MUTATIONS[name]
    monkeypatch.setattr(mod, attr, fn)
    if mod is moe:
        # the tests import these names directly
        for t in (tm, tg):
            if hasattr(t, attr):
                monkeypatch.setattr(t, attr, fn)
    assert _gate_pins() > 0, name
