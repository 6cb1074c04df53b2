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


def _requant_256(h):
    q, s, hd, alt = ORIG["requant_blockwise"](h * (448.0 / 256.0))
    return q, s, hd * (256.0 / 448.0), alt


def _mx_shift(h):
    """MX requant with the shared exponent off by one (floor(log2 amax) - 7)."""
    rows, I = h.shape
    h32 = codecs.fp32(h).reshape(rows, I // 32, 32)
    amax = np.max(np.abs(h32), axis=2).astype(np.float64)
    lg = np.floor(np.log2(np.where(amax > 0, amax, 1.0)))
    s = np.where(amax > 0, np.clip(lg - 7, -127, 127), -127).astype(np.int64)
    p = codecs.fp32(h32.astype(np.float64) * np.ldexp(1.0, -s)[:, :, None])
    q = codecs.e4m3_encode(p.astype(np.float64))
    hd = codecs.e4m3_decode(q) * np.ldexp(1.0, s)[:, :, None]
    return q.reshape(rows, I), (s + 127).astype(np.uint8), hd.reshape(rows, I), np.zeros((rows, I))


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


ORIG = {"requant_blockwise": moe.requant_blockwise, "requant_mx": moe.requant_mx,
        "dequant_w": moe.dequant_w, "dequant_x": moe.dequant_x,
        "e4m3_decode": codecs.e4m3_decode, "fp4_unpack": codecs.fp4_unpack,
        "e2m1_decode": codecs.e2m1_decode}

MUTATIONS = {
    "gate_up_swapped": (moe, "_swiglu", _swap_gate_up),
    "silu_sign": (moe, "_silu", _silu_sign),
    "requant_1_over_256": (moe, "requant_blockwise", _requant_256),
    "mx_exponent_off_by_one": (moe, "requant_mx", _mx_shift),
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
