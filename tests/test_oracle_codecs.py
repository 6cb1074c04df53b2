"""Pins for the oracle's number codecs (CPU only).

The codecs are checked against (a) hand-derived values from the format
definitions (tests/golden/codecs.json), (b) an independent implementation
(torch's float8_e4m3fn / bfloat16 casts), and (c) brute-force nearest search
over every representable value.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import codecs

GOLD = os.path.join(os.path.dirname(__file__), "golden", "codecs.json")


def _num(s):
    if s == "nan":
        return float("nan")
    return float(eval(s, {"__builtins__": {}}))  # arithmetic literals only


def _int(s):
    return int(s, 16) if s.startswith("0x") else int(s)


@pytest.fixture(scope="module")
def gold():
    with open(GOLD) as f:
        return json.load(f)


def test_e4m3_decode_golden(gold):
    for code, val in gold["e4m3_decode"].items():
        got = codecs.e4m3_decode(np.array([_int(code)], np.uint8))[0]
        want = _num(val)
        if math.isnan(want):
            assert math.isnan(got), code
        else:
            assert got == want, (code, got, want)


def test_e4m3_decode_vs_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    mine = codecs.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])
    # exactly two NaN codes, max finite 448
    assert nan.sum() == 2
    assert np.nanmax(mine) == 448.0 and np.nanmin(mine) == -448.0


def test_e4m3_encode_golden(gold):
    for val, code in gold["e4m3_encode"].items():
        got = codecs.e4m3_encode(np.array([_num(val)]))[0]
        assert got == _int(code), (val, hex(got), code)


def test_e4m3_roundtrip_every_code():
    codes = np.arange(256, dtype=np.uint8)
    vals = codecs.e4m3_decode(codes)
    fin = ~np.isnan(vals)
    back = codecs.e4m3_encode(vals[fin])
    assert np.array_equal(back, codes[fin])


def test_e4m3_midpoints_round_to_even():
    codes = np.arange(0, 0x7E, dtype=np.uint8)          # positive finite, below max
    lo = codecs.e4m3_decode(codes)
    hi = codecs.e4m3_decode(codes + 1)
    mid = (lo + hi) / 2.0
    got = codecs.e4m3_encode(mid)
    want = np.where(codes % 2 == 0, codes, codes + 1)
    assert np.array_equal(got, want.astype(np.uint8))
    # and the negative side mirrors it
    got_n = codecs.e4m3_encode(-mid)
    assert np.array_equal(got_n, (want | 0x80).astype(np.uint8))


def test_e4m3_encode_brute_force_nearest():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.normal(0, 100, 4000), rng.normal(0, 0.01, 2000),
                        rng.uniform(-600, 600, 1000)])
    got = codecs.e4m3_encode(v)
    table = codecs.e4m3_decode(np.arange(256, dtype=np.uint8))
    finite_codes = np.array([c for c in range(256) if not math.isnan(table[c])])
    for x, g in zip(v, got):
        xs = min(max(x, -448.0), 448.0)                  # saturation
        d = np.abs(table[finite_codes] - xs)
        best = d.min()
        cands = finite_codes[d == best]
        if len(cands) > 1:                               # tie: even mantissa
            cands = [c for c in cands if c % 2 == 0 or (c & 0x7F) == 0]
            if xs == 0:
                cands = [0x80 if math.copysign(1, x) < 0 else 0x00]
        assert g in cands, (x, hex(g), [hex(c) for c in cands])


def test_e4m3_encode_vs_torch_in_range():
    rng = np.random.default_rng(2)
    v = rng.uniform(-448, 448, 20000).astype(np.float32)
    v[:5000] = (v[:5000] * 1e-3).astype(np.float32)
    mine = codecs.e4m3_encode(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mine, ref)


def test_e8m0_golden(gold):
    for code, val in gold["e8m0_decode"].items():
        got = codecs.e8m0_decode(np.array([int(code)]))[0]
        want = _num(val)
        assert (math.isnan(got) and math.isnan(want)) or got == want


def test_bf16_golden(gold):
    for val, code in gold["bf16_encode"].items():
        got = codecs.bf16_encode(np.array([_num(val)]))[0]
        assert got == _int(code), (val, hex(got), code)


def test_bf16_vs_torch_for_fp32_inputs():
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.normal(0, 1, 20000), rng.normal(0, 1e-39, 2000),
                        rng.normal(0, 1e37, 2000)]).astype(np.float32)
    mine = codecs.bf16_encode(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    back = codecs.bf16_decode(mine)
    ref_back = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(back, ref_back)


def test_bf16_round_fp64_brute_force():
    """One rounding from fp64: the result is a bf16 value and no neighbour is
    closer; exact ties pick the even pattern."""
    rng = np.random.default_rng(4)
    v = rng.normal(0, 1, 3000) * np.exp2(rng.integers(-60, 60, 3000))
    bits = codecs.bf16_encode(v).astype(np.int64)
    for x, b in zip(v, bits):
        cands = [b - 1, b, b + 1]
        vals = [codecs.bf16_decode(np.array([c & 0xFFFF], np.uint16))[0] for c in cands]
        d = [abs(y - x) for y in vals]
        assert d[1] <= d[0] and d[1] <= d[2]
        if d[1] == d[0] or d[1] == d[2]:
            assert b % 2 == 0


def test_e2m1_decode_golden(gold):
    for code, val in gold["e2m1_decode"].items():
        got = codecs.e2m1_decode(np.array([_int(code)], np.uint8))[0]
        want = _num(val)
        assert got == want and math.copysign(1.0, got) == math.copysign(1.0, want), (code, got)


def test_e2m1_table_shape():
    t = codecs.E2M1_TABLE
    assert np.all(np.isfinite(t))
    assert np.array_equal(t[8:], -t[:8])                # sign bit
    assert np.all(np.diff(t[:8]) > 0)                   # codes 0..7 ascend
    assert t[:8].max() == 6.0 and t[1] == 0.5           # largest, smallest subnormal


def test_fp4_unpack_nibble_order():
    # element 2j in the low nibble of byte j, element 2j+1 in its high nibble
    got = codecs.fp4_unpack(np.array([[0x5A, 0x0F]], np.uint8))
    assert got.tolist() == [[0xA, 0x5, 0xF, 0x0]]
