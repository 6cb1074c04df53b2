"""Number-format codecs for the oracle, written from the format definitions.

Test infrastructure (see the package docstring): used only by the tests, the
smoke check and the CPU baseline.

Formats
-------
* e4m3 -- OCP 8-bit floating point "E4M3FN": 1 sign bit, 4 exponent bits with
  bias 7, 3 mantissa bits; exponent field 0 holds subnormals m * 2^-9; the
  all-ones code (S.1111.111) is NaN; there is no infinity, so the largest
  finite magnitude is 1.75 * 2^8 = 448.  The [DeepGEMM #88] page ("Before you
  merge" section) fixes 448 as the largest code in its requantization
  expression; the [prime-flash] page ("Two data types" table) names e4m3 for
  values.
* e8m0 -- OCP MX shared scale: an 8-bit biased exponent, value 2^(c - 127);
  code 255 is NaN.  [prime-flash] "Scale layout (mxfp8)" section: e8m0 block
  scales, block 32 along K.
* bfloat16 -- the top 16 bits of an IEEE binary32: 8 exponent bits (bias 127),
  7 stored mantissa bits, subnormals below 2^-126 with spacing 2^-133.
  [prime-flash] "Shapes" table: out is bf16; "Two data types" table: the bf16
  path.

* e2m1 -- OCP MX FP4 element "E2M1": 1 sign bit, 2 exponent bits with bias 1,
  1 mantissa bit; exponent field 0 holds the subnormal m * 0.5; no infinity
  and no NaN, so the magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6.  The
  [DeepGEMM #411] page ("Summary") keeps routed weights as packed MXFP4:
  E2M1 elements with one UE8M0 (= e8m0) exponent per 32 along K.  Packing:
  two elements per byte, the one with the lower index in the low nibble.

Rounding: every encoder rounds to nearest, ties to even, once, from the exact
fp64 input.  e4m3 saturates to +-448 (the reading that an out-of-range
product after scaling by 1/amax*448 must land on the largest code, since the
format has no infinity).  bfloat16 overflows to +-inf as IEEE rounding does.
"""

import numpy as np

E4M3_MAX = 448.0


def _e4m3_decode_one(code):
    """Value of one e4m3 code (0..255) from the bit fields; NaN for S.1111.111."""
    s = -1.0 if (code >> 7) & 1 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * (m / 8.0) * 2.0 ** -6  # subnormal: m * 2^-9
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


# 256-entry decode table built from the bit-field definition above.
E4M3_TABLE = np.array([_e4m3_decode_one(c) for c in range(256)], dtype=np.float64)


def e4m3_decode(codes):
    """uint8 e4m3 codes -> fp64 values (exact)."""
    codes = np.asarray(codes, dtype=np.uint8)
    return E4M3_TABLE[codes]


def e4m3_encode(values):
    """fp64 values -> uint8 e4m3 codes, round to nearest even, saturating.

    Magnitudes above 448 become 448.  NaN becomes the positive NaN code 0x7F.
    Zero keeps its sign.
    """
    v = np.asarray(values, dtype=np.float64)
    sign = np.signbit(v)
    a = np.abs(v)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, a)
    # binade exponent; below the smallest normal (2^-6) the spacing stays 2^-9
    with np.errstate(divide="ignore"):
        ex = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    ex = np.maximum(ex, -6.0)
    # guard against log2 rounding at exact binade edges
    ex = np.where(a >= 2.0 ** (ex + 1), ex + 1, ex)
    ex = np.where((a < 2.0 ** ex) & (ex > -6), ex - 1, ex)
    ulp = 2.0 ** (ex - 3)
    q = np.rint(a / ulp) * ulp          # exact scaling, one RNE rounding
    q = np.minimum(q, E4M3_MAX)         # saturate
    # encode magnitude
    normal = q >= 2.0 ** -6
    with np.errstate(divide="ignore"):
        qe = np.floor(np.log2(np.where(normal, q, 1.0)))
    qe = np.where(normal & (q >= 2.0 ** (qe + 1)), qe + 1, qe)
    qe = np.where(normal & (q < 2.0 ** qe), qe - 1, qe)
    mant_n = np.where(normal, q / 2.0 ** qe * 8.0 - 8.0, 0.0)
    code_n = (qe + 7).astype(np.int64) * 8 + np.rint(mant_n).astype(np.int64)
    code_s = np.rint(q / 2.0 ** -9).astype(np.int64)
    code = np.where(normal, code_n, code_s)
    code = np.where(sign, code | 0x80, code)
    code = np.where(nan, 0x7F, code)
    return code.astype(np.uint8)


def _e2m1_decode_one(code):
    """Value of one e2m1 code (0..15) from the bit fields."""
    s = -1.0 if (code >> 3) & 1 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        return s * m * 0.5                        # subnormal: m * 2^(1-1) * 0.5
    return s * (1.0 + m / 2.0) * 2.0 ** (e - 1)


# 16-entry decode table built from the bit-field definition above.
E2M1_TABLE = np.array([_e2m1_decode_one(c) for c in range(16)], dtype=np.float64)


def fp4_unpack(packed):
    """uint8 (..., C/2) packed e2m1 pairs -> uint8 codes (..., C): element 2j
    from the low nibble of byte j, element 2j+1 from its high nibble."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


def e2m1_decode(codes):
    """uint8 e2m1 codes (0..15) -> fp64 values (exact)."""
    return E2M1_TABLE[np.asarray(codes, dtype=np.uint8)]


def e8m0_decode(codes):
    """uint8 e8m0 codes -> fp64 powers of two 2^(c-127); 255 -> NaN."""
    c = np.asarray(codes, dtype=np.int64)
    out = np.ldexp(1.0, c - 127)
    return np.where(c == 255, np.nan, out)


def bf16_decode(bits):
    """uint16 bfloat16 bit patterns -> fp64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_round(values):
    """fp64 -> fp64 value of the nearest bfloat16 (ties to even), one rounding.

    Overflow past the largest finite bf16 goes to +-inf; NaN stays NaN.
    """
    v = np.asarray(values, dtype=np.float64)
    a = np.abs(v)
    fin = np.isfinite(a) & (a > 0)
    aa = np.where(fin, a, 1.0)
    ex = np.floor(np.log2(aa))
    ex = np.where(aa >= 2.0 ** (ex + 1), ex + 1, ex)
    ex = np.where(aa < 2.0 ** ex, ex - 1, ex)
    ex = np.maximum(ex, -126.0)            # subnormal spacing 2^-133
    ulp = 2.0 ** (ex - 7)
    q = np.rint(aa / ulp) * ulp
    q = np.where(q >= 2.0 ** 128, np.inf, q)
    q = np.where(fin, q, a)                # 0, inf, nan pass through
    return np.copysign(q, v)


def bf16_encode(values):
    """fp64 -> uint16 bfloat16 bit patterns (RNE, one rounding)."""
    q = bf16_round(values)
    # q is exactly representable in bf16, hence in fp32: take the top half
    return (q.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def bf16_half_ulp(values):
    """Half the bfloat16 spacing at each value's magnitude (for tolerances)."""
    a = np.abs(np.asarray(values, dtype=np.float64))
    aa = np.where(a > 0, a, 2.0 ** -126)
    ex = np.floor(np.log2(aa))
    ex = np.maximum(ex, -126.0)
    return 2.0 ** (ex - 8)


def fp32(values):
    """Round fp64 values to the nearest binary32 (RNE), returned as float32."""
    return np.asarray(values, dtype=np.float64).astype(np.float32)
