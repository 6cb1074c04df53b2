"""The caller-side MXFP4 weight quantizer (input generation, shared by the
tests and the benchmark): every element is the nearest E2M1 magnitude of its
scaled value (ties to the even code, saturating at 6) under the OCP shared
exponent floor(log2 amax) - 2, checked by brute force over the 16 codes."""

import math

import numpy as np
import torch

import datagen
from oracle import codecs


def _brute(vals):
    """Expected (codes, e8m0) of one 32-element block, by exhaustive search."""
    amax = max(abs(v) for v in vals)
    s = -127 if amax == 0 else max(-127, min(127, math.frexp(amax)[1] - 1 - 2))
    codes = []
    for v in vals:
        a = min(abs(v) * 2.0 ** -s, 6.0)
        best = min(abs(codecs.E2M1_TABLE[c] - a) for c in range(8))
        cands = [c for c in range(8) if abs(codecs.E2M1_TABLE[c] - a) == best]
        c = [c for c in cands if c % 2 == 0][0] if len(cands) > 1 else cands[0]
        codes.append(c | (8 if v < 0 else 0))
    return codes, s + 127


def test_quant_mxfp4_matches_brute_force():
    g = torch.Generator().manual_seed(5)
    w = torch.randn(6, 96, generator=g) * 0.3
    w[0, :32] = 0.0                                           # all-zero block
    w[1, :32] = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * 4)  # exact ties
    w[2, 32:64] *= 1e6                                        # large exponents
    packed, sc = datagen.quant_mxfp4(w)
    codes = codecs.fp4_unpack(packed.numpy())
    for r in range(w.shape[0]):
        for b in range(w.shape[1] // 32):
            want, e = _brute([float(v) for v in w[r, 32 * b:32 * b + 32]])
            got = codes[r, 32 * b:32 * b + 32].tolist()
            # a negative value that rounds to zero may carry either sign bit
            got = [c if codecs.E2M1_TABLE[c] != 0 else 0 for c in got]
            want = [c if codecs.E2M1_TABLE[c] != 0 else 0 for c in want]
            assert got == want, (r, b)
            assert int(sc[r, b]) == e, (r, b)


def test_quant_mxfp4_tie_rounding():
    # scaled values exactly between two codes go to the even code
    w = torch.tensor([[0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * 4])
    packed, sc = datagen.quant_mxfp4(w)
    assert int(sc[0, 0]) == 127                               # amax 6 -> 2^(2-2)
    vals = codecs.e2m1_decode(codecs.fp4_unpack(packed.numpy()))[0, :8]
    assert vals.tolist() == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0]
