"""Pins for the parity gate (CPU only): what it accepts and what it rejects.

The gate (oracle.moe.tolerance_check with moe_ref's allowance) must accept a
correct kernel's fp32 rounding differences and reject plausible kernel
mistakes.  The mistakes are planted in the oracle's own result on the CPU:
* one 128-wide K block of one route's activations dropped;
* one route's weight applied twice;
* one route dropped;
* an MX group decoded with the wrong shared exponent where the exponent is
  not a near-tie.
Each planted case must fail the gate with the allowance.  The half-spacing
term of the gate is pinned by hand-derived bfloat16 spacings.
"""

import math

import numpy as np
import pytest

import oracle.moe as om
from oracle import codecs
from tests.test_oracle_moe import run, small_case

TOL = {"bf16": 5e-3, "fp8_blockwise": 2e-2, "mxfp8": 2e-2, "mxfp4": 2e-2}


# ---------------------------------------------------------------------------
# the half-spacing term
# ---------------------------------------------------------------------------

def test_bf16_half_ulp_golden():
    """bfloat16 keeps 8 significant bits: the spacing in [2^e, 2^(e+1)) is
    2^(e-7), half of it 2^(e-8); below 2^-126 the spacing is 2^-133."""
    v = np.array([1.0, 1.99, 2.0, 0.75, 3.0 * 2.0 ** -130, 0.0, -6.0, 2.0 ** 100])
    want = np.array([2.0 ** -8, 2.0 ** -8, 2.0 ** -7, 2.0 ** -9, 2.0 ** -134, 2.0 ** -134,
                     2.0 ** -6, 2.0 ** 92])
    np.testing.assert_array_equal(codecs.bf16_half_ulp(v), want)


def test_gate_next_code_rejected_midpoint_accepted():
    """tol 0, no allowance: a value on the bf16 grid must come back exactly
    (its neighbour, one spacing off, fails); a value on a midpoint may come
    back as either neighbour (half a spacing off)."""
    ref = np.array([1.5, -0.375, 3.0])
    ok, _ = om.tolerance_check(codecs.bf16_encode(ref), ref, 0.0)
    assert ok
    nxt = ref + np.array([2.0 ** -7, 0.0, 0.0])
    ok, st = om.tolerance_check(codecs.bf16_encode(nxt), ref, 0.0)
    assert not ok and st["n_over_bound"] == 1
    mid = np.array([1.5 + 2.0 ** -8, -0.375, 3.0])
    for got in (1.5, 1.5 + 2.0 ** -7):
        ok, _ = om.tolerance_check(codecs.bf16_encode(np.array([got, -0.375, 3.0])), mid, 0.0)
        assert ok


def test_gate_half_spacing_at_the_binade_the_kernel_reaches():
    """ref just below 2 with a deviation bound of 2^-7 + 2^-11: the kernel's
    fp32 value can pass the midpoint 2 + 2^-7 of the binade above, where the
    spacing is 2^-6, and round up to 2 + 2^-6 (an error of 2^-6 + 2^-12, more
    than the deviation plus half a spacing at ref's own binade); 2 + 2^-5 is
    out of reach."""
    ref = np.array([2.0 - 2.0 ** -12] + [1.0] * 9)      # exact elements keep the mean error low
    allowance = np.array([2.0 ** -7 + 2.0 ** -11] + [0.0] * 9)
    for got, want in ((2.0, True), (2.0 + 2.0 ** -6, True), (2.0 + 2.0 ** -5, False)):
        ok, st = om.tolerance_check(codecs.bf16_encode(np.array([got] + [1.0] * 9)), ref, 0.0,
                                    allowance)
        assert ok == want, (got, st)


def test_gate_rejects_nan_and_large_mean_error():
    ref = np.linspace(-1, 1, 1000)
    bad = ref.copy()
    bad[3] = np.nan
    assert not om.tolerance_check(codecs.bf16_encode(bad), ref, 2e-2)[0]
    # every element 1% of rms high: inside the element bound, but the mean
    # relative error is about 1.7e-2 > 5e-3
    rms = math.sqrt(np.mean(ref * ref))
    shifted = ref + 0.01 * rms
    ok, st = om.tolerance_check(codecs.bf16_encode(shifted), ref, 2e-2)
    assert st["n_over_bound"] == 0 and not ok


# ---------------------------------------------------------------------------
# planted kernel mistakes
# ---------------------------------------------------------------------------

def _one_route(d, t, j, w=None):
    """Oracle output of route (t, j) alone (weight w, default its own)."""
    dj = dict(d)
    wts = np.zeros_like(d["topk_weights"])
    wts[t, j] = d["topk_weights"][t, j] if w is None else w
    dj["topk_weights"] = wts
    return run(dj, tokens=np.array([t]))["out64"][0]


def _gate(kind, mutated, ref):
    return om.tolerance_check(codecs.bf16_encode(mutated), ref["out64"], TOL[kind],
                              ref["allowance"])


CASES = [("fp8_blockwise", 4096, 512), ("fp8_blockwise", 1024, 256), ("mxfp8", 4096, 256),
         ("mxfp4", 2048, 256), ("bf16", 512, 256)]


@pytest.mark.parametrize("kind,K,I", CASES)
def test_gate_rejects_dropped_k_block(kind, K, I):
    d = small_case(kind, 8, K, I, 8, 4, seed="gate")
    ref = run(d)
    assert om.tolerance_check(ref["out_bf16"], ref["out64"], TOL[kind], ref["allowance"])[0]
    t, j = 2, 1
    y = _one_route(d, t, j)
    dx = dict(d)
    x = d["x"].copy()
    x[t, 128:256] = 0                           # one 128-wide block of K
    dx["x"] = x
    y_drop = _one_route(dx, t, j)
    mutated = ref["out64"].copy()
    mutated[t] += y_drop - y
    ok, st = _gate(kind, mutated, ref)
    assert not ok, st


@pytest.mark.parametrize("kind,K,I", CASES)
def test_gate_rejects_weight_applied_twice(kind, K, I):
    d = small_case(kind, 8, K, I, 8, 4, seed="gate")
    ref = run(d)
    t, j = 5, 3
    mutated = ref["out64"].copy()
    mutated[t] += _one_route(d, t, j)
    ok, st = _gate(kind, mutated, ref)
    assert not ok, st


@pytest.mark.parametrize("kind,K,I", CASES)
def test_gate_rejects_dropped_route(kind, K, I):
    d = small_case(kind, 8, K, I, 8, 4, seed="gate")
    ref = run(d)
    t, j = 0, 2
    mutated = ref["out64"].copy()
    mutated[t] -= _one_route(d, t, j)
    ok, st = _gate(kind, mutated, ref)
    assert not ok, st


@pytest.mark.parametrize("kind", ["mxfp8", "mxfp4"])
def test_gate_rejects_wrong_mx_exponent(kind, monkeypatch):
    """One route's intermediate: its first 32-wide group decoded with the
    shared exponent one too large (every value halved, saturating where it
    leaves e4m3's range) although the exponent is not a near-tie."""
    d = small_case(kind, 8, 2048, 256, 8, 4, seed="gate")
    ref = run(d, keep_h=True)
    t, j = 3, 0
    key = t * 4 + j
    e = int(d["topk_ids"][t, j])
    real = om._requant_mx
    state = {"done": False}

    def wrong(h, band):
        out = list(real(h, band))
        moved = out[6][0]
        hd = out[2].copy()
        rows = np.nonzero(np.all(np.isclose(hd, ref["h"][key][2][None, :], rtol=0, atol=0),
                                 axis=1))[0]
        if rows.size and not state["done"]:
            r = rows[0]
            assert not moved[r, 0]              # not a near-tie
            q = out[0][r, :32]
            s = int(out[1][r, 0]) - 127 + 1
            hd[r, :32] = codecs.e4m3_decode(q) * 2.0 ** s
            state["done"] = True
        out[2] = hd
        return tuple(out)

    monkeypatch.setattr(om, "_requant_mx", wrong)
    mutated = run(d)["out64"]
    assert state["done"] and int(d["topk_ids"][t, j]) == e
    ok, st = _gate(kind, mutated, ref)
    assert not ok, st


# ---------------------------------------------------------------------------
# per-route rows held in bf16 before the combine
# ---------------------------------------------------------------------------

def _rows_rounded(d, T, k, bits=8):
    """Emulated kernel: each route's row y_j (the oracle's exact value)
    rounded to `bits` significant bits (8: bf16, round to nearest even),
    then the weighted sum in fp64."""
    out = None
    for t in range(T):
        for j in range(k):
            y = _one_route(d, t, j, w=1.0)
            if bits == 8:
                yr = codecs.bf16_decode(codecs.bf16_encode(y))
            else:
                m, e = np.frexp(y)
                yr = np.ldexp(np.round(m * 2.0 ** bits) / 2.0 ** bits, e)
            if out is None:
                out = np.zeros((T, y.size))
            out[t] += d["topk_weights"][t, j] * yr
    return out


@pytest.mark.parametrize("kind,K,I", CASES)
def test_gate_accepts_bf16_route_rows(kind, K, I, monkeypatch):
    """Rows rounded to bf16 before the combine (the pages' two-byte combine
    buffer) pass the gate with no tolerance at all (tol 0: the allowance and
    the output's half spacing only); without the row-rounding term of the
    allowance the same output fails, so the term is what admits it."""
    T, k = 4, 4
    d = small_case(kind, T, K, I, 8, k, seed="rows")
    ref = run(d)
    emul = _rows_rounded(d, T, k)
    ok, st = om.tolerance_check(codecs.bf16_encode(emul), ref["out64"], 0.0, ref["allowance"])
    assert ok, st
    monkeypatch.setattr(om, "_row_rounding", lambda reach: np.zeros_like(reach))
    bare = run(d)
    ok, st = om.tolerance_check(codecs.bf16_encode(emul), ref["out64"], 0.0, bare["allowance"])
    assert not ok, st


@pytest.mark.parametrize("kind,K,I", CASES)
def test_gate_rejects_coarser_route_rows(kind, K, I):
    """Rows rounded to 6 significant bits (a plausible wrong row format: up
    to four times bf16's rounding error) fail the gate at tol 0."""
    T, k = 4, 4
    d = small_case(kind, T, K, I, 8, k, seed="rows")
    ref = run(d)
    emul = _rows_rounded(d, T, k, bits=6)
    ok, st = om.tolerance_check(codecs.bf16_encode(emul), ref["out64"], 0.0, ref["allowance"])
    assert not ok, st
