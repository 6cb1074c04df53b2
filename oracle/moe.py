"""Expert-FFN oracle in fp64, step by step (test infrastructure).

Test infrastructure (see the package docstring).

What is computed, and where the pages say it
--------------------------------------------
For every token t and route j with expert e = topk_ids[t, j] in [0, E):

  1. dequantize x[t], w1[e], w2[e] exactly into fp64
       * bf16 path: the bf16 values themselves;
       * blockwise FP8 path: e4m3 value times the fp32 scale of its block,
         1 x 128 for activations and 128 x 128 for weights (the blockwise W8A8
         format the [hpc-ops RFC] "Background" section names, with the block
         shapes of the blockwise configurations);
       * mxfp8 path: e4m3 value times the e8m0 scale of its 32-wide block along
         the contraction dimension ([prime-flash] "Scale layout (mxfp8)").
  2. gate/up GEMM: G = x[t] . w1[e]^T, N = 2I columns; gate = G[:I],
     up = G[I:] ([hpc-ops RFC] "Background" stage 2; [prime-flash] "Shapes":
     w1 is (E, N, K) with N the fused gate+up columns).
  3. SwiGLU: h = silu(gate) * up, silu(g) = g / (1 + e^-g)
     ([hpc-ops RFC] "Background" stage 3; [prime-flash] intro).
  4. requantize h before the down GEMM
       * blockwise: per row and 128 columns, amax clamped below at 1e-10,
         sf = amax * (1/448), sf_inv = 1/sf, q = e4m3(h * sf_inv), value q*sf
         ([DeepGEMM #88] "Before you merge": the requant scale expression and
         the per-128 grouping);
       * mxfp8: per row and 32 columns, OCP MX rule: shared exponent
         floor(log2 amax) - 8 (8 = exponent of e4m3's largest power of two),
         elements rounded to e4m3 with saturation ([prime-flash] intro: the
         intermediate is requantized to mxfp8 on chip; "Scale layout" names the
         OCP MX quantizer);
       * bf16: h rounded to bf16, since the down GEMM takes bf16 operands (the
         pages are silent; plainest reading).
  5. down GEMM: y = hq . w2[e]^T, w2 is (E, K, I) ([hpc-ops RFC] stage 4;
     [prime-flash] "Shapes").
  6. top-k weighted combine: out[t] = sum_j topk_weights[t, j] * y_j, the
     weight applied after the down GEMM, summed in fp64; the bf16 output is
     one rounding of that sum ([hpc-ops RFC] stage 5; [prime-flash] intro:
     "top-k weighted reduction").  Between the down GEMM and the combine a
     kernel may hold each route's row y_j in bf16: the pages' combine buffer
     takes two bytes per token, selected expert and hidden column ([DeepGEMM
     #88] "The rest of the memory numbers": 512 MiB at 8192 tokens on
     4096/2048/288/8).  The result here keeps y_j exact; ``dev_bound``
     covers that rounding (below).

Requantization decisions (rounding to e4m3 / bf16, the power-of-two MX scale)
are taken on h rounded to binary32, the precision the kernels hold h in; the
GEMMs and the combine stay in fp64.

The gate: how far a correct fp32 kernel may lie from this fp64 result
---------------------------------------------------------------------
The pages fix the method, not the summation order or precision of a kernel's
fp32 arithmetic, so a correct kernel's output differs from the fp64 result in
two ways, both modelled per element and returned beside the result:

* Arithmetic deviation (``dev_bound``).  A matrix-core GEMM sums its K
  products block by block (128 e4m3 or 32 bf16 products per instruction) and
  carries the running sum in fp32 from block to block (adding each block's
  scaled partial sum, for the blockwise format).  The model:
    - one instruction adds its products with a zero-mean error of standard
      deviation at most KAPPA * ||p||_2 (the 2-norm of its products), the
      errors of different instructions independent; KAPPA = 2^-14 for e4m3
      operands (the instruction does not round like an fp32 adder: it keeps a
      limited number of bits of the products it aligns), 2^-24 (binary32's
      unit roundoff u) for bf16 operands;
    - every addition to the running sum and every scale product rounds once
      in binary32, an error of at most u times its magnitude, taken as
      independent;
  so the result G of a GEMM deviates with standard deviation at most
      sigma_G = sqrt( KAPPA^2 * Q  +  u^2 * (steps + 2) * (|G| + 3 sqrt(Q))^2 ),
  Q = sum_k (a_k b_k)^2 over the dequantized operands, steps = K / block; it
  grows like sqrt(K).  The bound used is LAMBDA = 6 standard deviations
  (a Gaussian tail of 2e-9 per element).  Through SwiGLU this gives a band
  on each element of h (derivative of silu times sigma, plus the fp32
  evaluation of silu: exp2, one division, the products, about (|g| + 6) u
  relative).  The down GEMM's own deviation, the deviation of a blockwise
  group's scale (the kernel's amax lies within the band of its largest
  element), the fp32 combine of the top_k rows and the rounding of each
  route's row to bf16 before the combine (half a bf16 spacing at the largest
  magnitude the kernel's row can reach, times the route weight) are added
  to ``dev_bound`` per output element.
* Near-ties (``flip_bound``).  Where the kernel's h can lie on the other side
  of a requantization rounding boundary (within the band above), both
  neighbouring codes are correct roundings of h.  Each requantizer returns,
  per element, ``alt``: the dequantized distance to the other admissible
  result (0 where the decision is unambiguous).  An MX group whose largest
  element lies within its band of a power of two can take the other shared
  exponent, which moves all 32 elements at once: that group is one decision,
  with the exact signed effect of the other exponent on each output.  Per
  route and output column, the effects of the independent decisions add to
  at most min(their sum, the largest in full plus FLIP_LAMBDA = 3 times
  their root-sum-square): near-tie decisions are independent one-step
  choices of either sign, so many small ones add like a random walk.
  Routes add with their weights.

``moe_ref`` returns both bounds and their sum ``allowance``;
:func:`tolerance_check` accepts an output when every element lies within
tol * rms(out64) + allowance + half a bf16 spacing (at the largest magnitude
the kernel's fp32 value can reach) of the fp64 result, and the mean relative
error is at most 5e-3.

KAPPA is a property of the matrix instructions.  A GPU test of the
instructions themselves (tests/test_gpu_mfma_model.py) checks, on random and
adversarial operands, that their errors stay within the model.

The loop runs per expert so that only one expert's dequantized weights are
held at a time.
"""

import numpy as np
from scipy.special import erfc

from . import codecs

U32 = 2.0 ** -24           # binary32 unit roundoff
KAPPA = {"bf16": 2.0 ** -24, "e4m3": 2.0 ** -15}
BLOCK_K = {"bf16": 32, "e4m3": 128}
LAMBDA = 6.0
FLIP_LAMBDA = 3.0


def _operands(kind):
    """Operand class of the matrix instructions a kind uses (MXFP4 weights
    run the e4m3 instruction with an e2m1 B operand)."""
    return "bf16" if kind == "bf16" else "e4m3"


def _silu(g):
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def _swiglu(G, I):
    """silu(gate) * up with gate = first I columns, up = last I columns."""
    return _silu(G[:, :I]) * G[:, I:]


def dequant_x(kind, x, x_scale, rows):
    """fp64 activations for the given token rows."""
    if kind == "bf16":
        return codecs.bf16_decode(x[rows])
    v = codecs.e4m3_decode(x[rows])
    if kind == "fp8_blockwise":
        return v * np.repeat(x_scale[rows].astype(np.float64), 128, axis=1)
    if kind in ("mxfp8", "mxfp4"):   # MXFP4 weights take MX FP8 activations
        return v * np.repeat(codecs.e8m0_decode(x_scale[rows]), 32, axis=1)
    raise ValueError(kind)


def dequant_w(kind, w, w_scale, e):
    """fp64 weight matrix of expert e (rows = output features)."""
    if kind == "bf16":
        return codecs.bf16_decode(w[e])
    if kind == "mxfp4":
        v = codecs.e2m1_decode(codecs.fp4_unpack(w[e]))
        return v * np.repeat(codecs.e8m0_decode(w_scale[e]), 32, axis=1)
    v = codecs.e4m3_decode(w[e])
    if kind == "fp8_blockwise":
        s = w_scale[e].astype(np.float64)
        R, C = v.shape
        # each 128 x 128 block times its scale (in place, one pass)
        v.reshape(R // 128, 128, C // 128, 128)[...] *= s[:, None, :, None]
        return v
    if kind == "mxfp8":
        return v * np.repeat(codecs.e8m0_decode(w_scale[e]), 32, axis=1)
    raise ValueError(kind)


# ---------------------------------------------------------------------------
# arithmetic model
# ---------------------------------------------------------------------------

def gemm_sigma(kind, a, b, G):
    """Standard deviation of a kernel's fp32 value of G = a . b^T under the
    model of the module docstring (a: (m, K), b: (n, K) dequantized fp64)."""
    cls = _operands(kind)
    Q = (a * a) @ (b * b).T
    rq = np.sqrt(Q)
    steps = a.shape[1] / BLOCK_K[cls]
    chain = U32 * np.sqrt(steps + 2.0) * (np.abs(G) + 3.0 * rq)
    return np.sqrt((KAPPA[cls] * rq) ** 2 + chain ** 2)


def swiglu_band(G, sigma_G, I):
    """h = silu(gate) * up and the band within which a kernel's fp32 h lies:
    LAMBDA standard deviations of the propagated GEMM deviation (first order,
    plus the second-order terms at LAMBDA sigma) and the fp32 evaluation of
    silu and the product."""
    h = _swiglu(G, I)
    g, v = G[:, :I], G[:, I:]
    sg, sv = sigma_G[:, :I], sigma_G[:, I:]
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-g))
    silu = g * sig
    dsilu = sig * (1.0 + g * (1.0 - sig))          # d silu / dg, |.| < 1.1
    sigma_h = np.sqrt((dsilu * v * sg) ** 2 + (silu * sv) ** 2)
    second = LAMBDA ** 2 * (1.1 * sg * sv + 0.25 * sg * sg * np.abs(v))
    band = LAMBDA * sigma_h + second + (np.abs(g) + 6.0) * U32 * np.abs(h)
    return h, band


# ---------------------------------------------------------------------------
# requantizers
# ---------------------------------------------------------------------------

def _flip_prob(dist, band):
    """Probability that a kernel value, off by a zero-mean normal deviation of
    standard deviation band / LAMBDA, lies beyond a boundary at distance
    ``dist``: the upper tail Phi(-dist / sigma)."""
    sigma = np.maximum(band, 1e-300) / LAMBDA
    return 0.5 * erfc(np.asarray(dist, dtype=np.float64) / (sigma * np.sqrt(2.0)))


def _alt_e4m3(p, band):
    """For scaled values p (fp64, |p| <= 448 after saturation) and a band
    half-width in the same units: (distance in p units to the other admissible
    e4m3 value, 0 when p is farther than ``band`` from every rounding
    boundary; probability that a deviation of the model crosses that
    boundary)."""
    q0 = codecs.e4m3_decode(codecs.e4m3_encode(p))
    lo = codecs.e4m3_decode(codecs.e4m3_encode(p - band))
    hi = codecs.e4m3_decode(codecs.e4m3_encode(p + band))
    dlo, dhi = np.abs(lo - q0), np.abs(hi - q0)
    alt = np.maximum(dlo, dhi)
    # the boundary crossed lies halfway between q0 and its neighbour
    edge = np.where(dhi >= dlo, q0 + dhi / 2.0, q0 - dlo / 2.0)
    prob = np.where(alt > 0, _flip_prob(np.abs(edge - p), band), 0.0)
    return alt, prob


def _requant_blockwise(h, band):
    rows, I = h.shape
    h32 = codecs.fp32(h).reshape(rows, I // 128, 128)
    amax = np.max(np.abs(h32), axis=2)                        # exact in fp32
    amax = np.maximum(amax, np.float32(1e-10))
    sf = (amax * np.float32(1.0 / 448.0)).astype(np.float32)  # fp32 product
    sf_inv = (np.float64(1.0) / sf.astype(np.float64)).astype(np.float32)
    p = (h32 * sf_inv[:, :, None]).astype(np.float32)         # fp32 product
    q = codecs.e4m3_encode(p.astype(np.float64))
    sf64 = sf.astype(np.float64)
    hd = codecs.e4m3_decode(q) * sf64[:, :, None]
    b = band.reshape(rows, I // 128, 128)
    # the kernel's amax is its largest |h|, within the largest band of the
    # group; sf, 1/sf, the product and fp32(h) round once each
    rel = np.max(b, axis=2) / amax.astype(np.float64) + 4.0 * U32
    p64 = p.astype(np.float64)
    band_p = b * sf_inv.astype(np.float64)[:, :, None] + np.abs(p64) * rel[:, :, None]
    alt, prob = _alt_e4m3(p64, band_p)
    alt = alt * sf64[:, :, None]
    scale_dev = rel - 2.0 * U32                             # relative deviation of sf
    return (q.reshape(rows, I), sf, hd.reshape(rows, I), alt.reshape(rows, I),
            prob.reshape(rows, I), scale_dev, None)


def requant_blockwise(h, band=None):
    """Per row and 128 columns: (codes uint8, scales fp32, dequantized fp64,
    near-tie alternative distance fp64).  ``band``: per-element half-width
    within which a kernel's h may lie (none: exact h, every alt is 0)."""
    b = np.zeros(h.shape) if band is None else band
    return _requant_blockwise(h, b)[:4]


def _mx_exponent(amax):
    with np.errstate(divide="ignore"):
        lg = np.floor(np.log2(np.where(amax > 0, amax, 1.0)))
    return np.where(amax > 0, np.clip(lg - 8, -127, 127), -127).astype(np.int64)


def _mx_apply(h32, s):
    p = h32.astype(np.float64) * np.ldexp(1.0, -s)[:, :, None]
    p = codecs.fp32(p).astype(np.float64)   # binary32 product, as the kernels
    q = codecs.e4m3_encode(p)
    return q, codecs.e4m3_decode(q) * np.ldexp(1.0, s)[:, :, None], p


def _requant_mx(h, band):
    rows, I = h.shape
    h32 = codecs.fp32(h).reshape(rows, I // 32, 32)
    amax = np.max(np.abs(h32), axis=2).astype(np.float64)
    s = _mx_exponent(amax)
    q, hd, p = _mx_apply(h32, s)
    b = band.reshape(rows, I // 32, 32)
    # p = h * 2^-s is exact in binary32 above the subnormals; fp32(h) rounds
    alt, prob = _alt_e4m3(p, b * np.ldexp(1.0, -s)[:, :, None] + np.abs(p) * U32)
    alt = alt * np.ldexp(1.0, s)[:, :, None]
    # the shared exponent itself is a near-tie when the kernel's amax (within
    # the largest band of the group) can lie on the other side of a power of
    # two: then the whole group may take the other exponent
    adev = np.max(b, axis=2)
    s_lo = _mx_exponent(np.maximum(amax - adev, 0.0))
    s_hi = _mx_exponent(amax + adev)
    s_alt = np.where(s_hi != s, s_hi, s_lo)
    moved = s_alt != s
    dhd = np.zeros_like(hd)
    alt2 = np.zeros_like(hd)
    gprob = np.zeros(moved.shape)
    if np.any(moved):
        _, hd_a, p_a = _mx_apply(h32, s_alt)
        dhd = np.where(moved[:, :, None], hd_a - hd, 0.0)
        a2, _ = _alt_e4m3(p_a, b * np.ldexp(1.0, -s_alt)[:, :, None] + np.abs(p_a) * U32)
        alt2 = np.where(moved[:, :, None], a2 * np.ldexp(1.0, s_alt)[:, :, None], 0.0)
        # the power of two between the two exponents' ranges
        edge = np.ldexp(1.0, np.maximum(s, s_alt) + 8)
        gprob = np.where(moved, _flip_prob(np.abs(edge - amax), adev), 0.0)
    groups = (moved, dhd.reshape(rows, I), alt2.reshape(rows, I), gprob)
    return (q.reshape(rows, I), (s + 127).astype(np.uint8), hd.reshape(rows, I),
            alt.reshape(rows, I), prob.reshape(rows, I), None, groups)


def requant_mx(h, band=None):
    """Per row and 32 columns: (codes uint8, e8m0 codes uint8, dequantized
    fp64, near-tie alternative distance fp64).  With a ``band``, an element of
    a group whose shared exponent is a near-tie carries as ``alt`` the larger
    of its own near-tie distance and its move under the other exponent."""
    b = np.zeros(h.shape) if band is None else band
    q, s, hd, alt, _, _, (moved, dhd, alt2, _) = _requant_mx(h, b)
    alt = np.maximum(alt, np.abs(dhd) + alt2)
    return q, s, hd, alt


def _requant_bf16(h, band):
    h32 = codecs.fp32(h).astype(np.float64)
    hd = codecs.bf16_round(h32)
    bb = band + np.abs(h32) * U32
    lo = codecs.bf16_round(h32 - bb)
    hi = codecs.bf16_round(h32 + bb)
    dlo, dhi = np.abs(lo - hd), np.abs(hi - hd)
    alt = np.maximum(dlo, dhi)
    edge = np.where(dhi >= dlo, hd + dhi / 2.0, hd - dlo / 2.0)
    prob = np.where(alt > 0, _flip_prob(np.abs(edge - h32), bb), 0.0)
    return codecs.bf16_encode(hd), None, hd, alt, prob, None, None


def requant_bf16(h, band=None):
    """h rounded to binary32 then to bfloat16: (bits uint16, None, fp64,
    near-tie alternative distance fp64)."""
    b = np.zeros(h.shape) if band is None else band
    return _requant_bf16(h, b)[:4]


# ---------------------------------------------------------------------------
# near-tie aggregation
# ---------------------------------------------------------------------------

def route_flip_bound(alt, prob, w2d, groups=None):
    """Per-route near-tie allowance on the down GEMM's outputs.

    alt: (m, I) independent element near-tie distances, prob: (m, I) the
    probability that the element's decision goes the other way under the
    model's deviation; w2d: (K, I); groups: None or (moved (m, I/32) bool,
    dhd (m, I), alt2 (m, I), gprob (m, I/32)) for MX groups whose shared
    exponent is a near-tie.  For each row and output column a decision's
    effect is e_i = alt_i |w2_ci| for an element, and for a moved group
    |sum_i dhd_i w2_ci| plus its elements' larger near-tie distances times
    |w2_ci|.  Bound: min(sum_i e_i, max_i e_i + FLIP_LAMBDA *
    sqrt(sum_i prob_i e_i^2)): the largest effect in full, the others as a
    random walk of independent decisions, each taken with its probability.
    Returns (m, K)."""
    m, I = alt.shape
    K = w2d.shape[0]
    a = alt.copy()
    pr = prob.copy()
    aw2 = np.abs(w2d)
    gterms = [[] for _ in range(m)]
    if groups is not None:
        moved, dhd, alt2, gprob = groups
        for r, gi in zip(*np.nonzero(moved)):
            sl = slice(32 * gi, 32 * gi + 32)
            eff = np.abs(w2d[:, sl] @ dhd[r, sl]) + aw2[:, sl] @ np.maximum(a[r, sl], alt2[r, sl])
            # the group's exponent decision, or any of its element decisions
            gp = min(1.0, gprob[r, gi] + float(np.sum(pr[r, sl])))
            gterms[r].append((eff, gp))
            a[r, sl] = 0.0                     # counted inside the group term
            pr[r, sl] = 0.0
    lin = a @ aw2.T
    sq = (pr * a * a) @ (aw2 * aw2).T
    big = np.zeros((m, K))
    for r in range(m):
        nz = np.nonzero(a[r])[0]
        if nz.size:
            big[r] = np.max(aw2[:, nz] * a[r, nz][None, :], axis=1)
        for eff, gp in gterms[r]:
            lin[r] += eff
            sq[r] += gp * eff * eff
            big[r] = np.maximum(big[r], eff)
    return np.minimum(lin, big + FLIP_LAMBDA * np.sqrt(sq))


# ---------------------------------------------------------------------------
# the forward
# ---------------------------------------------------------------------------

def _shared_expert(e_routed, s):
    """Weight index of shared expert s: stored after the routed experts."""
    return e_routed + s


def _shared_weight():
    """Weight of a shared expert's output in the sum: the shared experts
    take every token and are not scaled by the router."""
    return 1.0


def _requantizer(kind):
    """The requantizer of a kind (looked up when called)."""
    return {"bf16": _requant_bf16, "fp8_blockwise": _requant_blockwise, "mxfp8": _requant_mx,
            "mxfp4": _requant_mx}.get(kind)


def _row_rounding(reach):
    """Largest change of a route's row element of magnitude at most `reach`
    when it is rounded to bf16 (round to nearest: half a spacing)."""
    return codecs.bf16_half_ulp(reach)


def moe_ref(kind, x, x_scale, w1, w1_scale, w2, w2_scale, topk_ids,
            topk_weights, tokens=None, exact_h=False, keep_h=False, h_perturb=None,
            n_shared=0):
    """Fused MoE forward, fp64.

    Arrays are numpy: bf16 data as uint16 bit patterns, e4m3 data as uint8
    codes, blockwise scales as float32, MX scales as uint8 e8m0 codes.
    Shapes: x (T, K); w1 (E, N, K); w2 (E, K, N/2); topk_ids, topk_weights
    (T, top_k).  ``mxfp4``: w1 (E, N, K/2) and w2 (E, K, N/4) packed e2m1
    pairs with e8m0 scales (E, N, K/32) and (E, K, N/64); x is MX FP8 and the
    intermediate is requantized to MX FP8, as on the mxfp8 path.

    ``tokens``: optional sorted array of token indices; only those outputs are
    computed (rows of the result follow that order).
    ``exact_h``: bf16 path only, skip the bf16 rounding of h (used by the
    dense-FFN special-case check).
    ``keep_h``: also return, per computed route (t, j), the requantized
    intermediate: codes, scales, dequantized values, near-tie distances and a
    dict of the decisions a kernel may take the other way: ``prob`` (per
    element), ``scale_rel`` (blockwise: bound on the relative deviation of
    each group's scale), ``moved`` / ``dhd`` / ``alt2`` (MX: groups whose
    shared exponent is a near-tie, the move of their values under the other
    exponent, and near-ties under it).
    ``h_perturb``: test hook, a function applied to each expert's fp64 h
    before requantization (to model a kernel's fp32 deviations); its second
    argument is the band of the arithmetic model for that h.
    ``n_shared``: the last n_shared experts of w1 / w2 are shared experts
    ([DeepGEMM #411] "Summary" fuses routed and shared L1 / L2; [DeepGEMM
    #88] "Performance" runs the shared expert as a separate GEMM): every
    token's output adds each shared expert's FFN with weight 1, computed
    exactly like a routed expert's.  Routed ids then count as local only in
    [0, E - n_shared).  With keep_h, shared route (t, s) is keyed
    T*top_k + t*n_shared + s.

    Returns a dict with ``out64`` (n, K) fp64, ``out_bf16`` (n, K) uint16,
    ``flip_bound``, ``dev_bound`` and ``allowance`` = their sum, each (n, K)
    fp64 (see the module docstring), and when ``keep_h`` a dict ``h`` mapping
    pair id t*top_k+j to (codes, scales, values, alt, info).
    """
    ids = np.asarray(topk_ids, dtype=np.int64)
    wts = np.asarray(topk_weights, dtype=np.float32).astype(np.float64)
    T, k_routed = ids.shape
    E_all = w1.shape[0]
    E = E_all - n_shared                                # routed experts
    if n_shared:
        # routes outside the routed experts are skipped; then one route per
        # (token, shared expert) with weight 1
        ids = np.where((ids >= 0) & (ids < E), ids, -1)
        sh = np.array([_shared_expert(E, s) for s in range(n_shared)], dtype=np.int64)
        ids = np.concatenate([ids, np.broadcast_to(sh, (T, n_shared))], axis=1)
        wts = np.concatenate([wts, np.full((T, n_shared), _shared_weight())], axis=1)
    k = ids.shape[1]
    K = w1.shape[2] * (2 if kind == "mxfp4" else 1)
    I = w1.shape[1] // 2
    if tokens is None:
        tokens = np.arange(T)
    tokens = np.asarray(tokens, dtype=np.int64)
    n = tokens.size
    out64 = np.zeros((n, K), dtype=np.float64)
    flip = np.zeros((n, K), dtype=np.float64)
    var_dev = np.zeros((n, K), dtype=np.float64)        # sum_j w_j^2 sigma_y^2
    lin_dev = np.zeros((n, K), dtype=np.float64)        # scale and combine terms
    local = {int(t): i for i, t in enumerate(tokens)}
    sel = ids[tokens]                                   # (n, k)
    hkeep = {}
    requant = _requantizer(kind)
    if requant is None:
        raise ValueError(kind)
    for e in np.unique(sel):
        if e < 0 or e >= E_all or (e >= E and not n_shared):
            continue                                    # not a local expert
        n_idx, j_idx = np.nonzero(sel == e)
        t_rows = tokens[n_idx]
        xd = dequant_x(kind, x, x_scale, t_rows)        # (m, K)
        w1d = dequant_w(kind, w1, w1_scale, e)          # (N, K)
        G = xd @ w1d.T                                  # (m, N)
        sG = gemm_sigma(kind, xd, w1d, G)
        del w1d
        h, band = swiglu_band(G, sG, I)
        if h_perturb is not None:
            h = h_perturb(h, band)
        if exact_h:
            q, s, hd, alt, prob, sdev, groups = (None, None, h, np.zeros_like(h),
                                                 np.zeros_like(h), None, None)
        else:
            q, s, hd, alt, prob, sdev, groups = requant(h, band)
        w2d = dequant_w(kind, w2, w2_scale, e)          # (K, I)
        y = hd @ w2d.T                                  # (m, K)
        fl = route_flip_bound(alt, prob, w2d, groups) if (np.any(alt) or (
            groups is not None and np.any(groups[0]))) else None
        sy = gemm_sigma(kind, hd, w2d, y)
        sd = None
        if sdev is not None:
            # a blockwise group's scale moves all of its 128 values together:
            # its signed contribution to each output, times its deviation
            sd = np.zeros_like(y)
            for gi in range(I // 128):
                sl = slice(128 * gi, 128 * gi + 128)
                sd += sdev[:, gi:gi + 1] * np.abs(hd[:, sl] @ w2d[:, sl].T)
        del w2d
        for r in range(t_rows.size):
            t = int(t_rows[r])
            j = int(j_idx[r])
            w = wts[t, j]
            i = local[t]
            out64[i] += w * y[r]
            var_dev[i] += (w * sy[r]) ** 2
            # the fp32 sum of the routes' rows (split-K over 128-wide slices
            # of I in the fused mode): at most k * I / 128 + 1 roundings
            lin_dev[i] += abs(w) * (U32 * (k * (I // 128 + 1) + 1) * np.abs(y[r]))
            # the row held in bf16 before the combine: the kernel's fp32 row
            # lies within its deviation and near-tie effects of y
            reach = np.abs(y[r]) + LAMBDA * sy[r]
            if sd is not None:
                lin_dev[i] += abs(w) * sd[r]
                reach = reach + sd[r]
            if fl is not None:
                flip[i] += abs(w) * fl[r]
                reach = reach + fl[r]
            lin_dev[i] += abs(w) * _row_rounding(reach)
            if keep_h:
                key = t * k_routed + j if j < k_routed else T * k_routed + t * n_shared + j - k_routed
                info = {"prob": prob[r]}
                if sdev is not None:
                    info["scale_rel"] = sdev[r]
                if groups is not None:
                    info["moved"], info["dhd"], info["alt2"] = (groups[0][r], groups[1][r],
                                                                groups[2][r])
                hkeep[key] = (None if q is None else q[r], None if s is None else s[r], hd[r],
                              alt[r], info)
    dev = LAMBDA * np.sqrt(var_dev) + lin_dev
    res = {"out64": out64, "out_bf16": codecs.bf16_encode(out64), "flip_bound": flip,
           "dev_bound": dev, "allowance": flip + dev}
    if keep_h:
        res["h"] = hkeep
    return res


def tolerance_check(out_bits, out64, tol, allowance=None):
    """Gate used by the parity tests (reading of the max-error and
    mean-relative-error bounds for a bf16 output).

    Element-wise: |out - out64| <= tol * rms(out64) + allowance + half a bf16
    spacing at |out64| + tol * rms + allowance (the kernel's fp32 value lies
    within tol * rms + allowance of out64 before its one rounding to bf16, so
    its rounding step is at most that binade's).  ``allowance`` is moe_ref's
    per-element near-tie and arithmetic allowance (None: 0).  Global:
    sum |out - out64| / sum |out64| <= 5e-3.  Every element must pass.
    Returns (ok, stats dict).
    """
    got = codecs.bf16_decode(out_bits)
    ref = np.asarray(out64, dtype=np.float64)
    err = np.abs(got - ref)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    dev = tol * rms + (0.0 if allowance is None else np.asarray(allowance, dtype=np.float64))
    bound = dev + codecs.bf16_half_ulp(np.abs(ref) + dev)
    strict = tol * rms + codecs.bf16_half_ulp(np.abs(ref) + tol * rms)
    finite = bool(np.all(np.isfinite(got)))
    max_ratio = float(np.max(err / np.where(rms > 0, rms, 1.0))) if ref.size else 0.0
    denom = float(np.sum(np.abs(ref)))
    mre = float(np.sum(err) / denom) if denom > 0 else 0.0
    n_bad = int(np.sum(err > bound))
    ok = finite and n_bad == 0 and mre <= 5e-3
    return ok, {"rms": rms, "max_err_over_rms": max_ratio, "mean_rel_err": mre,
                "n_over_bound": n_bad, "n_over_strict": int(np.sum(err > strict)),
                "max_allowance_over_rms": float(np.max(dev - tol * rms) / rms) if
                (ref.size and rms > 0) else 0.0,
                "finite": finite}
