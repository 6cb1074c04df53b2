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
     "top-k weighted reduction").

Requantization decisions (rounding to e4m3 / bf16, the power-of-two MX scale)
are taken on h rounded to binary32, the precision the kernels hold h in; the
GEMMs and the combine stay in fp64.

Near-ties.  A kernel computes h in fp32 with its own summation order, so its
h differs from this fp64 h by a small amount; where the scaled value sits
within that distance of a rounding boundary, both neighbouring codes are
correct roundings of h.  Each requantizer therefore also returns, per
element, ``alt``: the dequantized distance to the other admissible result (0
where the decision is unambiguous).  The band models the kernel's deviation
as REL_BAND = 2^-14 of |h| plus ABS_BAND = 2^-16 of the group's amax (the
relative part is three to four times the deviations of the group amax
measured on the GPU, 1-2e-5; the absolute part covers elements that are small
because of cancellation).  moe_ref turns the alts into a per-output allowance
``flip_bound``: for each route, the smaller of the plain sum of all near-ties'
effects on the output (sum_i alt_i |w2_ci|, which covers any combination) and
the largest single effect in full plus three times the root-sum-square of all
of them (near-ties are independent one-step decisions of either sign, so many
small ones add like a random walk), weighted by the route weight and summed
over routes.  :func:`tolerance_check`
adds it to the element-wise bound and separately requires that at most 0.1%
of the elements need it.

The loop runs per expert so that only one expert's dequantized weights are
held at a time.
"""

import numpy as np

from . import codecs


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
        return v * np.repeat(np.repeat(s, 128, axis=0), 128, axis=1)
    if kind == "mxfp8":
        return v * np.repeat(codecs.e8m0_decode(w_scale[e]), 32, axis=1)
    raise ValueError(kind)


REL_BAND = 2.0 ** -14
ABS_BAND = 2.0 ** -16


def _alt_e4m3(p, band):
    """For scaled values p (fp64, |p| <= 448 after saturation) and a band
    half-width in the same units: dequantized-unit distance (in p units) to
    the other admissible e4m3 value, 0 when p is farther than ``band`` from
    every rounding boundary."""
    q0 = codecs.e4m3_decode(codecs.e4m3_encode(p))
    lo = codecs.e4m3_decode(codecs.e4m3_encode(p - band))
    hi = codecs.e4m3_decode(codecs.e4m3_encode(p + band))
    return np.maximum(np.abs(lo - q0), np.abs(hi - q0))


def requant_blockwise(h):
    """Per row and 128 columns: (codes uint8, scales fp32, dequantized fp64,
    near-tie alternative distance fp64)."""
    rows, I = h.shape
    h32 = codecs.fp32(h).reshape(rows, I // 128, 128)
    amax = np.max(np.abs(h32), axis=2)                        # exact in fp32
    amax = np.maximum(amax, np.float32(1e-10))
    sf = (amax * np.float32(1.0 / 448.0)).astype(np.float32)  # fp32 product
    sf_inv = (np.float64(1.0) / sf.astype(np.float64)).astype(np.float32)
    p = (h32 * sf_inv[:, :, None]).astype(np.float32)         # fp32 product
    q = codecs.e4m3_encode(p.astype(np.float64))
    hd = codecs.e4m3_decode(q) * sf.astype(np.float64)[:, :, None]
    p64 = p.astype(np.float64)
    alt = _alt_e4m3(p64, np.abs(p64) * REL_BAND + 448.0 * ABS_BAND) * \
        sf.astype(np.float64)[:, :, None]
    return q.reshape(rows, I), sf, hd.reshape(rows, I), alt.reshape(rows, I)


def _mx_exponent(amax):
    with np.errstate(divide="ignore"):
        lg = np.floor(np.log2(np.where(amax > 0, amax, 1.0)))
    return np.where(amax > 0, np.clip(lg - 8, -127, 127), -127).astype(np.int64)


def _mx_apply(h32, s):
    p = h32.astype(np.float64) * np.ldexp(1.0, -s)[:, :, None]
    p = codecs.fp32(p).astype(np.float64)   # binary32 product, as the kernels
    q = codecs.e4m3_encode(p)
    return q, codecs.e4m3_decode(q) * np.ldexp(1.0, s)[:, :, None], p


def requant_mx(h):
    """Per row and 32 columns: (codes uint8, e8m0 codes uint8, dequantized
    fp64, near-tie alternative distance fp64)."""
    rows, I = h.shape
    h32 = codecs.fp32(h).reshape(rows, I // 32, 32)
    amax = np.max(np.abs(h32), axis=2).astype(np.float64)
    s = _mx_exponent(amax)
    q, hd, p = _mx_apply(h32, s)

    def band(pp, ss):
        return np.abs(pp) * REL_BAND + np.ldexp(amax * ABS_BAND, -ss)[:, :, None]

    alt = _alt_e4m3(p, band(p, s)) * np.ldexp(1.0, s)[:, :, None]
    # the shared exponent itself is a near-tie when amax lies within the band
    # of a power of two: the other exponent's result is admissible too
    s_lo = _mx_exponent(amax * (1.0 - REL_BAND))
    s_hi = _mx_exponent(amax * (1.0 + REL_BAND))
    for s_alt in (s_lo, s_hi):
        moved = s_alt != s
        if np.any(moved):
            _, hd_alt, p_alt = _mx_apply(h32, s_alt)
            a2 = np.abs(hd_alt - hd) + _alt_e4m3(p_alt, band(p_alt, s_alt)) * \
                np.ldexp(1.0, s_alt)[:, :, None]
            alt = np.where(moved[:, :, None], np.maximum(alt, a2), alt)
    return q.reshape(rows, I), (s + 127).astype(np.uint8), hd.reshape(rows, I), alt.reshape(rows, I)


def requant_bf16(h):
    """h rounded to binary32 then to bfloat16: (bits uint16, None, fp64,
    near-tie alternative distance fp64)."""
    rows, I = h.shape
    h32 = codecs.fp32(h).astype(np.float64)
    hd = codecs.bf16_round(h32)
    G = 128 if I % 128 == 0 else I
    amax = np.max(np.abs(h32).reshape(rows, I // G, G), axis=2)
    band = np.abs(h32) * REL_BAND + np.repeat(amax * ABS_BAND, G, axis=1)
    lo = codecs.bf16_round(h32 - band)
    hi = codecs.bf16_round(h32 + band)
    alt = np.maximum(np.abs(lo - hd), np.abs(hi - hd))
    return codecs.bf16_encode(hd), None, hd, alt


def _shared_expert(e_routed, s):
    """Weight index of shared expert s: stored after the routed experts."""
    return e_routed + s


def _shared_weight():
    """Weight of a shared expert's output in the sum: the shared experts
    take every token and are not scaled by the router."""
    return 1.0


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
    intermediate: codes, scales and dequantized values.
    ``h_perturb``: test hook, a function applied to each expert's fp64 h
    before requantization (to model a kernel's fp32 deviations).
    ``n_shared``: the last n_shared experts of w1 / w2 are shared experts
    ([DeepGEMM #411] "Summary" fuses routed and shared L1 / L2; [DeepGEMM
    #88] "Performance" runs the shared expert as a separate GEMM): every
    token's output adds each shared expert's FFN with weight 1, computed
    exactly like a routed expert's.  Routed ids then count as local only in
    [0, E - n_shared).  With keep_h, shared route (t, s) is keyed
    T*top_k + t*n_shared + s.

    Returns a dict with ``out64`` (n, K) fp64, ``out_bf16`` (n, K) uint16,
    ``flip_bound`` (n, K) fp64 (the near-tie allowance, see the module
    docstring), and when ``keep_h`` a dict ``h`` mapping pair id t*top_k+j to
    (codes, scales, values).
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
    out64 = np.zeros((tokens.size, K), dtype=np.float64)
    bound = np.zeros((tokens.size, K), dtype=np.float64)
    local = {int(t): i for i, t in enumerate(tokens)}
    sel = ids[tokens]                                   # (n, k)
    hkeep = {}
    if kind == "bf16":
        requant = requant_bf16
    elif kind == "fp8_blockwise":
        requant = requant_blockwise
    elif kind in ("mxfp8", "mxfp4"):
        requant = requant_mx
    else:
        raise ValueError(kind)
    for e in np.unique(sel):
        if e < 0 or e >= E_all or (e >= E and not n_shared):
            continue                                    # not a local expert
        n_idx, j_idx = np.nonzero(sel == e)
        t_rows = tokens[n_idx]
        xd = dequant_x(kind, x, x_scale, t_rows)        # (m, K)
        w1d = dequant_w(kind, w1, w1_scale, e)          # (N, K)
        G = xd @ w1d.T                                  # (m, N)
        del w1d
        h = _swiglu(G, I)
        if h_perturb is not None:
            h = h_perturb(h)
        if exact_h:
            q, s, hd, alt = None, None, h, np.zeros_like(h)
        else:
            q, s, hd, alt = requant(h)
        w2d = dequant_w(kind, w2, w2_scale, e)          # (K, I)
        y = hd @ w2d.T                                  # (m, K)
        yb = None
        if np.any(alt):
            aw2 = np.abs(w2d)
            lin = alt @ aw2.T
            yb = 3.0 * np.sqrt((alt * alt) @ (aw2 * aw2).T)
            for r in range(alt.shape[0]):
                nz = np.nonzero(alt[r])[0]
                if nz.size:
                    yb[r] += np.max(aw2[:, nz] * alt[r, nz][None, :], axis=1)
            yb = np.minimum(yb, lin)
            del aw2, lin
        del w2d
        for r in range(t_rows.size):
            t = int(t_rows[r])
            j = int(j_idx[r])
            out64[local[t]] += wts[t, j] * y[r]
            if yb is not None:
                bound[local[t]] += abs(wts[t, j]) * yb[r]
            if keep_h:
                key = t * k_routed + j if j < k_routed else T * k_routed + t * n_shared + j - k_routed
                hkeep[key] = (None if q is None else q[r], None if s is None else s[r], hd[r])
    res = {"out64": out64, "out_bf16": codecs.bf16_encode(out64), "flip_bound": bound}
    if keep_h:
        res["h"] = hkeep
    return res


def tolerance_check(out_bits, out64, tol, flip_bound=None):
    """Gate used by the parity tests (reading of the max-error and
    mean-relative-error bounds for a bf16 output).

    Element-wise: |out - out64| <= tol * rms(out64) + half a bf16 spacing at
    out64 (the output format's own rounding) + flip_bound (the near-tie
    allowance).  At most 0.1% of the elements may exceed the bound without
    the allowance.  Global: sum|out - out64| / sum|out64| <= 5e-3.
    Returns (ok, stats dict).
    """
    got = codecs.bf16_decode(out_bits)
    ref = np.asarray(out64, dtype=np.float64)
    err = np.abs(got - ref)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    strict = tol * rms + codecs.bf16_half_ulp(ref)
    bound = strict if flip_bound is None else strict + flip_bound
    n_strict = int(np.sum(err > strict))
    finite = bool(np.all(np.isfinite(got)))
    max_ratio = float(np.max(err / np.where(rms > 0, rms, 1.0))) if ref.size else 0.0
    denom = float(np.sum(np.abs(ref)))
    mre = float(np.sum(err) / denom) if denom > 0 else 0.0
    n_bad = int(np.sum(err > bound))
    ok = finite and n_bad == 0 and mre <= 5e-3 and n_strict <= max(1, ref.size // 1000)
    return ok, {"rms": rms, "max_err_over_rms": max_ratio, "mean_rel_err": mre,
                "n_over_bound": n_bad, "n_over_strict": n_strict, "finite": finite}
