"""The HIP path's stages pinned apart from each other.

* Exact arithmetic: small-integer operands with power-of-two scales make
  every partial sum of the gate/up GEMM an exactly representable binary32
  value, so the GEMM is exact in any summation order; the split mode's
  intermediate (codes and scales) must then equal the oracle's.  The only
  freedom left is the fp32 evaluation of silu (a few ulp), which could flip
  a code only on an exact rounding midpoint; a difference is accepted only
  there, and at most one.
* Down GEMM + combine: the oracle's own intermediate written into the
  workspace, then only the down GEMM and the combine run
  (fused_moe_down_combine): with no requantization decision left to the
  kernel, the output must lie within the arithmetic model's bound alone
  (tolerance 0, no near-tie allowance) of the oracle's.  [prime-flash]
  "Tests and benchmarks": the comparison isolates the kernel from the
  quantizer.
"""

import numpy as np
import pytest
import torch

import datagen
import mixture_experts_ffn_moe_amd as moe
from oracle import codecs
from oracle.moe import tolerance_check

from .gpu_helpers import oracle, out_bits, poisoned, say
from .test_gpu_moe import small_case

pytestmark = pytest.mark.gpu


def _ints(rng, shape, lo, hi):
    return rng.integers(lo, hi + 1, shape).astype(np.float64)


def exact_case(kind, T=48, K=512, I=256, E=6, k=2, seed=3):
    """Small integers, power-of-two scales; routing as the normal recipe."""
    rng = np.random.default_rng(seed)
    N = 2 * I
    ids, wts = datagen.make_routing(T, E, k, "normal", tag=f"exact-{kind}")
    xv = _ints(rng, (T, K), -4, 4)
    w1v = _ints(rng, (E, N, K), -4, 4)
    w2v = _ints(rng, (E, K, I), -4, 4)
    if kind == "bf16":
        def bf(v, s):
            return torch.from_numpy(codecs.bf16_encode(v * s).view(np.int16)).view(torch.bfloat16)
        x, w1, w2 = bf(xv, 1.0), bf(w1v, 2.0 ** -7), bf(w2v, 2.0 ** -7)
        xs = s1 = s2 = None
    else:
        x = torch.from_numpy(codecs.e4m3_encode(xv))
        w2 = torch.from_numpy(codecs.e4m3_encode(w2v))
        if kind == "mxfp4":
            # e2m1 integers -4..4 (codes of 0, 1, 2, 3, 4 and their negatives)
            v = np.clip(w1v, -4, 4)
            mag = {0: 0, 1: 2, 2: 4, 3: 5, 4: 6}
            nib = np.vectorize(lambda a: (8 if a < 0 else 0) | mag[int(abs(a))])(v).astype(np.uint8)
            w1 = torch.from_numpy(nib[..., 0::2] | (nib[..., 1::2] << 4))
            v2 = np.clip(w2v, -4, 4)
            nib2 = np.vectorize(lambda a: (8 if a < 0 else 0) | mag[int(abs(a))])(v2).astype(np.uint8)
            w2 = torch.from_numpy(nib2[..., 0::2] | (nib2[..., 1::2] << 4))
        else:
            w1 = torch.from_numpy(codecs.e4m3_encode(w1v))
        if kind == "fp8_blockwise":
            xs = torch.full((T, K // 128), 2.0 ** -2)
            s1 = torch.full((E, N // 128, K // 128), 2.0 ** -5)
            s2 = torch.full((E, K // 128, I // 128), 2.0 ** -5)
        else:
            xs = torch.full((T, K // 32), 127 - 2, dtype=torch.uint8)
            s1 = torch.full((E, N, K // 32), 127 - 5, dtype=torch.uint8)
            s2 = torch.full((E, K, I // 32), 127 - 5, dtype=torch.uint8)
    if kind != "bf16":
        x = x.view(torch.float8_e4m3fn)
        if kind != "mxfp4":
            w1 = w1.view(torch.float8_e4m3fn)
            w2 = w2.view(torch.float8_e4m3fn)
    c = datagen.Case(kind, T, K, I, E, k, x, xs, w1, s1, w2, s2, ids, wts)
    for f in ("x", "x_scale", "w1", "w1_scale", "w2", "w2_scale", "topk_ids", "topk_weights"):
        v = getattr(c, f)
        if v is not None:
            setattr(c, f, v.cuda())
    return c


def _intermediate(c, bm, tune=None):
    out0, ws, align0 = poisoned(c, bm, 1, tune)
    out, (sid, _, ntp) = moe.run_case(c, block_m=bm, split=1, out=out0, workspace=ws,
                                      align_out=align0, tune=tune)
    torch.cuda.synchronize()
    return ws.cpu().numpy(), sid.cpu().numpy(), int(ntp.item())


@pytest.mark.parametrize("kind", ["bf16", "fp8_blockwise", "mxfp8", "mxfp4"])
@pytest.mark.parametrize("bm", [16, 64])
def test_exact_arithmetic_intermediate(kind, bm):
    """The gate/up GEMM is exact here, so the only freedom left is the fp32
    evaluation of silu (a few ulp of h): a blockwise group's scale may move
    by that much (its amax element), and a decision (a code, an MX exponent)
    may go the other way only on a midpoint at that precision, which the
    24,576 codes of this case should not hold more than once."""
    c = exact_case(kind)
    K, I, E, k = c.K, c.I, c.E, c.top_k
    wsn, sid, n = _intermediate(c, bm)
    h_off, hs_off = moe.moe_workspace_layout(kind, c.T, K, 2 * I, E, k, bm)
    ref = oracle(c, keep_h=True)["h"]
    es = 2 if kind == "bf16" else 1
    sign = 0x8000 if es == 2 else 0x80
    decisions = 0
    total = 0
    for pos in range(n):
        rid = int(sid[pos])
        if rid < 0:
            continue
        q_ref, s_ref, _, _, _ = ref[rid]
        row = wsn[h_off + pos * I * es: h_off + (pos + 1) * I * es]
        if kind == "bf16":
            row = row.view(np.uint16)
        keep = np.ones(I, bool)
        if kind == "fp8_blockwise":
            srow = wsn[hs_off + pos * (I // 128) * 4: hs_off + (pos + 1) * (I // 128) * 4]
            rel = np.abs(srow.view(np.float32).astype(np.float64) / s_ref - 1.0)
            assert np.all(rel <= 2.0 ** -20), (pos, rel)
        elif kind != "bf16":
            srow = wsn[hs_off + pos * (I // 32): hs_off + (pos + 1) * (I // 32)]
            moved = srow != s_ref
            decisions += int(moved.sum())
            keep = ~np.repeat(moved, 32)
        diff = (row != q_ref) & keep
        a, b = row[diff].astype(np.int64), q_ref[diff].astype(np.int64)
        assert np.all(((a & sign) == (b & sign)) & (np.abs((a & (sign - 1)) - (b & (sign - 1))) == 1)), pos
        decisions += int(diff.sum())
        total += I
    say(f"      {kind} bm={bm}: {decisions} decisions differ of {total} codes")
    assert decisions <= 1


@pytest.mark.parametrize("kind,bm", [("bf16", 16), ("fp8_blockwise", 16), ("fp8_blockwise", 64),
                                     ("fp8_blockwise", 256), ("mxfp8", 16), ("mxfp8", 128),
                                     ("mxfp4", 16), ("mxfp4", 64)])
def test_down_combine_on_oracle_intermediate(kind, bm):
    T = 300 if bm >= 64 else 60
    c = small_case(kind, T=T, E=8, k=2, tag="gpu-stage")
    if bm == 256:
        c = small_case(kind, T=T, E=4, k=2, tag="gpu-stage", K=512, I=256)
    K, I, E, k = c.K, c.I, c.E, c.top_k
    say(f"[gpu] down + combine on the oracle's intermediate: {kind} T={T} K={K} I={I} bm={bm}")
    out0, ws, align0 = poisoned(c, bm, 1)
    sid, eid, ntp = moe.moe_align(c.topk_ids, E, bm, out=align0)
    torch.cuda.synchronize()
    ref = oracle(c, keep_h=True)
    h_off, hs_off = moe.moe_workspace_layout(kind, c.T, K, 2 * I, E, k, bm)
    wsn = ws.cpu().numpy()
    es = 2 if kind == "bf16" else 1
    sidn = sid.cpu().numpy()
    for pos in range(int(ntp.item())):
        rid = int(sidn[pos])
        if rid < 0:
            continue
        q, s, _, _, _ = ref["h"][rid]
        codes = q.view(np.uint8) if kind == "bf16" else q
        wsn[h_off + pos * I * es: h_off + (pos + 1) * I * es] = codes
        if kind == "fp8_blockwise":
            wsn[hs_off + pos * (I // 128) * 4: hs_off + (pos + 1) * (I // 128) * 4] = \
                s.astype(np.float32).view(np.uint8)
        elif kind != "bf16":
            wsn[hs_off + pos * (I // 32): hs_off + (pos + 1) * (I // 32)] = s
    ws.copy_(torch.from_numpy(wsn))
    out = moe.fused_moe_down_combine(kind, c.w2, c.w2_scale, sid, eid, ntp, c.topk_weights, k,
                                     bm, ws, c.T, out=out0)
    torch.cuda.synchronize()
    ok, stats = tolerance_check(out_bits(out), ref["out64"], 0.0, ref["dev_bound"])
    say(f"      stats {stats}")
    assert ok, stats
