"""Seeded synthetic inputs for the fused MoE forward.

This module is shared by the tests, the smoke check and the benchmark.  It
holds no step of the expert FFN itself; it only draws inputs and prepares them
the way an upstream caller would:

* activations x ~ N(0, 1) and expert weights (bf16: N(0, 0.02^2); FP8 and MX:
  N(0, 1/K) with K the hidden size);
* routing: router logits per token, softmax over all experts, top-k by
  descending logit, weights renormalized to sum to 1 in fp32 (the pages take
  routing as given; this stands in for a model's gate);
* caller-side input quantization.  The [prime-flash] page ("Scale layout")
  leaves producing e4m3 values and e8m0 exponents to the caller; here
  - blockwise: one fp32 scale per 1 x 128 block of x and per 128 x 128 block of
    w1/w2, scale = amax / 448 (amax floored at 1e-10), values cast to e4m3;
  - MX: one e8m0 exponent per 32 elements along the contraction dimension,
    exponent = floor(log2 amax) - 8 (OCP MX rule for e4m3), values saturated to
    +-448 and cast to e4m3.
  - MXFP4 weights ([DeepGEMM #411] "Summary": packed E2M1 with a UE8M0
    exponent per 32 along K): exponent = floor(log2 amax) - 2 (OCP MX rule
    for E2M1, whose largest magnitude is 1.5 * 2^2), values rounded to the
    nearest E2M1 magnitude with ties to the even code, saturated to +-6, two
    codes per byte (element 2j in the low nibble).  Activations stay MX FP8.
  All done with torch tensor ops, on the CPU or on the GPU.

Randomness: ``torch.Generator`` seeded from a CRC of (workload, tensor name,
token count where it applies), so one weight set serves every token count.
The public model shapes the workloads stand in for have no weights or router
outputs available; these draws replace them.
"""

import zlib
from dataclasses import dataclass, field
from typing import Optional

import torch

# Workloads, named by what they are.  The FFN shapes follow the model
# configurations the [DeepGEMM #88] page benchmarks (hidden / intermediate /
# routed experts / top-k), plus a narrow-intermediate MX shape (the
# [prime-flash] usage example's N=512 at K=4096) and a tiny bf16 shape.
WORKLOADS = {
    # tiny bf16 correctness shape
    "bf16-k512-i256-e8-top2": dict(
        kind="bf16", K=512, I=256, E=8, top_k=2, tokens=(32,),
        routing="normal", w_std=0.02),
    # DeepSeek-V4-Flash shape, decode-sized batches
    "fp8-k4096-i2048-e256-top6": dict(
        kind="fp8_blockwise", K=4096, I=2048, E=256, top_k=6,
        tokens=(8, 64, 256), routing="uniform"),
    # GLM-5.3-Flash shape, prefill-sized batches, 8 experts masked empty
    "fp8-k4096-i2048-e288-top8": dict(
        kind="fp8_blockwise", K=4096, I=2048, E=288, top_k=8,
        tokens=(1024, 2048, 4096, 8192), routing="normal_masked", n_masked=8),
    # DeepSeek-V4-Pro shape with Zipf(1.1)-skewed expert load
    "fp8-k7168-i3072-e384-top6": dict(
        kind="fp8_blockwise", K=7168, I=3072, E=384, top_k=6,
        tokens=(256, 1024, 4096), routing="zipf", zipf_s=1.1),
    # narrow local intermediate (N=512), MX FP8
    "mx-k4096-i256-e32-top8": dict(
        kind="mxfp8", K=4096, I=256, E=32, top_k=8,
        tokens=(8, 32, 128, 512), routing="uniform"),
    # the DeepSeek-V4-Flash decode shape with MXFP4 weights and MX FP8
    # activations (the weight format of the [DeepGEMM #411] page)
    "mxfp4-k4096-i2048-e256-top6": dict(
        kind="mxfp4", K=4096, I=2048, E=256, top_k=6,
        tokens=(8, 64, 256), routing="uniform"),
}


def _seed(*parts):
    return zlib.crc32("/".join(str(p) for p in parts).encode()) & 0x7FFFFFFF


def _gen(device, *parts):
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*parts))
    return g


# ---------------------------------------------------------------------------
# caller-side input quantizers (torch ops)
# ---------------------------------------------------------------------------

def quant_blockwise_rows(x):
    """(T, K) float32 -> (e4m3 (T, K), fp32 scales (T, K/128))."""
    T, K = x.shape
    xb = x.reshape(T, K // 128, 128)
    amax = xb.abs().amax(dim=2).clamp_min(1e-10)
    scale = amax * (1.0 / 448.0)
    q = (xb * (1.0 / scale)[:, :, None]).clamp(-448.0, 448.0)
    return q.reshape(T, K).to(torch.float8_e4m3fn), scale.float()


def quant_blockwise_mat(w):
    """(R, C) float32 -> (e4m3 (R, C), fp32 scales (R/128, C/128))."""
    R, C = w.shape
    wb = w.reshape(R // 128, 128, C // 128, 128)
    amax = wb.abs().amax(dim=(1, 3)).clamp_min(1e-10)
    scale = amax * (1.0 / 448.0)
    q = (wb * (1.0 / scale)[:, None, :, None]).clamp(-448.0, 448.0)
    return q.reshape(R, C).to(torch.float8_e4m3fn), scale.float()


def quant_mx(w):
    """(..., C) float32 -> (e4m3 (..., C), e8m0 uint8 (..., C/32))."""
    shp = w.shape
    wb = w.reshape(*shp[:-1], shp[-1] // 32, 32)
    amax = wb.abs().amax(dim=-1)
    _, ex = torch.frexp(amax)                 # amax = m * 2^ex, m in [0.5, 1)
    s = (ex.to(torch.int32) - 1) - 8
    s = torch.where(amax > 0, s.clamp(-127, 127), torch.full_like(s, -127))
    scaled = torch.ldexp(wb, (-s).to(wb.dtype)[..., None])
    q = scaled.clamp(-448.0, 448.0).reshape(shp).to(torch.float8_e4m3fn)
    return q, (s + 127).to(torch.uint8)


# E2M1 magnitudes by code and the midpoints between neighbouring codes
_E2M1_MIDS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


def quant_mxfp4(w):
    """(..., C) float32 -> (packed e2m1 uint8 (..., C/2), e8m0 uint8 (..., C/32))."""
    shp = w.shape
    wb = w.reshape(*shp[:-1], shp[-1] // 32, 32)
    amax = wb.abs().amax(dim=-1)
    _, ex = torch.frexp(amax)                 # amax = m * 2^ex, m in [0.5, 1)
    s = (ex.to(torch.int32) - 1) - 2
    s = torch.where(amax > 0, s.clamp(-127, 127), torch.full_like(s, -127))
    a = torch.ldexp(wb.abs(), (-s).to(wb.dtype)[..., None])   # exact: power-of-two scale
    mids = torch.tensor(_E2M1_MIDS, dtype=a.dtype, device=a.device)
    code = torch.bucketize(a, mids)           # ties go to the lower code ...
    lower = code.clamp(max=6)
    tie = (code < 7) & (a == mids[lower]) & (code % 2 == 1)
    code = code + tie.to(code.dtype)          # ... and to the upper one when it is even
    code = code | torch.where(wb < 0, 8, 0).to(code.dtype)
    code = code.to(torch.uint8).reshape(*shp[:-1], shp[-1] // 2, 2)
    packed = code[..., 0] | (code[..., 1] << 4)
    return packed, (s + 127).to(torch.uint8)


# ---------------------------------------------------------------------------
# routing
# ---------------------------------------------------------------------------

def make_router_logits(T, E, top_k, routing, device="cpu", tag="routing", **kw):
    """Router logits (T, E) fp32 of the given routing recipe ("uniform",
    "normal", "normal_masked" with -inf for n_masked seeded experts, "zipf")."""
    g = _gen(device, tag, T, E, top_k, routing)
    if routing == "uniform":
        logits = torch.rand(T, E, generator=g, device=device)
    else:
        logits = torch.randn(T, E, generator=g, device=device)
    if routing == "normal_masked":
        gm = _gen("cpu", tag, "mask", E)
        masked = torch.randperm(E, generator=gm)[: kw.get("n_masked", 8)]
        logits[:, masked.to(device)] = float("-inf")
    elif routing == "zipf":
        gz = _gen("cpu", tag, "zipf", E)
        rank = torch.randperm(E, generator=gz).to(torch.float64) + 1.0
        bias = (-kw.get("zipf_s", 1.1) * torch.log(rank)).float()
        logits = logits + bias.to(device)[None, :]
    return logits.float().contiguous()


def make_routing(T, E, top_k, routing, device="cpu", tag="routing", **kw):
    """topk_ids (T, top_k) int32 and topk_weights (T, top_k) fp32 for the
    expert FFN's inputs: the recipe's logits through torch's softmax and
    topk (a library stand-in for the model's gate)."""
    logits = make_router_logits(T, E, top_k, routing, device=device, tag=tag, **kw)
    probs = torch.softmax(logits, dim=1)
    w, ids = torch.topk(probs, top_k, dim=1, largest=True, sorted=True)
    w = w / w.sum(dim=1, keepdim=True)
    return ids.to(torch.int32).contiguous(), w.float().contiguous()


# ---------------------------------------------------------------------------
# cases
# ---------------------------------------------------------------------------

@dataclass
class Case:
    kind: str
    T: int
    K: int
    I: int
    E: int
    top_k: int
    x: torch.Tensor
    x_scale: Optional[torch.Tensor]
    w1: torch.Tensor
    w1_scale: Optional[torch.Tensor]
    w2: torch.Tensor
    w2_scale: Optional[torch.Tensor]
    topk_ids: torch.Tensor
    topk_weights: torch.Tensor
    extra: dict = field(default_factory=dict)
    n_shared: int = 0   # shared experts stored after the E routed ones in w1 / w2

    @property
    def N(self):
        return 2 * self.I


def make_weights(kind, K, I, E, device="cpu", tag="w", w_std=None, chunk=8):
    """Expert weights in the layout the kernels take.

    bf16: w1 (E, 2I, K), w2 (E, K, I) bf16.  Blockwise: e4m3 values plus fp32
    scales (E, 2I/128, K/128) and (E, K/128, I/128).  MX: e4m3 values plus e8m0
    scales (E, 2I, K/32) and (E, K, I/32).  MXFP4: packed e2m1 pairs
    (E, 2I, K/2) and (E, K, I/2) plus the same e8m0 scale shapes as MX.
    """
    N = 2 * I
    if kind == "bf16":
        std = 0.02 if w_std is None else w_std
        g = _gen(device, tag, kind, K, I, E, "w1")
        w1 = (torch.randn(E, N, K, generator=g, device=device) * std).to(torch.bfloat16)
        g = _gen(device, tag, kind, K, I, E, "w2")
        w2 = (torch.randn(E, K, I, generator=g, device=device) * std).to(torch.bfloat16)
        return w1, None, w2, None
    std = (1.0 / K) ** 0.5 if w_std is None else w_std
    if kind == "mxfp4":
        w1 = torch.empty(E, N, K // 2, dtype=torch.uint8, device=device)
        w2 = torch.empty(E, K, I // 2, dtype=torch.uint8, device=device)
    else:
        w1 = torch.empty(E, N, K, dtype=torch.float8_e4m3fn, device=device)
        w2 = torch.empty(E, K, I, dtype=torch.float8_e4m3fn, device=device)
    if kind == "fp8_blockwise":
        s1 = torch.empty(E, N // 128, K // 128, dtype=torch.float32, device=device)
        s2 = torch.empty(E, K // 128, I // 128, dtype=torch.float32, device=device)
    else:
        s1 = torch.empty(E, N, K // 32, dtype=torch.uint8, device=device)
        s2 = torch.empty(E, K, I // 32, dtype=torch.uint8, device=device)
    g1 = _gen(device, tag, kind, K, I, E, "w1")
    g2 = _gen(device, tag, kind, K, I, E, "w2")
    for e0 in range(0, E, chunk):
        e1 = min(E, e0 + chunk)
        a = torch.randn(e1 - e0, N, K, generator=g1, device=device) * std
        b = torch.randn(e1 - e0, K, I, generator=g2, device=device) * std
        for e in range(e0, e1):
            if kind == "fp8_blockwise":
                w1[e], s1[e] = quant_blockwise_mat(a[e - e0])
                w2[e], s2[e] = quant_blockwise_mat(b[e - e0])
            elif kind == "mxfp4":
                w1[e], s1[e] = quant_mxfp4(a[e - e0])
                w2[e], s2[e] = quant_mxfp4(b[e - e0])
            else:
                w1[e], s1[e] = quant_mx(a[e - e0])
                w2[e], s2[e] = quant_mx(b[e - e0])
        del a, b
    return w1, s1, w2, s2


def make_tokens(kind, T, K, device="cpu", tag="x"):
    """Activations x (T, K) and their scales for the given path."""
    g = _gen(device, tag, kind, T, K)
    x = torch.randn(T, K, generator=g, device=device)
    if kind == "bf16":
        return x.to(torch.bfloat16), None
    if kind == "fp8_blockwise":
        return quant_blockwise_rows(x)
    return quant_mx(x)


def make_case(kind, T, K, I, E, top_k, routing="uniform", device="cpu",
              tag="case", weights=None, n_shared=0, **kw):
    """A full input set.  ``weights`` may pass a (w1, s1, w2, s2) tuple to
    reuse one weight set across token counts.  ``n_shared`` adds that many
    shared experts after the E routed ones in the weights (routing stays over
    the E routed experts)."""
    if weights is None:
        weights = make_weights(kind, K, I, E + n_shared, device=device, tag=tag,
                               w_std=kw.get("w_std"))
    w1, s1, w2, s2 = weights
    x, xs = make_tokens(kind, T, K, device=device, tag=tag)
    ids, wts = make_routing(T, E, top_k, routing, device=device, tag=tag, **kw)
    return Case(kind, T, K, I, E, top_k, x, xs, w1, s1, w2, s2, ids, wts, n_shared=n_shared)


def make_workload_case(name, T, device="cpu", weights=None):
    spec = dict(WORKLOADS[name])
    kind = spec.pop("kind")
    K, I, E, k = spec.pop("K"), spec.pop("I"), spec.pop("E"), spec.pop("top_k")
    spec.pop("tokens")
    routing = spec.pop("routing")
    return make_case(kind, T, K, I, E, k, routing=routing, device=device,
                     tag=name, weights=weights, **spec)


class ExpertSubset:
    """Host copy of a few experts of an (E, ...) weight tensor: indexable by
    expert id and reporting the full shape; reading another expert raises."""

    def __init__(self, shape, parts):
        self.shape = shape
        self._parts = parts

    def __getitem__(self, e):
        return self._parts[int(e)]


def to_numpy(case, experts=None):
    """Host copies in the oracle's conventions: bf16 as uint16 bits, e4m3 as
    uint8 codes, scales as float32 / uint8.  ``experts`` limits the weight copy
    to those experts (see :class:`ExpertSubset`)."""
    import numpy as np

    def bits(t):
        if t is None:
            return None
        t = t.detach().contiguous().cpu()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16)
        if t.dtype == torch.float8_e4m3fn:
            return t.view(torch.uint8).numpy()
        return t.numpy()

    def wsel(t):
        if t is None or experts is None:
            return bits(t)
        return ExpertSubset(tuple(t.shape),
                            {int(e): bits(t[int(e)]) for e in experts})

    return dict(kind=case.kind, x=bits(case.x), x_scale=bits(case.x_scale),
                w1=wsel(case.w1), w1_scale=wsel(case.w1_scale),
                w2=wsel(case.w2), w2_scale=wsel(case.w2_scale),
                topk_ids=bits(case.topk_ids), topk_weights=bits(case.topk_weights),
                n_shared=case.n_shared)
