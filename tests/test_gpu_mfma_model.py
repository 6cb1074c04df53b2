"""The matrix instructions against the arithmetic model of the parity gate.

The gate accepts kernel outputs within an error model of the instructions
(oracle.moe.gemm_sigma): a 128-wide K step adds its products with a zero-mean
error of standard deviation at most KAPPA times the 2-norm of the products,
plus binary32 roundings of the running sum.  Here the instructions themselves
(moe_mfma_probe: one K step per 16 x 16 tile through the kernels' own
operand layout and wrappers) run on operands of the kinds the kernels see,
and their errors against exact fp64 sums must stay within the model:
root-mean-square of err / sigma at most 1, and no single error beyond
8 sigma.  The operand kinds: e4m3 codes of normal values scaled to amax 448
(activations and weights as quantized by block amax), codes of SwiGLU outputs
(the intermediate), tiny codes against normal ones, cancelling pairs,
accumulator inputs far larger than the products, MX scales, e2m1 weights,
bf16.  Outside the model: codes drawn uniformly over all e4m3 values, whose
products span 35 binades; the instruction then loses the small products
entirely (measured: 5.4e-5 of the 2-norm, RMS); that case is reported, not
asserted.
"""

import zlib

import numpy as np
import pytest
import torch

import mixture_experts_ffn_moe_amd as moe
from oracle import codecs
from oracle.moe import gemm_sigma

pytestmark = pytest.mark.gpu

NT = 2048


def _e4m3(v):
    return codecs.e4m3_encode(np.clip(v, -448.0, 448.0))


def _operands(name, rng):
    """(kind, A codes, B codes, A scales, B scales, C) as numpy arrays."""
    sa = sb = None
    c = np.zeros((NT, 16, 16), dtype=np.float32)
    shape = (NT, 16, 128)
    if name == "normal":
        a, b = _e4m3(rng.normal(0, 120, shape)), _e4m3(rng.normal(0, 120, shape))
    elif name == "swiglu":
        g, u = rng.normal(size=shape), rng.normal(size=shape)
        h = g / (1 + np.exp(-g)) * u
        a = _e4m3(h / np.max(np.abs(h), axis=2, keepdims=True) * 448.0)
        b = _e4m3(rng.normal(0, 120, shape))
    elif name == "small_by_normal":
        a, b = _e4m3(rng.normal(0, 0.05, shape)), _e4m3(rng.normal(0, 120, shape))
    elif name == "cancelling":
        a = _e4m3(rng.normal(0, 120, shape))
        a[:, :, 1::2] = a[:, :, 0::2] ^ 0x80
        b = _e4m3(rng.normal(0, 120, shape))
        b[:, :, 1::2] = b[:, :, 0::2]
        a[:, :, 127] = _e4m3(rng.normal(0, 1, (NT, 16)))
    elif name in ("large_c", "huge_c"):
        a, b = _e4m3(rng.normal(0, 120, shape)), _e4m3(rng.normal(0, 120, shape))
        c = (rng.normal(0, 1e4, c.shape) if name == "large_c"
             else np.full(c.shape, 2.0 ** 26)).astype(np.float32)
    elif name == "uniform_codes":
        a = rng.integers(0, 256, shape).astype(np.uint8)
        b = rng.integers(0, 256, shape).astype(np.uint8)
        for m in (a, b):
            m[(m & 0x7F) == 0x7F] = 0                 # no NaN codes
    if name.startswith("mx"):
        a = _e4m3(rng.normal(0, 120, shape))
        sa = rng.integers(120, 135, (NT, 16, 4)).astype(np.uint8)
        sb = rng.integers(120, 135, (NT, 16, 4)).astype(np.uint8)
        if name == "mxfp8":
            b = _e4m3(rng.normal(0, 120, shape))
        else:                                        # e2m1, two per byte
            nib = rng.integers(0, 16, (NT, 16, 128)).astype(np.uint8)
            b = (nib[:, :, 0::2] | (nib[:, :, 1::2] << 4)).astype(np.uint8)
    kind = {"mxfp8": "mxfp8", "mxfp4": "mxfp4"}.get(name, "fp8_blockwise")
    return kind, a, b, sa, sb, c


def _values(kind, a, b, sa, sb):
    av = codecs.e4m3_decode(a)
    if kind == "mxfp4":
        bv = codecs.e2m1_decode(codecs.fp4_unpack(b))
    else:
        bv = codecs.e4m3_decode(b)
    if sa is not None:
        av = av * np.repeat(codecs.e8m0_decode(sa), 32, axis=2)
        bv = bv * np.repeat(codecs.e8m0_decode(sb), 32, axis=2)
    return av, bv


def _check(kind, av, bv, c, d, label, assert_model=True):
    exact = c.astype(np.float64) + np.matmul(av, np.swapaxes(bv, 1, 2))
    sig = np.stack([gemm_sigma(kind, av[t], bv[t], exact[t]) for t in range(av.shape[0])])
    z = np.abs(d.astype(np.float64) - exact) / sig
    rms, mx = float(np.sqrt(np.mean(z * z))), float(np.max(z))
    print(f"{label}: rms err/sigma {rms:.3f}, max err/sigma {mx:.2f}", flush=True)
    if assert_model:
        assert rms <= 1.0 and mx <= 8.0, (label, rms, mx)
    return rms, mx


def _run(kind, a, b, sa, sb, c):
    dev = torch.device("cuda", 0)
    t = [None if v is None else torch.from_numpy(np.ascontiguousarray(v)).to(dev)
         for v in (a, b, sa, sb, c)]
    d = moe.moe_mfma_probe(kind, t[0], t[1], t[2], t[3], t[4])
    torch.cuda.synchronize()
    return d.cpu().numpy()


@pytest.mark.parametrize("name", ["normal", "swiglu", "small_by_normal", "cancelling", "large_c",
                                  "huge_c", "mxfp8", "mxfp4"])
def test_e4m3_instruction_within_model(name):
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    kind, a, b, sa, sb, c = _operands(name, rng)
    d = _run(kind, a, b, sa, sb, c)
    av, bv = _values(kind, a, b, sa, sb)
    _check(kind, av, bv, c, d, name)


def test_uniform_codes_reported():
    rng = np.random.default_rng(99)
    kind, a, b, sa, sb, c = _operands("uniform_codes", rng)
    d = _run(kind, a, b, sa, sb, c)
    av, bv = _values(kind, a, b, sa, sb)
    _check(kind, av, bv, c, d, "uniform codes (outside the model)", assert_model=False)


@pytest.mark.parametrize("with_c", [False, True])
def test_bf16_instruction_within_model(with_c):
    g = torch.Generator().manual_seed(5 + with_c)
    a = torch.randn(NT, 16, 128, generator=g).to(torch.bfloat16)
    b = torch.randn(NT, 16, 128, generator=g).to(torch.bfloat16)
    c = (torch.randn(NT, 16, 16, generator=g) * 100 if with_c else
         torch.zeros(NT, 16, 16)).float()
    dev = torch.device("cuda", 0)
    d = moe.moe_mfma_probe("bf16", a.to(dev), b.to(dev), None, None, c.to(dev))
    torch.cuda.synchronize()
    av = codecs.bf16_decode(a.view(torch.int16).numpy().view(np.uint16))
    bv = codecs.bf16_decode(b.view(torch.int16).numpy().view(np.uint16))
    _check("bf16", av, bv, c.numpy(), d.cpu().numpy(), f"bf16 C={'N(0,100^2)' if with_c else 0}")
