"""Schedule overrides (moe_tune) on the GPU.  Every supported override must
pass the oracle gate on poisoned outputs and workspace.  The prefetch depth
and the tiled kernels' stage count change only how far ahead the operands
are loaded, not the order of any sum, so those results must also equal the
library's own choice bit for bit."""

import numpy as np
import pytest
import torch

import mixture_experts_ffn_moe_amd as moe

from .gpu_helpers import check, out_bits, poisoned, say
from .test_gpu_moe import small_case

pytestmark = pytest.mark.gpu


def _bits(c, bm, split, tune):
    out0, ws, align0 = poisoned(c, bm, split, tune)
    out, _ = moe.run_case(c, block_m=bm, split=split, out=out0, workspace=ws, align_out=align0,
                          tune=tune)
    torch.cuda.synchronize()
    return out_bits(out)


@pytest.mark.parametrize("kind", ["bf16", "fp8_blockwise", "mxfp8", "mxfp4"])
@pytest.mark.parametrize("bm,split", [(16, 1), (32, 1), (16, 0)])
@pytest.mark.parametrize("depth", [1, 2, 4])
def test_prefetch_depth(kind, bm, split, depth):
    c = small_case(kind, T=40, E=8, k=2, tag="gpu-tune")
    tune = {"prefetch": depth, "k_groups": 1}
    check(c, bm, split, tune=tune, label="tune")
    if split == 1:
        assert np.array_equal(_bits(c, bm, split, tune), _bits(c, bm, split, {"k_groups": 1}))


@pytest.mark.parametrize("kind", ["bf16", "fp8_blockwise", "mxfp8", "mxfp4"])
@pytest.mark.parametrize("groups", [1, 2])
def test_k_groups(kind, groups):
    c = small_case(kind, T=40, E=8, k=2, tag="gpu-tune")
    check(c, 16, 1, tune={"k_groups": groups}, label="tune")


@pytest.mark.parametrize("kind", ["fp8_blockwise", "mxfp8", "mxfp4", "bf16"])
def test_k_split_over_workgroups(kind):
    c = small_case(kind, T=24, E=8, k=2, tag="gpu-tune-ks", K=2048, I=256)
    check(c, 16, 1, tune={"k_split": 4}, label="tune")
    check(c, 16, 1, tune={"k_split": 1}, label="tune")


@pytest.mark.parametrize("kind", ["fp8_blockwise", "mxfp8"])
@pytest.mark.parametrize("bm", [64, 128])
@pytest.mark.parametrize("K,I", [(512, 384), (256, 128), (768, 384)])
def test_tiled_stages(kind, bm, K, I):
    """Two and three LDS stages.  K and I give the two GEMMs walks of 4 and
    3, 2 and 1, 6 and 3 steps: as long as the pipeline or shorter, and not
    a whole number of rounds of its slots."""
    c = small_case(kind, T=300, E=8, k=2, tag="gpu-tune-tiled", K=K, I=I)   # tiled: K % 256 == 0
    check(c, bm, 1, tune={"stages": 2}, label="tune")
    a = _bits(c, bm, 1, {"stages": 2})
    b = _bits(c, bm, 1, {"stages": 3})
    say(f"      stages 2 against 3: {int((a != b).sum())} outputs differ")
    assert np.array_equal(a, b)


@pytest.mark.parametrize("kind", ["fp8_blockwise", "mxfp8"])
@pytest.mark.parametrize("K,I", [(8448, 256), (512, 8448), (16384, 256), (512, 16384)])
def test_tiled_long_k_walks(kind, K, I):
    """More than 64 K steps in one tiled GEMM (66: the gate/up GEMM at
    K = 8448, the down GEMM at I = 8448; 128, the most the blockwise format
    allows, at 16384): the weight block-scale rows held for the walk, and
    every later step's operands, past their first 64."""
    c = small_case(kind, T=70, E=2, k=1, tag="gpu-tune-long", K=K, I=I)
    for bm in (64, 128):
        check(c, bm, 1, label="long K walk")
