"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
binding, run the oracle on the same seeded inputs, compare."""

import sys

import numpy as np
import torch

import datagen
import mixture_experts_ffn_moe_amd as moe
from oracle.moe import moe_ref, tolerance_check

# max |err| <= TOL * rms(out_oracle) (+ half a bf16 ulp), mean relative error
# <= 5e-3: the bounds of the fused-MoE parity requirement for FP8 and bf16.
TOL = {"bf16": 5e-3, "fp8_blockwise": 2e-2, "mxfp8": 2e-2, "mxfp4": 2e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def out_bits(out):
    return out.view(torch.int16).cpu().numpy().view(np.uint16)


def oracle(case, tokens=None, keep_h=False):
    ids = case.topk_ids.cpu().numpy()
    sel = ids if tokens is None else ids[np.asarray(tokens)]
    experts = sorted(set(int(e) for e in np.unique(sel) if 0 <= e < case.E))
    experts += [case.E + s for s in range(case.n_shared)]
    d = datagen.to_numpy(case, experts=experts)
    return moe_ref(d["kind"], d["x"], d["x_scale"], d["w1"], d["w1_scale"], d["w2"],
                   d["w2_scale"], d["topk_ids"], d["topk_weights"], tokens=tokens,
                   keep_h=keep_h, n_shared=case.n_shared)


def check(case, block_m, split, tokens=None, ref=None, label=""):
    say(f"[gpu] {label} kind={case.kind} T={case.T} K={case.K} I={case.I} E={case.E} "
        f"k={case.top_k} block_m={block_m} split={split}")
    out, align = moe.run_case(case, block_m=block_m, split=split)
    torch.cuda.synchronize()
    if ref is None:
        ref = oracle(case, tokens)
    got = out_bits(out)
    if tokens is not None:
        got = got[np.asarray(tokens)]
    ok, stats = tolerance_check(got, ref["out64"], TOL[case.kind], ref["flip_bound"])
    say(f"      stats {stats}")
    assert ok, stats
    return out, align, ref
