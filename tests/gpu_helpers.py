"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
binding, run the oracle on the same seeded inputs, compare."""

import os
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


def oracle(case, tokens=None, keep_h=False, threads=1):
    """The fp64 oracle on the case's inputs (copied to the host), for all
    tokens or the given sorted ones.  threads > 1 evaluates each token on its
    own in a thread pool (numpy releases the interpreter lock in its array
    work) and stacks the rows; keep_h needs threads == 1."""
    ids = case.topk_ids.cpu().numpy()
    sel = ids if tokens is None else ids[np.asarray(tokens)]
    experts = sorted(set(int(e) for e in np.unique(sel) if 0 <= e < case.E))
    experts += [case.E + s for s in range(case.n_shared)]
    d = datagen.to_numpy(case, experts=experts)

    def run(toks):
        return moe_ref(d["kind"], d["x"], d["x_scale"], d["w1"], d["w1_scale"], d["w2"],
                       d["w2_scale"], d["topk_ids"], d["topk_weights"], tokens=toks,
                       keep_h=keep_h, n_shared=case.n_shared)

    if threads <= 1 or tokens is None or keep_h:
        return run(tokens)
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(threads) as ex:
        parts = list(ex.map(lambda t: run(np.array([t])), list(np.asarray(tokens))))
    return {k: np.concatenate([p[k] for p in parts]) for k in parts[0] if k != "h"}


def oracle_threads():
    """Worker threads for the oracle: the cores this process may use, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


SENTINEL = 0x7F7F7F7F


def poisoned(case, block_m, split, tune=None):
    """out full of NaN, the workspace full of 0xFF bytes (NaN as fp32, -1 as
    int32) and the planner outputs full of a sentinel: the library must write
    every element of out and of the plan, and clear what it counts on."""
    T, K = case.x.shape
    E_all = case.E + case.n_shared
    k_all = case.top_k + case.n_shared
    dev = case.x.device
    out = torch.full((T, K), float("nan"), dtype=torch.bfloat16, device=dev)
    need = moe.moe_workspace_size(case.kind, T, K, 2 * case.I, E_all, k_all, block_m, split,
                                  tune)
    ws = torch.full((max(need, 256),), 0xFF, dtype=torch.uint8, device=dev)
    rows, blocks = moe.moe_align_capacity(T, k_all, E_all, block_m)
    align = (torch.full((max(rows, 1),), SENTINEL, dtype=torch.int32, device=dev)[:rows],
             torch.full((max(blocks, 1),), SENTINEL, dtype=torch.int32, device=dev)[:blocks],
             torch.full((1,), SENTINEL, dtype=torch.int32, device=dev))
    return out, ws, align


def check(case, block_m, split, tokens=None, ref=None, label="", tune=None):
    say(f"[gpu] {label} kind={case.kind} T={case.T} K={case.K} I={case.I} E={case.E} "
        f"k={case.top_k} block_m={block_m} split={split} tune={tune}")
    out0, ws, align0 = poisoned(case, block_m, split, tune)
    out, align = moe.run_case(case, block_m=block_m, split=split, out=out0, workspace=ws,
                              align_out=align0, tune=tune)
    torch.cuda.synchronize()
    assert not bool((align[0] == SENTINEL).any()) and not bool((align[1] == SENTINEL).any())
    if ref is None:
        ref = oracle(case, tokens)
    got = out_bits(out)
    if tokens is not None:
        got = got[np.asarray(tokens)]
    ok, stats = tolerance_check(got, ref["out64"], TOL[case.kind], ref["allowance"])
    say(f"      stats {stats}")
    assert ok, stats
    return out, align, ref
