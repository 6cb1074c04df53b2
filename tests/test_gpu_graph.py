"""The planner and the forward captured in a HIP graph and replayed.

The C ABI calls enqueue on the caller's stream and, given preallocated
planner outputs, workspace and output, allocate nothing and never
synchronize, so ``torch.cuda.graph`` captures them (every clear in the path
is a fill kernel, not a memset node).  Each replay follows new token and
routing contents written in place and an eager call on those contents (eager
work between replays).  The split, ring and tiled modes fix their summation
order, so a replay must match the eager call bit for bit; the fused mode adds
each route's partial sums (one per intermediate slice) with atomics in no
fixed order, so its replays are checked against the fp64 oracle within the
parity tolerance instead."""

import pytest
import torch

import datagen
import mixture_experts_ffn_moe_amd as moe

from oracle.moe import tolerance_check

from .gpu_helpers import TOL, oracle, out_bits, say
from .test_gpu_moe import SHAPES, to_gpu

pytestmark = pytest.mark.gpu

# kind, T, E, top_k, block_m, split, shape overrides; together they run the
# streaming split kernels, the gate/up GEMM with K split over workgroups
# (K=2048, few tiles: streaming and 64-row tiled), the fused kernel, the
# LDS-tiled kernels at 64, 128 and 256 rows, the ring mode and the chunked
# planner (more than 16,384 routes)
CASES = [
    ("fp8_blockwise", 8, 16, 2, 16, 1, dict(K=2048, I=256)),
    ("fp8_blockwise", 200, 16, 4, 32, 1, {}),
    ("fp8_blockwise", 50, 8, 2, 16, 0, {}),
    ("fp8_blockwise", 300, 8, 4, 64, 1, {}),
    ("fp8_blockwise", 100, 8, 2, 16, 2, {}),
    ("bf16", 50, 8, 2, 16, 0, {}),
    ("bf16", 2100, 64, 8, 64, 1, dict(K=256, I=128)),
    ("mxfp8", 200, 8, 4, 32, 1, {}),
    ("mxfp4", 50, 8, 2, 16, 1, {}),
    ("mxfp8", 128, 8, 4, 64, 1, dict(K=2048, I=256)),
    ("fp8_blockwise", 600, 8, 2, 128, 1, dict(K=512, I=256)),
    ("fp8_blockwise", 1200, 4, 2, 256, 1, dict(K=512, I=256)),
]


def _case(kind, T, E, k, shp, tag):
    s = dict(SHAPES[kind])
    s.update(shp)
    return to_gpu(datagen.make_case(kind, T, s["K"], s["I"], E, k, routing="normal", tag=tag))


def _buffers(c, bm, split):
    rows, blocks = moe.moe_align_capacity(c.T, c.top_k, c.E, bm)
    dev = c.x.device
    align = (torch.empty(max(rows, 1), dtype=torch.int32, device=dev)[:rows],
             torch.empty(max(blocks, 1), dtype=torch.int32, device=dev)[:blocks],
             torch.empty(1, dtype=torch.int32, device=dev))
    need = moe.moe_workspace_size(c.kind, c.T, c.K, 2 * c.I, c.E, c.top_k, bm, split)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    out = torch.empty(c.T, c.K, dtype=torch.bfloat16, device=dev)
    return dict(block_m=bm, split=split, workspace=ws, out=out, align_out=align)


@pytest.mark.parametrize("kind,T,E,k,bm,split,shp", CASES,
                         ids=[f"{c[0]}-T{c[1]}-E{c[2]}-k{c[3]}-bm{c[4]}-s{c[5]}" for c in CASES])
def test_graph_replay_matches_eager(kind, T, E, k, bm, split, shp):
    say(f"[gpu] graph kind={kind} T={T} E={E} k={k} block_m={bm} split={split} {shp}")
    c = _case(kind, T, E, k, shp, "graph0")
    g_args = _buffers(c, bm, split)
    e_args = _buffers(c, bm, split)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the capture (allocates the planner scratch)
        moe.run_case(c, **g_args)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        moe.run_case(c, **g_args)
    torch.cuda.synchronize()

    for r in range(3):
        n = _case(kind, T, E, k, shp, f"graph{r + 1}")
        for f in ("x", "x_scale", "topk_ids", "topk_weights"):
            dst = getattr(c, f)
            if dst is not None:
                dst.copy_(getattr(n, f))
        eager, _ = moe.run_case(c, **e_args)
        torch.cuda.synchronize()
        want = out_bits(eager).copy()
        graph.replay()
        torch.cuda.synchronize()
        got = out_bits(g_args["out"])
        diff = int((got != want).sum())
        say(f"      replay {r}: {diff} of {got.size} outputs differ from the eager call")
        if split == 0:
            ref = oracle(c)
            ok, stats = tolerance_check(got, ref["out64"], TOL[kind], ref["allowance"])
            say(f"      oracle {stats}")
            assert ok, stats
        else:
            assert diff == 0
        assert torch.equal(g_args["align_out"][2], e_args["align_out"][2])
