"""C ABI checks that need no GPU: the library loads, exports every function
include/moe.h declares, and rejects bad arguments on the host before anything
is enqueued (each call below returns before its first HIP call)."""

import ctypes
import os
import re

import pytest

import mixture_experts_ffn_moe_amd as moe

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "moe.h")
FAKE = 1 << 20          # 16-byte aligned, never dereferenced (errors come first)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(\w+)\s*\(", text, flags=re.M)))


def test_header_symbols_exported():
    L = moe.lib()
    names = declared_functions()
    assert set(names) == set(moe.EXPORTED_SYMBOLS), names
    for n in names:
        assert hasattr(L, n), n


def test_capacity_closed_form():
    for T, k, E, bm in [(0, 2, 8, 16), (1, 6, 256, 16), (8192, 8, 288, 128), (37, 3, 5, 64)]:
        rows, blocks = moe.moe_align_capacity(T, k, E, bm)
        R = T * k
        assert rows == R + min(E, R) * (bm - 1)
        assert blocks == -(-rows // bm)


@pytest.mark.parametrize("args,status", [
    ((-1, 2, 8, 16), -2), ((4, 0, 8, 16), -2), ((4, 2, 0, 16), -2),
    ((4, 2, 8, 48), -3), ((4, 2, 8, 512), -3), ((1 << 29, 8, 8, 16), -2)])
def test_capacity_errors(args, status):
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_align_capacity(*args)
    assert ei.value.status == status


def test_align_errors_before_launch():
    L = moe.lib()
    P = ctypes.c_void_p
    # E > 1024
    assert L.moe_align(P(FAKE), 4, 2, 2000, 16, P(FAKE), P(FAKE), P(FAKE), None, 0, None) == -3
    # null outputs
    assert L.moe_align(P(FAKE), 4, 2, 8, 16, None, P(FAKE), P(FAKE), None, 0, None) == -1
    # misaligned
    assert L.moe_align(P(FAKE + 4), 4, 2, 8, 16, P(FAKE), P(FAKE), P(FAKE), None, 0,
                       None) == -4
    assert b"aligned" in L.moe_last_error()
    # misaligned workspace
    assert L.moe_align(P(FAKE), 4096, 8, 8, 16, P(FAKE), P(FAKE), P(FAKE), P(FAKE + 4), 1 << 20,
                       None) == -4


def test_align_workspace_size():
    """0 up to 16,384 routes (one workgroup plans), then 4 bytes per expert
    and chunk of 512 routes (the chunked planner)."""
    assert moe.moe_align_workspace_size(2048, 8, 288) == 0
    assert moe.moe_align_workspace_size(2049, 8, 288) == 4 * 33 * 288
    assert moe.moe_align_workspace_size(8192, 8, 288) == 4 * 128 * 288
    for bad in ((-1, 8, 288), (8, 0, 288), (8, 8, 0)):
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_align_workspace_size(*bad)
        assert ei.value.status == -2


def test_route_align_errors_before_launch():
    L = moe.lib()
    P = ctypes.c_void_p

    def call(T=4, E=8, k=2, bm=16, logits=FAKE, ids=FAKE, ws=FAKE, ws_bytes=256):
        return L.moe_route_align(P(logits) if logits else None, T, E, k, bm, P(ids) if ids else None,
                                 P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(ws) if ws else None,
                                 ws_bytes, None)
    assert moe.moe_route_align_workspace_size() == 256
    assert call(E=2000) == -3                  # E > 1024
    assert call(k=17, E=64) == -3              # top_k > 16
    assert call(k=9, E=8) == -3                # top_k > E
    assert call(bm=48) == -3
    assert call(T=-1) == -2
    assert call(logits=0) == -1
    assert call(ids=0) == -1
    assert call(ws=0) == -1
    assert call(logits=FAKE + 4) == -4         # misaligned
    assert call(ws_bytes=8) == -5
    assert b"workspace" in L.moe_last_error()


def _ffn(L, fn, K=4096, N=4096, T=8, E=16, k=2, bm=16, split=-1, ws=FAKE, ws_bytes=1 << 40,
         x=FAKE, sorted_ids=FAKE, scales=True, tune=None):
    P = ctypes.c_void_p
    tail = [P(sorted_ids), P(FAKE), P(FAKE), P(FAKE), P(FAKE), T, K, N, E, k, bm, split,
            None if tune is None else ctypes.byref(moe.MoeTune(**tune)),
            P(ws) if ws else None, ws_bytes, None]
    if fn == "fused_moe_bf16":
        return getattr(L, fn)(P(x), P(FAKE), P(FAKE), *tail)
    s = P(FAKE) if scales else None
    return getattr(L, fn)(P(x), s, P(FAKE), s, P(FAKE), s, *tail)


@pytest.mark.parametrize("fn", ["fused_moe_bf16", "fused_moe_fp8_blockwise", "fused_moe_mxfp8",
                                "fused_moe_mxfp4"])
def test_ffn_errors_before_launch(fn):
    L = moe.lib()
    assert _ffn(L, fn, K=4000) == -3                    # K % 128
    assert _ffn(L, fn, N=4095) == -2                    # odd N
    assert _ffn(L, fn, N=4096 + 128) == -3              # I % 128
    assert _ffn(L, fn, bm=24) == -3                     # block_m
    if fn in ("fused_moe_bf16", "fused_moe_mxfp4"):
        assert _ffn(L, fn, bm=256) == -3                # 256 needs e4m3 weights
    else:
        assert _ffn(L, fn, bm=256, K=384 * 2 + 128) == -3   # 256 needs K % 256 == 0
        assert _ffn(L, fn, bm=256, split=0) == -3       # 256 runs the split mode only
    assert _ffn(L, fn, T=-1) == -2
    assert _ffn(L, fn, k=0) == -2
    assert _ffn(L, fn, split=3) == -3
    assert _ffn(L, fn, split=2, bm=64) == -3            # the ring mode runs 16 or 32 rows
    assert _ffn(L, fn, split=2, ws_bytes=100) == -5     # not even one ring slot
    assert b"ring slot" in L.moe_last_error()
    assert _ffn(L, fn, x=0) == -1                       # null input
    assert _ffn(L, fn, x=FAKE + 8) == -4                # misaligned
    assert _ffn(L, fn, ws=0) == -5                      # no workspace
    assert _ffn(L, fn, ws_bytes=100) == -5              # workspace too small
    assert b"workspace" in L.moe_last_error()
    if fn != "fused_moe_bf16":
        assert _ffn(L, fn, scales=False) == -1
    # T == 0 is a successful no-op (no launch)
    assert _ffn(L, fn, T=0) == 0


@pytest.mark.parametrize("fn", ["fused_moe_bf16", "fused_moe_fp8_blockwise", "fused_moe_mxfp8",
                                "fused_moe_mxfp4"])
def test_tune_errors_before_launch(fn):
    """Every set field of moe_tune must name a variant the call's kernels
    have; otherwise MOE_ERR_UNSUPPORTED before any launch."""
    L = moe.lib()
    tiled = fn in ("fused_moe_fp8_blockwise", "fused_moe_mxfp8")
    for field, bad in (("k_groups", 3), ("k_split", 2), ("prefetch", 3), ("stages", 4),
                       ("k_groups", -1)):
        assert _ffn(L, fn, split=1, tune={field: bad}) == -3, (field, bad)
        assert b"tune." + field.encode() in L.moe_last_error()
    # a field for kernels the call does not run
    assert _ffn(L, fn, bm=64, split=1, tune={"k_groups": 2}) == -3
    assert _ffn(L, fn, bm=64, split=1, tune={"prefetch": 2}) == -3
    assert _ffn(L, fn, bm=16, split=2, tune={"prefetch": 2}) == -3     # ring mode
    assert _ffn(L, fn, bm=16, split=1, tune={"stages": 2}) == -3       # streaming kernels
    assert _ffn(L, fn, bm=64, split=0, tune={"stages": 2}) == -3       # fused mode
    if not tiled:
        assert _ffn(L, fn, bm=64, split=1, tune={"stages": 2}) == -3   # no tiled kernels
    assert _ffn(L, fn, K=1024, bm=16, split=1, tune={"k_split": 4}) == -3   # K / 128 < 16
    assert _ffn(L, fn, K=2176, bm=16, split=1, tune={"k_split": 4}) == -3   # not a multiple of 8
    assert _ffn(L, fn, bm=16, split=0, tune={"k_split": 4}) == -3
    assert _ffn(L, fn, bm=16, split=1, tune={"k_split": 4, "k_groups": 1}) == -3
    assert _ffn(L, fn, bm=16, split=1, tune={"k_split": 4, "prefetch": 2}) == -3
    assert _ffn(L, fn, K=128, bm=16, split=1, tune={"k_groups": 2}) == -3   # one K step
    # supported overrides pass the checks (the call then stops at T == 0)
    ok = [{"k_groups": 1}, {"k_groups": 2}, {"k_split": 4}, {"k_split": 1, "prefetch": 1},
          {"prefetch": 2}, {"prefetch": 4}, {"k_groups": 2, "prefetch": 4}]
    for t in ok:
        assert _ffn(L, fn, T=0, bm=16, split=1, tune=t) == 0, t
        assert _ffn(L, fn, T=0, bm=32, split=0, tune={k: v for k, v in t.items()
                                                         if k != "k_split"}) == 0, t
    # the gate/up K split: 16- and 32-row streaming blocks, and the 64-row
    # LDS-tiled kernels of the e4m3 dtypes
    assert _ffn(L, fn, T=0, bm=64, split=1, tune={"k_split": 4}) == (0 if tiled else -3)
    assert _ffn(L, fn, bm=128, split=1, tune={"k_split": 4}) == -3
    assert _ffn(L, fn, K=1024, bm=64, split=1, tune={"k_split": 4}) == -3   # K / 128 < 16
    if tiled:
        for st in (2, 3):
            assert _ffn(L, fn, T=0, bm=128, split=1, tune={"stages": st}) == 0
        assert _ffn(L, fn, bm=256, split=1, tune={"stages": 3}) == -3  # 256 rows: two stages
    # the same checks in moe_workspace_size, which also sizes the K-split sums
    dt = {"fused_moe_bf16": "bf16", "fused_moe_fp8_blockwise": "fp8_blockwise",
          "fused_moe_mxfp8": "mxfp8", "fused_moe_mxfp4": "mxfp4"}[fn]
    plain = moe.moe_workspace_size(dt, 2048, 4096, 4096, 256, 6, 16, 1, {"k_split": 1})
    split4 = moe.moe_workspace_size(dt, 2048, 4096, 4096, 256, 6, 16, 1, {"k_split": 4})
    assert split4 > plain
    with pytest.raises(moe.MoeError):
        moe.moe_workspace_size(dt, 8, 4096, 4096, 256, 6, 16, 1, {"prefetch": 3})


def test_workspace_sizes_grow_with_tokens():
    small = moe.moe_workspace_size("fp8_blockwise", 64, 4096, 4096, 256, 6, 16, split=1)
    big = moe.moe_workspace_size("fp8_blockwise", 4096, 4096, 4096, 256, 6, 64, split=1)
    fused = moe.moe_workspace_size("fp8_blockwise", 64, 4096, 4096, 256, 6, 16, split=0)
    assert 0 < small < big
    assert fused == 64 * 4096 * 4
    h, hs = moe.moe_workspace_layout("fp8_blockwise", 64, 4096, 4096, 256, 6, 16)
    assert h % 256 == 0 and hs > h


def test_heuristics():
    assert moe.moe_select_block_m(8, 6, 256) == 16
    assert moe.moe_select_block_m(8192, 8, 288, "fp8_blockwise", 4096) == 256  # 228 rows/expert
    assert moe.moe_select_block_m(8192, 8, 288, "mxfp8", 4096) == 256
    assert moe.moe_select_block_m(8192, 8, 288, "mxfp8", 4096 + 128) == 128
    assert moe.moe_select_block_m(8192, 8, 288, "bf16", 4096) == 128
    assert moe.moe_select_block_m(4096, 8, 288, "fp8_blockwise", 4096) == 128  # 114 rows/expert
    assert moe.moe_select_block_m(1024, 8, 288, "fp8_blockwise", 4096) == 64   # 28 rows/expert
    assert moe.moe_select_block_m(1024, 6, 384, "fp8_blockwise", 7168) == 64   # 16 rows/expert
    assert moe.moe_select_block_m(256, 8, 288, "fp8_blockwise", 4096) == 16    # 7 rows/expert
    assert moe.moe_select_block_m(256, 6, 256, "fp8_blockwise", 4096) == 16    # 6 rows/expert
    assert moe.moe_select_block_m(512, 8, 288, "fp8_blockwise", 4096) == 64    # 14 rows/expert
    assert moe.moe_select_block_m(64, 6, 256, "fp8_blockwise", 4096 + 128) == 16


def test_routed_heuristic():
    # the even-spread selector is the routed one with min(T*top_k, E) active experts
    for T, k, E in [(8, 6, 256), (256, 6, 256), (1024, 8, 288), (8192, 8, 288), (3, 2, 64)]:
        for kind in ("fp8_blockwise", "mxfp8", "bf16", "mxfp4"):
            act = min(T * k, E)
            assert (moe.moe_select_block_m(T, k, E, kind, 4096)
                    == moe.moe_select_block_m_routed(T, k, E, act, kind, 4096))
    # skewed routing: few active experts holding many rows each
    assert moe.moe_select_block_m_routed(256, 6, 384, 59, "fp8_blockwise", 7168) == 64
    assert moe.moe_select_block_m_routed(2048, 6, 384, 112, "fp8_blockwise", 7168) == 128
    # 203 rows per active expert but 64 per expert: not every expert fills 256 rows
    assert moe.moe_select_block_m_routed(4096, 6, 384, 121, "fp8_blockwise", 7168) == 128
    assert moe.moe_select_block_m_routed(8192, 8, 288, 280, "fp8_blockwise", 4096) == 256
    assert moe.moe_select_block_m_routed(0, 6, 256, 0, "fp8_blockwise", 4096) == 16
    for bad in (-1, 257):
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_select_block_m_routed(8, 6, 256, bad, "fp8_blockwise", 4096)
        assert ei.value.status == -2
    assert moe.moe_select_split("fp8_blockwise", 8, 4096, 4096, 256, 6, 16) == 1  # 6.4 GB of weights
    assert moe.moe_select_split("mxfp8", 8, 4096, 512, 32, 8, 16) == 1         # 100 MB
    assert moe.moe_select_split("bf16", 32, 512, 512, 8, 2, 16) == 0            # 6.3 MB: fused
    assert moe.moe_select_split("fp8_blockwise", 8192, 4096, 4096, 288, 8, 128) == 1


def test_align_ws_sizes_and_errors():
    assert moe.moe_align_ws_size(256, 6, 256) == 0                 # 1,536 routes: one workgroup
    assert moe.moe_align_ws_size(2048, 8, 288) == 0                # 16,384: still one
    assert moe.moe_align_ws_size(2049, 8, 288) == 4 * 33 * 288     # 16,392 routes, 33 chunks of 512
    assert moe.moe_align_ws_size(8192, 8, 288, 1) == 4 * 144 * 289  # 73,728 routes with a shared expert
    L = moe.lib()
    P = ctypes.c_void_p
    args = (P(FAKE), 8192, 8, 288, 0, 128, P(FAKE), P(FAKE), P(FAKE))
    assert L.moe_align_ws(*args, None, 0, None) == -5              # no workspace
    assert L.moe_align_ws(*args, P(FAKE), 100, None) == -5         # too small
    assert b"workspace" in L.moe_last_error()
    assert L.moe_align_ws(*args, P(FAKE + 8), 1 << 30, None) == -4  # misaligned workspace
    assert L.moe_align_ws(P(FAKE), 8192, 8, 2000, 0, 128, P(FAKE), P(FAKE), P(FAKE), P(FAKE),
                          1 << 30, None) == -3                     # E > 1024
    with pytest.raises(moe.MoeError):
        moe.moe_align_ws_size(8, 6, 256, -1)


def test_noalloc_rejects_before_launch():
    """The static-workspace entry point: a call needing more than its 64 MiB
    fails before any HIP call; so do the ordinary argument checks."""
    L = moe.lib()
    P = ctypes.c_void_p
    f = P(FAKE)
    assert L.fused_moe_fp8_blockwise_noalloc(*([f] * 11), 4096, 4096, 4096, 256, 6, 64, 1,
                                             None) == -5
    assert b"static scratch" in L.moe_last_error()
    assert L.fused_moe_fp8_blockwise_noalloc(*([f] * 11), 8, 4000, 4096, 256, 6, 16, 1,
                                             None) == -3   # K % 128
    assert L.fused_moe_fp8_blockwise_noalloc(*([f] * 11), 0, 4096, 4096, 256, 6, 16, 1,
                                             None) == 0    # T == 0: no-op
