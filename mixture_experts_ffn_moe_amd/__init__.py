"""MI355X (gfx950) fused MoE expert-FFN forward: Python binding.

Thin ctypes layer over the C ABI in ``include/moe.h`` (library
``libmoe_mi355x.so`` next to this file, built by
``python -m mixture_experts_ffn_moe_amd.build``).  The functions here only
marshal arguments: torch tensors provide device memory and the current HIP
stream; every step of the forward runs in the library's kernels.  There is no
fallback: if the library is missing, every call raises.

Entry points (same names as the C ABI):
  moe_align(topk_ids, num_experts, block_m)
      -> (sorted_token_ids, expert_ids, num_tokens_post_padded)
  fused_moe_bf16(x, w1, w2, sorted_token_ids, expert_ids,
                 num_tokens_post_padded, topk_weights, top_k, block_m, ...)
  fused_moe_fp8_blockwise(x, x_scale, w1, w1_scale, w2, w2_scale, ...)
  fused_moe_mxfp8(x, x_scale, w1, w1_scale, w2, w2_scale, ...)
  fused_moe_mxfp4(x, x_scale, w1, w1_scale, w2, w2_scale, ...)   (packed e2m1 weights)
plus the host helpers moe_align_capacity, moe_workspace_size,
moe_workspace_layout, moe_ring_layout, moe_select_split and moe_select_block_m.
``split=2`` runs the persistent ring mode (block_m 16 or 32).
"""

import ctypes
import os

import torch

__all__ = [
    "MoeError", "lib", "LIB_PATH", "MOE_BF16", "MOE_FP8_BLOCKWISE", "MOE_MXFP8", "MOE_MXFP4",
    "moe_align_capacity", "moe_align", "moe_select_split", "moe_select_block_m",
    "moe_select_block_m_routed", "moe_align_ws_size", "moe_align_ws",
    "moe_workspace_size", "moe_workspace_layout", "moe_ring_layout", "moe_ring_schedule",
    "fused_moe_bf16",
    "fused_moe_fp8_blockwise", "fused_moe_mxfp8", "fused_moe_mxfp4", "EXPORTED_SYMBOLS",
    "moe_route_align", "moe_route_align_workspace_size", "moe_align_shared", "fused_moe_shared",
    "moe_mfma_probe", "moe_align_workspace_size", "MoeTune", "fused_moe_down_combine",
    "fused_moe_fp8_blockwise_noalloc",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_mi355x.so")

MOE_BF16, MOE_FP8_BLOCKWISE, MOE_MXFP8, MOE_MXFP4 = 0, 1, 2, 3
_DTYPE_CODE = {"bf16": MOE_BF16, "fp8_blockwise": MOE_FP8_BLOCKWISE, "mxfp8": MOE_MXFP8,
               "mxfp4": MOE_MXFP4}

EXPORTED_SYMBOLS = (
    "moe_last_error", "moe_align_capacity", "moe_align", "moe_select_split",
    "moe_select_block_m", "moe_workspace_size", "moe_workspace_layout",
    "fused_moe_bf16", "fused_moe_fp8_blockwise", "fused_moe_mxfp8", "fused_moe_mxfp4",
    "moe_set_timing_events", "moe_route_align_workspace_size", "moe_route_align",
    "moe_align_shared", "fused_moe_shared", "moe_ring_layout", "moe_ring_schedule",
    "moe_select_block_m_routed", "moe_align_ws_size", "moe_align_ws", "moe_mfma_probe",
    "moe_align_workspace_size", "fused_moe_down_combine", "fused_moe_fp8_blockwise_noalloc",
)

_STATUS = {0: "MOE_OK", -1: "MOE_ERR_NULL", -2: "MOE_ERR_SHAPE", -3: "MOE_ERR_UNSUPPORTED",
           -4: "MOE_ERR_ALIGN", -5: "MOE_ERR_WORKSPACE", -6: "MOE_ERR_HIP"}


class MoeError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t


def lib():
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m mixture_experts_ffn_moe_amd.build` (no fallback path exists)")
    L = ctypes.CDLL(LIB_PATH)
    L.moe_last_error.restype = ctypes.c_char_p
    L.moe_last_error.argtypes = []
    L.moe_align_capacity.argtypes = [_I64, _I32, _I32, _I32, ctypes.POINTER(_I64),
                                     ctypes.POINTER(_I64)]
    L.moe_align.argtypes = [_P, _I64, _I32, _I32, _I32, _P, _P, _P, _P, _SZ, _P]
    L.moe_align_workspace_size.argtypes = [_I64, _I32, _I32, ctypes.POINTER(_SZ)]
    L.moe_select_split.argtypes = [_I32, _I64, _I64, _I64, _I32, _I32, _I32,
                                   ctypes.POINTER(_I32)]
    L.moe_select_block_m.argtypes = [_I32, _I64, _I64, _I32, _I32, ctypes.POINTER(_I32)]
    L.moe_align_ws_size.argtypes = [_I64, _I32, _I32, _I32, ctypes.POINTER(_SZ)]
    L.moe_align_ws.argtypes = [_P, _I64, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _SZ, _P]
    L.moe_select_block_m_routed.argtypes = [_I32, _I64, _I64, _I32, _I32, _I32,
                                            ctypes.POINTER(_I32)]
    L.moe_workspace_size.argtypes = [_I32, _I64, _I64, _I64, _I32, _I32, _I32, _I32, _P,
                                     ctypes.POINTER(_SZ)]
    L.moe_workspace_layout.argtypes = [_I32, _I64, _I64, _I64, _I32, _I32, _I32,
                                       ctypes.POINTER(_SZ), ctypes.POINTER(_SZ)]
    L.moe_ring_schedule.argtypes = [_I32, _I32, _I32, _I32, _I64, _I64, _P, _P, _P]
    L.moe_ring_layout.argtypes = [_I32, _I64, _I64, _I64, _I32, _I32, _I32, ctypes.POINTER(_SZ),
                                  ctypes.POINTER(_SZ), ctypes.POINTER(_I64)]
    tail = [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I32, _I32, _I32, _I32, _P, _P, _SZ, _P]
    L.fused_moe_bf16.argtypes = [_P, _P, _P] + tail
    L.fused_moe_fp8_blockwise.argtypes = [_P, _P, _P, _P, _P, _P] + tail
    L.fused_moe_mxfp8.argtypes = [_P, _P, _P, _P, _P, _P] + tail
    L.fused_moe_mxfp4.argtypes = [_P, _P, _P, _P, _P, _P] + tail
    L.fused_moe_fp8_blockwise_noalloc.argtypes = [_P] * 11 + [_I64, _I64, _I64, _I32, _I32,
                                                              _I32, _I32, _P]
    L.moe_set_timing_events.argtypes = [_P, _P, _I32]
    L.moe_mfma_probe.argtypes = [_I32, _P, _P, _P, _P, _P, _P, _I64, _P]
    L.fused_moe_down_combine.argtypes = [_I32, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64,
                                         _I32, _I32, _I32, _P, _SZ, _P]
    L.moe_route_align_workspace_size.argtypes = [ctypes.POINTER(_SZ)]
    L.moe_route_align.argtypes = [_P, _I64, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _SZ, _P]
    L.moe_align_shared.argtypes = [_P, _I64, _I32, _I32, _I32, _I32, _P, _P, _P, _P]
    L.fused_moe_shared.argtypes = [_I32, _P, _P, _P, _P, _P, _P, _I32] + tail
    for name in EXPORTED_SYMBOLS:
        if name != "moe_last_error":
            getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


class MoeTune(ctypes.Structure):
    """Schedule overrides (struct moe_tune of the C ABI); 0 keeps the
    library's choice: k_groups (1, 2), k_split (1, 4), prefetch (1, 2, 4),
    stages (2, 3)."""
    _fields_ = [("k_groups", _I32), ("k_split", _I32), ("prefetch", _I32), ("stages", _I32)]


def _tune(tune):
    """A MoeTune, a dict of its fields, or None -> pointer argument."""
    if tune is None:
        return None
    if isinstance(tune, dict):
        tune = MoeTune(**tune)
    return ctypes.byref(tune)


def _check(status):
    if status != 0:
        raise MoeError(status, lib().moe_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def moe_align_capacity(T, top_k, num_experts, block_m):
    rows, blocks = _I64(), _I64()
    _check(lib().moe_align_capacity(T, top_k, num_experts, block_m, ctypes.byref(rows),
                                    ctypes.byref(blocks)))
    return rows.value, blocks.value


def moe_set_timing_events(before, after, which=1):
    """Record the hipEvent_t handles ``before`` / ``after`` (ctypes.c_void_p
    or int) around one kernel of the next fused_moe_* calls of this thread
    (which=1: fused or gate/up kernel, 2: down kernel); ``None`` switches the
    hook off."""
    if before is None or after is None:
        _check(lib().moe_set_timing_events(None, None, 0))
        return
    _check(lib().moe_set_timing_events(before, after, which))


def moe_align_workspace_size(T, top_k, num_experts):
    out = _SZ()
    _check(lib().moe_align_workspace_size(T, top_k, num_experts, ctypes.byref(out)))
    return out.value


def moe_align(topk_ids, num_experts, block_m, stream=None, out=None, workspace=-1):
    """Planner: returns (sorted_token_ids, expert_ids, num_tokens_post_padded)
    as int32 device tensors (the last one of shape (1,)).  ``out`` may pass
    preallocated tensors of the capacities moe_align_capacity gives.
    ``workspace``: a device tensor of moe_align_workspace_size bytes (the
    chunked planner past 16,384 routes), None (one workgroup plans), or by
    default one cached per device."""
    T, k = topk_ids.shape
    rows, blocks = moe_align_capacity(T, k, num_experts, block_m)
    dev = topk_ids.device
    if out is not None:
        sorted_ids, expert_ids, ntp = out
    else:
        sorted_ids = torch.empty(max(rows, 1), dtype=torch.int32, device=dev)[:rows]
        expert_ids = torch.empty(max(blocks, 1), dtype=torch.int32, device=dev)[:blocks]
        ntp = torch.empty(1, dtype=torch.int32, device=dev)
    if isinstance(workspace, int):
        need = moe_align_workspace_size(T, k, num_experts)
        workspace = _cached_align_ws(dev, need) if need else None
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().moe_align(_ptr(topk_ids.contiguous()), T, k, num_experts, block_m,
                           _ptr(sorted_ids), _ptr(expert_ids), _ptr(ntp), _ptr(workspace), nbytes,
                           _stream(stream)))
    return sorted_ids, expert_ids, ntp


def moe_route_align_workspace_size():
    out = _SZ()
    _check(lib().moe_route_align_workspace_size(ctypes.byref(out)))
    return out.value


_route_ws = {}


def _cached_align_ws(dev, need):
    ws = _ALIGN_WS.get(dev)
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        _ALIGN_WS[dev] = ws
    return ws


def moe_route_align(logits, top_k, block_m, stream=None, out=None, workspace=None):
    """Router + planner in one launch: (T, E) fp32 logits -> (topk_ids,
    topk_weights, sorted_token_ids, expert_ids, num_tokens_post_padded).
    ``out`` may pass those five preallocated.  ``workspace``'s first 256
    bytes must hold zeros before its first use (each call leaves them zero);
    by default one zeroed buffer per device, large enough for the chunked
    planner of this call, is kept and reused, so calls on several streams of
    one device must pass their own."""
    T, E = logits.shape
    rows, blocks = moe_align_capacity(T, top_k, E, block_m)
    dev = logits.device
    if out is not None:
        ids, w, sorted_ids, expert_ids, ntp = out
    else:
        ids = torch.empty(T, top_k, dtype=torch.int32, device=dev)
        w = torch.empty(T, top_k, dtype=torch.float32, device=dev)
        sorted_ids = torch.empty(max(rows, 1), dtype=torch.int32, device=dev)[:rows]
        expert_ids = torch.empty(max(blocks, 1), dtype=torch.int32, device=dev)[:blocks]
        ntp = torch.empty(1, dtype=torch.int32, device=dev)
    if workspace is None:
        key = (dev.type, dev.index)
        need = moe_route_align_workspace_size() + moe_align_workspace_size(T, top_k, E)
        if key not in _route_ws or _route_ws[key].numel() < need:
            _route_ws[key] = torch.zeros(need, dtype=torch.uint8, device=dev)
        workspace = _route_ws[key]
    _check(lib().moe_route_align(_ptr(logits.contiguous()), T, E, top_k, block_m, _ptr(ids),
                                 _ptr(w), _ptr(sorted_ids), _ptr(expert_ids), _ptr(ntp),
                                 _ptr(workspace), workspace.numel(), _stream(stream)))
    return ids, w, sorted_ids, expert_ids, ntp


def moe_align_shared(topk_ids, num_experts, n_shared, block_m, stream=None, out=None):
    """Planner with ``n_shared`` shared experts (ids num_experts ..
    num_experts + n_shared - 1) that every token routes to after its routed
    experts; returns (sorted_token_ids, expert_ids, num_tokens_post_padded)."""
    T, k = topk_ids.shape
    rows, blocks = moe_align_capacity(T, k + n_shared, num_experts + n_shared, block_m)
    dev = topk_ids.device
    if out is not None:
        sorted_ids, expert_ids, ntp = out
    else:
        sorted_ids = torch.empty(max(rows, 1), dtype=torch.int32, device=dev)[:rows]
        expert_ids = torch.empty(max(blocks, 1), dtype=torch.int32, device=dev)[:blocks]
        ntp = torch.empty(1, dtype=torch.int32, device=dev)
    _check(lib().moe_align_shared(_ptr(topk_ids.contiguous()), T, k, num_experts, n_shared,
                                  block_m, _ptr(sorted_ids), _ptr(expert_ids), _ptr(ntp),
                                  _stream(stream)))
    return sorted_ids, expert_ids, ntp


def moe_align_ws_size(T, top_k, num_experts, n_shared=0):
    out = _SZ()
    _check(lib().moe_align_ws_size(T, top_k, num_experts, n_shared, ctypes.byref(out)))
    return out.value


_ALIGN_WS = {}


def moe_align_ws(topk_ids, num_experts, block_m, n_shared=0, stream=None, out=None,
                 workspace=None):
    """Planner for any route count (chunked launches past 16,384 routes);
    the outputs of moe_align / moe_align_shared.  Without ``workspace`` a
    cached one per device is used (calls on one device run in stream order)."""
    T, k = topk_ids.shape
    rows, blocks = moe_align_capacity(T, k + n_shared, num_experts + n_shared, block_m)
    dev = topk_ids.device
    if out is not None:
        sorted_ids, expert_ids, ntp = out
    else:
        sorted_ids = torch.empty(max(rows, 1), dtype=torch.int32, device=dev)[:rows]
        expert_ids = torch.empty(max(blocks, 1), dtype=torch.int32, device=dev)[:blocks]
        ntp = torch.empty(1, dtype=torch.int32, device=dev)
    need = moe_align_ws_size(T, k, num_experts, n_shared)
    if workspace is None and need:
        workspace = _cached_align_ws(dev, need)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().moe_align_ws(_ptr(topk_ids.contiguous()), T, k, num_experts, n_shared, block_m,
                              _ptr(sorted_ids), _ptr(expert_ids), _ptr(ntp), _ptr(workspace),
                              nbytes, _stream(stream)))
    return sorted_ids, expert_ids, ntp


def fused_moe_shared(dtype, x, x_scale, w1, w1_scale, w2, w2_scale, n_shared, sorted_token_ids,
                     expert_ids, num_tokens_post_padded, topk_weights, top_k, block_m, split=-1,
                     out=None, workspace=None, stream=None, tune=None):
    """Forward with shared experts: w1 / w2 (and scales) hold the routed
    experts followed by ``n_shared`` shared ones; planner outputs from
    moe_align_shared."""
    T, K = x.shape
    E_all, N, _ = w1.shape
    E = E_all - n_shared
    dev = w1.device
    if out is None:
        out = torch.empty(T, K, dtype=torch.bfloat16, device=dev)
    need = moe_workspace_size(dtype, T, K, N, E_all, top_k + n_shared, block_m, split, tune)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _check(lib().fused_moe_shared(_DTYPE_CODE.get(dtype, dtype), _ptr(x), _ptr(x_scale), _ptr(w1),
                                  _ptr(w1_scale), _ptr(w2), _ptr(w2_scale), n_shared,
                                  _ptr(sorted_token_ids), _ptr(expert_ids),
                                  _ptr(num_tokens_post_padded), _ptr(topk_weights), _ptr(out), T,
                                  K, N, E, top_k, block_m, split, _tune(tune), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def moe_select_split(dtype, T, K, N, num_experts, top_k, block_m):
    out = _I32()
    _check(lib().moe_select_split(_DTYPE_CODE.get(dtype, dtype), T, K, N, num_experts, top_k,
                                  block_m, ctypes.byref(out)))
    return out.value


def moe_select_block_m(T, top_k, num_experts, dtype="fp8_blockwise", K=4096):
    out = _I32()
    _check(lib().moe_select_block_m(_DTYPE_CODE.get(dtype, dtype), T, K, top_k, num_experts,
                                    ctypes.byref(out)))
    return out.value


def moe_select_block_m_routed(T, top_k, num_experts, active_experts, dtype="fp8_blockwise",
                              K=4096):
    """block_m from the number of experts that hold at least one route."""
    out = _I32()
    _check(lib().moe_select_block_m_routed(_DTYPE_CODE.get(dtype, dtype), T, K, top_k,
                                           num_experts, active_experts, ctypes.byref(out)))
    return out.value


def active_experts(topk_ids, num_experts):
    """Experts holding at least one route of topk_ids (a host-side count)."""
    ids = topk_ids.reshape(-1)
    valid = ids[(ids >= 0) & (ids < num_experts)]
    return int(torch.unique(valid).numel())


def moe_workspace_size(dtype, T, K, N, num_experts, top_k, block_m, split=-1, tune=None):
    out = _SZ()
    _check(lib().moe_workspace_size(_DTYPE_CODE.get(dtype, dtype), T, K, N, num_experts, top_k,
                                    block_m, split, _tune(tune), ctypes.byref(out)))
    return out.value


def moe_workspace_layout(dtype, T, K, N, num_experts, top_k, block_m):
    h, hs = _SZ(), _SZ()
    _check(lib().moe_workspace_layout(_DTYPE_CODE.get(dtype, dtype), T, K, N, num_experts,
                                      top_k, block_m, ctypes.byref(h), ctypes.byref(hs)))
    return h.value, hs.value


def moe_ring_layout(dtype, T, K, N, num_experts, top_k, block_m):
    """Ring-mode workspace: (bytes ahead of the ring, bytes per slot,
    default slots).  A split=2 call uses as many slots as its workspace
    holds, at most one per planner block."""
    fixed, slot, slots = _SZ(), _SZ(), _I64()
    _check(lib().moe_ring_layout(_DTYPE_CODE.get(dtype, dtype), T, K, N, num_experts, top_k,
                                 block_m, ctypes.byref(fixed), ctypes.byref(slot),
                                 ctypes.byref(slots)))
    return fixed.value, slot.value, slots.value


def moe_ring_schedule(n_blocks, up_per_block, down_per_block, lag, first=0, count=None):
    """Tickets first .. first+count-1 of the ring stream as three int32 numpy
    arrays (kind: 1 up, 2 down, 0 past the end; block; index)."""
    import numpy as np
    if count is None:
        count = n_blocks * (up_per_block + down_per_block) - first
    kind, block, index = (np.zeros(max(count, 0), np.int32) for _ in range(3))
    _check(lib().moe_ring_schedule(n_blocks, up_per_block, down_per_block, lag, first, count,
                                   kind.ctypes.data, block.ctypes.data, index.ctypes.data))
    return kind, block, index


def _run(fn, dtype, operands, w1, sorted_token_ids, expert_ids, num_tokens_post_padded,
         topk_weights, top_k, block_m, split, out, workspace, stream, T, K, tune=None):
    E, N, _ = w1.shape
    dev = w1.device
    if out is None:
        out = torch.empty(T, K, dtype=torch.bfloat16, device=dev)
    need = moe_workspace_size(dtype, T, K, N, E, top_k, block_m, split, tune)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _check(fn(*[_ptr(t) for t in operands], _ptr(sorted_token_ids), _ptr(expert_ids),
              _ptr(num_tokens_post_padded), _ptr(topk_weights), _ptr(out), T, K, N, E, top_k,
              block_m, split, _tune(tune), _ptr(workspace),
              workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def fused_moe_bf16(x, w1, w2, sorted_token_ids, expert_ids, num_tokens_post_padded,
                   topk_weights, top_k, block_m, split=-1, out=None, workspace=None,
                   stream=None, tune=None):
    T, K = x.shape
    return _run(lib().fused_moe_bf16, MOE_BF16, [x, w1, w2], w1, sorted_token_ids, expert_ids,
                num_tokens_post_padded, topk_weights, top_k, block_m, split, out, workspace,
                stream, T, K, tune)


def fused_moe_fp8_blockwise(x, x_scale, w1, w1_scale, w2, w2_scale, sorted_token_ids,
                            expert_ids, num_tokens_post_padded, topk_weights, top_k, block_m,
                            split=-1, out=None, workspace=None, stream=None, tune=None):
    T, K = x.shape
    return _run(lib().fused_moe_fp8_blockwise, MOE_FP8_BLOCKWISE,
                [x, x_scale, w1, w1_scale, w2, w2_scale], w1, sorted_token_ids, expert_ids,
                num_tokens_post_padded, topk_weights, top_k, block_m, split, out, workspace,
                stream, T, K, tune)


def fused_moe_fp8_blockwise_noalloc(x, x_scale, w1, w1_scale, w2, w2_scale, sorted_token_ids,
                                    expert_ids, num_tokens_post_padded, topk_weights, top_k,
                                    block_m, split=-1, out=None, stream=None):
    """fused_moe_fp8_blockwise with the library's static workspace (no
    workspace argument; the caller provides ``out``, or it is allocated here
    by torch before the call)."""
    T, K = x.shape
    E, N, _ = w1.shape
    if out is None:
        out = torch.empty(T, K, dtype=torch.bfloat16, device=x.device)
    _check(lib().fused_moe_fp8_blockwise_noalloc(
        _ptr(x), _ptr(x_scale), _ptr(w1), _ptr(w1_scale), _ptr(w2), _ptr(w2_scale),
        _ptr(sorted_token_ids), _ptr(expert_ids), _ptr(num_tokens_post_padded),
        _ptr(topk_weights), _ptr(out), T, K, N, E, top_k, block_m, split, _stream(stream)))
    return out


def fused_moe_mxfp8(x, x_scale, w1, w1_scale, w2, w2_scale, sorted_token_ids, expert_ids,
                    num_tokens_post_padded, topk_weights, top_k, block_m, split=-1, out=None,
                    workspace=None, stream=None, tune=None):
    T, K = x.shape
    return _run(lib().fused_moe_mxfp8, MOE_MXFP8, [x, x_scale, w1, w1_scale, w2, w2_scale], w1,
                sorted_token_ids, expert_ids, num_tokens_post_padded, topk_weights, top_k,
                block_m, split, out, workspace, stream, T, K, tune)


def fused_moe_mxfp4(x, x_scale, w1, w1_scale, w2, w2_scale, sorted_token_ids, expert_ids,
                    num_tokens_post_padded, topk_weights, top_k, block_m, split=-1, out=None,
                    workspace=None, stream=None, tune=None):
    """w1 (E, N, K/2) and w2 (E, K, N/4) uint8: packed e2m1 pairs."""
    T, K = x.shape
    return _run(lib().fused_moe_mxfp4, MOE_MXFP4, [x, x_scale, w1, w1_scale, w2, w2_scale], w1,
                sorted_token_ids, expert_ids, num_tokens_post_padded, topk_weights, top_k,
                block_m, split, out, workspace, stream, T, K, tune)


def fused_moe_down_combine(dtype, w2, w2_scale, sorted_token_ids, expert_ids,
                           num_tokens_post_padded, topk_weights, top_k, block_m, workspace, T,
                           out=None, stream=None):
    """Down GEMM + combine of the split mode on the intermediate the caller
    wrote into ``workspace`` (moe_workspace_layout offsets); returns out."""
    E, K, I = w2.shape[0], w2.shape[1], w2.shape[2] * (2 if dtype == "mxfp4" else 1)
    if out is None:
        out = torch.empty(T, K, dtype=torch.bfloat16, device=w2.device)
    _check(lib().fused_moe_down_combine(_DTYPE_CODE.get(dtype, dtype), _ptr(w2), _ptr(w2_scale),
                                        _ptr(sorted_token_ids), _ptr(expert_ids),
                                        _ptr(num_tokens_post_padded), _ptr(topk_weights),
                                        _ptr(out), T, K, 2 * I, E, top_k, block_m,
                                        _ptr(workspace),
                                        workspace.numel() * workspace.element_size(),
                                        _stream(stream)))
    return out


def moe_mfma_probe(dtype, a, b, a_scale=None, b_scale=None, c=None, stream=None, out=None):
    """One 128-wide K step of the dtype's matrix instruction per 16 x 16 tile
    (diagnostic): a, b are (n, 16, 128) uint8 / bf16 rows (MXFP4 b: (n, 16,
    64) packed bytes), scales (n, 16, 4) uint8 for the MX dtypes, c an
    optional (n, 16, 16) fp32 accumulator.  Returns d (n, 16, 16) fp32."""
    n = a.shape[0]
    if out is None:
        out = torch.empty(n, 16, 16, dtype=torch.float32, device=a.device)
    _check(lib().moe_mfma_probe(_DTYPE_CODE.get(dtype, dtype), _ptr(a), _ptr(b), _ptr(a_scale),
                                _ptr(b_scale), _ptr(c), _ptr(out), n, _stream(stream)))
    return out


def run_case(case, block_m=None, split=-1, stream=None, workspace=None, out=None,
             align_out=None, skip_align=False, tune=None):
    """Planner + forward for a ``datagen.Case``-like object (attributes kind,
    x, x_scale, w1, w1_scale, w2, w2_scale, topk_ids, topk_weights, E, top_k).
    Returns (out, (sorted_token_ids, expert_ids, num_tokens_post_padded)).
    ``skip_align`` runs the fused forward alone on ``align_out`` as an earlier
    call with the same routing and block_m filled it.  ``tune``: schedule
    overrides (MoeTune or a dict of its fields).  Without ``block_m`` the
    routed block-size choice needs the active-expert count, which this
    helper counts on the host (a synchronization)."""
    T = case.x.shape[0]
    if block_m is None:
        block_m = moe_select_block_m_routed(T, case.top_k, case.E,
                                            active_experts(case.topk_ids, case.E), case.kind,
                                            case.x.shape[1])
    S = getattr(case, "n_shared", 0)
    if skip_align:
        if align_out is None:
            raise ValueError("skip_align needs the align_out of an earlier call")
        align = tuple(align_out)
    elif S:
        align = moe_align_ws(case.topk_ids, case.E, block_m, n_shared=S, stream=stream,
                             out=align_out)
    else:
        align = moe_align(case.topk_ids, case.E, block_m, stream=stream, out=align_out)
    args = dict(top_k=case.top_k, block_m=block_m, split=split, out=out, workspace=workspace,
                stream=stream, tune=tune)
    if S:
        o = fused_moe_shared(case.kind, case.x, case.x_scale, case.w1, case.w1_scale, case.w2,
                             case.w2_scale, S, *align, case.topk_weights, **args)
    elif case.kind == "bf16":
        o = fused_moe_bf16(case.x, case.w1, case.w2, *align, case.topk_weights, **args)
    elif case.kind == "fp8_blockwise":
        o = fused_moe_fp8_blockwise(case.x, case.x_scale, case.w1, case.w1_scale, case.w2,
                                    case.w2_scale, *align, case.topk_weights, **args)
    elif case.kind == "mxfp8":
        o = fused_moe_mxfp8(case.x, case.x_scale, case.w1, case.w1_scale, case.w2,
                            case.w2_scale, *align, case.topk_weights, **args)
    else:
        o = fused_moe_mxfp4(case.x, case.x_scale, case.w1, case.w1_scale, case.w2,
                            case.w2_scale, *align, case.topk_weights, **args)
    return o, align
