// abi.hip -- host side of the C ABI declared in include/moe.h: argument
// validation (before anything is enqueued), capacities, workspace layout,
// mode / block heuristics, and the launches.
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/moe.h"
#include "device.h"
#include "launch.h"

namespace {

thread_local char g_err[512] = "";
thread_local TimingHook g_hook;

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return MOE_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool valid_block_m(int32_t bm) {
  return bm == 16 || bm == 32 || bm == 64 || bm == 128 || bm == 256;
}

int check_routes(int64_t T, int32_t top_k, int32_t E) {
  if (T < 0) return fail(MOE_ERR_SHAPE, "T must be >= 0 (got %lld)", (long long)T);
  if (top_k < 1) return fail(MOE_ERR_SHAPE, "top_k must be >= 1 (got %d)", top_k);
  if (E < 1) return fail(MOE_ERR_SHAPE, "E must be >= 1 (got %d)", E);
  if (T * (int64_t)top_k >= (int64_t(1) << 31))
    return fail(MOE_ERR_SHAPE, "T*top_k must be < 2^31");
  return MOE_OK;
}

void capacity(int64_t T, int32_t top_k, int32_t E, int32_t bm, int64_t* rows, int64_t* blocks) {
  const int64_t R = T * top_k;
  const int64_t r = R + (R < E ? R : (int64_t)E) * (bm - 1);
  *rows = r;
  *blocks = (r + bm - 1) / bm;
}

int check_ffn(int32_t dtype, int64_t T, int64_t K, int64_t N, int32_t E, int32_t top_k,
              int32_t block_m) {
  int rc = check_routes(T, top_k, E);
  if (rc) return rc;
  if (dtype < MOE_BF16 || dtype > MOE_MXFP4) return fail(MOE_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
  if (K <= 0 || N <= 0) return fail(MOE_ERR_SHAPE, "K and N must be > 0");
  if (N % 2) return fail(MOE_ERR_SHAPE, "N (fused gate+up width) must be even");
  if (K % 128) return fail(MOE_ERR_UNSUPPORTED, "K must be a multiple of 128 (got %lld)", (long long)K);
  if ((N / 2) % 128)
    return fail(MOE_ERR_UNSUPPORTED, "I = N/2 must be a multiple of 128 (got %lld)", (long long)(N / 2));
  // blockwise weight scales of one row of 128-blocks sit in two registers per lane
  if (dtype == MOE_FP8_BLOCKWISE && (K > 16384 || N / 2 > 16384))
    return fail(MOE_ERR_UNSUPPORTED, "blockwise FP8 needs K and I = N/2 <= 16384");
  if (!valid_block_m(block_m))
    return fail(MOE_ERR_UNSUPPORTED, "block_m must be 16, 32, 64, 128 or 256 (got %d)", block_m);
  if (block_m == 256 && (dtype == MOE_BF16 || dtype == MOE_MXFP4 || K % 256))
    return fail(MOE_ERR_UNSUPPORTED, "block_m 256 needs e4m3 weights and K %% 256 == 0");
  // 32-bit offsets inside one expert's weights and element indices of out
  if (N * K >= (int64_t(1) << 31) || T * K >= (int64_t(1) << 31))
    return fail(MOE_ERR_UNSUPPORTED, "per-expert weight or output element count must be < 2^31");
  int64_t rows, blocks;
  capacity(T, top_k, E, block_m, &rows, &blocks);
  if (blocks * block_m * (N / 2) * 2 >= (int64_t(1) << 32))
    return fail(MOE_ERR_UNSUPPORTED, "intermediate workspace must stay below 4 GiB");
  return MOE_OK;
}

int pick_split(int32_t dtype, int64_t T, int64_t K, int64_t N, int32_t E, int32_t top_k,
               int32_t block_m) {
  if (block_m == 256) return 1;
  // Measured on MI355X: wherever the weight stream sets the time the split
  // mode is faster (its down GEMM streams W2 through the register ring,
  // while the fused mode reads its W2 slice column chunk by chunk and adds
  // R*K*(I/128) fp32 atomics); e.g. K=4096, I=2048, E=256, top-6: 219 vs
  // 240 us at T=8, 833 vs 949 us at T=64.  The fused mode's one launch fewer
  // wins only when the whole call is tiny (bf16 K=512, I=256, E=8, T=32:
  // 37.5 vs 41.3 us).
  const double weight_bytes =
      (double)E * 3.0 * (double)K * (double)(N / 2) *
      (dtype == MOE_BF16 ? 2.0 : dtype == MOE_MXFP4 ? 0.5 : 1.0);
  return (T * top_k <= 512 && weight_bytes <= 32e6) ? 0 : 1;
}

// Gate/up K split over 4 workgroups per tile (split mode: 16- or 32-row
// streaming blocks, or 64-row LDS-tiled blocks of the e4m3 dtypes) where few
// (block, slice) tiles exist: at most 128 by the even-spread estimate, K/128
// a multiple of 8 and at least 16.  Measured (MXFP8, K=4096, I=256, E=32,
// top-8): see the kernels.
bool kw_supported(int32_t dtype, int64_t K, int64_t I, int32_t block_m, int split) {
  const int64_t KS = K / 128;
  if (split != 1 || KS % 8 || KS < 16) return false;
  if (block_m <= 32) return true;
  return block_m == 64 && tiled_supported(dtype, block_m, (int)K, (int)I);
}

int pick_kw(int32_t dtype, int64_t T, int64_t K, int64_t N, int32_t E, int32_t top_k,
            int32_t block_m, int split, const moe_tune* tune = nullptr) {
  if (tune && tune->k_split) return tune->k_split;
  if (!kw_supported(dtype, K, N / 2, block_m, split)) return 1;
  const int64_t R = T * top_k, S = (N / 2) / 128;
  const int64_t spread = R < E ? R : (int64_t)E;  // blocks if every route's expert differs
  if (block_m <= 32) return spread * S <= 128 ? 4 : 1;
  // 64-row tiles hold a CU each (their LDS): split while four workgroups per
  // tile still fit on the 256 CUs at once (MXFP8, K=4096, I=256, E=32,
  // top-8: gate/up GEMM 34.7 -> 26.6 us at T=128, 64 tiles; at T=512, 128
  // tiles, 36.4 against 56.0 us split)
  const int64_t blocks = spread > (R + block_m - 1) / block_m ? spread : (R + block_m - 1) / block_m;
  return blocks * S * 4 <= 256 ? 4 : 1;
}

// Schedule overrides: every set field must name a variant the call's
// kernels have (checked before anything is launched).
int check_tune(int32_t dtype, int64_t K, int64_t I, int32_t block_m, int split, const moe_tune* t) {
  if (!t) return MOE_OK;
  const bool streaming = block_m <= 32 || dtype == MOE_BF16 || dtype == MOE_MXFP4;
  if (t->k_groups) {
    if (t->k_groups != 1 && t->k_groups != 2)
      return fail(MOE_ERR_UNSUPPORTED, "tune.k_groups must be 0, 1 or 2 (got %d)", t->k_groups);
    if (block_m > 32 || split == 2)
      return fail(MOE_ERR_UNSUPPORTED, "tune.k_groups needs block_m 16 or 32 and split 0 or 1");
    if (t->k_groups == 2 && K < 256)
      return fail(MOE_ERR_UNSUPPORTED, "tune.k_groups = 2 needs K >= 256");
  }
  if (t->k_split) {
    if (t->k_split != 1 && t->k_split != 4)
      return fail(MOE_ERR_UNSUPPORTED, "tune.k_split must be 0, 1 or 4 (got %d)", t->k_split);
    if (t->k_split == 4 && !kw_supported(dtype, K, I, block_m, split))
      return fail(MOE_ERR_UNSUPPORTED,
                  "tune.k_split = 4 needs split 1, block_m 16 or 32 (or 64 with an e4m3 dtype), K/128 "
                  "a multiple of 8 and >= 16");
    if (t->k_split == 4 && t->k_groups == 1)
      return fail(MOE_ERR_UNSUPPORTED, "tune.k_split = 4 runs two K groups per workgroup");
  }
  if (t->prefetch) {
    if (t->prefetch != 1 && t->prefetch != 2 && t->prefetch != 4)
      return fail(MOE_ERR_UNSUPPORTED, "tune.prefetch must be 0, 1, 2 or 4 (got %d)", t->prefetch);
    if (block_m > 32 || split == 2 || t->k_split == 4)
      return fail(MOE_ERR_UNSUPPORTED,
                  "tune.prefetch needs block_m 16 or 32, split 0 or 1 and k_split 1");
  }
  if (t->stages) {
    if (t->stages != 2 && t->stages != 3)
      return fail(MOE_ERR_UNSUPPORTED, "tune.stages must be 0, 2 or 3 (got %d)", t->stages);
    if (streaming || split != 1 || block_m > 128 || K % 256)
      return fail(MOE_ERR_UNSUPPORTED,
                  "tune.stages needs the LDS-tiled kernels: e4m3 dtypes, split 1, block_m 64 or 128");
  }
  return MOE_OK;
}

struct Layout {
  size_t ctl, flags, tickets, part, hq, hs, yr, acc, total;
  size_t ring_fixed, slot_bytes;  // ring mode: bytes before the ring, bytes per slot
  int64_t slots;                  // ring mode: slots of the default size
};

// Scale bytes per intermediate row.
size_t h_scale_bytes(int32_t dtype, int64_t I) {
  return dtype == MOE_FP8_BLOCKWISE ? (size_t)(I / 128) * 4
         : (dtype == MOE_MXFP8 || dtype == MOE_MXFP4) ? (size_t)(I / 32) : 0;
}

Layout layout(int32_t dtype, int64_t T, int64_t K, int64_t N, int32_t E, int32_t top_k,
              int32_t block_m, int split, const moe_tune* tune = nullptr) {
  Layout L{};
  const int64_t I = N / 2;
  const size_t R = (size_t)T * top_k;
  const size_t es = dtype == MOE_BF16 ? 2 : 1;
  int64_t rows, blocks;
  capacity(T, top_k, E, block_m, &rows, &blocks);
  rows = blocks * block_m;  // whole blocks, so every block's rows exist
  size_t off = 0;
  if (split == 2) {
    // control words and flags first (one clear), then the per-route rows,
    // then the ring: slots of block_m rows, values then scales
    L.ctl = off;
    off += ring_ctl_bytes(blocks);
    L.flags = off;
    off = round_up(off + R * 4, 256);
    L.yr = off;
    off = round_up(off + R * (size_t)K * 2, 256);
    L.ring_fixed = off;
    L.slot_bytes = (size_t)block_m * ((size_t)I * es + h_scale_bytes(dtype, I));
    L.slots = ring_default_slots(blocks, (int)(I / 128));
    L.hq = off;
    L.hs = dtype == MOE_BF16 ? L.hq : L.hq + (size_t)L.slots * block_m * I * es;
    off += (size_t)L.slots * L.slot_bytes;
    L.total = round_up(off, 256);
    return L;
  }
  if (split) {
    L.flags = off;
    off = round_up(off + R * 4, 256);
    const int kw = pick_kw(dtype, T, K, N, E, top_k, block_m, split, tune);
    if (kw > 1) {  // tile tickets right after the flags (one clear)
      L.tickets = off;
      off = round_up(off + (size_t)blocks * (I / 128) * 4, 256);
    }
    L.hq = off;
    off = round_up(off + (size_t)rows * I * es, 256);
    L.hs = off;
    if (dtype == MOE_FP8_BLOCKWISE) off = round_up(off + (size_t)rows * (I / 128) * 4, 256);
    if (dtype == MOE_MXFP8 || dtype == MOE_MXFP4) off = round_up(off + (size_t)rows * (I / 32), 256);
    if (dtype == MOE_BF16) L.hs = L.hq;
    L.yr = off;
    off = round_up(off + R * (size_t)K * 2, 256);
    if (kw > 1) {  // per tile and workgroup: block_m rows x 256 gate/up sums
      L.part = off;
      off = round_up(off + (size_t)blocks * (I / 128) * kw * block_m * 256 * 4, 256);
    }
  } else {
    L.acc = off;
    off = round_up(off + (size_t)T * K * 4, 256);
  }
  L.total = off;
  return L;
}

int run_ffn(int32_t dtype, const void* x, const void* xs, const void* w1, const void* w1s,
            const void* w2, const void* w2s, const int32_t* sorted, const int32_t* expert_ids,
            const int32_t* ntp, const float* topk_w, void* out, int64_t T, int64_t K, int64_t N,
            int32_t E, int32_t top_k, int32_t block_m, int32_t split, const moe_tune* tune,
            void* ws, size_t ws_bytes, void* stream, int32_t n_shared = 0,
            bool down_only = false) {
  // E routed experts, then n_shared shared ones in the weights; every token
  // adds one route per shared expert.  Capacities and workspace follow the
  // totals.
  if (n_shared < 0) return fail(MOE_ERR_SHAPE, "n_shared must be >= 0");
  const int32_t E_all = E + n_shared, k_all = top_k + n_shared;
  int rc = check_ffn(dtype, T, K, N, E_all, k_all, block_m);
  if (rc) return rc;
  if (split < -1 || split > 2) return fail(MOE_ERR_UNSUPPORTED, "split must be -1, 0, 1 or 2");
  if (block_m == 256 && split == 0)
    return fail(MOE_ERR_UNSUPPORTED, "block_m 256 runs the split mode only");
  if (split == 2 && block_m > 32)
    return fail(MOE_ERR_UNSUPPORTED, "the ring mode runs block_m 16 or 32 (got %d)", block_m);
  const int sp = split < 0 ? pick_split(dtype, T, K, N, E_all, k_all, block_m) : split;
  rc = check_tune(dtype, K, N / 2, block_m, sp, tune);
  if (rc) return rc;
  if (T == 0) return ok();
  if (down_only) {
    // only w2 is read; the checks below see it in place of x and w1
    x = w1 = w2;
    xs = w1s = w2s;
  }
  if (!x || !w1 || !w2 || !sorted || !expert_ids || !ntp || !topk_w || !out)
    return fail(MOE_ERR_NULL, "a required pointer is NULL");
  if (dtype != MOE_BF16 && (!xs || !w1s || !w2s))
    return fail(MOE_ERR_NULL, "scale pointers are required for FP8 paths");
  const void* p16[] = {x, w1, w2, out, sorted, expert_ids, topk_w, ws};
  for (const void* p : p16)
    if (p && !aligned(p, 16)) return fail(MOE_ERR_ALIGN, "tensors must be 16-byte aligned");
  if (dtype == MOE_FP8_BLOCKWISE && (!aligned(xs, 4) || !aligned(w1s, 4) || !aligned(w2s, 4)))
    return fail(MOE_ERR_ALIGN, "fp32 scales must be 4-byte aligned");
  if (!aligned(ntp, 4)) return fail(MOE_ERR_ALIGN, "num_tokens_post_padded must be 4-byte aligned");
  Layout L = layout(dtype, T, K, N, E_all, k_all, block_m, sp, tune);
  int64_t rows, blocks;
  capacity(T, k_all, E_all, block_m, &rows, &blocks);
  if (sp == 2) {
    // the ring takes as many slots as the workspace holds (at least one, at
    // most one per block: then it never wraps)
    const size_t min_bytes = L.ring_fixed + L.slot_bytes;
    if (!ws) return fail(MOE_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", L.total);
    if (ws_bytes < min_bytes)
      return fail(MOE_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes (one ring slot)",
                  ws_bytes, min_bytes);
    int64_t slots = (int64_t)((ws_bytes - L.ring_fixed) / L.slot_bytes);
    if (slots > blocks) slots = blocks;
    L.slots = slots;
    if (dtype != MOE_BF16) L.hs = L.hq + (size_t)slots * block_m * (N / 2);  // e4m3 values
  } else {
    if (!ws) return fail(MOE_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", L.total);
    if (ws_bytes < L.total)
      return fail(MOE_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, L.total);
  }
  uint8_t* w = static_cast<uint8_t*>(ws);
  MoeArgs a{};
  a.x = static_cast<const uint8_t*>(x);
  a.xs = xs;
  a.w1 = static_cast<const uint8_t*>(w1);
  a.w1s = w1s;
  a.w2 = static_cast<const uint8_t*>(w2);
  a.w2s = w2s;
  a.sorted = sorted;
  a.expert_ids = expert_ids;
  a.ntp = ntp;
  a.topk_w = topk_w;
  a.out = static_cast<uint16_t*>(out);
  if (sp) {
    a.flags = reinterpret_cast<int32_t*>(w + L.flags);
    a.hq = w + L.hq;
    a.hs = w + L.hs;
    a.yr = reinterpret_cast<uint16_t*>(w + L.yr);
    a.h_rows = (int)(blocks * block_m);
    a.kw = pick_kw(dtype, T, K, N, E_all, k_all, block_m, sp, tune);
    if (a.kw > 1) {
      a.tickets = reinterpret_cast<int*>(w + L.tickets);
      a.part = reinterpret_cast<float*>(w + L.part);
    }
    if (sp == 2) {
      a.ctl = reinterpret_cast<int*>(w + L.ctl);
      a.ring = (int)L.slots;
      a.h_rows = (int)(L.slots * block_m);
    }
  } else {
    a.acc = reinterpret_cast<float*>(w + L.acc);
  }
  a.T = (int)T;
  a.K = (int)K;
  a.I = (int)(N / 2);
  a.E = E_all;
  a.top_k = top_k;
  a.n_shared = n_shared;
  a.blocks_cap = (int)blocks;
  if (tune) {
    a.ksplit = tune->k_groups;
    a.depth = tune->prefetch;
    a.stages = tune->stages;
  }
  static_assert(MOE_BF16 == KIND_BF16 && MOE_FP8_BLOCKWISE == KIND_FP8B && MOE_MXFP8 == KIND_MX &&
                    MOE_MXFP4 == KIND_MX4,
                "the moe_dtype values are the kernel kinds");
  const int kind = dtype;
  hipError_t e = down_only
                     ? launch_down_combine(kind, block_m, a, static_cast<hipStream_t>(stream))
                     : launch_moe(kind, block_m, sp, a, static_cast<hipStream_t>(stream), g_hook);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

// Workspace of fused_moe_fp8_blockwise_noalloc: device memory the library
// holds on every GPU it runs on until the process ends.  Host code never
// uses this name as an address (on the host it is a stand-in, not device
// memory): each device's address comes from hipGetSymbolAddress, taken once
// with that device current.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's copy of `scratch`, looked up on the first call made with the
// device current.
int scratch_for_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOE_ERR_UNSUPPORTED, "device %d beyond the %d this library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_last_error(void) { return g_err; }

int moe_align_capacity(int64_t T, int32_t top_k, int32_t E, int32_t block_m, int64_t* sorted_cap,
                       int64_t* blocks_cap) {
  if (!sorted_cap || !blocks_cap) return fail(MOE_ERR_NULL, "output pointers are NULL");
  int rc = check_routes(T, top_k, E);
  if (rc) return rc;
  if (!valid_block_m(block_m))
    return fail(MOE_ERR_UNSUPPORTED, "block_m must be 16, 32, 64, 128 or 256 (got %d)", block_m);
  capacity(T, top_k, E, block_m, sorted_cap, blocks_cap);
  return ok();
}

// Route counts from which the planner runs over chunks in three launches
// when the caller provides the workspace (measured, K=4096 I=2048 E=288
// top-8: the one-workgroup planner takes 165 us for 65,536 routes, 11 us for
// 1,536; the chunked one 29 us for 65,536).
constexpr int64_t kChunkedRoutes = 16384;

int moe_align_workspace_size(int64_t T, int32_t top_k, int32_t E, size_t* bytes) {
  if (!bytes) return fail(MOE_ERR_NULL, "bytes is NULL");
  int rc = check_routes(T, top_k, E);
  if (rc) return rc;
  const int64_t routes = T * (int64_t)top_k;
  *bytes = routes > kChunkedRoutes ? align_chunked_ws(routes, E) : 0;
  return ok();
}

int moe_align(const int32_t* topk_ids, int64_t T, int32_t top_k, int32_t E, int32_t block_m,
              int32_t* sorted_token_ids, int32_t* expert_ids, int32_t* num_tokens_post_padded,
              void* ws, size_t ws_bytes, void* stream) {
  int64_t rows, blocks;
  int rc = moe_align_capacity(T, top_k, E, block_m, &rows, &blocks);
  if (rc) return rc;
  if (E > 1024) return fail(MOE_ERR_UNSUPPORTED, "moe_align supports E <= 1024 (got %d)", E);
  if (!num_tokens_post_padded || (rows > 0 && (!sorted_token_ids || !expert_ids)) ||
      (T > 0 && !topk_ids))
    return fail(MOE_ERR_NULL, "a required pointer is NULL");
  const void* ps[] = {topk_ids, sorted_token_ids, expert_ids, ws};
  for (const void* p : ps)
    if (p && !aligned(p, 16)) return fail(MOE_ERR_ALIGN, "tensors must be 16-byte aligned");
  if (!aligned(num_tokens_post_padded, 4))
    return fail(MOE_ERR_ALIGN, "num_tokens_post_padded must be 4-byte aligned");
  size_t need = 0;
  rc = moe_align_workspace_size(T, top_k, E, &need);
  if (rc) return rc;
  hipError_t e;
  if (need > 0 && ws && ws_bytes >= need)
    e = launch_align_chunked(topk_ids, (int)(T * top_k), E, block_m, sorted_token_ids, expert_ids,
                             num_tokens_post_padded, (int)rows, (int)blocks,
                             static_cast<hipStream_t>(stream), (int)T, 0, static_cast<int*>(ws));
  else
    e = launch_align(topk_ids, (int)(T * top_k), E, block_m, sorted_token_ids, expert_ids,
                     num_tokens_post_padded, (int)rows, (int)blocks,
                     static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

int moe_align_shared(const int32_t* topk_ids, int64_t T, int32_t top_k, int32_t E,
                     int32_t n_shared, int32_t block_m, int32_t* sorted_token_ids,
                     int32_t* expert_ids, int32_t* num_tokens_post_padded, void* stream) {
  if (n_shared < 0) return fail(MOE_ERR_SHAPE, "n_shared must be >= 0");
  int64_t rows, blocks;
  int rc = moe_align_capacity(T, top_k + n_shared, E + n_shared, block_m, &rows, &blocks);
  if (rc) return rc;
  if (E + n_shared > 1024)
    return fail(MOE_ERR_UNSUPPORTED, "the planner supports E + n_shared <= 1024 (got %d)",
                E + n_shared);
  if (!num_tokens_post_padded || (rows > 0 && (!sorted_token_ids || !expert_ids)) ||
      (T > 0 && !topk_ids))
    return fail(MOE_ERR_NULL, "a required pointer is NULL");
  const void* ps[] = {topk_ids, sorted_token_ids, expert_ids};
  for (const void* p : ps)
    if (p && !aligned(p, 16)) return fail(MOE_ERR_ALIGN, "tensors must be 16-byte aligned");
  if (!aligned(num_tokens_post_padded, 4))
    return fail(MOE_ERR_ALIGN, "num_tokens_post_padded must be 4-byte aligned");
  hipError_t e = launch_align(topk_ids, (int)(T * top_k), E, block_m, sorted_token_ids,
                              expert_ids, num_tokens_post_padded, (int)rows, (int)blocks,
                              static_cast<hipStream_t>(stream), (int)T, n_shared);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

int fused_moe_shared(int32_t dtype, const void* x, const void* x_scale, const void* w1,
                     const void* w1_scale, const void* w2, const void* w2_scale,
                     int32_t n_shared, const int32_t* sorted_token_ids,
                     const int32_t* expert_ids, const int32_t* num_tokens_post_padded,
                     const float* topk_weights, void* out, int64_t T, int64_t K, int64_t N,
                     int32_t E, int32_t top_k, int32_t block_m, int32_t split,
                     const moe_tune* tune, void* workspace, size_t workspace_bytes,
                     void* stream) {
  if (dtype < MOE_BF16 || dtype > MOE_MXFP4) return fail(MOE_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
  return run_ffn(dtype, x, x_scale, w1, w1_scale, w2, w2_scale, sorted_token_ids, expert_ids,
                 num_tokens_post_padded, topk_weights, out, T, K, N, E, top_k, block_m, split,
                 tune, workspace, workspace_bytes, stream, n_shared);
}

int moe_align_ws_size(int64_t T, int32_t top_k, int32_t E, int32_t n_shared, size_t* bytes) {
  if (!bytes) return fail(MOE_ERR_NULL, "bytes is NULL");
  if (n_shared < 0) return fail(MOE_ERR_SHAPE, "n_shared must be >= 0");
  int rc = check_routes(T, top_k + n_shared, E + n_shared);
  if (rc) return rc;
  const int64_t routes = T * (int64_t)(top_k + n_shared);
  *bytes = routes > kChunkedRoutes ? align_chunked_ws(routes, E + n_shared) : 0;
  return ok();
}

int moe_align_ws(const int32_t* topk_ids, int64_t T, int32_t top_k, int32_t E, int32_t n_shared,
                 int32_t block_m, int32_t* sorted_token_ids, int32_t* expert_ids,
                 int32_t* num_tokens_post_padded, void* ws, size_t ws_bytes, void* stream) {
  size_t need = 0;
  int rc = moe_align_ws_size(T, top_k, E, n_shared, &need);
  if (rc) return rc;
  if (need == 0)
    return n_shared ? moe_align_shared(topk_ids, T, top_k, E, n_shared, block_m, sorted_token_ids,
                                       expert_ids, num_tokens_post_padded, stream)
                    : moe_align(topk_ids, T, top_k, E, block_m, sorted_token_ids, expert_ids,
                                num_tokens_post_padded, nullptr, 0, stream);
  int64_t rows, blocks;
  rc = moe_align_capacity(T, top_k + n_shared, E + n_shared, block_m, &rows, &blocks);
  if (rc) return rc;
  if (E + n_shared > 1024)
    return fail(MOE_ERR_UNSUPPORTED, "the planner supports E + n_shared <= 1024 (got %d)",
                E + n_shared);
  if (!num_tokens_post_padded || !sorted_token_ids || !expert_ids || !topk_ids)
    return fail(MOE_ERR_NULL, "a required pointer is NULL");
  const void* ps[] = {topk_ids, sorted_token_ids, expert_ids};
  for (const void* p : ps)
    if (!aligned(p, 16)) return fail(MOE_ERR_ALIGN, "tensors must be 16-byte aligned");
  if (!aligned(num_tokens_post_padded, 4))
    return fail(MOE_ERR_ALIGN, "num_tokens_post_padded must be 4-byte aligned");
  if (!ws) return fail(MOE_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (!aligned(ws, 16)) return fail(MOE_ERR_ALIGN, "the workspace must be 16-byte aligned");
  if (ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
  hipError_t e = launch_align_chunked(topk_ids, (int)(T * top_k), E, block_m, sorted_token_ids,
                                      expert_ids, num_tokens_post_padded, (int)rows, (int)blocks,
                                      static_cast<hipStream_t>(stream), (int)T, n_shared,
                                      static_cast<int*>(ws));
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

int moe_route_align_workspace_size(size_t* bytes) {
  if (!bytes) return fail(MOE_ERR_NULL, "bytes is NULL");
  *bytes = 256;
  return ok();
}

int moe_route_align(const float* logits, int64_t T, int32_t E, int32_t top_k, int32_t block_m,
                    int32_t* topk_ids, float* topk_weights, int32_t* sorted_token_ids,
                    int32_t* expert_ids, int32_t* num_tokens_post_padded, void* ws,
                    size_t ws_bytes, void* stream) {
  int64_t rows, blocks;
  int rc = moe_align_capacity(T, top_k, E, block_m, &rows, &blocks);
  if (rc) return rc;
  if (E > 1024) return fail(MOE_ERR_UNSUPPORTED, "moe_route_align supports E <= 1024 (got %d)", E);
  if (top_k > 16 || top_k > E)
    return fail(MOE_ERR_UNSUPPORTED, "moe_route_align needs top_k <= 16 and <= E (got %d)", top_k);
  if (T * (int64_t)E >= (int64_t(1) << 40)) return fail(MOE_ERR_SHAPE, "T*E too large");
  if (!num_tokens_post_padded || !ws || (rows > 0 && (!sorted_token_ids || !expert_ids)) ||
      (T > 0 && (!logits || !topk_ids || !topk_weights)))
    return fail(MOE_ERR_NULL, "a required pointer is NULL");
  const void* ps[] = {logits, topk_ids, topk_weights, sorted_token_ids, expert_ids};
  for (const void* p : ps)
    if (p && !aligned(p, 16)) return fail(MOE_ERR_ALIGN, "tensors must be 16-byte aligned");
  if (!aligned(num_tokens_post_padded, 4) || !aligned(ws, 16))
    return fail(MOE_ERR_ALIGN, "num_tokens_post_padded must be 4-byte and ws 16-byte aligned");
  if (ws_bytes < 256) return fail(MOE_ERR_WORKSPACE, "workspace too small: %zu < 256 bytes", ws_bytes);
  // past 16,384 routes, with room for the chunk counts after the ticket: the
  // router alone, then the chunked planner
  size_t chunk = 0;
  rc = moe_align_workspace_size(T, top_k, E, &chunk);
  if (rc) return rc;
  int* counts = (chunk > 0 && ws_bytes >= 256 + chunk)
                    ? reinterpret_cast<int*>(static_cast<uint8_t*>(ws) + 256) : nullptr;
  hipError_t e = launch_route_align(logits, (int)T, E, top_k, block_m, topk_ids, topk_weights,
                                    sorted_token_ids, expert_ids, num_tokens_post_padded,
                                    (int)rows, (int)blocks, static_cast<int*>(ws),
                                    static_cast<hipStream_t>(stream), counts);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

int fused_moe_down_combine(int32_t dtype, const void* w2, const void* w2_scale,
                           const int32_t* sorted_token_ids, const int32_t* expert_ids,
                           const int32_t* num_tokens_post_padded, const float* topk_weights,
                           void* out, int64_t T, int64_t K, int64_t N, int32_t E, int32_t top_k,
                           int32_t block_m, void* workspace, size_t workspace_bytes,
                           void* stream) {
  if (dtype < MOE_BF16 || dtype > MOE_MXFP4) return fail(MOE_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
  // the split mode's layout without schedule overrides: moe_workspace_layout's offsets
  return run_ffn(dtype, nullptr, nullptr, nullptr, nullptr, w2, w2_scale, sorted_token_ids,
                 expert_ids, num_tokens_post_padded, topk_weights, out, T, K, N, E, top_k, block_m,
                 1, nullptr, workspace, workspace_bytes, stream, 0, true);
}

int moe_set_timing_events(void* before, void* after, int32_t which) {
  if (which < 0 || which > 2) return fail(MOE_ERR_UNSUPPORTED, "which must be 0, 1 or 2");
  g_hook.before = static_cast<hipEvent_t>(before);
  g_hook.after = static_cast<hipEvent_t>(after);
  g_hook.which = which;
  return ok();
}

int moe_select_split(int32_t dtype, int64_t T, int64_t K, int64_t N, int32_t E, int32_t top_k,
                     int32_t block_m, int32_t* split) {
  if (!split) return fail(MOE_ERR_NULL, "split is NULL");
  *split = pick_split(dtype, T, K, N, E, top_k, block_m);
  return ok();
}

int moe_select_block_m_routed(int32_t dtype, int64_t T, int64_t K, int32_t top_k, int32_t E,
                              int32_t active_experts, int32_t* block_m) {
  if (!block_m) return fail(MOE_ERR_NULL, "block_m is NULL");
  int rc = check_routes(T, top_k, E);
  if (rc) return rc;
  if (active_experts < 0 || active_experts > E)
    return fail(MOE_ERR_SHAPE, "active_experts must lie in [0, E] (got %d)", active_experts);
  const int64_t R = T * top_k;
  const int64_t act = active_experts > 0 ? active_experts : 1;
  const double per = (double)R / (double)act;     // rows per active expert
  const double per_all = (double)R / (double)E;   // rows per expert, all experts
  if (dtype == MOE_FP8_BLOCKWISE && K % 256 == 0) {
    // measured (whole forward, blockwise FP8; K=4096, I=2048, E=256 / 288,
    // near-uniform routing; K=7168, I=3072, E=384, zipf routing):
    // - 16-row streaming blocks up to ~12 rows per active expert (6: 1135 us
    //   against 1189 for 64; 12: 1198 against 1206);
    // - 64-row LDS-tiled blocks up to ~64 (14.6: 1345 against 1450 for 16;
    //   29: 1407 against 1508 for 128; 26 under zipf: 961 against 1389 for 16);
    // - 256 rows only where every expert holds that many (234 per expert:
    //   2824 against 3166 for 128); under a skewed routing the long tail of
    //   small experts wastes most of a 256-row tile (zipf, 110 rows per active
    //   expert, 32 per expert: 3018 against 2714 for 128);
    // - 128 rows otherwise (117: 1972 against 2487 for 64 and 2376 for 256).
    *block_m = per <= 12 ? 16 : per <= 64 ? 64 : (per > 160 && per_all > 160) ? 256 : 128;
    return ok();
  }
  // MXFP8 (the MFMA applies the scales itself) and the streaming-only dtypes;
  // measured (MXFP8, K=4096, I=256, E=32): 69 us at 32 rows per expert with
  // 64-row tiles against 92 for 16 and 82 for 128; 88 us at 128 rows against
  // 101 for 128; 219 us at 512 rows with 256-row tiles against 253 for 128
  const bool big_ok = dtype == MOE_MXFP8 && K % 256 == 0;
  *block_m = per <= 16 ? 16 : per <= 160 ? 64 : (per <= 200 || !big_ok) ? 128 : 256;
  return ok();
}

int moe_select_block_m(int32_t dtype, int64_t T, int64_t K, int32_t top_k, int32_t E,
                       int32_t* block_m) {
  if (!block_m) return fail(MOE_ERR_NULL, "block_m is NULL");
  int rc = check_routes(T, top_k, E);
  if (rc) return rc;
  // routes spread evenly: min(R, E) experts hold routes
  const int64_t R = T * top_k;
  const int32_t act = (int32_t)(R < E ? (R > 0 ? R : 1) : E);
  return moe_select_block_m_routed(dtype, T, K, top_k, E, act, block_m);
}

int moe_workspace_size(int32_t dtype, int64_t T, int64_t K, int64_t N, int32_t E, int32_t top_k,
                       int32_t block_m, int32_t split, const moe_tune* tune, size_t* bytes) {
  if (!bytes) return fail(MOE_ERR_NULL, "bytes is NULL");
  int rc = check_ffn(dtype, T, K, N, E, top_k, block_m);
  if (rc) return rc;
  if (split < -1 || split > 2) return fail(MOE_ERR_UNSUPPORTED, "split must be -1, 0, 1 or 2");
  if (split == 2 && block_m > 32)
    return fail(MOE_ERR_UNSUPPORTED, "the ring mode runs block_m 16 or 32 (got %d)", block_m);
  const int sp = split < 0 ? pick_split(dtype, T, K, N, E, top_k, block_m) : split;
  rc = check_tune(dtype, K, N / 2, block_m, sp, tune);
  if (rc) return rc;
  *bytes = layout(dtype, T, K, N, E, top_k, block_m, sp, tune).total;
  return ok();
}

int moe_ring_layout(int32_t dtype, int64_t T, int64_t K, int64_t N, int32_t E, int32_t top_k,
                    int32_t block_m, size_t* fixed_bytes, size_t* slot_bytes,
                    int64_t* default_slots) {
  if (!fixed_bytes || !slot_bytes || !default_slots)
    return fail(MOE_ERR_NULL, "output pointers are NULL");
  int rc = check_ffn(dtype, T, K, N, E, top_k, block_m);
  if (rc) return rc;
  if (block_m > 32)
    return fail(MOE_ERR_UNSUPPORTED, "the ring mode runs block_m 16 or 32 (got %d)", block_m);
  const Layout L = layout(dtype, T, K, N, E, top_k, block_m, 2);
  *fixed_bytes = L.ring_fixed;
  *slot_bytes = L.slot_bytes;
  *default_slots = L.slots;
  return ok();
}

int moe_ring_schedule(int32_t n_blocks, int32_t up_per_block, int32_t down_per_block,
                      int32_t lag, int64_t first, int64_t count, int32_t* kind, int32_t* block,
                      int32_t* index) {
  if (count > 0 && (!kind || !block || !index)) return fail(MOE_ERR_NULL, "output pointers are NULL");
  if (n_blocks < 0 || up_per_block < 1 || down_per_block < 1 || lag < 0 || first < 0 || count < 0)
    return fail(MOE_ERR_SHAPE, "sizes must be non-negative (tasks per block positive)");
  const int64_t total = (int64_t)n_blocks * (up_per_block + down_per_block);
  if (total >= (int64_t(1) << 31)) return fail(MOE_ERR_SHAPE, "the stream must hold < 2^31 tasks");
  for (int64_t j = 0; j < count; ++j) {
    const int64_t t = first + j;
    const RingTask k = t < total ? ring_task((int)t, n_blocks, up_per_block, down_per_block, lag)
                                 : RingTask{0, 0, 0};
    kind[j] = k.kind;
    block[j] = k.b;
    index[j] = k.i;
  }
  return ok();
}

int moe_workspace_layout(int32_t dtype, int64_t T, int64_t K, int64_t N, int32_t E, int32_t top_k,
                         int32_t block_m, size_t* h_offset, size_t* hs_offset) {
  if (!h_offset || !hs_offset) return fail(MOE_ERR_NULL, "output pointers are NULL");
  int rc = check_ffn(dtype, T, K, N, E, top_k, block_m);
  if (rc) return rc;
  const Layout L = layout(dtype, T, K, N, E, top_k, block_m, 1);
  *h_offset = L.hq;
  *hs_offset = L.hs;
  return ok();
}

int fused_moe_bf16(const void* x, const void* w1, const void* w2, const int32_t* sorted_token_ids,
                   const int32_t* expert_ids, const int32_t* num_tokens_post_padded,
                   const float* topk_weights, void* out, int64_t T, int64_t K, int64_t N, int32_t E,
                   int32_t top_k, int32_t block_m, int32_t split, const moe_tune* tune,
                   void* workspace, size_t workspace_bytes, void* stream) {
  return run_ffn(MOE_BF16, x, nullptr, w1, nullptr, w2, nullptr, sorted_token_ids, expert_ids,
                 num_tokens_post_padded, topk_weights, out, T, K, N, E, top_k, block_m, split,
                 tune, workspace, workspace_bytes, stream);
}

int fused_moe_fp8_blockwise(const void* x, const float* x_scale, const void* w1,
                            const float* w1_scale, const void* w2, const float* w2_scale,
                            const int32_t* sorted_token_ids, const int32_t* expert_ids,
                            const int32_t* num_tokens_post_padded, const float* topk_weights,
                            void* out, int64_t T, int64_t K, int64_t N, int32_t E, int32_t top_k,
                            int32_t block_m, int32_t split, const moe_tune* tune, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return run_ffn(MOE_FP8_BLOCKWISE, x, x_scale, w1, w1_scale, w2, w2_scale, sorted_token_ids,
                 expert_ids, num_tokens_post_padded, topk_weights, out, T, K, N, E, top_k, block_m,
                 split, tune, workspace, workspace_bytes, stream);
}

int fused_moe_fp8_blockwise_noalloc(const void* x, const float* x_scale, const void* w1,
                                    const float* w1_scale, const void* w2, const float* w2_scale,
                                    const int32_t* sorted_token_ids, const int32_t* expert_ids,
                                    const int32_t* num_tokens_post_padded,
                                    const float* topk_weights, void* out, int64_t T, int64_t K,
                                    int64_t N, int32_t E, int32_t top_k, int32_t block_m,
                                    int32_t split, void* stream) {
  size_t need = 0;
  int rc = moe_workspace_size(MOE_FP8_BLOCKWISE, T, K, N, E, top_k, block_m, split, nullptr,
                              &need);
  if (rc) return rc;
  if (need > kScratchBytes)
    return fail(MOE_ERR_WORKSPACE,
                "the call needs %zu workspace bytes, beyond the %zu of the library's static "
                "scratch; use fused_moe_fp8_blockwise with a workspace",
                need, kScratchBytes);
  if (T == 0) return ok();
  void* ws = nullptr;
  rc = scratch_for_current_device(&ws);
  if (rc) return rc;
  return run_ffn(MOE_FP8_BLOCKWISE, x, x_scale, w1, w1_scale, w2, w2_scale, sorted_token_ids,
                 expert_ids, num_tokens_post_padded, topk_weights, out, T, K, N, E, top_k, block_m,
                 split, nullptr, ws, kScratchBytes, stream);
}

int fused_moe_mxfp8(const void* x, const uint8_t* x_scale, const void* w1, const uint8_t* w1_scale,
                    const void* w2, const uint8_t* w2_scale, const int32_t* sorted_token_ids,
                    const int32_t* expert_ids, const int32_t* num_tokens_post_padded,
                    const float* topk_weights, void* out, int64_t T, int64_t K, int64_t N,
                    int32_t E, int32_t top_k, int32_t block_m, int32_t split,
                    const moe_tune* tune, void* workspace, size_t workspace_bytes, void* stream) {
  return run_ffn(MOE_MXFP8, x, x_scale, w1, w1_scale, w2, w2_scale, sorted_token_ids, expert_ids,
                 num_tokens_post_padded, topk_weights, out, T, K, N, E, top_k, block_m, split,
                 tune, workspace, workspace_bytes, stream);
}

int fused_moe_mxfp4(const void* x, const uint8_t* x_scale, const void* w1, const uint8_t* w1_scale,
                    const void* w2, const uint8_t* w2_scale, const int32_t* sorted_token_ids,
                    const int32_t* expert_ids, const int32_t* num_tokens_post_padded,
                    const float* topk_weights, void* out, int64_t T, int64_t K, int64_t N,
                    int32_t E, int32_t top_k, int32_t block_m, int32_t split,
                    const moe_tune* tune, void* workspace, size_t workspace_bytes, void* stream) {
  return run_ffn(MOE_MXFP4, x, x_scale, w1, w1_scale, w2, w2_scale, sorted_token_ids, expert_ids,
                 num_tokens_post_padded, topk_weights, out, T, K, N, E, top_k, block_m, split,
                 tune, workspace, workspace_bytes, stream);
}

}  // extern "C"
