// launch.h -- internal host-side launchers (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

struct MoeArgs {
  const uint8_t* x;    // (T, K) activations
  const void* xs;      // activation scales (fp32 or e8m0), or null
  const uint8_t* w1;   // (E, N, K)
  const void* w1s;
  const uint8_t* w2;   // (E, K, I)
  const void* w2s;
  const int32_t* sorted;      // sorted_token_ids
  const int32_t* expert_ids;  // per block
  const int32_t* ntp;         // num_tokens_post_padded (device scalar)
  const float* topk_w;        // (T, top_k)
  uint16_t* out;              // (T, K) bf16 bits
  // workspace regions
  uint8_t* hq;     // split: (rows_cap, I) intermediate values
  uint8_t* hs;     // split: intermediate scales
  float* yr;       // split: (T*top_k, K) per-route down outputs
  int32_t* flags;  // split: (T*top_k) route placed flags
  float* acc;      // fused: (T, K) fp32 accumulator
  int T, K, I, E, top_k;
  int n_shared;    // shared experts: the last n_shared of the E experts
  int blocks_cap;  // planner block capacity (grid bound)
};

// Route ids: t * top_k + j for the routed experts (weight topk_w[id]), then
// T * top_k + t * n_shared + s for the shared ones (weight 1).
inline size_t total_routes(const MoeArgs& a) { return (size_t)a.T * (a.top_k + a.n_shared); }

__device__ __forceinline__ int route_token(const MoeArgs& p, int id) {
  const int R = p.T * p.top_k;
  return id < 0 ? 0 : id < R ? id / p.top_k : (id - R) / p.n_shared;  // padding rows: token 0
}

__device__ __forceinline__ float route_weight(const MoeArgs& p, int id) {
  return id < p.T * p.top_k ? p.topk_w[id] : 1.f;
}

// Planner; n_shared > 0 appends one route per (token, shared expert), the
// shared experts numbered E .. E + n_shared - 1 (T tokens: R = T * top_k).
hipError_t launch_align(const int32_t* topk_ids, int R, int E, int block_m,
                        int32_t* sorted, int32_t* expert_ids, int32_t* ntp,
                        int sorted_cap, int blocks_cap, hipStream_t stream, int T = 0,
                        int n_shared = 0);

// Router (softmax, top-k, renormalized weights) and planner in one launch;
// `ticket` is one int of workspace, zero before the call and after it.
hipError_t launch_route_align(const float* logits, int T, int E, int top_k, int block_m,
                              int32_t* topk_ids, float* topk_w, int32_t* sorted,
                              int32_t* expert_ids, int32_t* ntp, int sorted_cap, int blocks_cap,
                              int* ticket, hipStream_t stream);

// Events recorded around one kernel of a launch_moe sequence (profiling).
struct TimingHook {
  hipEvent_t before = nullptr, after = nullptr;
  int which = 0;  // 1: fused / gate-up kernel, 2: down kernel
};

hipError_t launch_moe(int kind, int block_m, int split, const MoeArgs& a,
                      hipStream_t stream, const TimingHook& hook);

// LDS-tiled split-mode kernels (moe_tiled.hip) for many rows per expert.
bool tiled_supported(int kind, int block_m, int K, int I);
hipError_t launch_tiled(int kind, int block_m, const MoeArgs& a, hipStream_t stream,
                        const TimingHook& hook);
