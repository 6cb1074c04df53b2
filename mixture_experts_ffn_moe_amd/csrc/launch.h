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
  int blocks_cap;  // planner block capacity (grid bound)
};

hipError_t launch_align(const int32_t* topk_ids, int R, int E, int block_m,
                        int32_t* sorted, int32_t* expert_ids, int32_t* ntp,
                        int sorted_cap, int blocks_cap, hipStream_t stream);

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
