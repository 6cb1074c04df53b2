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
  uint16_t* yr;    // split: (T*top_k, K) per-route down outputs, bf16 bits
  int32_t* flags;  // split: (T*top_k) route placed flags
  float* acc;      // fused: (T, K) fp32 accumulator
  int T, K, I, E, top_k;
  int n_shared;    // shared experts: the last n_shared of the E experts
  int blocks_cap;  // planner block capacity (grid bound)
  int h_rows;      // rows of the intermediate buffer (blocks_cap * block_m, or the ring's)
  // persistent ring mode: control words in the workspace (ticket, error flag,
  // then per block the finished up tiles and the finished down tiles), the
  // lag of a block's down tiles behind its up tiles in the task stream, and
  // the ring's size in blocks (block b's intermediate lives in slot b % ring)
  int* ctl;
  int lag, ring;
  // gate/up K split over kw workgroups (1: off): per-tile tickets (zero at
  // launch, right after the flags) and the workgroups' gate/up sums
  int kw;
  int* tickets;
  float* part;
  // schedule overrides (0: the library's choice): K groups of the streaming
  // gate/up kernels, their prefetch depth, the tiled kernels' stages
  int ksplit, depth, stages;
};

// Ring mode sizing ([DeepGEMM #88] "How it works": the lag follows from the
// work in flight, the ring from the lag).  The whole grid takes a ticket at
// once, and the stream opens with rounds of up tasks only (up_per_block
// tickets each), so a block's down tasks find its up tasks finished only if
// at least one grid's worth of tickets, with a margin, lies between them:
// lag * up_per_block >= 1.5 x the resident workgroups (measured: with a
// third less, half the grid polls at decode sizes).  A ring of twice the lag
// (plus 2) likewise leaves the down tasks of a slot's previous block time
// to finish before the slot is overwritten.  The default ring assumes a
// grid of 512 workgroups, twice the one per CU that the launch uses on
// 256 CUs, so the launch's own lag fits it with room to spare.
constexpr int kRingMaxResident = 512;
inline int ring_lag(int resident, int up_per_block) {
  return (3 * resident + 2 * up_per_block - 1) / (2 * up_per_block);
}
inline int64_t ring_default_slots(int64_t blocks_cap, int up_per_block) {
  const int64_t r = 2 * (int64_t)ring_lag(kRingMaxResident, up_per_block) + 2;
  return r < blocks_cap ? r : blocks_cap;
}
// One task of the ring stream.
struct RingTask {
  int kind;  // 0: none, 1: up (slice i of block b), 2: down (column tile i of block b)
  int b, i;
};

// Ticket t -> task, for nb blocks of S up and NT down tasks each: rounds
// r = 0, 1, .. hold the up tasks of block r (while r < nb), then the down
// tasks of block r - lag (once r >= lag); empty parts take no tickets, so
// tickets 0 .. nb * (S + NT) - 1 cover every task once.
__host__ __device__ inline RingTask ring_task(int t, int nb, int S, int NT, int lag) {
  const int h = lag < nb ? lag : nb;  // leading rounds with up tasks only
  if (t < h * S) return {1, t / S, t % S};
  t -= h * S;
  const int per = S + NT, m = nb - h;  // rounds with both kinds
  if (t < m * per) {
    const int r = h + t / per, i = t % per;
    return i < S ? RingTask{1, r, i} : RingTask{2, r - lag, i - S};
  }
  t -= m * per;
  const int b0 = nb - h;  // trailing rounds: down tasks only
  if (t < h * NT) return {2, b0 + t / NT, t % NT};
  return {0, 0, 0};
}

// control words: ticket, error word, per block finished up and down tasks
inline size_t ring_ctl_bytes(int64_t blocks_cap) {
  return ((size_t)(2 + 2 * blocks_cap) * 4 + 255) / 256 * 256;
}

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

// The same plan from three launches over chunks of route ids, for many
// routes; `counts` holds align_chunked_ws(routes, E + n_shared) bytes.
size_t align_chunked_ws(int64_t routes, int ET);
hipError_t launch_align_chunked(const int32_t* topk_ids, int R, int E, int block_m,
                                int32_t* sorted, int32_t* expert_ids, int32_t* ntp,
                                int sorted_cap, int blocks_cap, hipStream_t stream, int T,
                                int n_shared, int* counts);

// Router (softmax, top-k, renormalized weights) and planner in one launch;
// `ticket` is one int of workspace, zero before the call and after it.  With
// `chunk_counts` (align_chunked_ws(T * top_k, E) bytes) the launch only
// routes, and the chunked planner follows.
hipError_t launch_route_align(const float* logits, int T, int E, int top_k, int block_m,
                              int32_t* topk_ids, float* topk_w, int32_t* sorted,
                              int32_t* expert_ids, int32_t* ntp, int sorted_cap, int blocks_cap,
                              int* ticket, hipStream_t stream, int* chunk_counts = nullptr);

// Events recorded around one kernel of a launch_moe sequence (profiling).
struct TimingHook {
  hipEvent_t before = nullptr, after = nullptr;
  int which = 0;  // 1: fused / gate-up kernel, 2: down kernel
};

hipError_t launch_moe(int kind, int block_m, int split, const MoeArgs& a,
                      hipStream_t stream, const TimingHook& hook);

// The split mode's down GEMM and combine alone, on the intermediate the
// workspace already holds.
hipError_t launch_down_combine(int kind, int block_m, const MoeArgs& a, hipStream_t stream);

// LDS-tiled split-mode kernels (moe_tiled.hip) for many rows per expert.
bool tiled_supported(int kind, int block_m, int K, int I);
hipError_t launch_tiled(int kind, int block_m, const MoeArgs& a, hipStream_t stream,
                        const TimingHook& hook);
hipError_t launch_tiled_down(int kind, int block_m, const MoeArgs& a, hipStream_t stream);
