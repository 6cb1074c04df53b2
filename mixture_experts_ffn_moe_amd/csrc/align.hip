// align.hip -- planner: route ids grouped by expert, padded to block_m.
//
// [hpc-ops RFC] "Design": the planner builds the expert histogram, the prefix
// sums and the row-to-token mapping; it is a separate launch because the
// histogram and the prefix sums are grid-wide dependencies.  [prime-flash]
// "Shapes": sorted_token_ids holds flat ids token*top_k + route, grouped by
// expert and padded to block_m with -1.
//
// One workgroup of 8 waves does the whole job, so every dependency is a
// workgroup barrier (no grid-wide synchronization, no atomics on global
// memory, and a deterministic result):
//   1. each wave counts the experts of its contiguous share of the route ids
//      into its own LDS histogram;
//   2. per expert: total count, block-padded count, exclusive prefix sum over
//      experts (expert order ascending), and each wave's starting position
//      inside the expert's segment (earlier waves first);
//   3. expert_ids gets the owner of each block (-1 past the last block); every
//      slot of sorted_token_ids was set to -1 with the histogram clear, so
//      the padding needs no pass of its own;
//   4. each wave walks its share in order, 64 ids at a time; lanes holding
//      the same expert find each other with ballots over the expert id's
//      bits, take consecutive slots in lane order, and the last of them
//      advances the wave's cursor.  Steps 1 and 4 visit ids in the same order,
//      so ids inside an expert come out ascending.
#include "device.h"
#include "launch.h"

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBatch = 8;

// Expert of route i: routed ids[i] for i < R_routed (valid in [0, E_routed),
// else -1), then route R_routed + t * S + s goes to shared expert E_routed + s.
__device__ __forceinline__ int route_expert(const int32_t* __restrict__ ids, int i, int R_routed,
                                            int E_routed, int S) {
  if (i < R_routed) {
    const int e = ids[i];
    return (unsigned)e < (unsigned)E_routed ? e : -1;
  }
  return E_routed + (i - R_routed) % S;
}

// The planner on one workgroup of kWaves waves; smem holds
// kWaves * ET + 2 * ET + kWaves + 1 ints, ET = E + S.
// Routes: ids[0 .. R) name routed experts (valid in [0, E)); with S shared
// experts, route R + t * S + s (t < T) goes to expert E + s.
__device__ __forceinline__ void align_body(const int32_t* __restrict__ ids, int R, int E_routed,
                                           int bm, int32_t* __restrict__ sorted,
                                           int32_t* __restrict__ expert_ids,
                                           int32_t* __restrict__ ntp_out, int sorted_cap,
                                           int blocks_cap, int* smem, int T, int S) {
  const int E = E_routed + S;  // every expert, shared ones last
  const int R_routed = R;
  auto expert_of = [=](int i) { return route_expert(ids, i, R_routed, E_routed, S); };
  R = R_routed + T * S;        // every route, shared ones last
  int* cnt = smem;                     // [kWaves][E]: counts, then cursors
  int* off = smem + kWaves * E;        // [E]: segment start
  int* tot = off + E;                  // [E]: route count
  int* wsum = tot + E;                 // [kWaves + 1]: scan scratch
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  for (int i = tid; i < kWaves * E; i += kThreads) cnt[i] = 0;
  // every slot starts as padding; the scatter below (after several barriers)
  // overwrites the slots that hold a route
  for (int q = tid; q < sorted_cap; q += kThreads) sorted[q] = -1;
  __syncthreads();

  const int seg = (R + kWaves - 1) / kWaves;
  const int lo = min(R, w * seg), hi = min(R, lo + seg);
  // ids are read kBatch chunks of 64 at a time so that the global loads
  // overlap instead of costing one memory latency per chunk; a wave whose
  // share is one batch keeps it in registers for the scatter
  const bool one = hi - lo <= 64 * kBatch;
  int keep[kBatch];
  for (int base = lo; base < hi; base += 64 * kBatch) {
    int eb[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = base + u * 64 + lane;
      eb[u] = i < hi ? expert_of(i) : -1;
      keep[u] = eb[u];
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if ((unsigned)eb[u] < (unsigned)E) atomicAdd(&cnt[w * E + eb[u]], 1);
  }
  __syncthreads();

  // padded counts, two experts per thread (E <= 1024), then a block scan
  const int e0 = 2 * tid, e1 = 2 * tid + 1;
  int c0 = 0, c1 = 0;
  if (e0 < E)
    for (int v = 0; v < kWaves; ++v) c0 += cnt[v * E + e0];
  if (e1 < E)
    for (int v = 0; v < kWaves; ++v) c1 += cnt[v * E + e1];
  const int p0 = (c0 + bm - 1) / bm * bm, p1 = (c1 + bm - 1) / bm * bm;
  int x = p0 + p1;  // inclusive scan inside the wave
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int v = 0; v < kWaves; ++v) {
      const int t = wsum[v];
      wsum[v] = run;
      run += t;
    }
    wsum[kWaves] = run;
  }
  __syncthreads();
  const int excl = wsum[w] + x - (p0 + p1);
  if (e0 < E) { off[e0] = excl; tot[e0] = c0; }
  if (e1 < E) { off[e1] = excl + p0; tot[e1] = c1; }
  const int ntp = wsum[kWaves];
  __syncthreads();

  // per-wave cursors: segment start plus the counts of earlier waves
  for (int e = tid; e < E; e += kThreads) {
    int run = off[e];
    for (int v = 0; v < kWaves; ++v) {
      const int c = cnt[v * E + e];
      cnt[v * E + e] = run;
      run += c;
    }
    // the expert of each block (the padding slots were filled at the start)
    const int pend = off[e] + (tot[e] + bm - 1) / bm * bm;
    for (int q = off[e] / bm; q < pend / bm; ++q) expert_ids[q] = e;
  }
  for (int q = ntp / bm + tid; q < blocks_cap; q += kThreads) expert_ids[q] = -1;
  if (tid == 0) *ntp_out = ntp;
  __syncthreads();

  // stable scatter, chunks of 64 ids in order, kBatch chunks loaded at once
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base0 = lo; base0 < hi; base0 += 64 * kBatch) {
    int eb[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = base0 + u * 64 + lane;
      eb[u] = one ? keep[u] : i < hi ? expert_of(i) : -1;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = base0 + u * 64 + lane;
      const int e = eb[u];
      const bool ok = (unsigned)e < (unsigned)E;
      unsigned long long peers = __ballot(ok);
      for (int bit = 0; (1 << bit) < E; ++bit) {
        const bool set = (e >> bit) & 1;
        const unsigned long long m = __ballot(ok && set);
        peers &= set ? m : ~m;
      }
      if (ok) {
        const int rank = __popcll(peers & below);
        const int cur = cnt[w * E + e];
        sorted[cur + rank] = i;
        __builtin_amdgcn_wave_barrier();
        if (lane == 63 - __clzll(peers)) cnt[w * E + e] = cur + __popcll(peers);
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
}

__global__ void __launch_bounds__(kThreads)
k_align(const int32_t* __restrict__ ids, int R, int E, int bm, int32_t* __restrict__ sorted,
        int32_t* __restrict__ expert_ids, int32_t* __restrict__ ntp_out, int sorted_cap,
        int blocks_cap, int T, int S) {
  extern __shared__ int smem[];
  align_body(ids, R, E, bm, sorted, expert_ids, ntp_out, sorted_cap, blocks_cap, smem, T, S);
}

// ---------------------------------------------------------------------------
// The same plan for many routes, from three launches over chunks of
// kChunk consecutive route ids (one workgroup runs the steps above in
// 8.8 us for 1,536 routes but 165 us for 65,536): per-chunk expert counts;
// one workgroup turns them into per-chunk cursors (segment start plus the
// counts of earlier chunks) and the block owners (the count launch has set
// every slot to -1); one wave per chunk then
// scatters its ids in order.  Chunks are contiguous and taken in order, so
// the result is the one-workgroup plan, bit for bit.  counts: C * ET ints
// of workspace, C = ceil(routes / kChunk).
// ---------------------------------------------------------------------------

constexpr int kChunk = 512;

// Also sets its share of sorted_token_ids to -1 (the padding; the scatter
// overwrites the slots that hold a route).
__global__ void __launch_bounds__(256)
k_align_count(const int32_t* __restrict__ ids, int R_routed, int E_routed, int T, int S,
              int* __restrict__ counts, int32_t* __restrict__ sorted, int sorted_cap) {
  extern __shared__ int h[];
  const int ET = E_routed + S, R = R_routed + T * S;
  const int share = (sorted_cap + (int)gridDim.x - 1) / (int)gridDim.x;
  const int f_lo = (int)blockIdx.x * share, f_hi = min(sorted_cap, f_lo + share);
  for (int q = f_lo + (int)threadIdx.x; q < f_hi; q += 256) sorted[q] = -1;
  for (int e = threadIdx.x; e < ET; e += 256) h[e] = 0;
  __syncthreads();
  const int lo = blockIdx.x * kChunk, hi = min(R, lo + kChunk);
  for (int i = lo + (int)threadIdx.x; i < hi; i += 256) {
    const int e = route_expert(ids, i, R_routed, E_routed, S);
    if (e >= 0) atomicAdd(&h[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < ET; e += 256) counts[(size_t)blockIdx.x * ET + e] = h[e];
}

__global__ void __launch_bounds__(kThreads)
k_align_plan(int ET, int C, int bm, int* __restrict__ counts, int32_t* __restrict__ sorted,
             int32_t* __restrict__ expert_ids, int32_t* __restrict__ ntp_out, int sorted_cap,
             int blocks_cap) {
  __shared__ int wsum[kWaves + 1];
  extern __shared__ int off[];  // [ET]
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // totals and padded counts, two experts per thread (ET <= 1024), block scan
  // (the chunk loops are unrolled so that their loads overlap: one load per
  // memory latency made this kernel the planner's slowest step)
  const int e0 = 2 * tid, e1 = 2 * tid + 1;
  int c0 = 0, c1 = 0;
  if (e0 < ET) {
#pragma unroll 16
    for (int c = 0; c < C; ++c) c0 += counts[(size_t)c * ET + e0];
  }
  if (e1 < ET) {
#pragma unroll 16
    for (int c = 0; c < C; ++c) c1 += counts[(size_t)c * ET + e1];
  }
  const int p0 = (c0 + bm - 1) / bm * bm, p1 = (c1 + bm - 1) / bm * bm;
  int x = p0 + p1;
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int v = 0; v < kWaves; ++v) {
      const int t = wsum[v];
      wsum[v] = run;
      run += t;
    }
    wsum[kWaves] = run;
  }
  __syncthreads();
  const int excl = wsum[w] + x - (p0 + p1);
  if (e0 < ET) off[e0] = excl;
  if (e1 < ET) off[e1] = excl + p0;
  const int ntp = wsum[kWaves];
  __syncthreads();
  for (int e = tid; e < ET; e += kThreads) {
    int run = off[e];
    int c = 0;
    for (; c + 16 <= C; c += 16) {  // 16 loads in flight, then the running sums
      int t[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) t[u] = counts[(size_t)(c + u) * ET + e];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        counts[(size_t)(c + u) * ET + e] = run;
        run += t[u];
      }
    }
    for (; c < C; ++c) {
      const int t = counts[(size_t)c * ET + e];
      counts[(size_t)c * ET + e] = run;
      run += t;
    }
    // run is now the end of the expert's routes; its blocks (the padding
    // slots were set to -1 by the count launch)
    const int pend = off[e] + (run - off[e] + bm - 1) / bm * bm;
    for (int q = off[e] / bm; q < pend / bm; ++q) expert_ids[q] = e;
  }
  if (C == 0)  // no count launch ran
    for (int q = tid; q < sorted_cap; q += kThreads) sorted[q] = -1;
  for (int q = ntp / bm + tid; q < blocks_cap; q += kThreads) expert_ids[q] = -1;
  if (tid == 0) *ntp_out = ntp;
}

__global__ void __launch_bounds__(64)
k_align_scatter(const int32_t* __restrict__ ids, int R_routed, int E_routed, int T, int S,
                const int* __restrict__ counts, int32_t* __restrict__ sorted) {
  extern __shared__ int cur[];
  const int ET = E_routed + S, R = R_routed + T * S;
  const int lane = threadIdx.x;
  for (int e = lane; e < ET; e += 64) cur[e] = counts[(size_t)blockIdx.x * ET + e];
  __syncthreads();
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int lo = blockIdx.x * kChunk, hi = min(R, lo + kChunk);
  for (int base = lo; base < hi; base += 64) {
    const int i = base + lane;
    const int e = i < hi ? route_expert(ids, i, R_routed, E_routed, S) : -1;
    const bool ok = e >= 0;
    unsigned long long peers = __ballot(ok);
    for (int bit = 0; (1 << bit) < ET; ++bit) {
      const bool set = (e >> bit) & 1;
      const unsigned long long m = __ballot(ok && set);
      peers &= set ? m : ~m;
    }
    if (ok) {
      const int rank = __popcll(peers & below);
      const int c = cur[e];
      sorted[c + rank] = i;
      __builtin_amdgcn_wave_barrier();
      if (lane == 63 - __clzll(peers)) cur[e] = c + __popcll(peers);
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// ---------------------------------------------------------------------------
// Router + planner in one launch.
//
// The gate's routing ([prime-flash] "Usage": it arrives at the planner as
// topk_ids and topk_weights; [hpc-ops RFC] "Results so far": normalized
// routing weights) is computed from the router logits, then the planner runs
// on it.  The planner needs every token's routes (grid-wide histogram and
// prefix, [hpc-ops RFC] "Design"), so the workgroups route their tokens,
// publish them, and take a ticket; the last one to arrive runs the planner on
// the whole routing.  No workgroup waits for another.
//
// Routing of one token by one wave: lane l holds logits l, l + 64, ... (EPL
// of them); k rounds each pick the largest logit not yet taken, ties to the
// lower expert id, by a wave-wide arg-max; the selected ids come out in
// descending logit order.  Weights: the softmax over all experts renormalized
// over the selection equals exp(l_j - l_max) / sum over the selection of
// exp(l_i - l_max), in fp32 with the library expf and an IEEE division.
// ---------------------------------------------------------------------------

constexpr int kMaxTopK = 16;

// (v, i) beats (bv, bi): larger logit, or equal logit and lower id; i < 0 is
// "nothing" and never beats anything
__device__ __forceinline__ bool beats(float v, int i, float bv, int bi) {
  return i >= 0 && (bi < 0 || v > bv || (v == bv && i < bi));
}

// one DPP step of the row-wide arg-max: (bv, bi) against its partner lane
template <int CTRL>
__device__ __forceinline__ void argmax_step(float& bv, int& bi) {
  const float ov = __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, bv), __builtin_bit_cast(int, bv),
                                         CTRL, 0xF, 0xF, false));
  const int oi = __builtin_amdgcn_update_dpp(bi, bi, CTRL, 0xF, 0xF, false);
  if (beats(ov, oi, bv, bi)) bv = ov, bi = oi;
}

// Wave-wide arg-max: xor 1 and xor 2 inside quads, then the half-row and row
// mirrors (every lane of a 16-lane row holds the row's best), then the four
// rows' results read out and combined (uniform over the wave).
__device__ __forceinline__ void wave_argmax(float& bv, int& bi) {
  argmax_step<0xB1>(bv, bi);   // quad_perm [1, 0, 3, 2]
  argmax_step<0x4E>(bv, bi);   // quad_perm [2, 3, 0, 1]
  argmax_step<0x141>(bv, bi);  // row_half_mirror
  argmax_step<0x140>(bv, bi);  // row_mirror
  float rv[4];
  int ri[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    rv[q] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, bv), 16 * q));
    ri[q] = __builtin_amdgcn_readlane(bi, 16 * q);
  }
  if (beats(rv[1], ri[1], rv[0], ri[0])) rv[0] = rv[1], ri[0] = ri[1];
  if (beats(rv[3], ri[3], rv[2], ri[2])) rv[2] = rv[3], ri[2] = ri[3];
  if (beats(rv[2], ri[2], rv[0], ri[0])) rv[0] = rv[2], ri[0] = ri[2];
  bv = rv[0];
  bi = ri[0];
}

template <int EPL>
__device__ __forceinline__ void load_token(const float* __restrict__ row, int E, int lane,
                                           float (&v)[EPL]) {
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + 64 * j;
    v[j] = e < E ? row[e] : 0.f;
  }
}

template <int EPL>
__device__ __forceinline__ void route_token(const float (&v)[EPL], int E, int k,
                                            int32_t* __restrict__ ids_out,
                                            float* __restrict__ w_out, int lane) {
  uint32_t taken = 0;  // bit j: slot j is taken (or lies past E)
#pragma unroll
  for (int j = 0; j < EPL; ++j)
    if (lane + 64 * j >= E) taken |= 1u << j;
  float sv[kMaxTopK];
  int si[kMaxTopK];
#pragma unroll
  for (int r = 0; r < kMaxTopK; ++r) {
    if (r >= k) break;
    float bv = 0.f;
    int bi = -1;
#pragma unroll
    for (int j = 0; j < EPL; ++j)  // ascending ids: a later equal logit never wins
      if (!((taken >> j) & 1u) && beats(v[j], lane + 64 * j, bv, bi)) bv = v[j], bi = lane + 64 * j;
    wave_argmax(bv, bi);
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    sv[r] = bv;
    si[r] = bi;
  }
  float ex[kMaxTopK];
  float sum = 0.f;
#pragma unroll
  for (int r = 0; r < kMaxTopK; ++r) {
    if (r >= k) break;
    ex[r] = expf(sv[r] - sv[0]);
    sum += ex[r];
  }
#pragma unroll
  for (int r = 0; r < kMaxTopK; ++r) {
    if (r >= k) break;
    if (lane == r) {
      ids_out[r] = si[r];
      w_out[r] = ex[r] / sum;
    }
  }
}

// tokens whose logits a wave loads at once (registers: NB * EPL per lane)
template <int EPL>
constexpr int route_batch() { return EPL <= 2 ? 4 : EPL <= 8 ? 2 : 1; }

template <int EPL>
__global__ void __launch_bounds__(kThreads)
k_route_align(const float* __restrict__ logits, int T, int E, int top_k, int bm,
              int32_t* __restrict__ topk_ids, float* __restrict__ topk_w,
              int32_t* __restrict__ sorted, int32_t* __restrict__ expert_ids,
              int32_t* __restrict__ ntp_out, int sorted_cap, int blocks_cap,
              int* __restrict__ ticket, int tokens_per_wg, int plan) {
  extern __shared__ int smem[];
  __shared__ int is_last;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int t0 = blockIdx.x * tokens_per_wg;
  const int t1 = min(T, t0 + tokens_per_wg);
  constexpr int NB = route_batch<EPL>();
  for (int t = t0 + w; t < t1; t += kWaves * NB) {
    float v[NB][EPL];
#pragma unroll
    for (int b = 0; b < NB; ++b)
      if (t + b * kWaves < t1) load_token<EPL>(logits + (size_t)(t + b * kWaves) * E, E, lane, v[b]);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int tb = t + b * kWaves;
      if (tb < t1)
        route_token<EPL>(v[b], E, top_k, topk_ids + (size_t)tb * top_k,
                         topk_w + (size_t)tb * top_k, lane);
    }
  }
  if (!plan) return;  // the chunked planner runs in launches of its own
  if (gridDim.x == 1) {
    // one workgroup routed every token: a workgroup barrier publishes them
    __syncthreads();
  } else {
    // release this workgroup's routes device-wide, then take a ticket
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) is_last = atomicAdd(ticket, 1) == (int)gridDim.x - 1;
    __syncthreads();
    if (!is_last) return;
    // acquire the other workgroups' routes; leave the ticket at zero for the
    // next call (an atomic, so that it reaches the point where the next
    // call's atomics are performed)
    __threadfence();
    if (threadIdx.x == 0) atomicExch(ticket, 0);
  }
  align_body(topk_ids, T * top_k, E, bm, sorted, expert_ids, ntp_out, sorted_cap, blocks_cap,
             smem, T, 0);
}

}  // namespace

hipError_t launch_route_align(const float* logits, int T, int E, int top_k, int block_m,
                              int32_t* topk_ids, float* topk_w, int32_t* sorted,
                              int32_t* expert_ids, int32_t* ntp, int sorted_cap, int blocks_cap,
                              int* ticket, hipStream_t stream, int* chunk_counts) {
  const size_t smem = (size_t)(kWaves * E + 2 * E + kWaves + 1) * sizeof(int);
  // one token per wave up to 256 workgroups, then more tokens per wave
  const int want = (T + kWaves - 1) / kWaves;
  const int groups = want < 1 ? 1 : (want > 256 ? 256 : want);
  const int per = (T + groups - 1) / groups;
  const int epl = (E + 63) / 64;
#define MOE_ROUTE(N)                                                                          \
  hipLaunchKernelGGL(k_route_align<N>, dim3(groups), dim3(kThreads), smem, stream, logits, T, E, \
                     top_k, block_m, topk_ids, topk_w, sorted, expert_ids, ntp, sorted_cap,   \
                     blocks_cap, ticket, per, chunk_counts ? 0 : 1)
  if (epl <= 1) MOE_ROUTE(1);
  else if (epl <= 2) MOE_ROUTE(2);
  else if (epl <= 4) MOE_ROUTE(4);
  else if (epl <= 8) MOE_ROUTE(8);
  else MOE_ROUTE(16);
#undef MOE_ROUTE
  if (chunk_counts)
    return launch_align_chunked(topk_ids, T * top_k, E, block_m, sorted, expert_ids, ntp,
                                sorted_cap, blocks_cap, stream, T, 0, chunk_counts);
  return hipGetLastError();
}

size_t align_chunked_ws(int64_t routes, int ET) {
  const int64_t C = (routes + kChunk - 1) / kChunk;
  return (size_t)(C > 0 ? C : 1) * ET * sizeof(int);
}

hipError_t launch_align_chunked(const int32_t* topk_ids, int R, int E, int block_m,
                                int32_t* sorted, int32_t* expert_ids, int32_t* ntp,
                                int sorted_cap, int blocks_cap, hipStream_t stream, int T,
                                int n_shared, int* counts) {
  const int ET = E + n_shared;
  const int routes = R + T * n_shared;
  const int C = (routes + kChunk - 1) / kChunk;
  const size_t hsm = (size_t)ET * sizeof(int);
  if (C > 0)
    hipLaunchKernelGGL(k_align_count, dim3(C), dim3(256), hsm, stream, topk_ids, R, E, T,
                       n_shared, counts, sorted, sorted_cap);
  hipLaunchKernelGGL(k_align_plan, dim3(1), dim3(kThreads), hsm, stream, ET, C, block_m, counts,
                     sorted, expert_ids, ntp, sorted_cap, blocks_cap);
  if (C > 0)
    hipLaunchKernelGGL(k_align_scatter, dim3(C), dim3(64), hsm, stream, topk_ids, R, E, T,
                       n_shared, counts, sorted);
  return hipGetLastError();
}

hipError_t launch_align(const int32_t* topk_ids, int R, int E, int block_m, int32_t* sorted,
                        int32_t* expert_ids, int32_t* ntp, int sorted_cap, int blocks_cap,
                        hipStream_t stream, int T, int n_shared) {
  const int ET = E + n_shared;
  const size_t smem = (size_t)(kWaves * ET + 2 * ET + kWaves + 1) * sizeof(int);
  hipLaunchKernelGGL(k_align, dim3(1), dim3(kThreads), smem, stream, topk_ids, R, E, block_m,
                     sorted, expert_ids, ntp, sorted_cap, blocks_cap, T, n_shared);
  return hipGetLastError();
}
