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
//   3. padding slots of each segment and the tail up to the capacity get -1,
//      expert_ids gets the owner of each block (-1 past the last block);
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

__global__ void __launch_bounds__(kThreads)
k_align(const int32_t* __restrict__ ids, int R, int E, int bm, int32_t* __restrict__ sorted,
        int32_t* __restrict__ expert_ids, int32_t* __restrict__ ntp_out, int sorted_cap,
        int blocks_cap) {
  extern __shared__ int smem[];
  int* cnt = smem;                     // [kWaves][E]: counts, then cursors
  int* off = smem + kWaves * E;        // [E]: segment start
  int* tot = off + E;                  // [E]: route count
  int* wsum = tot + E;                 // [kWaves + 1]: scan scratch
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  for (int i = tid; i < kWaves * E; i += kThreads) cnt[i] = 0;
  __syncthreads();

  const int seg = (R + kWaves - 1) / kWaves;
  const int lo = min(R, w * seg), hi = min(R, lo + seg);
  // ids are read kBatch chunks of 64 at a time so that the global loads
  // overlap instead of costing one memory latency per chunk
  for (int base = lo; base < hi; base += 64 * kBatch) {
    int eb[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = base + u * 64 + lane;
      eb[u] = i < hi ? ids[i] : -1;
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
    // padding inside the segment and the expert of each block
    const int pend = off[e] + (tot[e] + bm - 1) / bm * bm;
    for (int q = off[e] + tot[e]; q < pend; ++q) sorted[q] = -1;
    for (int q = off[e] / bm; q < pend / bm; ++q) expert_ids[q] = e;
  }
  for (int q = ntp + tid; q < sorted_cap; q += kThreads) sorted[q] = -1;
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
      eb[u] = i < hi ? ids[i] : -1;
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

}  // namespace

hipError_t launch_align(const int32_t* topk_ids, int R, int E, int block_m, int32_t* sorted,
                        int32_t* expert_ids, int32_t* ntp, int sorted_cap, int blocks_cap,
                        hipStream_t stream) {
  const size_t smem = (size_t)(kWaves * E + 2 * E + kWaves + 1) * sizeof(int);
  hipLaunchKernelGGL(k_align, dim3(1), dim3(kThreads), smem, stream, topk_ids, R, E, block_m,
                     sorted, expert_ids, ntp, sorted_cap, blocks_cap);
  return hipGetLastError();
}
