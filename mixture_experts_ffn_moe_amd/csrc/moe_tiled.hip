// moe_tiled.hip -- LDS-tiled split-mode kernels for many rows per expert
// (block_m 64 and 128, e4m3 paths: blockwise FP8 and MXFP8).
//
// Same computation as k_up / k_down in moe_kernels.hip ([hpc-ops RFC]
// "Background" stages 2-4; [prime-flash] introduction, split=True), organized
// for the regime where each expert holds many rows, so that the MFMA pipes
// rather than the operand loads set the pace:
//
//  * A (activation rows) and B (weight rows) of one 128-wide K step are
//    staged in LDS with direct-to-LDS 16-byte buffer loads (no VGPR staging),
//    NSTAGE steps in flight.  Every wave then reads its MFMA fragments from
//    LDS, so each operand byte crosses the L2 -> CU path once per workgroup.
//  * LDS rows are 128 bytes (8 chunks of 16 bytes); chunk q of row r is stored
//    at chunk q ^ (r & 7).  Measured on gfx950 with the fragment pattern (lane
//    (g, r) reading chunks g and 4 + g of row r of a 16-row group), this plain
//    xor reads at 216 B/clk/CU, lane-contiguous addresses at 191, and the xor
//    with an extra (r >> 3) & 1 term that spreads 16 rows over 16 bank groups
//    at 127 (its lanes g, r and g + 1, r + 8 meet in one bank group).  The
//    loads write LDS in lane order, so each lane fetches the logical chunk
//    that belongs in its slot.
//  * Workgroup tile: block_m rows x (128 gate + 128 up) for k_up_t,
//    block_m rows x 256 output columns for k_down_t; 4 waves arranged
//    (block_m / 64) x (4 / (block_m / 64)); a wave owns 64 rows.
//  * Blockwise scales: the activation row scales of each step ride along in
//    LDS (4-byte direct loads); weight block scales are wave-uniform scalar
//    loads.  MX: the e8m0 dwords of each row (4 K blocks per step) ride along
//    in LDS and feed the block-scaled MFMA.
//  * Workgroup ids are remapped so that consecutive tiles (the slices of one
//    block, then the next block of the same expert) land on one XCD and share
//    its L2.
#include "device.h"
#include "launch.h"

namespace {

constexpr int kRowBytes = 128;  // one K step of e4m3
constexpr int kChunks = 8;      // 16-byte chunks per row

__device__ __forceinline__ int swz(int row) { return row & 7; }

// Workgroup barrier without the release fence __syncthreads() carries: that
// fence waits for every outstanding vector load, including the direct-to-LDS
// loads of later pipeline stages.  Stage completion is tracked with explicit
// vmcnt waits instead; the empty asm keeps the compiler from moving memory
// accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS reads are done
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Logical tile index of workgroup `bid`.  The hardware dispatches workgroup
// ids round-robin over the 8 XCDs; the `valid` tiles that have a planner
// block (read on the device) are split into 8 contiguous runs, run x on XCD
// x, so consecutive tiles share that XCD's L2 and every XCD gets an equal
// share.  (Splitting the whole grid instead, whose blocks past the padded
// count are empty, left the last XCDs idle: at K=4096, I=2048, E=288,
// top-8, T=8192 only 656 of 798 blocks hold routes.)  -1: past the runs.
__device__ __forceinline__ int xcd_remap(int bid, int valid) {
  const int per = (valid + 7) / 8;
  const int j = bid / 8;
  return j < per ? (bid % 8) * per + j : -1;
}

template <int KIND, int BM, int BN, int NS>
struct TileCfg {
  // waves per workgroup: two per SIMD from 128 rows up, so that one wave's
  // LDS reads and blockwise promotion overlap the other's MFMAs (128 rows,
  // K=4096, I=2048, E=288, top-8: 4.04 against 4.56 ms at T=8192 with one
  // wave per SIMD); 64-row tiles keep one 64 x 64 tile per wave
  static constexpr int NW = BM >= 128 ? 8 : 4;
  static constexpr int WM = BM / 64;            // wave rows (64 rows each)
  static constexpr int WN = NW / WM;            // wave columns
  static constexpr int MI = 4;                  // 16-row subtiles per wave
  static constexpr int NI = BN / WN / 16;       // 16-column subtiles per wave
  static constexpr int A_BYTES = BM * kRowBytes;
  static constexpr int B_BYTES = BN * kRowBytes;
  // Row scales (fp32, or 4 x e8m0 per row): each wave stages SA_ROWS rows in
  // 64 four-byte slots (every lane loads; the slots past SA_ROWS are padding).
  static constexpr int SA_BYTES = NW * 256;
  static constexpr int SB_BYTES = (KIND == KIND_MX) ? NW * 256 : 0;  // MX weight scales
  static constexpr int STAGE = A_BYTES + B_BYTES + SA_BYTES + SB_BYTES;
  static constexpr int A_INSTR = A_BYTES / 1024 / NW;  // 16-byte DMA instructions per wave
  static constexpr int B_INSTR = B_BYTES / 1024 / NW;
  static constexpr int SA_ROWS = BM / NW;              // scale rows staged per wave
  static constexpr int SB_ROWS = BN / NW;
  static constexpr int S_INSTR = 1 + ((KIND == KIND_MX) ? 1 : 0);
  static constexpr int LOADS = A_INSTR + B_INSTR + S_INSTR;  // per wave per stage
  static constexpr int THREADS = NW * 64;
  static_assert(SA_ROWS <= 64 && SB_ROWS <= 64, "one scale instruction per wave");
};

// Operand sources of one tile GEMM.
struct TileSrc {
  desc_t ra, rb, rsa, rsb;
  const float* bsc;  // FP8B: weight block-scale row of the wave's n-block (index: step)
  const float* bsc2; // FP8B k_up_t: the up half's block-scale row
};

// Issue the DMA loads of K step `ks` into stage slot `st` of the pipeline
// area at LDS address `lds` (a wave-uniform byte address).
//  a_off[t] / b_off[t]: this lane's byte offsets of its A / B chunks (t-th load)
//  sa_off / sb_off    : this lane's scale row offsets; sa_step bytes per step
template <int KIND, int BM, int BN, int NS>
__device__ __forceinline__ void tile_load(const TileSrc& src, uint32_t lds, int st, int ks,
                                          const uint32_t (&a_off)[TileCfg<KIND, BM, BN, NS>::A_INSTR],
                                          uint32_t sa_off, uint32_t sa_step,
                                          const uint32_t (&b_off)[TileCfg<KIND, BM, BN, NS>::B_INSTR],
                                          uint32_t sb_off) {
  using C = TileCfg<KIND, BM, BN, NS>;
  const uint32_t w = (uint32_t)wave_id();
  const uint32_t stage = lds + (uint32_t)(st * C::STAGE);
  const uint32_t soff = (uint32_t)ks * kRowBytes;
#pragma unroll
  for (int t = 0; t < C::A_INSTR; ++t) dma16(src.ra, stage + (w + C::NW * t) * 1024, a_off[t], soff);
#pragma unroll
  for (int t = 0; t < C::B_INSTR; ++t)
    dma16(src.rb, stage + C::A_BYTES + (w + C::NW * t) * 1024, b_off[t], soff);
  // row scales: wave w stages rows [w * SA_ROWS, (w + 1) * SA_ROWS) in its 64
  // slots.  All lanes load (lanes past SA_ROWS fill padding from an in-bounds
  // row): a lane-dependent branch around the asm would put its scalar
  // operands in vector registers.
  dma4(src.rsa, stage + C::A_BYTES + C::B_BYTES + w * 256, sa_off, (uint32_t)ks * sa_step);
  if constexpr (KIND == KIND_MX)
    dma4(src.rsb, stage + C::A_BYTES + C::B_BYTES + C::SA_BYTES + w * 256, sb_off, (uint32_t)ks * 4);
}

// Per-lane DMA offsets of the A and B tiles: lane slot (w + 4t) * 64 + lane
// holds row slot / 8, physical chunk slot % 8, which carries logical chunk
// (slot % 8) ^ swz(row).
template <int NW>
__device__ __forceinline__ void dma_rows(int t_idx, int& row, int& qchunk) {
  const int lane = threadIdx.x & 63, w = wave_id();
  const int slot = (w + NW * t_idx) * 64 + lane;
  row = slot / kChunks;
  qchunk = (slot % kChunks) ^ swz(row);
}

// Fragment of row `row` (tile-relative) from a staged tile at `base`.
__device__ __forceinline__ void lds_frag(Frag<KIND_FP8B>& f, const uint8_t* base, int row, int g) {
  const uint8_t* r = base + row * kRowBytes;
  const int s = swz(row);
  f.c[0] = *reinterpret_cast<const uint4*>(r + ((g ^ s) << 4));
  f.c[1] = *reinterpret_cast<const uint4*>(r + (((4 + g) ^ s) << 4));
}

// LDS slot of a row's staged scale: wave row / ROWS, lane row % ROWS.
template <int ROWS>
__device__ __forceinline__ int scale_slot(int row) { return (row / ROWS) * 64 + row % ROWS; }

// Compute one staged K step (stage at `stage`, logical step ks).
template <int KIND, int BM, int BN, int NS>
__device__ __forceinline__ void tile_step(const uint8_t* stage, int ks, const StepScales& sc1,
                                          const StepScales& sc2, int up_split,
                                          f32x4 (&acc)[4][TileCfg<KIND, BM, BN, NS>::NI]) {
  using C = TileCfg<KIND, BM, BN, NS>;
  constexpr int MI = C::MI, NI = C::NI;
  const int lane = threadIdx.x & 63, wid = wave_id();
  const int wn = wid % C::WN, wm = wid / C::WN;
  const int g = lane >> 4, r16 = lane & 15;
  const uint8_t* ta = stage;
  const uint8_t* tb = stage + C::A_BYTES;
  const uint8_t* tsa = stage + C::A_BYTES + C::B_BYTES;
  const uint8_t* tsb = tsa + C::SA_BYTES;
  // With one wave per SIMD nothing else hides LDS latency, so every fragment
  // of the step is requested before the first MFMA (reads complete in order
  // and each MFMA waits only for its own operands).  With two waves per SIMD
  // the register budget is halved; B fragments are then read per column
  // and the other wave covers the wait.
  constexpr bool B_AHEAD = C::NW == 4;
  auto brow_of = [&](int ni) {
    return (ni < up_split ? 0 : BN / 2 - up_split * 16) + wn * (up_split * 16) + ni * 16 + r16;
  };
  Frag<KIND_FP8B> fa[MI];
  Frag<KIND_FP8B> fbs[B_AHEAD ? NI : 1];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) lds_frag(fa[mi], ta, wm * 64 + mi * 16 + r16, g);
  if constexpr (B_AHEAD) {
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) lds_frag(fbs[ni], tb, brow_of(ni), g);
  }
  auto frag_b = [&](int ni) -> Frag<KIND_FP8B> {
    if constexpr (B_AHEAD) {
      return fbs[ni];
    } else {
      Frag<KIND_FP8B> fb;
      lds_frag(fb, tb, brow_of(ni), g);
      return fb;
    }
  };
  if constexpr (KIND == KIND_FP8B) {
    float sa[MI][4];
    const float s1 = sc1.at(ks);
    const float s2 = sc2.at(ks);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        sa[mi][i4] = reinterpret_cast<const float*>(tsa)[scale_slot<C::SA_ROWS>(wm * 64 + mi * 16 + 4 * g + i4)];
    // MFMAs of subtile column ni go into their own temporaries and are
    // promoted one column later, so the MFMA pipe never waits on a
    // promotion (the tile products are independent of each other).
    f32x4 t[2][MI];
    auto issue = [&](int ni, f32x4 (&tt)[MI]) {
      const Frag<KIND_FP8B> fb = frag_b(ni);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        tt[mi] = mfma_step<KIND_FP8B>(fa[mi], fb, z);
      }
    };
    auto promote = [&](int ni, const f32x4 (&tt)[MI]) {
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
          acc[mi][ni][i4] += tt[mi][i4] * (sa[mi][i4] * (ni < up_split ? s1 : s2));
    };
    if constexpr (C::NW == 8) {
      // two waves share each SIMD and fill each other's MFMA gaps; no
      // lookahead, which keeps the wave within 256 registers
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        issue(ni, t[0]);
        promote(ni, t[0]);
      }
    } else {
      issue(0, t[0]);
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        if (ni + 1 < NI) issue(ni + 1, t[(ni + 1) & 1]);
        promote(ni, t[ni & 1]);
      }
    }
  } else {  // MX
    int xa[MI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
      xa[mi] = (reinterpret_cast<const uint32_t*>(tsa)[scale_slot<C::SA_ROWS>(wm * 64 + mi * 16 + r16)] >>
                (8 * g)) & 0xff;
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const Frag<KIND_FP8B> fb = frag_b(ni);
      const int xb =
          (reinterpret_cast<const uint32_t*>(tsb)[scale_slot<C::SB_ROWS>(brow_of(ni))] >> (8 * g)) & 0xff;
      Frag<KIND_MX> fbm, fam;
      fbm.c[0] = fb.c[0];
      fbm.c[1] = fb.c[1];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        fam.c[0] = fa[mi].c[0];
        fam.c[1] = fa[mi].c[1];
        acc[mi][ni] = mfma_step_mx(fam, fbm, acc[mi][ni], xa[mi], xb);
      }
    }
  }
}

// One workgroup tile: acc[mi][ni] over all K steps, visiting the steps from
// a staggered start, NS stages in flight (stage slots in one LDS array).
template <int KIND, int BM, int BN, int NS>
__device__ __forceinline__ void tile_gemm(const TileSrc& src, uint8_t* smem, int ksteps,
                                          const uint32_t (&a_off)[TileCfg<KIND, BM, BN, NS>::A_INSTR],
                                          uint32_t sa_off, uint32_t sa_step,
                                          const uint32_t (&b_off)[TileCfg<KIND, BM, BN, NS>::B_INSTR],
                                          uint32_t sb_off, int up_split, int group,
                                          f32x4 (&acc)[4][TileCfg<KIND, BM, BN, NS>::NI]) {
  using C = TileCfg<KIND, BM, BN, NS>;
  constexpr int MI = C::MI, NI = C::NI;
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};
  StepScales sc1{0.f, 0.f}, sc2{0.f, 0.f};
  if constexpr (KIND == KIND_FP8B) {
    sc1.load(src.bsc, ksteps);
    sc2.load(src.bsc2 ? src.bsc2 : src.bsc, ksteps);
    // wait here: the compiler would place this wait at the first use, inside
    // the K loop, where it would also drain the pipeline's loads every pass
    wait_vmcnt<0>();
  }
  // All tiles of one expert start at the same step and walk K in step: the
  // slices (or column tiles) of one block then read its gathered activation
  // rows at nearly the same time and share them in L2, and the blocks of one
  // expert share its weight rows.  (Starting each slice at its own step let
  // the weight stream evict the activation rows between their reads: 7.0
  // against 5.3 GB fetched by the gate/up GEMM at K=4096, I=2048, E=288,
  // top-8, T=8192.)  Other experts start elsewhere, which spreads the weight
  // rows read at one moment over the HBM channels.
  const int rot = (int)((((uint32_t)group * 2654435761u) >> 16) % (uint32_t)ksteps);
  auto step_at = [&](int i) { const int k = i + rot; return k >= ksteps ? k - ksteps : k; };
  const uint32_t lbase = lds_addr(smem);
  auto load = [&](int slot, int i) {
    tile_load<KIND, BM, BN, NS>(src, lbase, slot, step_at(i), a_off, sa_off, sa_step, b_off, sb_off);
  };
#pragma unroll
  for (int u = 0; u < NS - 1; ++u)
    if (u < ksteps) load(u, u);
  int slot = 0;
  for (int i = 0; i < ksteps; ++i) {
    // step i has landed once only the later steps' loads may be pending
    if (i + NS - 2 < ksteps) wait_vmcnt<C::LOADS * (NS - 2)>();
    else wait_vmcnt<0>();
    lds_barrier();
    const int ahead = slot + NS - 1;
    if (i + NS - 1 < ksteps) load(ahead >= NS ? ahead - NS : ahead, i + NS - 1);
    tile_step<KIND, BM, BN, NS>(smem + slot * C::STAGE, step_at(i), sc1, sc2, up_split, acc);
    slot = slot + 1 == NS ? 0 : slot + 1;
  }
  __syncthreads();  // the caller reuses the LDS
}


// gate/up GEMM + SwiGLU + requantization, one (block, 128-wide slice) tile
template <int KIND, int BM, int NS>
__global__ void __launch_bounds__(BM >= 128 ? 512 : 256) __attribute__((amdgpu_waves_per_eu(1, BM >= 128 ? 2 : 1))) k_up_t(MoeArgs p) {
  using C = TileCfg<KIND, BM, 256, NS>;
  constexpr int MI = C::MI, NI = C::NI, HALF = NI / 2;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * C::STAGE];
  __shared__ int ids[BM];
  __shared__ float lds_amax[C::WN * BM];
  const int S = p.I / 128;
  const int logical = xcd_remap(blockIdx.x, (*p.ntp / BM) * S);
  if (logical < 0) return;
  const int b = logical / S, s = logical % S;
  if (b >= p.blocks_cap || b * BM >= *p.ntp) return;
  const int e = __builtin_amdgcn_readfirstlane(p.expert_ids[b]);  // uniform: descriptors in SGPRs
  if ((unsigned)e >= (unsigned)p.E) return;
  const int lane = threadIdx.x & 63, wid = wave_id();
  const int wn = wid % C::WN, wm = wid / C::WN;
  const int g = lane >> 4, r16 = lane & 15;
  if (threadIdx.x < BM) ids[threadIdx.x] = p.sorted[b * BM + threadIdx.x];
  __syncthreads();
  const int K = p.K, I = p.I, N = 2 * I, KS = K / 128;

  TileSrc src;
  src.ra = make_desc(p.x, (uint32_t)((size_t)p.T * K));
  src.rb = make_desc(p.w1 + (size_t)e * N * K, (uint32_t)((size_t)N * K));
  uint32_t a_off[C::A_INSTR], b_off[C::B_INSTR];
#pragma unroll
  for (int t = 0; t < C::A_INSTR; ++t) {
    int row, q;
    dma_rows<C::NW>(t, row, q);
    a_off[t] = (uint32_t)route_token(p, ids[row]) * K + q * 16;
  }
#pragma unroll
  for (int t = 0; t < C::B_INSTR; ++t) {
    int row, q;
    dma_rows<C::NW>(t, row, q);  // rows [0,128): gate slice rows; [128,256): up slice rows
    const int n = (row < 128 ? s * 128 + row : I + s * 128 + row - 128);
    b_off[t] = (uint32_t)n * K + q * 16;
  }
  const int srow = wid * C::SA_ROWS + lane;  // scale row this lane stages
  uint32_t sa_off = 0, sa_step = 4, sb_off = 0;
  if constexpr (KIND == KIND_FP8B) {
    src.rsa = make_desc(p.xs, (uint32_t)((size_t)p.T * KS * 4));
    sa_off = (uint32_t)route_token(p, ids[srow < BM ? srow : 0]) * KS * 4;
    src.bsc = reinterpret_cast<const float*>(p.w1s) + ((size_t)e * (N / 128) + s) * KS;
    src.bsc2 = reinterpret_cast<const float*>(p.w1s) + ((size_t)e * (N / 128) + S + s) * KS;
  } else {
    src.rsa = make_desc(p.xs, (uint32_t)((size_t)p.T * (K / 32)));
    sa_off = (uint32_t)route_token(p, ids[srow < BM ? srow : 0]) * (K / 32);
    src.rsb = make_desc(reinterpret_cast<const uint8_t*>(p.w1s) + (size_t)e * N * (K / 32),
                        (uint32_t)((size_t)N * (K / 32)));
    const int brow = min(wid * C::SB_ROWS + lane, 255);  // B scale row this lane stages
    const int n = (brow < 128 ? s * 128 + brow : I + s * 128 + brow - 128);
    sb_off = (uint32_t)n * (K / 32);
    src.bsc = nullptr;
    src.bsc2 = nullptr;
  }
  f32x4 acc[MI][NI];
  tile_gemm<KIND, BM, 256, NS>(src, smem, KS, a_off, sa_off, sa_step, b_off, sb_off, HALF,
                               e, acc);

  // SwiGLU: gate subtile j pairs with up subtile HALF + j (same columns)
  float h[MI][HALF][4];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int j = 0; j < HALF; ++j)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) h[mi][j][i4] = swiglu(acc[mi][j][i4], acc[mi][HALF + j][i4]);

  // requantize; stage codes in LDS as (BM x 128) bytes, then store rows
  uint8_t* q = smem;  // reuse the pipeline LDS
  constexpr int QROW = 128 + 16;
  const size_t pos0 = (size_t)b * BM;
  if constexpr (KIND == KIND_FP8B) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        float a = 0.f;
#pragma unroll
        for (int j = 0; j < HALF; ++j) a = __builtin_fmaxf(a, __builtin_fabsf(h[mi][j][i4]));
        a = wave_max16(a);
        if (r16 == 0) lds_amax[wn * BM + wm * 64 + mi * 16 + 4 * g + i4] = a;
      }
    __syncthreads();
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int row = wm * 64 + mi * 16 + 4 * g + i4;
        float a = lds_amax[row];
        if constexpr (C::WN == 4)
          a = __builtin_fmaxf(__builtin_fmaxf(a, lds_amax[BM + row]),
                              __builtin_fmaxf(lds_amax[2 * BM + row], lds_amax[3 * BM + row]));
        else
          a = __builtin_fmaxf(a, lds_amax[BM + row]);
        a = __builtin_fmaxf(a, 1e-10f);
        const float f = a * (1.0f / 448.0f);
        const float inv = 1.0f / f;
#pragma unroll
        for (int j = 0; j < HALF; ++j)
          q[row * QROW + wn * HALF * 16 + j * 16 + r16] = (uint8_t)f32_to_e4m3(h[mi][j][i4] * inv);
        if (wn == 0 && r16 == 0) reinterpret_cast<float*>(p.hs)[(pos0 + row) * (I / 128) + s] = f;
      }
  } else {  // MX: groups of 32 columns = subtile pairs (2j, 2j+1) of this wave
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int row = wm * 64 + mi * 16 + 4 * g + i4;
#pragma unroll
        for (int jg = 0; jg < HALF / 2; ++jg) {
          float a = __builtin_fmaxf(__builtin_fabsf(h[mi][2 * jg][i4]),
                                    __builtin_fabsf(h[mi][2 * jg + 1][i4]));
          a = wave_max16(a);
          const int se = mx_shared_exp(a);
#pragma unroll
          for (int jj = 0; jj < 2; ++jj)
            q[row * QROW + wn * HALF * 16 + (2 * jg + jj) * 16 + r16] =
                (uint8_t)f32_to_e4m3(__builtin_amdgcn_ldexpf(h[mi][2 * jg + jj][i4], -se));
          if (r16 == 0) p.hs[(pos0 + row) * (I / 32) + s * 4 + wn * (HALF / 2) + jg] = (uint8_t)(se + 127);
        }
      }
  }
  __syncthreads();
  // coalesced store of the slice: each thread writes 16-byte row chunks
  for (int c = threadIdx.x; c < BM * 8; c += C::THREADS) {
    const int row = c / 8, ch = c % 8;
    *reinterpret_cast<uint4*>(p.hq + (pos0 + row) * I + s * 128 + ch * 16) =
        *reinterpret_cast<const uint4*>(q + row * QROW + ch * 16);
  }
  if (s == 0 && threadIdx.x < BM) {
    const int id = ids[threadIdx.x];
    if (id >= 0) p.flags[id] = 1;
  }
}

// down GEMM, one (block, 256 output columns) tile, fp32 per-route rows
template <int KIND, int BM, int NS>
__global__ void __launch_bounds__(BM >= 128 ? 512 : 256) __attribute__((amdgpu_waves_per_eu(1, BM >= 128 ? 2 : 1))) k_down_t(MoeArgs p) {
  using C = TileCfg<KIND, BM, 256, NS>;
  constexpr int MI = C::MI, NI = C::NI;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * C::STAGE];
  __shared__ int ids[BM];
  const int K = p.K, I = p.I, IS = I / 128;
  const int NT = K / 256;
  const int logical = xcd_remap(blockIdx.x, (*p.ntp / BM) * NT);
  if (logical < 0) return;
  const int b = logical / NT, ct = logical % NT;
  if (b >= p.blocks_cap || b * BM >= *p.ntp) return;
  const int e = __builtin_amdgcn_readfirstlane(p.expert_ids[b]);  // uniform: descriptors in SGPRs
  if ((unsigned)e >= (unsigned)p.E) return;
  const int lane = threadIdx.x & 63, wid = wave_id();
  const int wn = wid % C::WN, wm = wid / C::WN;
  const int g = lane >> 4, r16 = lane & 15;
  if (threadIdx.x < BM) ids[threadIdx.x] = p.sorted[b * BM + threadIdx.x];
  __syncthreads();
  const size_t rows_cap = (size_t)p.blocks_cap * BM;
  TileSrc src;
  src.ra = make_desc(p.hq, (uint32_t)(rows_cap * I));
  src.rb = make_desc(p.w2 + (size_t)e * K * I, (uint32_t)((size_t)K * I));
  uint32_t a_off[C::A_INSTR], b_off[C::B_INSTR];
#pragma unroll
  for (int t = 0; t < C::A_INSTR; ++t) {
    int row, q;
    dma_rows<C::NW>(t, row, q);
    a_off[t] = (uint32_t)((size_t)b * BM + row) * I + q * 16;
  }
#pragma unroll
  for (int t = 0; t < C::B_INSTR; ++t) {
    int row, q;
    dma_rows<C::NW>(t, row, q);
    b_off[t] = (uint32_t)(ct * 256 + row) * I + q * 16;
  }
  const int srow = wid * C::SA_ROWS + lane;
  uint32_t sa_off = 0, sa_step = 4, sb_off = 0;
  const int c0 = ct * 256 + wn * (256 / C::WN);  // this wave's first output column
  if constexpr (KIND == KIND_FP8B) {
    src.rsa = make_desc(p.hs, (uint32_t)(rows_cap * IS * 4));
    sa_off = (uint32_t)((size_t)b * BM + (srow < BM ? srow : 0)) * IS * 4;
    src.bsc = reinterpret_cast<const float*>(p.w2s) + ((size_t)e * (K / 128) + c0 / 128) * IS;
    src.bsc2 = nullptr;
  } else {
    src.rsa = make_desc(p.hs, (uint32_t)(rows_cap * (I / 32)));
    sa_off = (uint32_t)((size_t)b * BM + (srow < BM ? srow : 0)) * (I / 32);
    src.rsb = make_desc(reinterpret_cast<const uint8_t*>(p.w2s) + (size_t)e * K * (I / 32),
                        (uint32_t)((size_t)K * (I / 32)));
    sb_off = (uint32_t)(ct * 256 + (wid * C::SB_ROWS + lane) % 256) * (I / 32);
    src.bsc = nullptr;
    src.bsc2 = nullptr;
  }
  f32x4 acc[MI][NI];
  // all NI subtiles of a wave are contiguous output columns (no gate/up split)
  tile_gemm<KIND, BM, 256, NS>(src, smem, IS, a_off, sa_off, sa_step, b_off, sb_off, NI,
                               e, acc);
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int id = ids[wm * 64 + mi * 16 + 4 * g + i4];
      if (id < 0) continue;
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) p.yr[(size_t)id * K + c0 + ni * 16 + r16] = acc[mi][ni][i4];
    }
}

template <int KIND, int BM>
hipError_t launch_tiled_kind(const MoeArgs& a, hipStream_t st, const TimingHook& hk) {
  constexpr int NS = BM == 256 ? 2 : 3;
  constexpr int TH = TileCfg<KIND, BM, 256, NS>::THREADS;
  const int S = a.I / 128;
  const unsigned g_up = (unsigned)(((size_t)a.blocks_cap * S + 7) / 8 * 8);
  const unsigned g_dn = (unsigned)(((size_t)a.blocks_cap * (a.K / 256) + 7) / 8 * 8);
  if (hk.which == 1 && hk.before) (void)hipEventRecord(hk.before, st);
  hipLaunchKernelGGL((k_up_t<KIND, BM, NS>), dim3(g_up), dim3(TH), 0, st, a);
  if (hk.which == 1 && hk.after) (void)hipEventRecord(hk.after, st);
  if (hk.which == 2 && hk.before) (void)hipEventRecord(hk.before, st);
  hipLaunchKernelGGL((k_down_t<KIND, BM, NS>), dim3(g_dn), dim3(TH), 0, st, a);
  if (hk.which == 2 && hk.after) (void)hipEventRecord(hk.after, st);
  return hipGetLastError();
}

}  // namespace

bool tiled_supported(int kind, int block_m, int K, int I) {
  return (kind == KIND_FP8B || kind == KIND_MX) &&
         (block_m == 64 || block_m == 128 || block_m == 256) && K % 256 == 0 && I % 128 == 0;
}

hipError_t launch_tiled(int kind, int block_m, const MoeArgs& a, hipStream_t st,
                        const TimingHook& hk) {
  if (kind == KIND_FP8B) {
    if (block_m == 256) return launch_tiled_kind<KIND_FP8B, 256>(a, st, hk);
    if (block_m == 128) return launch_tiled_kind<KIND_FP8B, 128>(a, st, hk);
    return launch_tiled_kind<KIND_FP8B, 64>(a, st, hk);
  }
  if (block_m == 256) return launch_tiled_kind<KIND_MX, 256>(a, st, hk);
  if (block_m == 128) return launch_tiled_kind<KIND_MX, 128>(a, st, hk);
  return launch_tiled_kind<KIND_MX, 64>(a, st, hk);
}
