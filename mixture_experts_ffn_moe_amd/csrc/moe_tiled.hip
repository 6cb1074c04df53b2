// moe_tiled.hip -- LDS-tiled split-mode kernels for many rows per expert
// (block_m 64, 128 and 256, e4m3 paths: blockwise FP8 and MXFP8).
//
// Same computation as k_up / k_down in moe_kernels.hip ([hpc-ops RFC]
// "Background" stages 2-4; [prime-flash] introduction, split=True), organized
// for the regime where each expert holds many rows, so that the MFMA pipes
// rather than the operand loads set the pace:
//
//  * A (activation rows) and B (weight rows) of one 128-wide K step are
//    staged in LDS with direct-to-LDS 16-byte buffer loads (no VGPR staging),
//    NS steps in flight.  Every wave then reads its MFMA fragments from LDS,
//    so each operand byte crosses the L2 -> CU path once per workgroup.  Only
//    some waves issue those loads (see TileCfg::LW).
//  * LDS rows are 128 bytes (8 chunks of 16 bytes); chunk q of row r is stored
//    at chunk q ^ (r & 7).  Measured on gfx950 with the fragment pattern (lane
//    (g, r) reading chunks g and 4 + g of row r of a 16-row group), this plain
//    xor reads at 216 B/clk/CU, lane-contiguous addresses at 191, and the xor
//    with an extra (r >> 3) & 1 term that spreads 16 rows over 16 bank groups
//    at 127 (its lanes g, r and g + 1, r + 8 meet in one bank group).  The
//    loads write LDS in lane order, so each lane fetches the logical chunk
//    that belongs in its slot.
//  * Workgroup tile: block_m rows x (128 gate + 128 up) for k_up_t,
//    block_m rows x 256 (or 128) output columns for k_down_t; a wave owns 64
//    rows, 4 waves at block_m 64, 8 (two per SIMD) from 128 on.
//  * Blockwise scales: the activation row scales of each step ride along in
//    LDS (4-byte direct loads); the weight block-scale rows of the tile are
//    loaded into LDS once.  MX: the e8m0 dwords of each row (4 K blocks per
//    step) ride along in LDS and feed the block-scaled MFMA.
//  * Workgroup ids are remapped so that consecutive tiles (the slices of one
//    block, then the next block of the same expert) land on one XCD and share
//    its L2; where eight consecutive blocks belong to one expert, the slices
//    run outermost over those blocks (tile_coords).
//  * With few tiles (64-row blocks), the gate/up GEMM splits K over four
//    workgroups per tile, reduced in a fixed order by the last one.
#include "device.h"
#include "launch.h"

namespace {

constexpr int kRowBytes = 128;  // one K step of e4m3
constexpr int kChunks = 8;      // 16-byte chunks per row
constexpr int kScaleRow = 128;  // K steps of a weight block-scale row in LDS (K, I <= 16384)

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

// Block b, column tile ct and expert e of logical tile `tile` (NT column
// tiles per block: gate/up slices or down output tiles; nb planner blocks
// hold routes).  Blocks go in aligned groups of kGroup.  A group whose
// blocks all belong to one expert (a heavily loaded expert under skewed
// routing) is walked column tile by column tile, its kGroup blocks inner, so
// the workgroups that run together on one XCD read a few weight slices and
// a few blocks' rows, both shared in its L2; block by block, every block
// re-read the expert's whole weights from beyond L2 (K=7168, I=3072, E=384,
// top-6, zipf, T=4096: 31 blocks of 128 rows on the busiest expert).  Other
// groups, and the last partial one, go block by block.  Either order is a
// permutation of the same tiles, so the result does not depend on it.
constexpr int kGroup = 8;
__device__ __forceinline__ void tile_coords(int tile, int NT, int nb, const int32_t* expert_ids,
                                            int& b, int& ct, int& e) {
  const int b0 = tile / (kGroup * NT) * kGroup;
  const int lane = threadIdx.x & 63;
  int eid = -1;  // lane j < kGroup: expert of block b0 + j (one load for the group)
  if (lane < kGroup && b0 + lane < nb) eid = expert_ids[b0 + lane];
  const int e_first = __builtin_amdgcn_readlane(eid, 0);
  const int e_last = __builtin_amdgcn_readlane(eid, kGroup - 1);
  if (b0 + kGroup <= nb && e_first == e_last) {
    const int r = tile - b0 * NT;
    ct = r / kGroup;
    b = b0 + r % kGroup;
    e = e_first;
  } else {
    b = tile / NT;
    ct = tile % NT;
    e = __builtin_amdgcn_readlane(eid, b - b0);
  }
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
  // Waves that issue the tile's DMA loads (waves 0 .. LW-1).  With two
  // waves per SIMD only the first wave of each SIMD loads (twice the
  // instructions), so the other never holds its MFMAs behind a queue of
  // vector-memory issues (K=4096, I=2048, E=288, top-8, T=8192, 256-row
  // tiles: gate/up GEMM 1.54 -> 1.43 ms).  With one wave per SIMD (64-row
  // tiles), blockwise FP8 loads from two SIMDs and leaves the other two to
  // compute (K=7168, I=3072, E=384, top-6, zipf, T=256: 941 -> 909 us per
  // call); MX keeps four, as its weight scales then need one instruction
  // per 64 rows.
  static constexpr int LW = NW == 8 ? 4 : (KIND == KIND_MX ? NW : 2);
  static constexpr int A_BYTES = BM * kRowBytes;
  static constexpr int B_BYTES = BN * kRowBytes;
  // Row scales (fp32, or 4 x e8m0 per row): each loading wave stages
  // SA_ROWS rows in 64 four-byte slots (every lane loads; the slots past
  // SA_ROWS are padding).
  static constexpr int SA_BYTES = LW * 256;
  static constexpr int SB_BYTES = (KIND == KIND_MX) ? LW * 256 : 0;  // MX weight scales
  static constexpr int STAGE = A_BYTES + B_BYTES + SA_BYTES + SB_BYTES;
  static constexpr int A_INSTR = A_BYTES / 1024 / LW;  // 16-byte DMA instructions per loading wave
  static constexpr int B_INSTR = B_BYTES / 1024 / LW;
  static constexpr int SA_ROWS = BM / LW;              // scale rows staged per loading wave
  static constexpr int SB_ROWS = BN / LW;
  static constexpr int S_INSTR = 1 + ((KIND == KIND_MX) ? 1 : 0);
  static constexpr int LOADS = A_INSTR + B_INSTR + S_INSTR;  // per loading wave per stage
  static constexpr int THREADS = NW * 64;
  static_assert(SA_ROWS <= 64 && (KIND != KIND_MX || SB_ROWS <= 64), "one scale instruction per wave");
};

// Operand sources of one tile GEMM.
struct TileSrc {
  desc_t ra, rb, rsa, rsb;
  // FP8B: block-scale rows (index: step) of the tile's two 128-row weight
  // blocks: k_up_t's gate and up slices, k_down_t's two column blocks
  const float* bsc;
  const float* bsc2;
};

// Issue the DMA loads of K step `ks` into stage slot `st` of the pipeline
// area at LDS address `lds` (a wave-uniform byte address).
//  a_off[t] + a_soff[t]: this lane's byte offset of its A chunk (t-th load),
//                       a lane part and a wave-uniform part (zero where the
//                       rows are gathered)
//  b_off + b_soff[t]  : the same for B, a lane offset plus a wave-uniform
//                       offset per load (the weight rows of one tile are
//                       contiguous, so only the lane part varies)
//  sa_off / sb_off    : this lane's scale row offsets; sa_step bytes per step
// PART 0 issues the whole stage; 1 only the weight side (B and its MX
// scales), 2 only the activation side (A and its row scales), so that a
// tile can request its first weights before it knows its activation rows.
template <int KIND, int BM, int BN, int NS, int PART = 0>
__device__ __forceinline__ void tile_load(const TileSrc& src, uint32_t lds, int st, int ks,
                                          const uint32_t (&a_off)[TileCfg<KIND, BM, BN, NS>::A_INSTR],
                                          const uint32_t (&a_soff)[TileCfg<KIND, BM, BN, NS>::A_INSTR],
                                          uint32_t sa_off, uint32_t sa_step, uint32_t b_off,
                                          const uint32_t (&b_soff)[TileCfg<KIND, BM, BN, NS>::B_INSTR],
                                          uint32_t sb_off) {
  using C = TileCfg<KIND, BM, BN, NS>;
  const uint32_t w = (uint32_t)wave_id();
  if (w >= (uint32_t)C::LW) return;
  const uint32_t stage = lds + (uint32_t)(st * C::STAGE);
  const uint32_t soff = (uint32_t)ks * kRowBytes;
  if constexpr (PART != 1) {
#pragma unroll
    for (int t = 0; t < C::A_INSTR; ++t)
      dma16(src.ra, stage + (w + C::LW * t) * 1024, a_off[t], soff + a_soff[t]);
  }
  if constexpr (PART != 2) {
#pragma unroll
    for (int t = 0; t < C::B_INSTR; ++t)
      dma16(src.rb, stage + C::A_BYTES + (w + C::LW * t) * 1024, b_off, soff + b_soff[t]);
  }
  // row scales: wave w stages rows [w * SA_ROWS, (w + 1) * SA_ROWS) in its 64
  // slots.  All lanes load (lanes past SA_ROWS fill padding from an in-bounds
  // row): a lane-dependent branch around the asm would put its scalar
  // operands in vector registers.
  if constexpr (PART != 1)
    dma4(src.rsa, stage + C::A_BYTES + C::B_BYTES + w * 256, sa_off, (uint32_t)ks * sa_step);
  if constexpr (KIND == KIND_MX && PART != 2)
    dma4(src.rsb, stage + C::A_BYTES + C::B_BYTES + C::SA_BYTES + w * 256, sb_off, (uint32_t)ks * 4);
}

// Per-lane DMA offsets of the A and B tiles, LW loading waves: lane slot
// (w + LW t) * 64 + lane holds row slot / 8, physical chunk slot % 8, which
// carries logical chunk (slot % 8) ^ swz(row).
template <int LW>
__device__ __forceinline__ void dma_rows(int t_idx, int& row, int& qchunk) {
  const int lane = threadIdx.x & 63, w = wave_id();
  const int slot = (w + LW * t_idx) * 64 + lane;
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

// Compute one staged K step (stage at `stage`, logical step ks).  wsc: the
// blockwise weight scales of the tile's two 128-row weight blocks in LDS,
// step ks of the first at wsc[ks], of the second at wsc[kScaleRow + ks].
template <int KIND, int BM, int BN, int NS, bool B_NEXT>
__device__ __forceinline__ void tile_step(const uint8_t* stage, int ks, const float* wsc,
                                          int up_split,
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
    const float s1 = wsc[ks];
    const float s2 = wsc[kScaleRow + ks];
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
    if constexpr (C::NW == 8 && B_NEXT) {
      // two waves share each SIMD and fill each other's MFMA gaps; column
      // ni + 1's B fragment is read while column ni's MFMAs run (K=4096,
      // I=2048, E=288, top-8, T=8192, 256-row tiles: gate/up GEMM 1.70 ->
      // 1.58 ms, down GEMM 0.96 -> 0.86 ms)
      Frag<KIND_FP8B> fb2[2];
      lds_frag(fb2[0], tb, brow_of(0), g);
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        if (ni + 1 < NI) lds_frag(fb2[(ni + 1) & 1], tb, brow_of(ni + 1), g);
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
          const f32x4 z = {0.f, 0.f, 0.f, 0.f};
          t[0][mi] = mfma_step<KIND_FP8B>(fa[mi], fb2[ni & 1], z);
        }
        promote(ni, t[0]);
      }
    } else if constexpr (C::NW == 8) {
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

// One workgroup tile: acc[mi][ni] over the K steps [k0, k0 + ksteps),
// visiting them from a staggered start, NS stages in flight (stage slots in
// one LDS array).  kscale: K steps of the weight block-scale rows staged.
// The tile's first requests go out before anything waits: the blockwise
// weight-scale rows of the tile's two 128-row weight blocks (src.bsc and
// src.bsc2, into `wsc`, 2 x kScaleRow floats of LDS; the wave reads them
// from row wsc_row on) and the weight side of the first stage; then `activation_offsets()` runs (it may wait
// for the tile's rows and fill a_off / sa_off, which are read only after
// it), then the activation side of the first stage and the other stages.
// Every load is a direct-to-LDS load issued from asm, so the K loop's
// explicit waits are the only ones.
template <int KIND, int BM, int BN, int NS, bool B_NEXT, typename F>
__device__ __forceinline__ void tile_gemm(const TileSrc& src, uint8_t* smem, float* wsc, int wsc_row,
                                          int ksteps, int k0, int kscale,
                                          const uint32_t (&a_off)[TileCfg<KIND, BM, BN, NS>::A_INSTR],
                                          const uint32_t (&a_soff)[TileCfg<KIND, BM, BN, NS>::A_INSTR],
                                          const uint32_t& sa_off, uint32_t sa_step, uint32_t b_off,
                                          const uint32_t (&b_soff)[TileCfg<KIND, BM, BN, NS>::B_INSTR],
                                          uint32_t sb_off, int up_split, int group,
                                          F&& activation_offsets, const bool& live,
                                          f32x4 (&acc)[4][TileCfg<KIND, BM, BN, NS>::NI]) {
  using C = TileCfg<KIND, BM, BN, NS>;
  constexpr int MI = C::MI, NI = C::NI;
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (KIND == KIND_FP8B) {
    // each row: lanes load steps lane and 64 + lane (past ksteps the
    // descriptor's bound returns zeros)
    const int lane = threadIdx.x & 63;
    const uint32_t m0 = lds_addr(wsc);
    const uint32_t bytes = (uint32_t)kscale * 4;
    const desc_t r1 = make_desc(src.bsc, bytes);
    const desc_t r2 = make_desc(src.bsc2 ? src.bsc2 : src.bsc, bytes);
    dma4(r1, m0, lane * 4, 0);
    dma4(r1, m0 + 256, 256 + lane * 4, 0);
    dma4(r2, m0 + kScaleRow * 4, lane * 4, 0);
    dma4(r2, m0 + kScaleRow * 4 + 256, 256 + lane * 4, 0);
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
  auto step_at = [&](int i) { const int k = i + rot; return k0 + (k >= ksteps ? k - ksteps : k); };
  const uint32_t lbase = lds_addr(smem);
  auto load = [&](int slot, int i) {
    tile_load<KIND, BM, BN, NS>(src, lbase, slot, step_at(i), a_off, a_soff, sa_off, sa_step, b_off, b_soff,
                                sb_off);
  };
  // stage 0 in two parts around the activation offsets (the wait counts
  // below count whole stages issued after the one awaited: unchanged)
  tile_load<KIND, BM, BN, NS, 1>(src, lbase, 0, step_at(0), a_off, a_soff, sa_off, sa_step, b_off, b_soff,
                                 sb_off);
  activation_offsets();
  tile_load<KIND, BM, BN, NS, 2>(src, lbase, 0, step_at(0), a_off, a_soff, sa_off, sa_step, b_off, b_soff,
                                 sb_off);
#pragma unroll
  for (int u = 1; u < NS - 1; ++u)
    if (u < ksteps) load(u, u);
  const float* wsc_r = wsc + wsc_row * kScaleRow;
  int slot = 0;
  for (int i = 0; i < ksteps; ++i) {
    // step i has landed once only the later steps' loads may be pending
    if (i + NS - 2 < ksteps) wait_vmcnt<C::LOADS * (NS - 2)>();
    else wait_vmcnt<0>();
    lds_barrier();
    const int ahead = slot + NS - 1;
    if (i + NS - 1 < ksteps) load(ahead >= NS ? ahead - NS : ahead, i + NS - 1);
    // blockwise: a wave whose 64 rows are all padding keeps its share of the
    // loads and barriers but computes nothing (its sums stay zero; padding
    // rows are never stored as results).  MX accumulates in place in the
    // MFMA, and a branch around it costs the 256-row tiles register spills.
    if (KIND != KIND_FP8B || live)
      tile_step<KIND, BM, BN, NS, B_NEXT>(smem + slot * C::STAGE, step_at(i), wsc_r, up_split, acc);
    slot = slot + 1 == NS ? 0 : slot + 1;
  }
  __syncthreads();  // the caller reuses the LDS
}


// gate/up GEMM + SwiGLU + requantization, one (block, 128-wide slice) tile.
// KW > 1 (64-row tiles, few tiles): KW workgroups per tile, workgroup kw
// summing the K steps [kw KS/KW, (kw+1) KS/KW).  Each stores its raw sums in
// the workspace with device-scope stores and takes a ticket; the last of the
// tile's workgroups adds the KW sums in the order kw = 0, 1, .. (the result
// does not depend on which one is last) and runs the epilogue.
template <int KIND, int BM, int NS, int KW>
__global__ void __launch_bounds__(BM >= 128 ? 512 : 256) __attribute__((amdgpu_waves_per_eu(1, BM >= 128 ? 2 : 1))) k_up_t(MoeArgs p) {
  using C = TileCfg<KIND, BM, 256, NS>;
  constexpr int MI = C::MI, NI = C::NI, HALF = NI / 2;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * C::STAGE];
  __shared__ int ids[C::NW * 64];  // route id of row r at scale_slot<SA_ROWS>(r)
  __shared__ float lds_amax[C::WN * BM];
  __shared__ float wsc[2 * kScaleRow];
  const int S = p.I / 128;
  // the KW workgroups of a tile are consecutive, on one XCD
  const int nb = *p.ntp / BM;
  const int logical = xcd_remap(blockIdx.x, nb * S * KW);
  if (logical < 0) return;
  const int tile = logical / KW, kw = logical % KW;
  int b, s, e;  // e uniform: descriptors in SGPRs
  tile_coords(tile, S, nb, p.expert_ids, b, s, e);
  if (b >= p.blocks_cap) return;
  if ((unsigned)e >= (unsigned)p.E) return;
  const int lane = threadIdx.x & 63, wid = wave_id();
  const int wn = wid % C::WN, wm = wid / C::WN;
  const int g = lane >> 4, r16 = lane & 15;
  const int srow = wid * C::SA_ROWS + lane;  // row whose id and scales this lane stages
  // the block's route ids, into LDS with the wave's scale-row layout; the
  // weight loads go out before anything waits for them
  dma4(make_desc(p.sorted, (uint32_t)((size_t)p.blocks_cap * BM * 4)), lds_addr(ids) + wid * 256,
       (uint32_t)(b * BM + (srow < BM ? srow : 0)) * 4, 0);
  auto id_of = [&](int r) { return ids[scale_slot<C::SA_ROWS>(r)]; };
  const int K = p.K, I = p.I, N = 2 * I, KS = K / 128;

  TileSrc src;
  src.ra = make_desc(p.x, (uint32_t)((size_t)p.T * K));
  src.rb = make_desc(p.w1 + (size_t)e * N * K, (uint32_t)((size_t)N * K));
  uint32_t a_off[C::A_INSTR], a_soff[C::A_INSTR], b_soff[C::B_INSTR];
#pragma unroll
  for (int t = 0; t < C::A_INSTR; ++t) a_soff[t] = 0;  // gathered rows: all in a_off
  // B rows [0,128): the gate slice's weight rows; [128,256): the up slice's.
  // Load t's rows are load 0's plus LW * 8 * t, all on one side of 128.
  int brow0, bq;
  dma_rows<C::LW>(0, brow0, bq);
  const uint32_t b_off = (uint32_t)(s * 128 + brow0) * K + bq * 16;
#pragma unroll
  for (int t = 0; t < C::B_INSTR; ++t) {
    const int d = C::LW * 8 * t;
    b_soff[t] = (uint32_t)(d < 128 ? d : I - 128 + d) * K;
  }
  uint32_t sa_off = 0, sa_step = 4, sb_off = 0;
  const uint32_t sa_row = KIND == KIND_FP8B ? KS * 4 : K / 32;  // bytes per activation scale row
  if constexpr (KIND == KIND_FP8B) {
    src.rsa = make_desc(p.xs, (uint32_t)((size_t)p.T * KS * 4));
    src.bsc = reinterpret_cast<const float*>(p.w1s) + ((size_t)e * (N / 128) + s) * KS;
    src.bsc2 = reinterpret_cast<const float*>(p.w1s) + ((size_t)e * (N / 128) + S + s) * KS;
  } else {
    src.rsa = make_desc(p.xs, (uint32_t)((size_t)p.T * (K / 32)));
    src.rsb = make_desc(reinterpret_cast<const uint8_t*>(p.w1s) + (size_t)e * N * (K / 32),
                        (uint32_t)((size_t)N * (K / 32)));
    const int brow = min(wid * C::SB_ROWS + lane, 255);  // B scale row this lane stages
    const int n = (brow < 128 ? s * 128 + brow : I + s * 128 + brow - 128);
    sb_off = (uint32_t)n * (K / 32);
    src.bsc = nullptr;
    src.bsc2 = nullptr;
  }
  // the gathered activation rows, once the route ids have arrived: issued
  // after them, the weight-scale rows (blockwise: 4 loads) and, in a
  // loading wave, the weight side of the first stage (B, and the MX weight
  // scales) may be pending
  bool live = true;  // this wave's rows hold a route (set once the route ids have arrived)
  auto activation_offsets = [&]() {
    if (wid < C::LW) wait_vmcnt<(KIND == KIND_FP8B ? 4 : 0) + C::B_INSTR + (KIND == KIND_MX ? 1 : 0)>();
    else wait_vmcnt<(KIND == KIND_FP8B ? 4 : 0)>();
    lds_barrier();
    live = __ballot(id_of(wm * 64 + lane) >= 0) != 0;
#pragma unroll
    for (int t = 0; t < C::A_INSTR; ++t) {
      int row, q;
      dma_rows<C::LW>(t, row, q);
      a_off[t] = (uint32_t)route_token(p, id_of(row)) * K + q * 16;
    }
    sa_off = (uint32_t)route_token(p, id_of(srow < BM ? srow : 0)) * sa_row;
  };
  f32x4 acc[MI][NI];
  tile_gemm<KIND, BM, 256, NS, true>(src, smem, wsc, 0, KS / KW, kw * (KS / KW), KS, a_off, a_soff,
                                     sa_off, sa_step, b_off, b_soff, sb_off, HALF, e,
                                     activation_offsets, live, acc);
  if constexpr (KW > 1) {
    constexpr int PER = MI * NI * 4;  // floats per lane
    __shared__ int last;
    float* const pt = p.part + (size_t)tile * KW * (C::THREADS * PER);
    float* const dst = pt + ((size_t)kw * C::NW + wid) * PER * 64 + lane;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          __hip_atomic_store(dst + ((mi * NI + ni) * 4 + i) * 64, acc[mi][ni][i], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    // the sums have been acknowledged device-wide before the ticket moves
    asm volatile("" ::: "memory");
    wait_vmcnt<0>();
    asm volatile("" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) last = atomicAdd(p.tickets + tile, 1) == KW - 1;
    __syncthreads();
    if (!last) return;
    const float* const src_p = pt + (size_t)wid * PER * 64 + lane;
#pragma unroll
    for (int q = 0; q < KW; ++q)
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float v = __hip_atomic_load(src_p + (size_t)q * C::NW * PER * 64 + ((mi * NI + ni) * 4 + i) * 64,
                                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            acc[mi][ni][i] = q == 0 ? v : acc[mi][ni][i] + v;
          }
  }

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
          q[row * QROW + wn * HALF * 16 + j * 16 + r16] = (uint8_t)f32_to_e4m3_in_range(h[mi][j][i4] * inv);
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
    const int id = id_of(threadIdx.x);
    if (id >= 0) p.flags[id] = 1;
  }
}

// down GEMM, one (block, BN output columns) tile, bf16 per-route rows.
// BN = 128 for short K walks at 64-row tiles (two workgroups then share a
// CU; see the launcher), 256 otherwise.
template <int KIND, int BM, int NS, int BN>
__global__ void __launch_bounds__(BM >= 128 ? 512 : 256)
__attribute__((amdgpu_waves_per_eu(1, BM >= 128 || BN == 128 ? 2 : 1))) k_down_t(MoeArgs p) {
  using C = TileCfg<KIND, BM, BN, NS>;
  constexpr int MI = C::MI, NI = C::NI;
  constexpr int YROW = BN * 2 + 16;  // bytes per staged bf16 output row (epilogue)
  constexpr int SMEM = NS * C::STAGE > BM * YROW ? NS * C::STAGE : BM * YROW;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM];
  __shared__ int ids[C::NW * 64];  // route id of row r at scale_slot<SA_ROWS>(r)
  __shared__ float wsc[2 * kScaleRow];
  const int K = p.K, I = p.I, IS = I / 128;
  const int NT = K / BN;
  const int nb = *p.ntp / BM;
  const int logical = xcd_remap(blockIdx.x, nb * NT);
  if (logical < 0) return;
  int b, ct, e;  // e uniform: descriptors in SGPRs
  tile_coords(logical, NT, nb, p.expert_ids, b, ct, e);
  if (b >= p.blocks_cap) return;
  if ((unsigned)e >= (unsigned)p.E) return;
  const int lane = threadIdx.x & 63, wid = wave_id();
  const int wn = wid % C::WN, wm = wid / C::WN;
  const int g = lane >> 4, r16 = lane & 15;
  const int srow = wid * C::SA_ROWS + lane;  // row whose id and scales this lane stages
  // the block's route ids are needed only to store the result: loaded into
  // LDS ahead of the K walk, whose last wait covers them
  dma4(make_desc(p.sorted, (uint32_t)((size_t)p.blocks_cap * BM * 4)), lds_addr(ids) + wid * 256,
       (uint32_t)(b * BM + (srow < BM ? srow : 0)) * 4, 0);
  const size_t rows_cap = (size_t)p.blocks_cap * BM;
  TileSrc src;
  src.ra = make_desc(p.hq, (uint32_t)(rows_cap * I));
  src.rb = make_desc(p.w2 + (size_t)e * K * I, (uint32_t)((size_t)K * I));
  // the block's H rows are contiguous: load t's rows are load 0's plus
  // LW * 8 * t, a wave-uniform offset, as for the weight rows
  uint32_t a_off[C::A_INSTR], a_soff[C::A_INSTR], b_soff[C::B_INSTR];
  int arow0, aq;
  dma_rows<C::LW>(0, arow0, aq);
  const uint32_t a_off0 = (uint32_t)((size_t)b * BM + arow0) * I + aq * 16;
#pragma unroll
  for (int t = 0; t < C::A_INSTR; ++t) {
    a_off[t] = a_off0;
    a_soff[t] = (uint32_t)(C::LW * 8 * t) * I;
  }
  int brow0, bq;
  dma_rows<C::LW>(0, brow0, bq);
  const uint32_t b_off = (uint32_t)(ct * BN + brow0) * I + bq * 16;
#pragma unroll
  for (int t = 0; t < C::B_INSTR; ++t) b_soff[t] = (uint32_t)(C::LW * 8 * t) * I;
  uint32_t sa_off = 0, sa_step = 4, sb_off = 0;
  const int c0 = ct * BN + wn * (BN / C::WN);  // this wave's first output column
  if constexpr (KIND == KIND_FP8B) {
    src.rsa = make_desc(p.hs, (uint32_t)(rows_cap * IS * 4));
    sa_off = (uint32_t)((size_t)b * BM + (srow < BM ? srow : 0)) * IS * 4;
    // the tile's 128-column weight blocks (two at BN = 256); the wave's is c0 / 128
    src.bsc = reinterpret_cast<const float*>(p.w2s) + ((size_t)e * (K / 128) + (BN / 128) * ct) * IS;
    src.bsc2 = BN == 256 ? src.bsc + IS : src.bsc;
  } else {
    src.rsa = make_desc(p.hs, (uint32_t)(rows_cap * (I / 32)));
    sa_off = (uint32_t)((size_t)b * BM + (srow < BM ? srow : 0)) * (I / 32);
    src.rsb = make_desc(reinterpret_cast<const uint8_t*>(p.w2s) + (size_t)e * K * (I / 32),
                        (uint32_t)((size_t)K * (I / 32)));
    sb_off = (uint32_t)(ct * BN + (wid * C::SB_ROWS + lane) % BN) * (I / 32);
    src.bsc = nullptr;
    src.bsc2 = nullptr;
  }
  f32x4 acc[MI][NI];
  // all NI subtiles of a wave are contiguous output columns (no gate/up split)
  // once the route ids have arrived (issued first; the weight-scale rows,
  // blockwise, and in a loading wave the weight side of the first stage may
  // be pending): does this wave's row range hold a route
  bool live = true;
  auto rows_live = [&]() {
    if (wid < C::LW) wait_vmcnt<(KIND == KIND_FP8B ? 4 : 0) + C::B_INSTR + (KIND == KIND_MX ? 1 : 0)>();
    else wait_vmcnt<(KIND == KIND_FP8B ? 4 : 0)>();
    lds_barrier();
    live = __ballot(ids[scale_slot<C::SA_ROWS>(wm * 64 + lane)] >= 0) != 0;
  };
  tile_gemm<KIND, BM, BN, NS, true>(src, smem, wsc, c0 / 128 - (BN / 128) * ct, IS, 0, IS, a_off, a_soff, sa_off, sa_step,
                                     b_off, b_soff, sb_off, NI, e, rows_live, live, acc);
  // the tile's rows rounded to bf16, staged in LDS (rows of 2 BN bytes plus
  // 16 bytes of padding), then written out as whole 2 BN-byte row pieces with
  // non-temporal stores: the combine reads them once, much later, so they
  // need not displace the weight stream in L2 (K=4096, I=2048, E=288,
  // top-8: 1-2% of this kernel at T = 4096 and 8192)
  const int cw = wn * (BN / C::WN);  // this wave's first column within the tile
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      uint16_t* yrow = reinterpret_cast<uint16_t*>(smem + (wm * 64 + mi * 16 + 4 * g + i4) * YROW);
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) yrow[cw + ni * 16 + r16] = f32_to_bf16(acc[mi][ni][i4]);
    }
  __syncthreads();
  for (int c = threadIdx.x; c < BM * (BN / 8); c += C::THREADS) {
    const int row = c / (BN / 8), ch = c % (BN / 8);
    const int id = ids[scale_slot<C::SA_ROWS>(row)];
    if (id < 0) continue;
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(smem + row * YROW + ch * 16),
                                reinterpret_cast<u32x4*>(p.yr + (size_t)id * K + ct * BN + ch * 8));
  }
}

template <int KIND, int BM, int NS, int BN>
void launch_down_bn(const MoeArgs& a, hipStream_t st) {
  constexpr int TH = TileCfg<KIND, BM, BN, NS>::THREADS;
  const unsigned g_dn = (unsigned)(((size_t)a.blocks_cap * (a.K / BN) + 7) / 8 * 8);
  hipLaunchKernelGGL((k_down_t<KIND, BM, NS, BN>), dim3(g_dn), dim3(TH), 0, st, a);
}

// Output columns per down-GEMM tile: 256, or 128 at 64-row tiles whose K
// walk is short (I <= 512).  There the tile's fixed costs (first loads,
// epilogue) outweigh its four steps, and 128 columns bring its LDS to 77 KiB
// in three stages, so two workgroups share a CU and overlap them (MXFP8,
// K=4096, I=256, E=32, top-8: down GEMM 18.2 -> 14.5 us at T=128, 35.3 ->
// 25.8 us at T=512).  Over longer walks the halved tile reads its
// activation rows twice as often (blockwise FP8, I=2048: 454 against 478 us
// at T=1024).
template <int KIND, int BM, int NS>
void launch_down_t(const MoeArgs& a, hipStream_t st) {
  if constexpr (BM == 64) {
    if (a.I <= 512) return launch_down_bn<KIND, BM, NS, 128>(a, st);
  }
  launch_down_bn<KIND, BM, NS, 256>(a, st);
}

template <int KIND, int BM, int NS>
hipError_t launch_tiled_ns(const MoeArgs& a, hipStream_t st, const TimingHook& hk) {
  constexpr int TH = TileCfg<KIND, BM, 256, NS>::THREADS;
  const int S = a.I / 128;
  const int kw = a.kw > 1 ? a.kw : 1;
  if (kw != 1 && (BM != 64 || kw != 4)) return hipErrorInvalidValue;
  const unsigned g_up = (unsigned)(((size_t)a.blocks_cap * S * kw + 7) / 8 * 8);
  if (hk.which == 1 && hk.before) (void)hipEventRecord(hk.before, st);
  if constexpr (BM == 64) {
    if (kw == 4) hipLaunchKernelGGL((k_up_t<KIND, BM, NS, 4>), dim3(g_up), dim3(TH), 0, st, a);
    else hipLaunchKernelGGL((k_up_t<KIND, BM, NS, 1>), dim3(g_up), dim3(TH), 0, st, a);
  } else {
    hipLaunchKernelGGL((k_up_t<KIND, BM, NS, 1>), dim3(g_up), dim3(TH), 0, st, a);
  }
  if (hk.which == 1 && hk.after) (void)hipEventRecord(hk.after, st);
  if (hk.which == 2 && hk.before) (void)hipEventRecord(hk.before, st);
  launch_down_t<KIND, BM, NS>(a, st);
  if (hk.which == 2 && hk.after) (void)hipEventRecord(hk.after, st);
  return hipGetLastError();
}

template <int KIND, int BM>
hipError_t launch_tiled_down_kind(const MoeArgs& a, hipStream_t st) {
  launch_down_t<KIND, BM, BM == 256 ? 2 : 3>(a, st);
  return hipGetLastError();
}

// Stages: two for 256-row tiles (the LDS holds no third), three otherwise,
// or the caller's two for 64- and 128-row tiles.
template <int KIND, int BM>
hipError_t launch_tiled_kind(const MoeArgs& a, hipStream_t st, const TimingHook& hk) {
  if constexpr (BM == 256) {
    return launch_tiled_ns<KIND, BM, 2>(a, st, hk);
  } else {
    if (a.stages == 2) return launch_tiled_ns<KIND, BM, 2>(a, st, hk);
    return launch_tiled_ns<KIND, BM, 3>(a, st, hk);
  }
}

}  // namespace

bool tiled_supported(int kind, int block_m, int K, int I) {
  return (kind == KIND_FP8B || kind == KIND_MX) &&
         (block_m == 64 || block_m == 128 || block_m == 256) && K % 256 == 0 && I % 128 == 0;
}

hipError_t launch_tiled_down(int kind, int block_m, const MoeArgs& a, hipStream_t st) {
  if (kind == KIND_FP8B) {
    if (block_m == 256) return launch_tiled_down_kind<KIND_FP8B, 256>(a, st);
    if (block_m == 128) return launch_tiled_down_kind<KIND_FP8B, 128>(a, st);
    return launch_tiled_down_kind<KIND_FP8B, 64>(a, st);
  }
  if (block_m == 256) return launch_tiled_down_kind<KIND_MX, 256>(a, st);
  if (block_m == 128) return launch_tiled_down_kind<KIND_MX, 128>(a, st);
  return launch_tiled_down_kind<KIND_MX, 64>(a, st);
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
