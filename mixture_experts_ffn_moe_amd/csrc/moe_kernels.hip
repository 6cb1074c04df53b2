// moe_kernels.hip -- expert FFN kernels for gfx950 (bf16, blockwise FP8, MXFP8).
//
// Stages ([hpc-ops RFC] "Background": gather, gate/up GroupGEMM, SiLU * gate
// with FP8 requantization, down GroupGEMM, top-k weighted reduction):
//
//   split mode ([prime-flash] introduction, split=True):
//     k_zero     clear the per-route "placed" flags
//     k_up       per (block_m rows of one expert, 128-wide slice of I):
//                gather x rows, gate/up GEMM on MFMA, SwiGLU, requantize,
//                write the intermediate slice (+ scales) to the workspace
//     k_down     per (block_m rows, 256 output columns): intermediate . w2^T
//                over all of I (no split-K), per-route result rows in bf16
//                (the pages' combine buffer)
//     k_combine  out[t] = bf16(sum_j w[t,j] * y[t,j]) in route order, in
//                fp32 (deterministic)
//   fused mode ([prime-flash] introduction, split=False):
//     k_zero     clear the fp32 (T, K) accumulator
//     k_fused    per (block_m rows, 128-wide slice of I): k_up's work with
//                the requantized slice kept in LDS, then the slice's
//                partial down GEMM over all K output columns, weighted by
//                the route weight and added into the accumulator (fp32
//                atomics: split-K over I)
//     k_finalize accumulator -> bf16 out
//
// Blockwise FP8 promotion: each 128-wide K step is one MFMA into a zeroed
// tile, then acc += tile * (row scale * weight block scale) in fp32 (one
// scale group and one rescale per step).  MX: the e8m0 scales go straight
// into the block-scaled MFMA.  bf16: plain MFMA accumulation.
//
// Waves: a workgroup has 4 waves per 64 rows (256 threads for block_m <= 64,
// 512 for block_m = 128).  Wave (wm, wn) owns rows [64*wm, 64*wm+64) of the
// block and, in the up GEMM, gate and up columns [32*wn, 32*wn+32) of the
// slice, so SwiGLU pairs gate and up inside one wave's accumulators.
#include "device.h"
#include "launch.h"

namespace {

constexpr int kSlice = 128;  // width of an I slice (= blockwise scale group)
constexpr int kCombineCols = 2048;  // output columns per combine workgroup (8 per thread)

// Operands of a wave's GEMM: A rows (l % 16 of each 16-row subtile) and B
// rows (l % 16 of each 16-column subtile) as buffer resources plus per-lane
// 32-bit byte offsets (row offset + 16 * lane group); the K step's offset is
// the wave-uniform soffset.
template <int MI, int NI>
struct Operand {
  __amdgpu_buffer_rsrc_t ra, rb;
  uint32_t a[MI], b[NI];
  // FP8B: fp32 scale of each of the lane's C rows (byte offsets, step stride
  // 4 bytes); the weight block-scale rows (at most two distinct 128-column
  // blocks per wave) and which of them each n-subtile uses
  __amdgpu_buffer_rsrc_t rsa;
  uint32_t as[MI][4];
  const float* bsrow[2];
  int bsel[NI];
  // MX: e8m0 rows of the lane's A row and B row, 4 bytes (one per 32-wide
  // block) per step; the same buffers as descriptors for direct-to-LDS loads
  __amdgpu_buffer_rsrc_t rxa, rxb;
  uint32_t ax[MI], bx[NI];
  desc_t dxa, dxb;
};

// MX scales staged in LDS.  Each wave copies, before its K walk, the e8m0
// bytes of its K range for every row it multiplies (NI*16 weight rows, then
// MI*16 activation rows) into a private LDS region, with direct-to-LDS loads
// that move whole 128-byte lines; a scale run (4 steps, 16 bytes of a row) is
// then one LDS read.  Fetched from memory instead, every run is a load that
// touches 16 rows' lines for 16 bytes each, which measured at 14% of the
// MXFP4 up GEMM.  Rows are `4 * ksteps` bytes, in 16-byte chunks; chunk q of
// row i sits in slot (q + (i % 16)) mod (chunks per row), so a run's 16 rows
// fall on different banks.
constexpr int kStageMax = 65536;  // dynamic LDS per workgroup for the regions

// Bytes of one wave's region for a K walk of `ksteps` steps (0: not staged,
// the runs come from memory).  Staging needs whole runs (ksteps % 4 == 0).
__host__ __device__ constexpr int stage_bytes(int ksteps, int mi, int waves) {
  const int cpr = ksteps / 4;
  const int bytes = 4 * 16 * cpr * 16 + (mi * 16 * cpr + 63) / 64 * 1024;
  return (ksteps % 4 == 0 && ksteps > 0 && bytes * waves <= kStageMax) ? bytes : 0;
}

struct Stage {
  const uint8_t* lds;  // the wave's region
  int rbs;             // bytes per row (4 per step)
  int cpr;             // 16-byte chunks per row
  int rm;              // this lane's slot rotation, (l % 16) % cpr
  int a_off;           // offset of the activation rows in the region
  uint32_t lane_row;   // (l % 16) * rbs
};

// MX scales travel in runs: one Q-dword load brings Q consecutive K steps of a
// row's e8m0 bytes, where Q (4, 2 or 1) divides the ring depth.  One byte per
// lane per step would cost a load instruction per operand row and step, each
// touching 16 rows' cache lines, and those requests (not bytes) measured as
// the streaming kernels' limit.
template <int D>
constexpr int scale_run() { return D % 4 == 0 ? 4 : D % 2 == 0 ? 2 : 1; }

template <int KIND, int MI, int NI, int D>
struct Ring {
  static constexpr int Q = scale_run<D>();
  Frag<KIND> fa[D][MI];
  FragB<KIND> fb[D][NI];
  float sa[D][MI][4];
  // MX: the rows' scale runs in flight, and the lane's byte of each step of
  // the run being computed (copied out when the run starts, so that its slot
  // can be refilled at once)
  uint32_t qa[D / Q][MI][Q];
  uint32_t qb[D / Q][NI][Q];
  int xa[MI][Q];
  int xb[NI][Q];
};

template <int Q, int CP = 0>
__device__ __forceinline__ void load_run(uint32_t (&q)[Q], __amdgpu_buffer_rsrc_t r, uint32_t voff,
                                         uint32_t soff) {
  if constexpr (Q == 4) {
    const uint4 v = buf_load16<CP>(r, voff, soff);
    q[0] = v.x, q[1] = v.y, q[2] = v.z, q[3] = v.w;
  } else if constexpr (Q == 2) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, CP);
    q[0] = v[0], q[1] = v[1];
  } else {
    q[0] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, CP);
  }
}

// MX scale run of the walk's steps [4q, 4q + 4) from the staged rows
template <int KIND, int MI, int NI, int D>
__device__ __forceinline__ void stage_read(Ring<KIND, MI, NI, D>& r, int slot, int q,
                                           const Stage& st) {
  int sl = q + st.rm;
  sl = sl >= st.cpr ? sl - st.cpr : sl;
  const uint8_t* base = st.lds + st.lane_row + 16 * sl;
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
    const uint4 v = *reinterpret_cast<const uint4*>(base + ni * 16 * st.rbs);
    r.qb[slot / 4][ni][0] = v.x, r.qb[slot / 4][ni][1] = v.y;
    r.qb[slot / 4][ni][2] = v.z, r.qb[slot / 4][ni][3] = v.w;
  }
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    const uint4 v = *reinterpret_cast<const uint4*>(base + st.a_off + mi * 16 * st.rbs);
    r.qa[slot / 4][mi][0] = v.x, r.qa[slot / 4][mi][1] = v.y;
    r.qa[slot / 4][mi][2] = v.z, r.qa[slot / 4][mi][3] = v.w;
  }
}

// CPA: cache policy of the activation-side loads (values and scales).
template <int KIND, int MI, int NI, int D, bool STAGED = false, int CPA = 0>
__device__ __forceinline__ void ring_load(Ring<KIND, MI, NI, D>& r, int slot, int ks,
                                          const Operand<MI, NI>& op) {
  const uint32_t soff = (uint32_t)ks * KindTraits<KIND>::STEP_BYTES;
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) load_frag<KIND, CPA>(r.fa[slot][mi], op.ra, op.a[mi], soff);
#pragma unroll
  for (int ni = 0; ni < NI; ++ni)
    load_frag_b<KIND>(r.fb[slot][ni], op.rb, op.b[ni], (uint32_t)ks * BTraits<KIND>::STEP_BYTES);
  if constexpr (KIND == KIND_FP8B) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int i = 0; i < 4; ++i) r.sa[slot][mi][i] = buf_loadf<CPA>(op.rsa, op.as[mi][i], ks * 4);
  }
  // a run starts at every Q-th slot (slot is a constant once the ring loop is
  // unrolled, so this is no branch)
  constexpr int Q = Ring<KIND, MI, NI, D>::Q;
  if constexpr (is_mx(KIND) && !STAGED) {
    if (slot % Q == 0) {
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
        load_run<Q, CPA>(r.qa[slot / Q][mi], op.rxa, op.ax[mi], ks * 4);
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) load_run<Q>(r.qb[slot / Q][ni], op.rxb, op.bx[ni], ks * 4);
    }
  }
}

template <int KIND, int MI, int NI, int D>
__device__ __forceinline__ void ring_compute(Ring<KIND, MI, NI, D>& r, int slot, int ks,
                                             const Operand<MI, NI>& op,
                                             const StepScales (&sc)[2], f32x4 (&acc)[MI][NI]) {
  if constexpr (KIND == KIND_FP8B) {
    float sb[2];
    sb[0] = sc[0].at(ks);
    sb[1] = sc[1].at(ks);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        f32x4 t = mfma_step<KIND>(r.fa[slot][mi], r.fb[slot][ni], z);
        const float w = op.bsel[ni] ? sb[1] : sb[0];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[mi][ni][i] += t[i] * (r.sa[slot][mi][i] * w);
      }
  } else if constexpr (is_mx(KIND)) {
    constexpr int Q = Ring<KIND, MI, NI, D>::Q;
    if (slot % Q == 0) {
      // lane group g's byte of each step: K block g of the step
      const uint32_t sh = (threadIdx.x >> 1) & 0x18u;  // 8 * (lane / 16)
#pragma unroll
      for (int j = 0; j < Q; ++j) {
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
          r.xa[mi][j] = (int)__builtin_amdgcn_ubfe(r.qa[slot / Q][mi][j], sh, 8);
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          r.xb[ni][j] = (int)__builtin_amdgcn_ubfe(r.qb[slot / Q][ni][j], sh, 8);
      }
    }
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        acc[mi][ni] = mfma_step_scaled<KIND>(r.fa[slot][mi], r.fb[slot][ni], acc[mi][ni],
                                             r.xa[mi][slot % Q], r.xb[ni][slot % Q]);
  } else {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        acc[mi][ni] = mfma_step<KIND>(r.fa[slot][mi], r.fb[slot][ni], acc[mi][ni]);
  }
}

// Start step of a K walk.  A dot product may visit its K steps in any
// order, and walks that all start at step 0 read the same offset of rows
// 4 KiB apart at the same time, which concentrates the traffic on a few HBM
// channels (measured: 1.8 TB/s against 6.2 TB/s with staggered starts).
// Each tile therefore starts at a step hashed from its tile index (its grid
// position in the split kernels, the same index in the persistent ring), so
// a tile's summation order, hence its rounding, does not depend on which
// workgroup runs it.
__device__ __forceinline__ int stagger(uint32_t tile, int nsteps) {
  return (int)(((tile * 2654435761u) >> 16) % (uint32_t)nsteps);
}

// acc[mi][ni] = sum over the 128-wide K steps [k_first, k_first + ksteps) of
// A rows . B rows (with the dtype's scales), D steps of operands prefetched
// into registers, visiting the steps from the tile's staggered start.
// STAGED (MX, runs of 4): the scale runs come from the wave's LDS region,
// filled here with the rows of a_row(i) / b_row(i) (byte offsets of the
// i-th activation / weight row's scales in their buffers).  CPA: cache
// policy of every activation-side load.
template <int KIND, int MI, int NI, int D, bool STAGED = false, int CPA = 0, class AR = int,
          class BR = int>
__device__ __forceinline__ void gemm_steps(const Operand<MI, NI>& op, int k_first, int ksteps,
                                           uint32_t tile, f32x4 (&acc)[MI][NI],
                                           const Stage* st = nullptr,
                                           AR a_row = 0, BR b_row = 0) {
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};
  StepScales sc[2] = {{0.f, 0.f}, {0.f, 0.f}};
  if constexpr (KIND == KIND_FP8B) {
    sc[0].load(op.bsrow[0] + k_first, ksteps);
    sc[1].load(op.bsrow[1] + k_first, ksteps);
    // wait here, not at the first use inside the loop, where it would also
    // drain the operand ring every pass
    wait_vmcnt<0>();
  }
  // MX scale runs are contiguous in K only if no run straddles the wrap, so
  // the rotation moves in whole runs (and stays 0 if runs do not tile the walk)
  constexpr int Q = is_mx(KIND) ? Ring<KIND, MI, NI, D>::Q : 1;
  const int rot = ksteps % Q == 0 ? Q * stagger(tile, ksteps / Q) : 0;
  auto rel = [&](int i) { const int k = i + rot; return k >= ksteps ? k - ksteps : k; };
  Ring<KIND, MI, NI, D> r;
  // The steady-state loop loads unconditionally, so the count of loads in
  // flight is the same at every step and the compiler's waits stay precise
  // (a conditional load inside the loop makes it wait for every load at the
  // join).  The last steps, fewer than 2D, run in an unrolled tail.
  // the prologue fills every slot unconditionally too (with fewer steps than
  // slots the spare slots re-load a wrapped, in-bounds step nobody uses):
  // a skipped load here would leave the loop's first waits conservative
  if constexpr (STAGED) {
    static_assert(is_mx(KIND) && Ring<KIND, MI, NI, D>::Q == 4 && NI == 4, "staged MX runs");
    // copy the scale rows: chunk c = 64 t + lane of a section is row c / cpr,
    // slot c % cpr, which holds the row's chunk (slot - rotation) mod cpr
    const int lane = threadIdx.x & 63, cpr = st->cpr;
    const uint32_t m0 = lds_addr(st->lds);
    const uint32_t koff = 4u * (uint32_t)k_first;
    for (int t = 0; t < cpr; ++t) {  // NI * 16 * cpr / 64 instructions
      const int c = t * 64 + lane, ri = c / cpr, ch = c - ri * cpr, rot_i = (ri & 15) % cpr;
      const int gq = ch >= rot_i ? ch - rot_i : ch + cpr - rot_i;
      dma16(op.dxb, m0 + t * 1024, b_row(ri) + 16 * gq, koff);
    }
    const int na = (MI * 16 * cpr + 63) / 64;
    for (int t = 0; t < na; ++t) {
      const int c = t * 64 + lane, ri = c / cpr, ch = c - ri * cpr, rot_i = (ri & 15) % cpr;
      const int gq = ch >= rot_i ? ch - rot_i : ch + cpr - rot_i;
      // lanes past the last row fill padding with a valid row's bytes
      dma16<CPA>(op.dxa, m0 + st->a_off + t * 1024,
                 a_row(ri < MI * 16 ? ri : MI * 16 - 1) + 16 * gq, koff);
    }
  }
#pragma unroll
  for (int d = 0; d < D; ++d)
    ring_load<KIND, MI, NI, D, STAGED, CPA>(r, d, k_first + rel(d < ksteps ? d : d % ksteps), op);
  if constexpr (STAGED) {
    // Wait for the copy once, after the first D steps of operand loads are
    // in flight (the empty asm keeps them above the wait).  Vector loads
    // complete in order, so a wait for "at most the loads issued after the
    // copy" would do as well; the full wait measured no slower and does not
    // depend on that count.
    asm volatile("" ::: "memory");
    wait_vmcnt<0>();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int d = 0; d < D; d += 4) stage_read(r, d, rel(d < ksteps ? d : d % ksteps) / 4, *st);
  }
  int ks = 0;
  for (; ks + 2 * D <= ksteps; ks += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      ring_compute<KIND>(r, d, rel(ks + d), op, sc, acc);
      ring_load<KIND, MI, NI, D, STAGED, CPA>(r, d, k_first + rel(ks + d + D), op);
      if constexpr (STAGED) {
        if (d % 4 == 0) stage_read(r, d, rel(ks + d + D) / 4, *st);
      }
    }
  }
#pragma unroll
  for (int d = 0; d < 2 * D; ++d) {
    const int k = ks + d;
    if (k < ksteps) {
      ring_compute<KIND>(r, d % D, rel(k), op, sc, acc);
      if (k + D < ksteps) {
        ring_load<KIND, MI, NI, D, STAGED, CPA>(r, d % D, k_first + rel(k + D), op);
        if constexpr (STAGED) {
          if (d % 4 == 0) stage_read(r, d % D, rel(k + D) / 4, *st);
        }
      }
    }
  }
}

// The region of the wave `w` of a workgroup of `waves` waves (dynamic LDS)
extern __shared__ __attribute__((aligned(16))) uint8_t mx_stage[];

__device__ __forceinline__ Stage make_stage(int ksteps, int mi, int waves, int w) {
  Stage st;
  const int bytes = stage_bytes(ksteps, mi, waves);
  st.lds = mx_stage + w * bytes;
  st.cpr = ksteps / 4;
  st.rbs = 4 * ksteps;
  const int r16 = threadIdx.x & 15;
  st.rm = r16 % st.cpr;
  st.a_off = 4 * 16 * st.cpr * 16;
  st.lane_row = (uint32_t)(r16 * st.rbs);
  return st;
}

// Region bytes per wave of the up GEMM (K groups of K / 128 / ksplit steps)
__host__ __device__ constexpr int up_stage_bytes(int K, int mi, int ksplit, int waves) {
  return (K / 128) % ksplit == 0 ? stage_bytes(K / 128 / ksplit, mi, waves) : 0;
}

template <int BM, int KSPLIT = 1>
struct BlockShape {
  static constexpr int MI = (BM < 64 ? BM : 64) / 16;  // 16-row subtiles per wave
  static constexpr int WM = (BM + 63) / 64;            // wave rows
  static constexpr int WG = 4 * WM;                    // waves per K group
  static constexpr int THREADS = 64 * WG * KSPLIT;
  // LDS floats for the partial sums of groups 1..KSPLIT-1 (4 gate/up subtile columns)
  static constexpr int RED = KSPLIT > 1 ? (KSPLIT - 1) * WG * MI * 4 * 4 * 64 : 1;
};


// Gate/up GEMM + SwiGLU for one (block, slice) tile (index `tile` for the
// stagger of its K walk): h[mi][j] holds the
// lane's C elements of gate/up column pair j (columns 32*wn + 16*j + l%16 of
// the slice), rows 64*wm + 16*mi + 4*(l/16) + i.
// RANGE: only the K steps [k0, k0 + kn), and no SwiGLU: the raw gate (ni <
// 2) and up (ni >= 2) sums go to part[mi][ni] (K group 0 holds them).  The
// default form is kept apart under `if constexpr`: the full-K kernels'
// register allocation moves with any change to their code.
template <int KIND, int BM, int D, int KSPLIT, bool RANGE = false>
__device__ __forceinline__ void up_tile(const MoeArgs& p, int e, int s, uint32_t tile,
                                        const int* ids, f32x4 (&h)[BlockShape<BM>::MI][2],
                                        float* red, int k0 = 0, int kn = 0,
                                        f32x4 (*part)[4] = nullptr) {
  using B = BlockShape<BM, KSPLIT>;
  constexpr int MI = B::MI;
  constexpr int ES = KindTraits<KIND>::ES;
  // wave-uniform wave index: the K range (hence every load's soffset) derives
  // from it and must stay in scalar registers
  const int lane = threadIdx.x & 63, wid = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int kg = KSPLIT > 1 ? wid / B::WG : 0, wig = KSPLIT > 1 ? wid % B::WG : wid;
  const int wn = wig & 3, wm = wig >> 2;
  const int g = lane >> 4, r16 = lane & 15;
  const int K = p.K, I = p.I, N = 2 * p.I;
  const int KS = K / 128, S = I / kSlice;
  Operand<MI, 4> op;
  op.ra = make_rsrc(p.x, (uint32_t)((size_t)p.T * K * ES));
  op.rb = make_rsrc(p.w1 + (size_t)e * N * BTraits<KIND>::row_bytes(K),
                    (uint32_t)(N * BTraits<KIND>::row_bytes(K)));
  if constexpr (KIND == KIND_FP8B) op.rsa = make_rsrc(p.xs, (uint32_t)((size_t)p.T * KS * 4));
  if constexpr (is_mx(KIND)) {
    op.rxa = make_rsrc(p.xs, (uint32_t)((size_t)p.T * (K / 32)));
    op.rxb = make_rsrc(reinterpret_cast<const uint8_t*>(p.w1s) + (size_t)e * N * (K / 32),
                       (uint32_t)((size_t)N * (K / 32)));
    op.dxa = make_desc(p.xs, (uint32_t)((size_t)p.T * (K / 32)));
    op.dxb = make_desc(reinterpret_cast<const uint8_t*>(p.w1s) + (size_t)e * N * (K / 32),
                       (uint32_t)((size_t)N * (K / 32)));
  }
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    const int row = wm * 64 + mi * 16 + r16;
    const int tok = route_token(p, ids[row]);
    op.a[mi] = (uint32_t)tok * K * ES + 16 * g;
    if constexpr (KIND == KIND_FP8B) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int crow = wm * 64 + mi * 16 + 4 * g + i;
        op.as[mi][i] = (uint32_t)route_token(p, ids[crow]) * KS * 4;
      }
    }
    if constexpr (is_mx(KIND)) op.ax[mi] = (uint32_t)tok * (K / 32);
  }
#pragma unroll
  for (int ni = 0; ni < 4; ++ni) {
    const int n = (ni < 2 ? 0 : I) + s * kSlice + 32 * wn + 16 * (ni & 1) + r16;
    op.b[ni] = (uint32_t)(n * BTraits<KIND>::row_bytes(K)) + 16 * g;
    if constexpr (KIND == KIND_FP8B) op.bsel[ni] = ni < 2 ? 0 : 1;  // gate block, up block
    if constexpr (is_mx(KIND)) op.bx[ni] = (uint32_t)n * (K / 32);
  }
  if constexpr (KIND == KIND_FP8B) {
    op.bsrow[0] = reinterpret_cast<const float*>(p.w1s) + ((size_t)e * (N / 128) + s) * KS;
    op.bsrow[1] = reinterpret_cast<const float*>(p.w1s) + ((size_t)e * (N / 128) + S + s) * KS;
  }
  f32x4 acc[MI][4];
  int k_lo, k_hi;
  if constexpr (RANGE) {
    k_lo = k0 + kg * kn / KSPLIT;
    k_hi = k0 + (kg + 1) * kn / KSPLIT;
  } else {
    k_lo = kg * KS / KSPLIT;
    k_hi = (kg + 1) * KS / KSPLIT;
  }
  bool done = false;
  if constexpr (is_mx(KIND) && scale_run<D>() == 4) {
    constexpr int W = B::THREADS / 64;
    if (up_stage_bytes(RANGE ? kn * 128 : K, MI, KSPLIT, W) > 0) {
      const Stage st = make_stage(k_hi - k_lo, MI, W, wid);
      const uint32_t rs = (uint32_t)(K / 32);
      auto a_row = [&](int ri) { return (uint32_t)route_token(p, ids[wm * 64 + ri]) * rs; };
      auto b_row = [&](int ri) {
        const int ni = ri >> 4;
        return (uint32_t)((ni < 2 ? 0 : I) + s * kSlice + 32 * wn + 16 * (ni & 1) + (ri & 15)) * rs;
      };
      gemm_steps<KIND, MI, 4, D, true>(op, k_lo, k_hi - k_lo, tile, acc, &st, a_row, b_row);
      done = true;
    }
  }
  if (!done) gemm_steps<KIND, MI, 4, D>(op, k_lo, k_hi - k_lo, tile, acc);
  if constexpr (KSPLIT > 1) {
    // partial sums of groups 1.. go through LDS (lane-contiguous floats);
    // group 0 adds them in group order
    constexpr int PER = MI * 4 * 4;  // floats per lane
    if (kg > 0) {
      float* dst = red + ((size_t)((kg - 1) * B::WG + wig) * PER) * 64 + lane;
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
          for (int i = 0; i < 4; ++i) dst[((mi * 4 + ni) * 4 + i) * 64] = acc[mi][ni][i];
    }
    __syncthreads();
    if (kg == 0) {
#pragma unroll
      for (int gk = 1; gk < KSPLIT; ++gk) {
        const float* src = red + ((size_t)((gk - 1) * B::WG + wig) * PER) * 64 + lane;
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
          for (int ni = 0; ni < 4; ++ni)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[mi][ni][i] += src[((mi * 4 + ni) * 4 + i) * 64];
      }
    }
  }
  if constexpr (RANGE) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) part[mi][ni] = acc[mi][ni];
  } else {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) h[mi][j][i] = swiglu(acc[mi][j][i], acc[mi][2 + j][i]);
  }
}

// Requantize the tile: codes[mi][j][i] (bf16 bits or e4m3 code) and the
// per-row scale (FP8B: fp32 sf of the whole 128-wide slice; MX: e8m0 of this
// wave's 32 columns).  FP8B reduces amax over the 4 waves through LDS.
template <int KIND, int BM>
__device__ __forceinline__ void requant_tile(const f32x4 (&h)[BlockShape<BM>::MI][2],
                                             uint32_t (&codes)[BlockShape<BM>::MI][2][4],
                                             float (&sf)[BlockShape<BM>::MI][4],
                                             int (&sx)[BlockShape<BM>::MI][4],
                                             float* lds_amax /* [4][BM] */) {
  constexpr int MI = BlockShape<BM>::MI;
  constexpr int WG = BlockShape<BM>::WG;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wig = wid % WG;  // waves past the first K group hold no result
  const int wn = wig & 3, wm = wig >> 2;
  const int g = lane >> 4, r16 = lane & 15;
  if constexpr (KIND == KIND_BF16) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) codes[mi][j][i] = f32_to_bf16(h[mi][j][i]);
    return;
  } else {
    float am[MI][4];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        am[mi][i] = wave_max16(__builtin_fmaxf(__builtin_fabsf(h[mi][0][i]),
                                               __builtin_fabsf(h[mi][1][i])));
    if constexpr (KIND == KIND_FP8B) {
      if (r16 == 0 && wid < WG) {
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            lds_amax[wn * BM + wm * 64 + mi * 16 + 4 * g + i] = am[mi][i];
      }
      __syncthreads();
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = wm * 64 + mi * 16 + 4 * g + i;
          float a = __builtin_fmaxf(__builtin_fmaxf(lds_amax[row], lds_amax[BM + row]),
                                    __builtin_fmaxf(lds_amax[2 * BM + row], lds_amax[3 * BM + row]));
          a = __builtin_fmaxf(a, 1e-10f);
          const float f = a * (1.0f / 448.0f);
          const float inv = 1.0f / f;
          sf[mi][i] = f;
#pragma unroll
          for (int j = 0; j < 2; ++j) codes[mi][j][i] = f32_to_e4m3_in_range(h[mi][j][i] * inv);
        }
    } else {  // MX: this wave's 32 columns form one group
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int se = mx_shared_exp(am[mi][i]);
          sx[mi][i] = se + 127;
#pragma unroll
          for (int j = 0; j < 2; ++j)
            codes[mi][j][i] = f32_to_e4m3(__builtin_amdgcn_ldexpf(h[mi][j][i], -se));
        }
    }
  }
}

// ---------------------------------------------------------------------------
// split mode
// ---------------------------------------------------------------------------

// Gate/up GEMM, SwiGLU and requantization of the tile (block b of expert
// e, slice s; tile index b * S + s), written to intermediate rows
// hrow0 .. hrow0 + block_m - 1;
// ids holds the block's route ids in LDS.  Every wave of the workgroup
// calls it (it has workgroup barriers).
// Store of the intermediate: plain, or (DEV) a relaxed device-scope atomic
// store, written where every XCD reads the same data.
template <bool DEV, class T>
__device__ __forceinline__ void store_h(T* ptr, T v) {
  if constexpr (DEV) __hip_atomic_store(ptr, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *ptr = v;
}

// GIVEN: the SwiGLU tile comes in as hg (no GEMM here).
template <int KIND, int BM, int D, int KSPLIT, bool DEV = false, bool GIVEN = false>
__device__ __forceinline__ void up_block(const MoeArgs& p, int e, int s, uint32_t tile,
                                         size_t hrow0, const int* ids, float* lds_amax,
                                         float* red, const f32x4 (*hg)[2] = nullptr) {
  using B = BlockShape<BM, KSPLIT>;
  constexpr int MI = B::MI;
  constexpr int ES = KindTraits<KIND>::ES;
  f32x4 h[MI][2];
  if constexpr (GIVEN) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) h[mi][0] = hg[mi][0], h[mi][1] = hg[mi][1];
  } else {
    up_tile<KIND, BM, D, KSPLIT>(p, e, s, tile, ids, h, red);
  }
  uint32_t codes[MI][2][4];
  float sf[MI][4];
  int sx[MI][4];
  requant_tile<KIND, BM>(h, codes, sf, sx, lds_amax);

  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (wid >= B::WG) return;  // the other K groups hold no result (no barrier follows)
  const int wn = wid & 3, wm = wid >> 2;
  const int g = lane >> 4, r16 = lane & 15;
  const int I = p.I;
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = wm * 64 + mi * 16 + 4 * g + i;
      const size_t pos = hrow0 + row;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = s * kSlice + 32 * wn + 16 * j + r16;
        if constexpr (ES == 2)
          store_h<DEV>(reinterpret_cast<uint16_t*>(p.hq) + pos * I + col, (uint16_t)codes[mi][j][i]);
        else
          store_h<DEV>(p.hq + pos * I + col, (uint8_t)codes[mi][j][i]);
      }
      if (r16 == 0) {
        if constexpr (KIND == KIND_FP8B) {
          if (wn == 0) store_h<DEV>(reinterpret_cast<float*>(p.hs) + pos * (I / 128) + s, sf[mi][i]);
        }
        if constexpr (is_mx(KIND)) store_h<DEV>(p.hs + pos * (I / 32) + s * 4 + wn, (uint8_t)sx[mi][i]);
      }
    }
  if (s == 0 && threadIdx.x < BM) {
    const int id = ids[threadIdx.x];
    if (id >= 0) p.flags[id] = 1;
  }
}

template <int KIND, int BM, int D, int KSPLIT>
__global__ void __launch_bounds__((BlockShape<BM, KSPLIT>::THREADS))
k_up(MoeArgs p) {
  using B = BlockShape<BM, KSPLIT>;
  const int S = p.I / kSlice;
  const int b = blockIdx.x / S, s = blockIdx.x % S;
  if (b * BM >= *p.ntp) return;
  const int e = p.expert_ids[b];
  if ((unsigned)e >= (unsigned)p.E) return;
  __shared__ int ids[BM];
  __shared__ float lds_amax[4 * BM];
  __shared__ float red[B::RED];
  if (threadIdx.x < BM) ids[threadIdx.x] = p.sorted[b * BM + threadIdx.x];
  __syncthreads();
  up_block<KIND, BM, D, KSPLIT>(p, e, s, blockIdx.x, (size_t)b * BM, ids, lds_amax, red);
}

// Gate/up with K split over KW workgroups, for calls with few (block,
// slice) tiles, where one workgroup per tile leaves most CUs idle and walks
// all of K alone (MXFP8, K=4096, I=256, E=32, T=8: 60 tiles on 256 CUs).
// Workgroup (t, kw) sums the K steps [kw*KS/KW, (kw+1)*KS/KW) of tile t and
// stores the raw gate/up sums in the workspace with device-scope stores;
// the last of the tile's workgroups to count itself in (a ticket per tile,
// zero at launch) adds the KW sums in the order kw = 0, 1, .. and runs
// SwiGLU, requantization and the stores of the tile.  The fixed order keeps
// the result deterministic.
template <int KIND, int BM, int D, int KSPLIT, int KW>
__global__ void __launch_bounds__((BlockShape<BM, KSPLIT>::THREADS))
k_up_sk(MoeArgs p) {
  using B = BlockShape<BM, KSPLIT>;
  constexpr int MI = B::MI;
  constexpr int PER = MI * 16;  // floats per lane: a wave's gate/up sums
  const int S = p.I / kSlice;
  const int t = blockIdx.x / KW, kw = blockIdx.x % KW;
  const int b = t / S, s = t % S;
  if (b * BM >= *p.ntp) return;
  const int e = p.expert_ids[b];
  if ((unsigned)e >= (unsigned)p.E) return;
  __shared__ int ids[BM];
  __shared__ float lds_amax[4 * BM];
  __shared__ float red[B::RED];
  __shared__ int last;
  if (threadIdx.x < BM) ids[threadIdx.x] = p.sorted[b * BM + threadIdx.x];
  __syncthreads();
  const int kn = p.K / 128 / KW;
  f32x4 h[MI][2];
  f32x4 part[MI][4];
  up_tile<KIND, BM, D, KSPLIT, true>(p, e, s, blockIdx.x, ids, h, red, kw * kn, kn, part);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  float* const pt = p.part + (size_t)t * KW * (B::WG * PER * 64);
  if (wid < B::WG) {  // K group 0 holds the workgroup's sums
    float* dst = pt + ((size_t)kw * B::WG + wid) * PER * 64 + lane;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          __hip_atomic_store(dst + ((mi * 4 + ni) * 4 + i) * 64, part[mi][ni][i], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
  }
  // the sums have been acknowledged device-wide before the ticket moves
  asm volatile("" ::: "memory");
  wait_vmcnt<0>();
  asm volatile("" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) last = atomicAdd(p.tickets + t, 1) == KW - 1;
  __syncthreads();
  if (!last) return;
  if (wid < B::WG) {
    const float* src = pt + (size_t)wid * PER * 64 + lane;
    f32x4 acc[MI][4];
#pragma unroll
    for (int q = 0; q < KW; ++q)
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float v = __hip_atomic_load(src + (size_t)q * B::WG * PER * 64 +
                                                  ((mi * 4 + ni) * 4 + i) * 64,
                                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            acc[mi][ni][i] = q == 0 ? v : acc[mi][ni][i] + v;
          }
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) h[mi][j][i] = swiglu(acc[mi][j][i], acc[mi][2 + j][i]);
  }
  up_block<KIND, BM, D, KSPLIT, false, true>(p, e, s, 0, (size_t)b * BM, ids, lds_amax, red, h);
}

// Down GEMM of the tile (block b of expert e, output columns ct*256 ..
// ct*256 + 255; tile index b * NT + ct) from intermediate rows hrow0 ..:
// per-route rows of yr, rounded to bf16.
// CPA: cache policy of the intermediate's loads.
template <int KIND, int BM, int D, int CPA = 0>
__device__ __forceinline__ void down_block(const MoeArgs& p, int e, int ct, uint32_t tile,
                                           size_t hrow0, const int* ids) {
  constexpr int MI = BlockShape<BM>::MI;
  constexpr int ES = KindTraits<KIND>::ES;
  const int K = p.K, I = p.I;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wn = wid & 3, wm = wid >> 2;
  const int g = lane >> 4, r16 = lane & 15;
  const int c0 = ct * 256 + 64 * wn;  // this wave's 64 output columns
  if (c0 >= K) return;
  const int IS = I / 128;
  Operand<MI, 4> op;
  op.ra = make_rsrc(p.hq, (uint32_t)((size_t)p.h_rows * I * ES));
  op.rb = make_rsrc(p.w2 + (size_t)e * K * BTraits<KIND>::row_bytes(I),
                    (uint32_t)(K * BTraits<KIND>::row_bytes(I)));
  if constexpr (KIND == KIND_FP8B)
    op.rsa = make_rsrc(p.hs, (uint32_t)((size_t)p.h_rows * IS * 4));
  if constexpr (is_mx(KIND)) {
    op.rxa = make_rsrc(p.hs, (uint32_t)((size_t)p.h_rows * (I / 32)));
    op.rxb = make_rsrc(reinterpret_cast<const uint8_t*>(p.w2s) + (size_t)e * K * (I / 32),
                       (uint32_t)((size_t)K * (I / 32)));
    op.dxa = make_desc(p.hs, (uint32_t)((size_t)p.h_rows * (I / 32)));
    op.dxb = make_desc(reinterpret_cast<const uint8_t*>(p.w2s) + (size_t)e * K * (I / 32),
                       (uint32_t)((size_t)K * (I / 32)));
  }
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    const uint32_t pos = (uint32_t)hrow0 + wm * 64 + mi * 16 + r16;
    op.a[mi] = pos * I * ES + 16 * g;
    if constexpr (KIND == KIND_FP8B) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t cpos = (uint32_t)hrow0 + wm * 64 + mi * 16 + 4 * g + i;
        op.as[mi][i] = cpos * IS * 4;
      }
    }
    if constexpr (is_mx(KIND)) op.ax[mi] = pos * (I / 32);
  }
#pragma unroll
  for (int ni = 0; ni < 4; ++ni) {
    const int c = c0 + 16 * ni + r16;
    op.b[ni] = (uint32_t)(c * BTraits<KIND>::row_bytes(I)) + 16 * g;
    if constexpr (KIND == KIND_FP8B) op.bsel[ni] = 0;
    if constexpr (is_mx(KIND)) op.bx[ni] = (uint32_t)c * (I / 32);
  }
  if constexpr (KIND == KIND_FP8B) {
    op.bsrow[0] = reinterpret_cast<const float*>(p.w2s) + ((size_t)e * (K / 128) + c0 / 128) * IS;
    op.bsrow[1] = op.bsrow[0];
  }
  f32x4 acc[MI][4];
  bool done = false;
  if constexpr (is_mx(KIND) && scale_run<D>() == 4) {
    constexpr int W = BlockShape<BM>::THREADS / 64;
    if (stage_bytes(IS, MI, W) > 0) {
      const Stage st = make_stage(IS, MI, W, wave_id());
      const uint32_t rs = (uint32_t)(I / 32), b0 = (uint32_t)hrow0 + wm * 64;
      auto a_row = [&](int ri) { return (b0 + ri) * rs; };
      auto b_row = [&](int ri) { return (uint32_t)(c0 + ri) * rs; };
      gemm_steps<KIND, MI, 4, D, true, CPA>(op, 0, IS, tile, acc, &st, a_row, b_row);
      done = true;
    }
  }
  if (!done) gemm_steps<KIND, MI, 4, D, false, CPA>(op, 0, IS, tile, acc);
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = ids[wm * 64 + mi * 16 + 4 * g + i];
      if (id < 0) continue;
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) p.yr[(size_t)id * K + c0 + 16 * ni + r16] = f32_to_bf16(acc[mi][ni][i]);
    }
}

template <int KIND, int BM, int D>
__global__ void __launch_bounds__(BlockShape<BM>::THREADS)
k_down(MoeArgs p) {
  const int NT = (p.K + 255) / 256;
  const int b = blockIdx.x / NT, ct = blockIdx.x % NT;
  if (b * BM >= *p.ntp) return;
  const int e = p.expert_ids[b];
  if ((unsigned)e >= (unsigned)p.E) return;
  __shared__ int ids[BM];
  if (threadIdx.x < BM) ids[threadIdx.x] = p.sorted[b * BM + threadIdx.x];
  __syncthreads();
  down_block<KIND, BM, D>(p, e, ct, blockIdx.x, (size_t)b * BM, ids);
}

// ---------------------------------------------------------------------------
// persistent ring mode ([DeepGEMM #88] "How it works" and "Why the order
// and not the pool size"): one resident grid takes tasks from a ticket.
// The stream holds, per block of rows in planner order, its up tasks (one
// per 128-wide slice of I) followed, lag blocks later, by its down tasks
// (one per 256 output columns).  Block b's intermediate lives in
// ring slot b % ring: its up tasks first wait until the down tasks of block
// b - ring have read the slot, and its down tasks wait until all its up
// tasks have written it.  Every wait is on a lower ticket, and tickets are
// taken in order by running workgroups, so the lowest unfinished ticket can
// always run: the stream drains for any grid size and any lag < ring.  The
// arithmetic per tile is the split mode's, so results are bitwise equal.
// ---------------------------------------------------------------------------

constexpr int kRingSpinLimit = 1 << 20;  // ~1 s of polling: only a broken invariant gets there

// Thread 0 polls *w until it reaches v (bounded; past the bound it raises
// the error word and goes on, and once the word is up no wait polls again,
// so the kernel always ends soon).
__device__ __forceinline__ void ring_wait(int* w, int v, int* err) {
  if (threadIdx.x != 0) return;
  if (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) return;
  for (int n = 0; __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < v; ++n) {
    if (n == kRingSpinLimit) {
      atomicOr(err, 1);
      return;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// Waves per SIMD: two where the larger task body fits half the register
// file (as the split kernels at 16 rows), else one.  MXFP8 at 16 rows needs
// slightly more than half once both bodies share one kernel.
template <int KIND, int BM>
constexpr int ring_waves_per_simd() { return BM <= 16 && KIND != KIND_MX ? 2 : 1; }

// p.ctl: [0] ticket, [1] error word, then blocks_cap finished-up counts and
// blocks_cap finished-down counts; all zero at launch.
template <int KIND, int BM, int D>
__global__ void __launch_bounds__(BlockShape<BM>::THREADS)
__attribute__((amdgpu_waves_per_eu(ring_waves_per_simd<KIND, BM>())))
k_ring(MoeArgs p) {
  using B = BlockShape<BM>;
  const int S = p.I / kSlice, NT = (p.K + 255) / 256;
  const int nb = *p.ntp / BM;
  const int total = nb * (S + NT);
  int* const ticket = p.ctl;
  int* const err = p.ctl + 1;
  int* const up_done = p.ctl + 2;
  int* const down_done = up_done + p.blocks_cap;
  __shared__ int ids[BM];
  __shared__ float lds_amax[4 * BM];
  __shared__ float red[B::RED];
  __shared__ int next;
  if (threadIdx.x == 0) next = atomicAdd(ticket, 1);
  __syncthreads();
  for (;;) {
    // wave-uniform: every index and offset derived from it stays scalar
    const int t = __builtin_amdgcn_readfirstlane(next);
    if (t >= total) break;
    // no memory operation of the last task is left in flight: the streaming
    // loops then start from a known count of outstanding loads, which keeps
    // their waits counted (with an unknown count they wait for every load)
    wait_vmcnt<0>();
    __syncthreads();  // every thread holds t; the last task's LDS is dead
    // the next task's ticket, taken now and read after this task's last barrier
    if (threadIdx.x == 0) next = atomicAdd(ticket, 1);
    const RingTask k = ring_task(t, nb, S, NT, p.lag);
    const int e = p.expert_ids[k.b];
    const size_t hrow0 = (size_t)(k.b % p.ring) * BM;
    if (threadIdx.x < BM) ids[threadIdx.x] = p.sorted[k.b * BM + threadIdx.x];
    if (k.kind == 1) {
      // the slot's previous block has been read: its down tasks consumed
      // the loaded values before they counted themselves done
      if (k.b >= p.ring) ring_wait(down_done + (k.b - p.ring), NT, err);
      __syncthreads();
      if ((unsigned)e < (unsigned)p.E)
        up_block<KIND, BM, D, 1, true>(p, e, k.i, (uint32_t)(k.b * S + k.i), hrow0, ids, lds_amax,
                                       red);
      // the slice's device-scope stores have completed (been acknowledged)
      // before the count that publishes them moves
      asm volatile("" ::: "memory");
      wait_vmcnt<0>();
      asm volatile("" ::: "memory");
      __syncthreads();
      if (threadIdx.x == 0) atomicAdd(up_done + k.b, 1);
    } else {
      ring_wait(up_done + k.b, S, err);
      __syncthreads();
      // the intermediate is read with device-scope loads, past any stale
      // copy in this CU's or this XCD's cache
      if ((unsigned)e < (unsigned)p.E)
        down_block<KIND, BM, D, kDeviceScope>(p, e, k.i, (uint32_t)(k.b * NT + k.i), hrow0, ids);
      __syncthreads();
      if (threadIdx.x == 0) atomicAdd(down_done + k.b, 1);
    }
  }
}

// out[t, c:c+8] = bf16(sum_j w[t,j] * y[t*top_k+j, c:c+8] + sum_s y[shared s of t]),
// j then s ascending.  The routes are taken eight at a time: the placed
// flags, weights and rows of all eight are requested before any is added,
// so a token costs one memory round trip per eight routes rather than two
// per route (a row whose flag is clear is loaded but not added: it lies in
// the per-route buffer, and its contents are undefined).
__global__ void __launch_bounds__(256) k_combine(MoeArgs p) {
  const int K = p.K;
  const int CT = (K + kCombineCols - 1) / kCombineCols;
  const int t = blockIdx.x / CT;
  const int c = (blockIdx.x % CT) * kCombineCols + threadIdx.x * 8;  // 8 columns per thread
  if (c >= K) return;
  float s[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) s[u] = 0.f;
  // route r of the token: routed r < top_k (its weight), then shared (weight 1)
  const int nr = p.top_k + p.n_shared;
  auto route_id = [&](int r) -> size_t {
    return r < p.top_k ? (size_t)t * p.top_k + r
                       : (size_t)p.T * p.top_k + (size_t)t * p.n_shared + (r - p.top_k);
  };
  constexpr int kBatch = 8;
  for (int r0 = 0; r0 < nr; r0 += kBatch) {
    uint4 y[kBatch];
    float w[kBatch];
    int placed[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int r = r0 + u;
      placed[u] = 0;
      if (r < nr) {
        const size_t id = route_id(r);
        placed[u] = p.flags[id];
        w[u] = r < p.top_k ? p.topk_w[id] : 1.0f;
        y[u] = *reinterpret_cast<const uint4*>(p.yr + id * K + c);
      }
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (!placed[u]) continue;
      const uint32_t v[4] = {y[u].x, y[u].y, y[u].z, y[u].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        s[2 * q] += w[u] * __uint_as_float(v[q] << 16);
        s[2 * q + 1] += w[u] * __uint_as_float(v[q] & 0xFFFF0000u);
      }
    }
  }
  uint4 o;
  o.x = (uint32_t)f32_to_bf16(s[0]) | ((uint32_t)f32_to_bf16(s[1]) << 16);
  o.y = (uint32_t)f32_to_bf16(s[2]) | ((uint32_t)f32_to_bf16(s[3]) << 16);
  o.z = (uint32_t)f32_to_bf16(s[4]) | ((uint32_t)f32_to_bf16(s[5]) << 16);
  o.w = (uint32_t)f32_to_bf16(s[6]) | ((uint32_t)f32_to_bf16(s[7]) << 16);
  *reinterpret_cast<uint4*>(p.out + (size_t)t * K + c) = o;
}

// ---------------------------------------------------------------------------
// fused mode
// ---------------------------------------------------------------------------

template <int KIND, int BM, int D, int KSPLIT>
__global__ void __launch_bounds__((BlockShape<BM, KSPLIT>::THREADS))
k_fused(MoeArgs p) {
  using B = BlockShape<BM, KSPLIT>;
  constexpr int MI = B::MI;
  constexpr int ES = KindTraits<KIND>::ES;
  constexpr int QROW = 128 * ES + 16;  // LDS row stride of the slice (bytes)
  const int S = p.I / kSlice;
  const int b = blockIdx.x / S, s = blockIdx.x % S;
  if (b * BM >= *p.ntp) return;
  const int e = p.expert_ids[b];
  if ((unsigned)e >= (unsigned)p.E) return;
  __shared__ int ids[BM];
  __shared__ float lds_amax[4 * BM];
  __shared__ float lds_sf[BM];
  __shared__ uint8_t lds_sx[BM * 4];
  __shared__ __attribute__((aligned(16))) uint8_t lds_q[BM * QROW];
  __shared__ float red[B::RED];
  if (threadIdx.x < BM) ids[threadIdx.x] = p.sorted[b * BM + threadIdx.x];
  __syncthreads();
  f32x4 h[MI][2];
  up_tile<KIND, BM, D, KSPLIT>(p, e, s, blockIdx.x, ids, h, red);
  uint32_t codes[MI][2][4];
  float sf[MI][4];
  int sx[MI][4];
  requant_tile<KIND, BM>(h, codes, sf, sx, lds_amax);

  const int lane = threadIdx.x & 63, wid = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int kg = KSPLIT > 1 ? wid / B::WG : 0, wig = KSPLIT > 1 ? wid % B::WG : wid;
  const int wn = wig & 3, wm = wig >> 2;
  const int g = lane >> 4, r16 = lane & 15;
  const int K = p.K, I = p.I;
  if (kg == 0) {  // the first K group holds the slice
  #pragma unroll
    for (int mi = 0; mi < MI; ++mi)
  #pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wm * 64 + mi * 16 + 4 * g + i;
  #pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = 32 * wn + 16 * j + r16;
          if constexpr (ES == 2)
            *reinterpret_cast<uint16_t*>(lds_q + row * QROW + col * 2) = (uint16_t)codes[mi][j][i];
          else
            lds_q[row * QROW + col] = (uint8_t)codes[mi][j][i];
        }
        if (r16 == 0) {
          if constexpr (KIND == KIND_FP8B) {
            if (wn == 0) lds_sf[row] = sf[mi][i];
          }
          if constexpr (is_mx(KIND)) lds_sx[row * 4 + wn] = (uint8_t)sx[mi][i];
        }
      }
  }
  __syncthreads();

  // partial down GEMM of this slice: rows of this wave x all K columns
  Frag<KIND> fa[MI];
  int xa[MI];
  float rsf[MI][4];
  int ctok[MI][4];
  float cw[MI][4];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    const int row = wm * 64 + mi * 16 + r16;
#pragma unroll
    for (int c = 0; c < KindTraits<KIND>::NCHUNK; ++c)
      fa[mi].c[c] = *reinterpret_cast<const uint4*>(lds_q + row * QROW + c * 64 + 16 * g);
    if constexpr (is_mx(KIND)) xa[mi] = lds_sx[row * 4 + g];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int crow = wm * 64 + mi * 16 + 4 * g + i;
      const int id = ids[crow];
      ctok[mi][i] = id >= 0 ? route_token(p, id) : -1;
      cw[mi][i] = id >= 0 ? route_weight(p, id) : 0.f;
      if constexpr (KIND == KIND_FP8B) rsf[mi][i] = lds_sf[crow];
    }
  }
  const int IS = I / 128;
  const int nchunks = K / 64;  // 64-column chunks, round-robin over the wave columns
  const __amdgpu_buffer_rsrc_t rw2 =
      make_rsrc(p.w2 + (size_t)e * K * BTraits<KIND>::row_bytes(I),
                (uint32_t)(K * BTraits<KIND>::row_bytes(I)));
  const uint32_t soff = (uint32_t)s * BTraits<KIND>::STEP_BYTES;  // this slice's K step of w2 rows
  const int qrot = stagger(blockIdx.x, nchunks);
  for (int qi = wn + 4 * kg; qi < nchunks; qi += 4 * KSPLIT) {
    const int q = (qi + qrot) % nchunks;  // staggered start, see stagger()
    const int c0 = q * 64;
    FragB<KIND> fb[4];
    int xb[4];
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const int c = c0 + 16 * ni + r16;
      load_frag_b<KIND>(fb[ni], rw2, (uint32_t)(c * BTraits<KIND>::row_bytes(I)) + 16 * g, soff);
      if constexpr (is_mx(KIND))
        xb[ni] = reinterpret_cast<const uint8_t*>(p.w2s)[((size_t)e * K + c) * (I / 32) + 4 * s + g];
    }
    float swb = 1.f;
    if constexpr (KIND == KIND_FP8B)
      swb = reinterpret_cast<const float*>(p.w2s)[((size_t)e * (K / 128) + c0 / 128) * IS + s];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
        if constexpr (is_mx(KIND)) {
          y = mfma_step_scaled<KIND>(fa[mi], fb[ni], y, xa[mi], xb[ni]);
              } else {
          y = mfma_step<KIND>(fa[mi], fb[ni], y);
        }
        const int c = c0 + 16 * ni + r16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (ctok[mi][i] < 0) continue;
          float v = y[i];
          if constexpr (KIND == KIND_FP8B) v *= rsf[mi][i] * swb;
          atomicAdd(p.acc + (size_t)ctok[mi][i] * K + c, v * cw[mi][i]);
        }
      }
  }
}

__global__ void __launch_bounds__(256) k_finalize(MoeArgs p) {
  const size_t n4 = (size_t)p.T * p.K / 4;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
    const float4 v = reinterpret_cast<const float4*>(p.acc)[i];
    uint2 o;
    o.x = (uint32_t)f32_to_bf16(v.x) | ((uint32_t)f32_to_bf16(v.y) << 16);
    o.y = (uint32_t)f32_to_bf16(v.z) | ((uint32_t)f32_to_bf16(v.w) << 16);
    reinterpret_cast<uint2*>(p.out)[i] = o;
  }
}

__global__ void __launch_bounds__(256) k_zero(uint4* ptr, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
    ptr[i] = make_uint4(0, 0, 0, 0);
}

inline unsigned grid_for(size_t n, size_t per_block) {
  size_t g = (n + per_block - 1) / per_block;
  if (g > 65536) g = 65536;
  if (g == 0) g = 1;
  return (unsigned)g;
}

// Register-prefetch depth (K steps in flight per wave), sized so that the
// operand ring, the accumulators and the scales fit the register file without
// spills (a bf16 fragment is twice an e4m3 one).
template <int KIND, int BM, int KSPLIT = 1>
constexpr int prefetch_depth() {
  // two K groups put two waves on each SIMD, which halves each wave's
  // registers (four groups would leave too few for any prefetch)
  // MX depths are even (4 where registers allow) so that the scale runs are
  // 4 (or 2) steps long; measured at 16 rows: MXFP4 depth 4 beat 6 and 8.
  if constexpr (KIND == KIND_BF16) return BM <= 32 && KSPLIT == 1 ? 2 : 1;
  else if constexpr (KIND == KIND_MX4 && KSPLIT == 2) return BM == 16 ? 4 : 2;
  else if constexpr (KIND == KIND_MX4) return BM <= 32 ? 4 : BM == 64 ? 2 : 1;
  else if constexpr (KIND == KIND_MX && KSPLIT == 2) return BM == 16 ? 4 : 2;
  else if constexpr (KIND == KIND_MX) return BM == 16 ? 4 : BM <= 64 ? 2 : 1;
  else if constexpr (KSPLIT == 2) return BM == 16 ? 3 : 2;
  else return BM == 16 ? 4 : BM == 32 ? 3 : BM == 64 ? 2 : 1;
}

inline void mark(const TimingHook& h, int which, bool after, hipStream_t st) {
  if (h.which == which && h.before && h.after) (void)hipEventRecord(after ? h.after : h.before, st);
}

// Launch of the up-GEMM kernel (k_up or k_fused) with KSPLIT K groups and a
// prefetch depth of D K steps.
template <int KIND, int BM, int KSPLIT, int D>
void launch_up_d(int split, const MoeArgs& a, unsigned grid, hipStream_t st) {
  constexpr int TH = BlockShape<BM, KSPLIT>::THREADS;
  constexpr int MI = BlockShape<BM, KSPLIT>::MI, W = TH / 64;
  const size_t lds = is_mx(KIND) && scale_run<D>() == 4
                         ? (size_t)W * up_stage_bytes(a.K, MI, KSPLIT, W) : 0;
  if (split) hipLaunchKernelGGL((k_up<KIND, BM, D, KSPLIT>), dim3(grid), dim3(TH), lds, st, a);
  else hipLaunchKernelGGL((k_fused<KIND, BM, D, KSPLIT>), dim3(grid), dim3(TH), lds, st, a);
}

// The depth from the register budget, or the caller's (1, 2 or 4; the host
// checks that it asked only at block_m 16 or 32).
template <int KIND, int BM, int KSPLIT>
void launch_up(int split, const MoeArgs& a, unsigned grid, hipStream_t st) {
  if constexpr (BM <= 32) {
    switch (a.depth) {
      case 1: return launch_up_d<KIND, BM, KSPLIT, 1>(split, a, grid, st);
      case 2: return launch_up_d<KIND, BM, KSPLIT, 2>(split, a, grid, st);
      case 4: return launch_up_d<KIND, BM, KSPLIT, 4>(split, a, grid, st);
      default: break;
    }
  }
  launch_up_d<KIND, BM, KSPLIT, prefetch_depth<KIND, BM, KSPLIT>()>(split, a, grid, st);
}

// Down GEMM of the split mode (streaming kernel) at depth D.
template <int KIND, int BM, int D>
void launch_down_d(const MoeArgs& a, hipStream_t st) {
  constexpr int THREADS = BlockShape<BM>::THREADS, W = THREADS / 64;
  const int NT = (a.K + 255) / 256;
  const size_t lds = is_mx(KIND) && scale_run<D>() == 4
                         ? (size_t)W * stage_bytes(a.I / 128, BlockShape<BM>::MI, W) : 0;
  hipLaunchKernelGGL((k_down<KIND, BM, D>), dim3((unsigned)a.blocks_cap * NT), dim3(THREADS), lds,
                     st, a);
}

// The caller's depth, else the register budget's, capped by the walk: a
// down GEMM over I = 256 has two K steps, and the 16-row MX kernel's depth
// of 4 then costs its staged scale runs for nothing (MXFP8 K=4096, I=256,
// E=32, top-8, whole call at T=8: 45 against 41 us with depth 2).
template <int KIND, int BM>
void launch_down(const MoeArgs& a, hipStream_t st) {
  if constexpr (BM <= 32) {
    int depth = a.depth;
    const int walk = a.I / 128;
    if (!depth && walk < prefetch_depth<KIND, BM>()) depth = walk >= 2 ? 2 : 1;
    switch (depth) {
      case 1: return launch_down_d<KIND, BM, 1>(a, st);
      case 2: return launch_down_d<KIND, BM, 2>(a, st);
      case 4: return launch_down_d<KIND, BM, 4>(a, st);
      default: break;
    }
  }
  launch_down_d<KIND, BM, prefetch_depth<KIND, BM>()>(a, st);
}

// K groups for the up GEMM: with few (block, slice) tiles (a narrow
// intermediate, or few routes) one workgroup per tile leaves most CUs idle
// and each CU streams from few waves.  Tiles are estimated as one block per
// routed expert (decode sizes) times the slices.
template <int BM>
int pick_ksplit(const MoeArgs& a) {
  if constexpr (BM > 32) {
    return 1;
  } else {
    const size_t R = total_routes(a);
    const size_t tiles = (R < (size_t)a.E ? R : (size_t)a.E) * (size_t)(a.I / kSlice);
    if (a.K / 128 < 8) return 1;  // too few K steps to share out
    return tiles <= 256 ? 2 : 1;
  }
}

// Gate/up with K split over workgroups (k_up_sk): 4 workgroups per tile,
// two K groups each (K/128 a multiple of 8; the host checks).
constexpr int kUpKW = 4;
template <int KIND, int BM>
void launch_up_sk(const MoeArgs& a, hipStream_t st) {
  constexpr int KSPLIT = 2;
  constexpr int TH = BlockShape<BM, KSPLIT>::THREADS;
  constexpr int D = prefetch_depth<KIND, BM, KSPLIT>();
  constexpr int MI = BlockShape<BM, KSPLIT>::MI, W = TH / 64;
  const int S = a.I / kSlice;
  const size_t lds = is_mx(KIND) && scale_run<D>() == 4
                         ? (size_t)W * up_stage_bytes(a.K / kUpKW, MI, KSPLIT, W) : 0;
  hipLaunchKernelGGL((k_up_sk<KIND, BM, D, KSPLIT, kUpKW>),
                     dim3((unsigned)a.blocks_cap * S * kUpKW), dim3(TH), lds, st, a);
}

template <int KIND, int BM>
void launch_up_any(int split, const MoeArgs& a, unsigned grid, hipStream_t st) {
  if constexpr (BM <= 32) {
    const int ks = a.ksplit ? a.ksplit : pick_ksplit<BM>(a);
    if (ks == 2) return launch_up<KIND, BM, 2>(split, a, grid, st);
  }
  launch_up<KIND, BM, 1>(split, a, grid, st);
}

// Persistent grid of k_ring for a dynamic LDS size (cached per device and
// size): one workgroup per CU, provided one fits.  Measured (K=4096,
// I=2048, E=256, top-6, blockwise FP8): 242 / 927 / 1190 us at T = 8 / 64
// / 256 with one per CU against 326 / 1058 / 1334 us with the two that fit;
// the second workgroup mostly waits for up tasks that the first has not
// finished, while one per CU keeps the waits near zero.
template <int KIND, int BM, int D>
int ring_grid(size_t lds) {
  struct Entry {
    int dev;
    size_t lds;
    int n;
  };
  static thread_local Entry cache[8];
  static thread_local int used = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  for (int i = 0; i < used; ++i)
    if (cache[i].dev == dev && cache[i].lds == lds) return cache[i].n;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_ring<KIND, BM, D>,
                                                   BlockShape<BM>::THREADS, lds) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (per_cu < 1 || cus < 1) return 0;
  cache[used < 8 ? used++ : 7] = Entry{dev, lds, cus};
  return cus;
}

// Ring mode: clear the control words and flags (adjacent in the
// workspace), one resident grid over the lag-ordered task stream, then the
// combine.
template <int KIND, int BM>
hipError_t launch_ring(const MoeArgs& a0, hipStream_t st, const TimingHook& hk) {
  constexpr int THREADS = BlockShape<BM>::THREADS, W = THREADS / 64;
  constexpr int D = prefetch_depth<KIND, BM>();
  constexpr int MI = BlockShape<BM>::MI;
  MoeArgs a = a0;
  const int S = a.I / kSlice, per = S + (a.K + 255) / 256;
  if (a.ring < 1 || reinterpret_cast<uint8_t*>(a.flags) !=
                        reinterpret_cast<uint8_t*>(a.ctl) + ring_ctl_bytes(a.blocks_cap))
    return hipErrorInvalidValue;
  size_t lds = 0;
  if constexpr (is_mx(KIND) && scale_run<D>() == 4) {
    const size_t up = (size_t)W * up_stage_bytes(a.K, MI, 1, W);
    const size_t dn = (size_t)W * stage_bytes(a.I / 128, MI, W);
    lds = up > dn ? up : dn;
  }
  const int g = ring_grid<KIND, BM, D>(lds);
  if (g <= 0) return hipErrorInvalidDeviceFunction;
  const int lag = ring_lag(g, S);
  a.lag = lag < a.ring - 1 ? lag : a.ring - 1;
  const size_t tasks = (size_t)a.blocks_cap * per;
  const unsigned grid = (unsigned)((size_t)g < tasks ? (size_t)g : tasks);
  const size_t n16 = (ring_ctl_bytes(a.blocks_cap) + total_routes(a) * 4 + 15) / 16;
  hipLaunchKernelGGL(k_zero, dim3(grid_for(n16, 256)), dim3(256), 0, st,
                     reinterpret_cast<uint4*>(a.ctl), n16);
  mark(hk, 1, false, st);
  hipLaunchKernelGGL((k_ring<KIND, BM, D>), dim3(grid), dim3(THREADS), lds, st, a);
  mark(hk, 1, true, st);
  const int CT = (a.K + kCombineCols - 1) / kCombineCols;
  hipLaunchKernelGGL(k_combine, dim3((unsigned)(a.T * CT)), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int KIND, int BM>
hipError_t launch_kind_bm(int split, const MoeArgs& a, hipStream_t st, const TimingHook& hk) {
  constexpr int THREADS = BlockShape<BM>::THREADS;
  constexpr int D = prefetch_depth<KIND, BM>();
  const int S = a.I / kSlice;
  const size_t R = total_routes(a);
  if (split == 2) {
    if constexpr (BM <= 32) return launch_ring<KIND, BM>(a, st, hk);
    else return hipErrorInvalidValue;
  }
  if (split) {
    size_t fbytes = (R * 4 + 15) / 16;
    if (a.kw > 1) {
      // the tile tickets follow the flags: one clear for both (streaming
      // blocks, or the 64-row tiled kernels)
      if (BM > 64 || (BM == 64 && !tiled_supported(KIND, BM, a.K, a.I))) return hipErrorInvalidValue;
      if (a.kw != kUpKW || reinterpret_cast<uint8_t*>(a.tickets) <
                               reinterpret_cast<uint8_t*>(a.flags) + R * 4)
        return hipErrorInvalidValue;
      fbytes = ((size_t)(reinterpret_cast<uint8_t*>(a.tickets) -
                         reinterpret_cast<uint8_t*>(a.flags)) +
                (size_t)a.blocks_cap * S * 4 + 15) / 16;
    }
    hipLaunchKernelGGL(k_zero, dim3(grid_for(fbytes, 256)), dim3(256), 0, st,
                       reinterpret_cast<uint4*>(a.flags), fbytes);
    if (tiled_supported(KIND, BM, a.K, a.I)) {
      hipError_t e = launch_tiled(KIND, BM, a, st, hk);
      if (e != hipSuccess) return e;
      const int CT = (a.K + kCombineCols - 1) / kCombineCols;
      hipLaunchKernelGGL(k_combine, dim3((unsigned)(a.T * CT)), dim3(256), 0, st, a);
      return hipGetLastError();
    }
    mark(hk, 1, false, st);
    if constexpr (BM <= 32) {
      if (a.kw > 1) launch_up_sk<KIND, BM>(a, st);
      else launch_up_any<KIND, BM>(1, a, (unsigned)a.blocks_cap * S, st);
    } else {
      launch_up_any<KIND, BM>(1, a, (unsigned)a.blocks_cap * S, st);
    }
    mark(hk, 1, true, st);
    mark(hk, 2, false, st);
    launch_down<KIND, BM>(a, st);
    mark(hk, 2, true, st);
    const int CT = (a.K + kCombineCols - 1) / kCombineCols;
    hipLaunchKernelGGL(k_combine, dim3((unsigned)(a.T * CT)), dim3(256), 0, st, a);
  } else {
    const size_t n16 = (size_t)a.T * a.K * 4 / 16;
    hipLaunchKernelGGL(k_zero, dim3(grid_for(n16, 256)), dim3(256), 0, st,
                       reinterpret_cast<uint4*>(a.acc), n16);
    mark(hk, 1, false, st);
    launch_up_any<KIND, BM>(0, a, (unsigned)a.blocks_cap * S, st);
    mark(hk, 1, true, st);
    hipLaunchKernelGGL(k_finalize, dim3(grid_for((size_t)a.T * a.K / 4, 256)), dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

// Flags of the routes a plan placed (what the gate/up kernels set), for a
// down GEMM that runs without them.
__global__ void __launch_bounds__(256) k_flag_routes(MoeArgs p) {
  const int n = *p.ntp;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) {
    const int id = p.sorted[i];
    if (id >= 0) p.flags[id] = 1;
  }
}

// The split mode's down GEMM and combine alone, on the intermediate already
// in the workspace.
template <int KIND, int BM>
hipError_t launch_down_combine_bm(const MoeArgs& a, hipStream_t st) {
  const size_t fbytes = (total_routes(a) * 4 + 15) / 16;
  hipLaunchKernelGGL(k_zero, dim3(grid_for(fbytes, 256)), dim3(256), 0, st,
                     reinterpret_cast<uint4*>(a.flags), fbytes);
  hipLaunchKernelGGL(k_flag_routes, dim3(grid_for((size_t)a.blocks_cap * BM, 256)), dim3(256), 0,
                     st, a);
  if (tiled_supported(KIND, BM, a.K, a.I)) {
    hipError_t e = launch_tiled_down(KIND, BM, a, st);
    if (e != hipSuccess) return e;
  } else if constexpr (BM <= 128) {
    launch_down<KIND, BM>(a, st);
  } else {
    return hipErrorInvalidValue;
  }
  const int CT = (a.K + kCombineCols - 1) / kCombineCols;
  hipLaunchKernelGGL(k_combine, dim3((unsigned)(a.T * CT)), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int KIND>
hipError_t launch_down_combine_kind(int block_m, const MoeArgs& a, hipStream_t st) {
  switch (block_m) {
    case 16: return launch_down_combine_bm<KIND, 16>(a, st);
    case 32: return launch_down_combine_bm<KIND, 32>(a, st);
    case 64: return launch_down_combine_bm<KIND, 64>(a, st);
    case 128: return launch_down_combine_bm<KIND, 128>(a, st);
    case 256: return launch_down_combine_bm<KIND, 256>(a, st);
    default: return hipErrorInvalidValue;
  }
}

// block_m 256 exists only as the LDS-tiled split mode (e4m3, K % 256 == 0)
template <int KIND>
hipError_t launch_tiled_only(const MoeArgs& a, hipStream_t st, const TimingHook& hk) {
  if (!tiled_supported(KIND, 256, a.K, a.I)) return hipErrorInvalidValue;
  const size_t R = total_routes(a);
  const size_t fbytes = (R * 4 + 15) / 16;
  hipLaunchKernelGGL(k_zero, dim3(grid_for(fbytes, 256)), dim3(256), 0, st,
                     reinterpret_cast<uint4*>(a.flags), fbytes);
  hipError_t e = launch_tiled(KIND, 256, a, st, hk);
  if (e != hipSuccess) return e;
  const int CT = (a.K + kCombineCols - 1) / kCombineCols;
  hipLaunchKernelGGL(k_combine, dim3((unsigned)(a.T * CT)), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int KIND>
hipError_t launch_kind(int block_m, int split, const MoeArgs& a, hipStream_t st,
                       const TimingHook& hk) {
  switch (block_m) {
    case 256: return launch_tiled_only<KIND>(a, st, hk);
    case 16: return launch_kind_bm<KIND, 16>(split, a, st, hk);
    case 32: return launch_kind_bm<KIND, 32>(split, a, st, hk);
    case 64: return launch_kind_bm<KIND, 64>(split, a, st, hk);
    case 128: return launch_kind_bm<KIND, 128>(split, a, st, hk);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_down_combine(int kind, int block_m, const MoeArgs& a, hipStream_t st) {
  switch (kind) {
    case KIND_BF16: return launch_down_combine_kind<KIND_BF16>(block_m, a, st);
    case KIND_FP8B: return launch_down_combine_kind<KIND_FP8B>(block_m, a, st);
    case KIND_MX: return launch_down_combine_kind<KIND_MX>(block_m, a, st);
    case KIND_MX4: return launch_down_combine_kind<KIND_MX4>(block_m, a, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_moe(int kind, int block_m, int split, const MoeArgs& a, hipStream_t st,
                      const TimingHook& hk) {
  switch (kind) {
    case KIND_BF16: return launch_kind<KIND_BF16>(block_m, split, a, st, hk);
    case KIND_FP8B: return launch_kind<KIND_FP8B>(block_m, split, a, st, hk);
    case KIND_MX: return launch_kind<KIND_MX>(block_m, split, a, st, hk);
    case KIND_MX4: return launch_kind<KIND_MX4>(block_m, split, a, st, hk);
    default: return hipErrorInvalidValue;
  }
}
