// device.h -- gfx950 device helpers shared by the MoE kernels.
//
// MFMA operand layout used throughout (16x16 tiles, wave64):
//   A (rows x K) : lane l supplies row (l % 16); B (K x cols): lane l supplies
//   column (l % 16).  Per 128-wide K step a lane holds, for its row/column,
//   the bytes at offsets c*64 + 16*g .. +16 of the step (g = l / 16 is the
//   lane group, c = 0..NCHUNK-1).  For e4m3 (NCHUNK = 2) this is the
//   instruction's own K order of v_mfma_*_16x16x128_f8f6f4, so the MX scale
//   a lane passes (lane group g) is the scale of the 32-wide K block g of the
//   step.  For bf16 (NCHUNK = 4) chunk c feeds the c-th 16x16x32 MFMA of the
//   step; A and B use the same order, so the contraction covers the 128
//   elements once.
//   C/D : lane l holds column (l % 16), rows 4*(l/16) + i, i = 0..3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// KIND_MX4: MXFP4 weights (packed e2m1, two per byte, element 2j in the low
// nibble, e8m0 per 32 along K) against MX FP8 activations.  Measured on
// gfx950 with a one-wave in-bounds probe: with B in format e2m1 (blgp = 4)
// the instruction reads four registers per lane; lane (column l % 16, group
// g = l / 16) holds K [32g, 32g + 32) of the step, lower index in the low
// nibble, and its e8m0 scale covers exactly that K block.  A keeps the e4m3
// layout above.  So a weight row's step is one 64-byte chunk at 16 * g.
enum : int { KIND_BF16 = 0, KIND_FP8B = 1, KIND_MX = 2, KIND_MX4 = 3 };

// e8m0 block scales go into the MFMA (MX activations)
constexpr bool is_mx(int kind) { return kind == KIND_MX || kind == KIND_MX4; }

// A operand (activations, intermediate): bf16 or e4m3
template <int KIND>
struct KindTraits {
  static constexpr int ES = (KIND == KIND_BF16) ? 2 : 1;  // bytes per element
  static constexpr int NCHUNK = (KIND == KIND_BF16) ? 4 : 2;  // 16B chunks / lane / step
  static constexpr int STEP_BYTES = 128 * ES;                 // bytes of one row per K step
};

// B operand (weights): as A except for MXFP4
template <int KIND>
struct BTraits {
  static constexpr int NCHUNK = KIND == KIND_MX4 ? 1 : KindTraits<KIND>::NCHUNK;
  static constexpr int STEP_BYTES = KIND == KIND_MX4 ? 64 : KindTraits<KIND>::STEP_BYTES;
  // bytes of a weight row of `len` elements
  static constexpr size_t row_bytes(size_t len) {
    return KIND == KIND_MX4 ? len / 2 : len * KindTraits<KIND>::ES;
  }
};

// One lane's share of a 16-row (or 16-column) operand for one 128-wide K step.
template <int KIND>
struct Frag {
  uint4 c[KindTraits<KIND>::NCHUNK];
};

template <int KIND>
struct FragB {
  uint4 c[BTraits<KIND>::NCHUNK];
};

// Buffer resource over [base, base + bytes): loads past the end return 0.
// Word 3 = 0x00020000 is the raw (untyped) dword format of CDNA buffers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// Cache policy of a buffer access: 0, or kDeviceScope (the sc1 bit), which
// makes a load read, and a store write, at the point where all XCDs see the
// same data (the per-CU and per-XCD caches are not coherent with each other).
constexpr int kDeviceScope = 16;

template <int CP = 0>
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, CP));
}

template <int CP = 0>
__device__ __forceinline__ float buf_loadf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, CP));
}

__device__ __forceinline__ int buf_loadu8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return (int)__builtin_amdgcn_raw_buffer_load_b8(r, (int)voff, (int)soff, 0);
}

// Fragment of one row for one K step: `voff` is the row's byte offset plus
// 16 * lane group, `soff` the step's byte offset (wave-uniform).
template <int KIND, int CP = 0>
__device__ __forceinline__ void load_frag(Frag<KIND>& f, __amdgpu_buffer_rsrc_t r, uint32_t voff,
                                          uint32_t soff) {
#pragma unroll
  for (int c = 0; c < KindTraits<KIND>::NCHUNK; ++c) f.c[c] = buf_load16<CP>(r, voff + c * 64, soff);
}

template <int KIND>
__device__ __forceinline__ void load_frag_b(FragB<KIND>& f, __amdgpu_buffer_rsrc_t r, uint32_t voff,
                                            uint32_t soff) {
#pragma unroll
  for (int c = 0; c < BTraits<KIND>::NCHUNK; ++c) f.c[c] = buf_load16(r, voff + c * 64, soff);
}

template <int KIND>
__device__ __forceinline__ void load_frag_ptr(Frag<KIND>& f, const uint8_t* row_step_ptr, int g) {
#pragma unroll
  for (int c = 0; c < KindTraits<KIND>::NCHUNK; ++c)
    f.c[c] = *reinterpret_cast<const uint4*>(row_step_ptr + c * 64 + 16 * g);
}

template <int KIND>
__device__ __forceinline__ void zero_frag(Frag<KIND>& f) {
#pragma unroll
  for (int c = 0; c < KindTraits<KIND>::NCHUNK; ++c) f.c[c] = make_uint4(0, 0, 0, 0);
}

__device__ __forceinline__ i32x8 as_i32x8(const uint4& lo, const uint4& hi) {
  i32x8 v;
  v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
  v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
  return v;
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& v) {
  return __builtin_bit_cast(bf16x8, v);
}

// acc += A . B over one 128-wide K step, no scales (bf16 and e4m3).
template <int KIND, class FB>
__device__ __forceinline__ f32x4 mfma_step(const Frag<KIND>& a, const FB& b, f32x4 acc) {
  if constexpr (KIND == KIND_BF16) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a.c[c]), as_bf16x8(b.c[c]), acc, 0, 0, 0);
    return acc;
  } else {
    // format 0 = e4m3 for both operands; zero scale operands select the
    // unscaled instruction
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
        as_i32x8(a.c[0], a.c[1]), as_i32x8(b.c[0], b.c[1]), acc, 0, 0, 0, 0, 0, 0);
  }
}

// acc += (A * 2^(sa-127)) . (B * 2^(sb-127)) with per-lane e8m0 scales
// (lane group g: K block g of the step).
__device__ __forceinline__ f32x4 mfma_step_mx(const Frag<KIND_MX>& a, const Frag<KIND_MX>& b,
                                              f32x4 acc, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
      as_i32x8(a.c[0], a.c[1]), as_i32x8(b.c[0], b.c[1]), acc, 0, 0, 0, sa, 0, sb);
}

// The same with B in e2m1 (format 4: only the first four registers are read).
// e4m3 A x e2m1 B (blgp 4), emitted with its wait states.  Measured on the
// MI355X: where the compiler read the accumulator of this instruction 7
// instructions and 7 wait states after it (copying it between registers),
// the copy held the value from before the instruction, and the down GEMM
// lost one K step of one row in every 16-column tile; whether it happened
// depended on the code around it.  The instruction issues at the e4m3 rate
// (measured), slower than an e2m1 x e2m1 one, and the compiler's wait states
// after it are too few.  Written as asm with 32 wait states after it (and 5
// before, for operands written just before), nothing reads its result
// sooner: every reader depends on the asm's output.  The accumulator stays
// in accumulation registers (D = C).
__device__ __forceinline__ f32x4 mfma_step_mx4(const Frag<KIND_MX4>& a, const FragB<KIND_MX4>& b,
                                               f32x4 acc, int sa, int sb) {
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  const i32x8 av = as_i32x8(a.c[0], a.c[1]);
  const i32x4 bv = __builtin_bit_cast(i32x4, b.c[0]);
  asm volatile(
      "s_nop 4\n\t"
      "v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0] blgp:4\n\t"
      "s_nop 15\n\t"
      "s_nop 15"
      : "+a"(acc)
      : "v"(av), "v"(bv), "v"(sa), "v"(sb));
  return acc;
}

// MX-scaled step for either MX kind (the B fragment type follows the kind).
template <int KIND>
__device__ __forceinline__ f32x4 mfma_step_scaled(const Frag<KIND>& a, const FragB<KIND>& b,
                                                  f32x4 acc, int sa, int sb) {
  if constexpr (KIND == KIND_MX4) {
    return mfma_step_mx4(a, b, acc, sa, sb);
  } else {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
        as_i32x8(a.c[0], a.c[1]), as_i32x8(b.c[0], b.c[1]), acc, 0, 0, 0, sa, 0, sb);
  }
}

// silu(g) * u in fp32: g / (1 + 2^(-g*log2 e)) with the hardware exp2 and a
// refined hardware reciprocal in place of an IEEE division (about 10 VALU
// instructions fewer per element; the result is within about one ulp).
__device__ __forceinline__ float swiglu(float g, float u) {
  // e^-g as 2^(-g log2 e), the exponent capped at 126 so that 1 + e and its
  // reciprocal stay finite and normal (past the cap silu(g) is below 1e-36)
  const float e = __builtin_amdgcn_exp2f(__builtin_fminf(-g * 1.4426950408889634f, 126.0f));
  const float d = 1.0f + e;
  // 1 / d: the hardware reciprocal (1 ulp) refined by one Newton step
  float r = __builtin_amdgcn_rcpf(d);
  r = __builtin_fmaf(__builtin_fmaf(-d, r, 1.0f), r, r);
  return g * r * u;
}

// fp32 -> e4m3 code, round to nearest even, saturating at +-448.  The
// hardware conversion rounds to nearest even but returns NaN past the 464
// midpoint, so the value is clamped first.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  v = __builtin_fminf(__builtin_fmaxf(v, -448.0f), 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, 0.0f, 0, false) & 0xFFu;
}

// The same for a value already within the range: h * (1 / (amax / 448))
// with |h| <= amax is at most 448 plus a few ulp, far below the 464 midpoint,
// so it rounds as the clamped value would.
__device__ __forceinline__ uint32_t f32_to_e4m3_in_range(float v) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, 0.0f, 0, false) & 0xFFu;
}

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float v) {
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// floor(log2 a) - 8 clamped to [-127, 127] for a >= 0 (a == 0 or subnormal
// gives -127): the OCP MX shared exponent for e4m3 elements.
__device__ __forceinline__ int mx_shared_exp(float a) {
  uint32_t bits = __float_as_uint(a);
  int ef = (int)((bits >> 23) & 0xFFu);
  if (ef == 0) return -127;
  int s = ef - 127 - 8;
  return s < -127 ? -127 : (s > 127 ? 127 : s);
}

// max of v and the value lane movement CTRL (a DPP control) brings in
template <int CTRL>
__device__ __forceinline__ float max_dpp(float v) {
  const int u = __builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true);
  return __builtin_fmaxf(v, __int_as_float(u));
}

__device__ __forceinline__ float wave_max16(float v) {
  // max over the 16 lanes sharing l / 16, which form one DPP row: swap
  // neighbours, then pairs (each quad holds its max), then rotate the row
  // by 4 and by 8 (each lane meets every quad); no LDS traffic
  v = max_dpp<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v = max_dpp<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v = max_dpp<0x124>(v);  // row_ror 4
  v = max_dpp<0x128>(v);  // row_ror 8
  return v;
}

// s_waitcnt vmcnt(n) (gfx9 encoding: vmcnt in bits 3:0 and 15:14), other counters untouched
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

typedef int desc_t __attribute__((ext_vector_type(4)));

// Raw buffer descriptor: base address, no stride, `bytes` records (loads past
// them return zeros), 32-bit data format.
__device__ __forceinline__ desc_t make_desc(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  return desc_t{__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xffff)),
                __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000};
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint8_t*)p);
}

// Direct-to-LDS buffer loads: lane L's bytes land at M0 + L * size.  They are
// issued from asm so that the only waits on them are the explicit vmcnt waits
// of the pipeline: the compiler cannot always tell which LDS stage such a
// load writes and would otherwise wait for every load in flight before an LDS
// read.  They have no destination register; VMEM loads complete in order, so
// the compiler's own vmcnt waits stay correct (at worst stricter).  M0 is set
// in the same statement; the compiler sets it right before each of its own
// uses.
// The scalar operands pass through readfirstlane: the compiler may hold a
// wave-uniform value in a vector register, which an "s" operand cannot take
// (the read folds away for values already in scalar registers).
template <int CP = 0>
__device__ __forceinline__ void dma16(desc_t r, uint32_t m0, uint32_t voff, uint32_t soff) {
  if constexpr (CP == kDeviceScope)
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen sc1 lds"
                 :: "s"(__builtin_amdgcn_readfirstlane(m0)), "v"(voff), "s"(r),
                    "s"(__builtin_amdgcn_readfirstlane(soff)) : "memory");
  else
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(__builtin_amdgcn_readfirstlane(m0)), "v"(voff), "s"(r),
                    "s"(__builtin_amdgcn_readfirstlane(soff)) : "memory");
}

__device__ __forceinline__ void dma4(desc_t r, uint32_t m0, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :: "s"(__builtin_amdgcn_readfirstlane(m0)), "v"(voff), "s"(r),
                  "s"(__builtin_amdgcn_readfirstlane(soff)) : "memory");
}

// Wave index as a wave-uniform (scalar) value, so that addresses derived from
// it (LDS stage offsets for M0, row bases) stay in scalar registers.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// Weight block scales of one n-block for every K step, held lane-indexed in
// registers (lane j holds step j, and step 64 + j in the second register), so
// the K loop reads them with readlane instead of memory loads (at most 128
// steps: K <= 16384).
struct StepScales {
  float lo, hi;
  __device__ __forceinline__ void load(const float* row, int nsteps) {
    const int lane = threadIdx.x & 63;
    lo = lane < nsteps ? row[lane] : 0.f;
    hi = 64 + lane < nsteps ? row[64 + lane] : 0.f;
  }
  __device__ __forceinline__ float at(int ks) const {
    const float v = ks < 64 ? lo : hi;
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), ks & 63));
  }
};
