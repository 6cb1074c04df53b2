// probe.hip -- moe_mfma_probe: one 128-wide K step of the matrix instructions
// the kernels use, on caller-given operands (a diagnostic, not a step of the
// forward).  The parity tests accept kernel outputs within an error model of
// these instructions (how far their sums may lie from the exact ones); this
// entry point lets a test measure the instructions themselves against it.
#include <cstring>

#include "../../include/moe.h"
#include "device.h"

namespace {

// One wave per tile: D = C + A . B^T over one 128-wide K step, through the
// same operand layout and instruction wrappers as the kernels.
template <int KIND>
__global__ void __launch_bounds__(64) k_probe(const uint8_t* a, const uint8_t* b, const uint8_t* sa,
                                               const uint8_t* sb, const float* c, float* d) {
  const size_t t = blockIdx.x;
  const int l = threadIdx.x, r = l % 16, g = l / 16;
  Frag<KIND> fa;
  load_frag_ptr<KIND>(fa, a + (t * 16 + r) * KindTraits<KIND>::STEP_BYTES, g);
  f32x4 acc;
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = c ? c[(t * 16 + 4 * g + i) * 16 + r] : 0.f;
  if constexpr (KIND == KIND_MX4) {
    FragB<KIND> fb;
    fb.c[0] = *reinterpret_cast<const uint4*>(b + (t * 16 + r) * 64 + 16 * g);
    acc = mfma_step_mx4(fa, fb, acc, sa[(t * 16 + r) * 4 + g], sb[(t * 16 + r) * 4 + g]);
  } else {
    Frag<KIND> fb;
    load_frag_ptr<KIND>(fb, b + (t * 16 + r) * KindTraits<KIND>::STEP_BYTES, g);
    if constexpr (KIND == KIND_MX)
      acc = mfma_step_mx(fa, fb, acc, sa[(t * 16 + r) * 4 + g], sb[(t * 16 + r) * 4 + g]);
    else
      acc = mfma_step<KIND>(fa, fb, acc);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) d[(t * 16 + 4 * g + i) * 16 + r] = acc[i];
}

}  // namespace

extern "C" int moe_mfma_probe(int32_t dtype, const void* a, const void* b, const uint8_t* a_scale,
                              const uint8_t* b_scale, const float* c, float* d, int64_t n_tiles,
                              void* stream) {
  if (dtype < MOE_BF16 || dtype > MOE_MXFP4) return MOE_ERR_UNSUPPORTED;
  if (n_tiles < 0 || n_tiles > (int64_t(1) << 24)) return MOE_ERR_SHAPE;
  if (n_tiles == 0) return MOE_OK;
  if (!a || !b || !d || ((dtype == MOE_MXFP8 || dtype == MOE_MXFP4) && (!a_scale || !b_scale)))
    return MOE_ERR_NULL;
  const void* ps[] = {a, b, c, d};
  for (const void* p : ps)
    if (p && reinterpret_cast<uintptr_t>(p) % 16) return MOE_ERR_ALIGN;
  const auto* A = static_cast<const uint8_t*>(a);
  const auto* B = static_cast<const uint8_t*>(b);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)n_tiles), block(64);
  switch (dtype) {
    case MOE_BF16:
      hipLaunchKernelGGL(k_probe<KIND_BF16>, grid, block, 0, st, A, B, a_scale, b_scale, c, d);
      break;
    case MOE_FP8_BLOCKWISE:
      hipLaunchKernelGGL(k_probe<KIND_FP8B>, grid, block, 0, st, A, B, a_scale, b_scale, c, d);
      break;
    case MOE_MXFP8:
      hipLaunchKernelGGL(k_probe<KIND_MX>, grid, block, 0, st, A, B, a_scale, b_scale, c, d);
      break;
    default:
      hipLaunchKernelGGL(k_probe<KIND_MX4>, grid, block, 0, st, A, B, a_scale, b_scale, c, d);
      break;
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
