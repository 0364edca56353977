// mfma_ceiling.hip -- sustained bf16 matrix-core rate on this card, for the
// benchmark's context figures (not part of the attention library).
//
// "Memory-bound vs compute-bound" (sections "Common mistakes" and
// "Measurement practice") recommends judging a kernel against a rate
// measured on the same card instead of the datasheet peak.  This kernel
// issues nothing but independent bf16 MFMAs on operands held in registers,
// so its rate is what the matrix cores sustain at the clock the card runs
// them at: with constant operands the datapath barely toggles, with random
// operands it draws the power real data draws.
//
// Each wave keeps independent accumulators (8 of 32x32, 16 of 16x16) and runs
// `iters` rounds (a multiple of 8) of as many MFMAs, 262144 flops a round, over
// 8 A and 8 B fragments loaded once from `src` (256 B per lane);
// the accumulators are summed into `dst` at the end so nothing is dead.
// Two workgroups of 4 waves per CU (two waves per SIMD), grid = 2 x CUs.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int SHAPE>
__global__ __launch_bounds__(256) void mfma_loop_kernel(const bf16x8* __restrict__ src,
                                                         float* __restrict__ dst, int iters) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  bf16x8 a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = src[(size_t)((wave * 16 + i) & 1023) * 64 + lane];
    b[i] = src[(size_t)((wave * 16 + 8 + i) & 1023) * 64 + lane];
  }
  float sum = 0.0f;
  if constexpr (SHAPE == 32) {
    f32x16 c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) c[i][e] = 0.0f;
    for (int it = 0; it < iters; it += 8) {
#pragma unroll
      for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int i = 0; i < 8; ++i)
          c[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[(i + r) & 7], c[i], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) sum += c[i][e];
  } else {
    f32x4 c[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) c[i][e] = 0.0f;
    for (int it = 0; it < iters; it += 8) {
#pragma unroll
      for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          c[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i & 7], b[(i + r) & 7], c[i], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) sum += c[i][e];
  }
  dst[(size_t)wave * 64 + lane] = sum;
}

}  // namespace

// Flops one call of mfma_ceiling_run performs (for the caller's rate).
extern "C" double mfma_ceiling_flops(int shape, int n_cu, int iters) {
  const double waves = 2.0 * n_cu * 4.0;
  const double per_round = shape == 32 ? 8.0 * 32 * 32 * 16 * 2 : 16.0 * 16 * 16 * 32 * 2;
  return waves * per_round * iters;
}

// Launch the loop on `stream`: shape 32 (v_mfma_f32_32x32x16_bf16) or 16
// (v_mfma_f32_16x16x32_bf16); src holds 1024 x 64 16-byte fragments (1 MiB),
// dst 2 n_cu x 4 x 64 floats.  Returns 0, or -1 on a bad argument or a
// failed launch.
extern "C" int mfma_ceiling_run(int shape, const void* src, float* dst, int n_cu, int iters,
                                hipStream_t stream) {
  if (!src || !dst || n_cu < 1 || iters < 8 || iters % 8 || (shape != 32 && shape != 16))
    return -1;
  const dim3 grid(2 * n_cu), block(256);
  if (shape == 32)
    hipLaunchKernelGGL(mfma_loop_kernel<32>, grid, block, 0, stream,
                       static_cast<const bf16x8*>(src), dst, iters);
  else
    hipLaunchKernelGGL(mfma_loop_kernel<16>, grid, block, 0, stream,
                       static_cast<const bf16x8*>(src), dst, iters);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
