// Measured issue rate of the matrix-core instructions the expert kernels use,
// the measured denominator beside the data-sheet peaks: every wave issues
// rounds of independent MFMAs on register operands (no memory traffic inside
// the loop), over enough workgroups to fill every SIMD several times.
#include <hip/hip_runtime.h>

#include "common.h"

namespace ftmoe {

namespace {

typedef int intx8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef short bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kPeakBlocks = 1024, kPeakThreads = 256;

// KIND 0: scaled 32x32x64, FP4 x FP4; KIND 3: 32x32x16 bf16 (4 accumulators
// of 16 values each); KIND 1: scaled 16x16x128, FP8 x FP8; KIND 2: 16x16x32
// bf16 (8 of 4 each); KIND 4: 16x16x4 fp64, the router's (8 of 4 doubles).
// Operands depend on the lane and the seed, so nothing folds; the sums are
// written out so that nothing is dead.
template <int KIND>
__global__ __launch_bounds__(kPeakThreads) void k_mfma_peak(float* out, int iters, int seed) {
  const int v = int(threadIdx.x) ^ seed;
  const intx8 A = {v, v + 1, v + 2, v + 3, v + 4, v + 5, v + 6, v + 7};
  const intx8 B = {v * 3, v * 5, v * 7, v * 9, v, v, v, v};
  float s = 0.f;
  if constexpr (KIND == 4) {
    typedef double f64x4 __attribute__((ext_vector_type(4)));
    const double a = double(v) * 0.5, b = double(v) * 0.25 + 1.0;
    f64x4 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = {0.0, 0.0, 0.0, 0.0};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, acc[i], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 8; ++i) s += float(acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3]);
  } else if constexpr (KIND == 0 || KIND == 3) {
    const bf16x8 a16 = {short(v), 1, 2, 3, 4, 5, 6, 7}, b16 = {short(v), 7, 6, 5, 4, 3, 2, 1};
    floatx16 acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[i][j] = 0.f;
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (KIND == 0)
          acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, acc[i], 4, 4, 0, 127, 0, 127);
        else
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a16, b16, acc[i], 0, 0, 0);
      }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 16; ++j) s += acc[i][j];
  } else {
    const bf16x8 a16 = {short(v), 1, 2, 3, 4, 5, 6, 7}, b16 = {short(v), 7, 6, 5, 4, 3, 2, 1};
    floatx4 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = {0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if constexpr (KIND == 1)
          acc[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, acc[i], 0, 0, 0, 127, 0, 127);
        else
          acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a16, b16, acc[i], 0, 0, 0);
      }
#pragma unroll
    for (int i = 0; i < 8; ++i) s += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
  }
  out[blockIdx.x * kPeakThreads + threadIdx.x] = s;
}

}  // namespace

// flops of one kernel run of the given kind
double mfma_peak_flops(int kind, int iters) {
  const double waves = double(kPeakBlocks) * (kPeakThreads / 64);
  if (kind == 0) return waves * iters * 4 * (32.0 * 32 * 64 * 2);
  if (kind == 3) return waves * iters * 4 * (32.0 * 32 * 16 * 2);
  if (kind == 1) return waves * iters * 8 * (16.0 * 16 * 128 * 2);
  if (kind == 4) return waves * iters * 8 * (16.0 * 16 * 4 * 2);
  return waves * iters * 8 * (16.0 * 16 * 32 * 2);
}

hipError_t launch_mfma_peak(int kind, int iters, int seed, float* out, hipStream_t s) {
  const dim3 g(kPeakBlocks), b(kPeakThreads);
  switch (kind) {
    case 0: hipLaunchKernelGGL(k_mfma_peak<0>, g, b, 0, s, out, iters, seed); break;
    case 1: hipLaunchKernelGGL(k_mfma_peak<1>, g, b, 0, s, out, iters, seed); break;
    case 2: hipLaunchKernelGGL(k_mfma_peak<2>, g, b, 0, s, out, iters, seed); break;
    case 3: hipLaunchKernelGGL(k_mfma_peak<3>, g, b, 0, s, out, iters, seed); break;
    case 4: hipLaunchKernelGGL(k_mfma_peak<4>, g, b, 0, s, out, iters, seed); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

size_t mfma_peak_out_bytes() { return size_t(kPeakBlocks) * kPeakThreads * sizeof(float); }

}  // namespace ftmoe
