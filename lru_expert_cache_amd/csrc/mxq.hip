// MX activation quantiser: bf16 rows -> element codes + one E8M0 scale per 32
// elements along the row (OCP Microscaling Formats v1.0, "conversion from a
// vector of scalars": X = 2^(floor(log2 amax) - emax_elem); each element is
// v / X rounded to nearest-even on the element grid and clamped to +-max;
// an all-zero block gets scale 2^-127).  Used by the prefill activation
// modes, where both the expert inputs x and the SwiGLU outputs h are fed to
// the block-scaled MFMA as MXFP4 (E2M1, emax 2, max 6) or MXFP8 (E4M3,
// emax 8, max 448).  Every step is exact in fp32: the inputs are bf16, the
// scale is a power of two and the grid rounding uses rintf.
//
// Output layout (row-major, the B operand of v_mfma_scale_f32_16x16x128_f8f6f4
// as stored): FP4 codes [R][K/2] (even element in the low nibble), FP8 codes
// [R][K]; scales [R][K/32].
#include "common.h"

namespace ftmoe {

namespace {

__device__ inline float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// floor(log2(a)) for a > 0 (normal or subnormal fp32)
__device__ inline int ilog2f(float a) {
  int e;
  (void)frexpf(a, &e);
  return e - 1;
}

// E2M1 code of a (already scaled) value: nearest-even on {0,.5,1,1.5,2,3,4,6}, clamped.
__device__ inline uint32_t to_e2m1(float v) {
  const float a = fabsf(v);
  uint32_t code;
  if (!(a > 0.0f)) {
    code = 0;
  } else {
    const int e = max(ilog2f(a), 0);
    const float q = ldexpf(1.0f, e - 1);
    float r = rintf(a / q) * q;
    r = fminf(r, 6.0f);
    // magnitude -> 3-bit code
    if (r < 1.0f)
      code = r > 0.0f ? 1u : 0u;  // 0.5 -> 1
    else {
      const int er = ilog2f(r);             // 0, 1 or 2
      const uint32_t m = (r > ldexpf(1.0f, er)) ? 1u : 0u;  // 1.5 * 2^er
      code = uint32_t(er + 1) * 2u + m;
    }
    if (v < 0.0f && code) code |= 8u;
  }
  return code;
}

// E4M3 ("FN") code of a scaled value: nearest-even, clamped to +-448.
__device__ inline uint32_t to_e4m3(float v) {
  const float a = fabsf(v);
  if (!(a > 0.0f)) return 0;
  const int e = max(ilog2f(a), -6);
  const float q = ldexpf(1.0f, e - 3);
  float r = rintf(a / q) * q;
  r = fminf(r, 448.0f);
  uint32_t code;
  if (r == 0.0f) {
    code = 0;
  } else {
    const int er = ilog2f(r);
    if (er < -6) {
      code = uint32_t(r * 512.0f);  // subnormal: m * 2^-9
    } else {
      const uint32_t m = uint32_t((r / ldexpf(1.0f, er) - 1.0f) * 8.0f);
      code = (uint32_t(er + 7) << 3) | m;
    }
  }
  return (v < 0.0f ? 0x80u : 0u) | code;
}

// One thread per 32-element block.
template <bool FP4>
__global__ __launch_bounds__(256) void k_mx_quant(const uint16_t* __restrict__ in, int rows, int K,
                                                  uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int nblk = K / 32;
  const int64_t b = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (b >= int64_t(rows) * nblk) return;
  const int64_t row = b / nblk;
  const int kb = int(b % nblk);
  const uint4* src = reinterpret_cast<const uint4*>(in + row * K + int64_t(kb) * 32);
  uint32_t w[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = src[i];
    w[4 * i] = v.x;
    w[4 * i + 1] = v.y;
    w[4 * i + 2] = v.z;
    w[4 * i + 3] = v.w;
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    amax = fmaxf(amax, fabsf(bf16_to_f32(w[i] & 0xFFFFu)));
    amax = fmaxf(amax, fabsf(bf16_to_f32(w[i] >> 16)));
  }
  const int emax = FP4 ? 2 : 8;
  int sexp = amax > 0.0f ? ilog2f(amax) - emax : -127;
  sexp = max(-127, min(127, sexp));
  scales[row * nblk + kb] = uint8_t(sexp + 127);
  if (FP4) {
    uint32_t out[4] = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t c0 = to_e2m1(ldexpf(bf16_to_f32(w[i] & 0xFFFFu), -sexp));
      const uint32_t c1 = to_e2m1(ldexpf(bf16_to_f32(w[i] >> 16), -sexp));
      out[i / 4] |= (c0 | (c1 << 4)) << (8 * (i % 4));
    }
    *reinterpret_cast<uint4*>(codes + row * (K / 2) + int64_t(kb) * 16) = make_uint4(out[0], out[1], out[2], out[3]);
  } else {
    uint32_t out[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t c0 = to_e4m3(ldexpf(bf16_to_f32(w[i] & 0xFFFFu), -sexp));
      const uint32_t c1 = to_e4m3(ldexpf(bf16_to_f32(w[i] >> 16), -sexp));
      out[i / 2] |= (c0 | (c1 << 8)) << (16 * (i % 2));
    }
    uint4* dst = reinterpret_cast<uint4*>(codes + row * K + int64_t(kb) * 32);
    dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
    dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
  }
}

}  // namespace

hipError_t launch_mx_quant(const uint16_t* in, int rows, int K, bool fp4, uint8_t* codes, uint8_t* scales,
                           hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int64_t blocks = int64_t(rows) * (K / 32);
  const dim3 grid(unsigned((blocks + 255) / 256));
  if (fp4)
    hipLaunchKernelGGL(k_mx_quant<true>, grid, dim3(256), 0, s, in, rows, K, codes, scales);
  else
    hipLaunchKernelGGL(k_mx_quant<false>, grid, dim3(256), 0, s, in, rows, K, codes, scales);
  return hipGetLastError();
}

}  // namespace ftmoe
