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
// Output: the MX GEMM's activation tiles (see MxQuantArgs): each source row
// is quantised once and written to the tile slot of every grouped row that
// reads it (the k expert rows of a token, and its shared-expert row).
#include "common.h"
#include "gmem.h"

namespace ftmoe {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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

// One thread per 32-element block of a source row: quantise it, then store
// its codes and scale byte at each destination slot.
template <bool FP4>
__global__ __launch_bounds__(256) void k_mx_quant_tiles(MxQuantArgs a) {
  const int nblk = a.K / 32, nkb = a.K / 128;
  const int64_t b = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (b >= int64_t(a.rows) * nblk) return;
  const int64_t row = b / nblk;
  const int kb32 = int(b % nblk);
  const uint4* src = reinterpret_cast<const uint4*>(a.in + row * a.K + int64_t(kb32) * 32);
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
  const uint8_t sbyte = uint8_t(sexp + 127);
  // codes: FP4 16 bytes (K 32 kb32 .. + 31), FP8 32 bytes
  uint32_t out[FP4 ? 4 : 8] = {};
  if constexpr (FP4) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t c0 = to_e2m1(ldexpf(bf16_to_f32(w[i] & 0xFFFFu), -sexp));
      const uint32_t c1 = to_e2m1(ldexpf(bf16_to_f32(w[i] >> 16), -sexp));
      out[i / 4] |= (c0 | (c1 << 4)) << (8 * (i % 4));
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t c0 = to_e4m3(ldexpf(bf16_to_f32(w[i] & 0xFFFFu), -sexp));
      const uint32_t c1 = to_e4m3(ldexpf(bf16_to_f32(w[i] >> 16), -sexp));
      out[i / 2] |= (c0 | (c1 << 8)) << (16 * (i % 2));
    }
  }
  // block kb32 = step kb, 32-block q4 of the step
  const int kb = kb32 >> 2, q4 = kb32 & 3;
  auto put = [&](int slot) {
    const int tile = slot / kMxTileRows, i = slot - tile * kMxTileRows;
    const int64_t blk = int64_t(tile) * nkb + kb;
    a.out_scales[blk * kMxTileScaleBytes + i * 4 + q4] = sbyte;
    uint8_t* sub = a.out_codes + blk * mx_tile_code_bytes(FP4) + (i >> 4) * (FP4 ? 1024 : 2048);
    const int n = i & 15;
    if constexpr (FP4) {
      gstore<u32x4>(sub + (16 * q4 + n) * 16, u32x4{out[0], out[1], out[2], out[3]});
    } else {
      // K 32 q4 .. + 31 of the step: half q4 / 2, lanes q = 2 q4 - 4 h and q + 1
      const int h = q4 >> 1, q = 2 * q4 - 4 * h;
      gstore<u32x4>(sub + h * 1024 + (16 * q + n) * 16, u32x4{out[0], out[1], out[2], out[3]});
      gstore<u32x4>(sub + h * 1024 + (16 * (q + 1) + n) * 16, u32x4{out[4], out[5], out[6], out[7]});
    }
  };
  if (a.pair_row) {
    for (int j = 0; j < a.k; ++j) put(a.row_slot[a.pair_row[row * a.k + j]]);
    if (a.shared_row0 >= 0) put(a.row_slot[a.shared_row0 + row]);
  } else {
    put(a.row_slot[row]);
  }
}

}  // namespace

hipError_t launch_mx_quant_tiles(const MxQuantArgs& a, bool fp4, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  if (a.K % 128) return hipErrorInvalidValue;
  const int64_t blocks = int64_t(a.rows) * (a.K / 32);
  const dim3 grid(unsigned((blocks + 255) / 256));
  if (fp4)
    hipLaunchKernelGGL(k_mx_quant_tiles<true>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_mx_quant_tiles<false>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace ftmoe
