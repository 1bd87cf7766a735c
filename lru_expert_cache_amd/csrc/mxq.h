// MX block quantisation of bf16 values (device code shared by the activation
// quantiser and the gate/up GEMM's epilogue, so that both give the same codes):
// one 32-element block gets X = 2^(floor(log2 amax) - emax_elem) as its E8M0
// scale (2^-127 for an all-zero block) and each element v / X rounded to
// nearest-even on the element grid, saturated at +-max (OCP Microscaling
// Formats v1.0, the rule for a block of scalars; E2M1: emax 2, max 6; E4M3:
// emax 8, max 448).  The bf16 inputs and power-of-two X make v / X exact.
#pragma once
#include "common.h"
#include "gmem.h"

namespace ftmoe {
namespace mxq {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short short2v __attribute__((ext_vector_type(2)));

__device__ inline float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// floor(log2(a)) for a > 0 (normal or subnormal fp32)
__device__ inline int ilog2f(float a) {
  int e;
  (void)frexpf(a, &e);
  return e - 1;
}

// Element codes from gfx950's scaled down-converts: v_cvt_scalef32_pk_fp4_f32
// and _pk_fp8_f32 compute v / X with round-to-nearest-even on the element grid
// (X a power of two, read from the exponent of the scale operand).  Measured
// against a plain software rounding for every finite bf16 input at X = 2^-127
// .. 2^127: identical codes once (a) FP8 inputs are clamped to +-448 X (the
// convert turns values past 448 into the NaN code, where the MX rule
// saturates; FP4 saturates at 6 by itself) and (b) a negative value that
// rounds to zero is given code +0 rather than -0 (the same number).
// 8 E2M1 codes (element 2i in the low nibble of byte i) with -0 made +0
__device__ inline uint32_t fp4x8(const float* v, float X) {
  uint32_t o = 0;
  o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, v[0], v[1], X, 0);
  o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, v[2], v[3], X, 1);
  o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, v[4], v[5], X, 2);
  o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, v[6], v[7], X, 3);
  // a nibble keeps its sign bit only if its magnitude bits are not all zero
  const uint32_t nz = ((o & 0x77777777u) + 0x77777777u) & 0x88888888u;
  return o & (nz | 0x77777777u);
}
// 4 E4M3 codes (element i in byte i), saturated at +-448, -0 made +0
__device__ inline uint32_t fp8x4(const float* v, float X) {
  const float lim = 448.0f * X;
  float c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) c[i] = fminf(fmaxf(v[i], -lim), lim);
  short2v lo = {0, 0};
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, c[0], c[1], X, false);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, c[2], c[3], X, true);
  const uint32_t o = uint32_t(uint16_t(lo[0])) | (uint32_t(uint16_t(lo[1])) << 16);
  const uint32_t nz = ((o & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) & 0x80808080u;
  return o & (nz | 0x7F7F7F7Fu);
}

// One 32-element block, given as 16 dwords of bf16 pairs (element 2i in the
// low half of dword i): its codes into out (FP4 4 dwords, FP8 8) and its
// E8M0 scale byte as the result.
template <bool FP4>
__device__ inline uint8_t quant_block(const uint32_t (&w)[16], uint32_t (&out)[FP4 ? 4 : 8]) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    amax = fmaxf(amax, fabsf(bf16_to_f32(w[i] & 0xFFFFu)));
    amax = fmaxf(amax, fabsf(bf16_to_f32(w[i] >> 16)));
  }
  const int emax = FP4 ? 2 : 8;
  int sexp = amax > 0.0f ? ilog2f(amax) - emax : -127;
  sexp = max(-127, min(127, sexp));
  const float X = ldexpf(1.0f, sexp);
  float v[32];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    v[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
    v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
  }
#pragma unroll
  for (int i = 0; i < (FP4 ? 4 : 8); ++i) out[i] = FP4 ? fp4x8(v + 8 * i, X) : fp8x4(v + 4 * i, X);
  return uint8_t(sexp + 127);
}

// Stores a quantised block into the MX GEMM's activation tile layout: block
// blk = (row tile, K step) of row i of the tile, 32-block q4 of the step.
template <bool FP4>
__device__ inline void store_tile_block(uint8_t* codes, uint8_t* scales, int64_t blk, int i, int q4,
                                        const uint32_t (&out)[FP4 ? 4 : 8], uint8_t sbyte) {
  scales[blk * kMxTileScaleBytes + i * 4 + q4] = sbyte;
  uint8_t* sub = codes + blk * mx_tile_code_bytes(FP4) + (i >> 4) * (FP4 ? 1024 : 2048);
  const int n = i & 15;
  if constexpr (FP4) {
    gstore<u32x4>(sub + (16 * q4 + n) * 16, u32x4{out[0], out[1], out[2], out[3]});
  } else {
    // K 32 q4 .. + 31 of the step: half q4 / 2, lanes q = 2 q4 - 4 h and q + 1
    const int h = q4 >> 1, q = 2 * q4 - 4 * h;
    gstore<u32x4>(sub + h * 1024 + (16 * q + n) * 16, u32x4{out[0], out[1], out[2], out[3]});
    gstore<u32x4>(sub + h * 1024 + (16 * (q + 1) + n) * 16, u32x4{out[4], out[5], out[6], out[7]});
  }
}

}  // namespace mxq
}  // namespace ftmoe
