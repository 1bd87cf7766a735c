// Per-token top-k with renormalised softmax weights, one wavefront per token.
// Shared by the stand-alone top-k kernel and the resolve kernel.
//
// Selection: the k largest fp64 logits, larger first, lower expert index on
// ties.  Weights: softmax of the selected logits after rounding them to fp32,
// evaluated in fp64 and rounded to fp32 (equal to the full softmax
// renormalised over the top-k).  The gap between ranks k and k+1 is reported
// so callers can check that the selection is not decided by rounding.
#pragma once

#include "common.h"

namespace ftmoe {

// Top-k of one token by one wavefront: each lane holds up to 8 logits; k
// rounds of a wave-wide argmax (larger logit first, lower index on ties), then
// one more for the gap to rank k+1.  Lane 0 writes sel[0..k), w[0..k), *gap.
__device__ inline void wave_topk(const double* __restrict__ zrow, int E, int k, int32_t* __restrict__ sel,
                          float* __restrict__ w, double* __restrict__ gap) {
  const int lane = threadIdx.x & 63;
  constexpr int kPer = kMaxExperts / 64;
  const double NEG = -__builtin_inf();
  double v[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? zrow[e] : NEG;
  }
  double zsel[kMaxTopK + 1];
  int isel[kMaxTopK + 1];
  double zk1 = 0.0, zk = 0.0;
  const int rounds = k < E ? k + 1 : k;
#pragma unroll
  for (int r = 0; r < kMaxTopK + 1; ++r) {
    if (r < rounds) {
      double bv = NEG;
      int bi = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int e = lane + 64 * i;
        if (e < E && v[i] != NEG && (v[i] > bv || (v[i] == bv && e < bi))) {
          bv = v[i];
          bi = e;
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const double ov = __shfl_xor(bv, off, 64);
        const int oi = __shfl_xor(bi, off, 64);
        if (ov > bv || (ov == bv && oi < bi)) {
          bv = ov;
          bi = oi;
        }
      }
      zsel[r] = bv;
      isel[r] = bi;
      if (r == k - 1) zk1 = bv;
      if (r == k) zk = bv;
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        if (lane + 64 * i == bi) v[i] = NEG;
    }
  }
  if (lane == 0) {
    const double z0 = double(float(zsel[0]));
    double ex[kMaxTopK];
    double den = 0.0;
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j < k) {
        ex[j] = exp(double(float(zsel[j])) - z0);
        den += ex[j];
      }
    }
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j < k) {
        sel[j] = isel[j];
        w[j] = float(ex[j] / den);
      }
    }
    *gap = k < E ? zk1 - zk : __builtin_inf();
  }
}

}  // namespace ftmoe
