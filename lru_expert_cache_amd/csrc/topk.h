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

// Top-k of one token by one wavefront: k+1 rounds of a wave-wide argmax
// (larger logit first, lower expert index on ties).  Each lane keeps the best
// of its own logits (experts lane, lane+64, ...); a round reduces the 64 lane
// bests with DPP row permutations (quad xor 1, quad xor 2, half-row mirror,
// row mirror: every lane ends with the best of its row of 16) and the two row
// broadcasts (lane 15 of rows 0 and 2 into rows 1 and 3, then lane 31 into
// rows 2 and 3), reads lane 63, and only the winning lane refreshes its best.
// No LDS round trips and no divergent branches in the reduction.
// ROWS: rows of 16 lanes that take part (the others see their own value).
template <int CTRL, int ROWS = 0xF>
__device__ __attribute__((always_inline)) inline void dpp_best(double& v, int& i) {
  const uint64_t b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(int(uint32_t(b)), int(uint32_t(b)), CTRL, ROWS, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(int(uint32_t(b >> 32)), int(uint32_t(b >> 32)), CTRL, ROWS, 0xF, false);
  const int oi = __builtin_amdgcn_update_dpp(i, i, CTRL, ROWS, 0xF, false);
  const double ov = __longlong_as_double((int64_t(uint32_t(hi)) << 32) | uint32_t(lo));
  const bool take = (ov > v) | ((ov == v) & (oi < i));
  v = take ? ov : v;
  i = take ? oi : i;
}

__device__ __attribute__((always_inline)) inline double readlane_f64(double v, int src) {
  const uint64_t b = __double_as_longlong(v);
  const uint32_t lo = __builtin_amdgcn_readlane(uint32_t(b), src);
  const uint32_t hi = __builtin_amdgcn_readlane(uint32_t(b >> 32), src);
  return __longlong_as_double((int64_t(hi) << 32) | lo);
}

// kPer: logits per lane (E <= 64 * kPer).
// sel2 / w2 / gap2: optional second copy of the results (an LDS mirror), or null.
template <int kPer>
__device__ __attribute__((always_inline)) inline void wave_topk_n(const double* __restrict__ zrow, int E, int k,
                                                                  int32_t* __restrict__ sel, float* __restrict__ w,
                                                                  double* __restrict__ gap, int32_t* sel2,
                                                                  float* w2, double* gap2) {
  const int lane = threadIdx.x & 63;
  const double NEG = -__builtin_inf();
  double v[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = lane + 64 * j;
    const double x = e < E ? zrow[e] : NEG;
    v[j] = x == 0.0 ? 0.0 : x;  // -0 and +0 compare equal; keep one spelling
  }
  // this lane's best (value, expert)
  double bv = NEG;
  int bi = 0x7fffffff;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = lane + 64 * j;
    const bool take = (v[j] > bv) | ((v[j] == bv) & (e < bi));
    bv = take ? v[j] : bv;
    bi = take ? e : bi;
  }
  const int rounds = k < E ? k + 1 : k;
  double myz = 0.0, zk1 = 0.0, zk = 0.0;
  for (int r = 0; r < rounds; ++r) {
    double rv = bv;
    int ri = bi;
    dpp_best<0xB1>(rv, ri);        // quad_perm [1,0,3,2]
    dpp_best<0x4E>(rv, ri);        // quad_perm [2,3,0,1]
    dpp_best<0x141>(rv, ri);       // row_half_mirror
    dpp_best<0x140>(rv, ri);       // row_mirror: every lane holds its row's best
    dpp_best<0x142, 0xA>(rv, ri);  // row_bcast:15 into rows 1 and 3
    dpp_best<0x143, 0xC>(rv, ri);  // row_bcast:31 into rows 2 and 3: lane 63 holds the best
    const double wv = readlane_f64(rv, 63);
    const int wi = __builtin_amdgcn_readlane(ri, 63);
    if (r < k && lane == 0) {
      sel[r] = wi;
      if (sel2) sel2[r] = wi;
    }
    if (lane == r) myz = wv;
    if (r == k - 1) zk1 = wv;
    if (r == k) zk = wv;
    if ((wi & 63) == lane) {  // the winner drops the taken logit and refreshes its best
      bv = NEG;
      bi = 0x7fffffff;
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int e = lane + 64 * j;
        if (e == wi) v[j] = NEG;
        const bool take = (v[j] > bv) | ((v[j] == bv) & (e < bi));
        bv = take ? v[j] : bv;
        bi = take ? e : bi;
      }
    }
  }
  // weights: lane j < k holds the logit of rank j
  const double f0 = double(float(readlane_f64(myz, 0)));
  const double ex = lane < k ? exp(double(float(myz)) - f0) : 0.0;
  double den = 0.0;
  for (int j = 0; j < k; ++j) den += readlane_f64(ex, j);
  if (lane < k) {
    w[lane] = float(ex / den);
    if (w2) w2[lane] = float(ex / den);
  }
  if (lane == 0) {
    *gap = k < E ? zk1 - zk : __builtin_inf();
    if (gap2) *gap2 = k < E ? zk1 - zk : __builtin_inf();
  }
}

__device__ __attribute__((always_inline)) inline void wave_topk(const double* __restrict__ zrow, int E, int k,
                                                                int32_t* __restrict__ sel, float* __restrict__ w,
                                                                double* __restrict__ gap, int32_t* sel2 = nullptr,
                                                                float* w2 = nullptr, double* gap2 = nullptr) {
  static_assert(kMaxExperts <= 512, "at most 8 logits per lane");
  if (E <= 128)
    wave_topk_n<2>(zrow, E, k, sel, w, gap, sel2, w2, gap2);
  else if (E <= 256)
    wave_topk_n<4>(zrow, E, k, sel, w, gap, sel2, w2, gap2);
  else
    wave_topk_n<8>(zrow, E, k, sel, w, gap, sel2, w2, gap2);
}

}  // namespace ftmoe
