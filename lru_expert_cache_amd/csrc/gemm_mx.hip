// Grouped expert GEMM of a prefill chunk on gfx950's block-scaled MFMA,
// v_mfma_scale_f32_16x16x128_f8f6f4, with MXFP4 weights and MX-quantised
// activations (MXFP4 or MXFP8, the prefill activation modes).
//
// Both operands arrive in the form the instruction takes, with no conversion:
//   A = a 16x128 weight tile of the device layout: lane 16q+r holds row r,
//       K 32q..32q+31 as 16 bytes of E2M1 codes, and its E8M0 scale byte;
//   B = 16 activation rows of the row-major quantised rows: lane 16q+n holds
//       row n and the row's E8M0 scale of 32-block q.  FP4: K 32q..32q+31 as
//       16 bytes (dwords 0-3).  FP8: the 8-bit operand splits K in two halves,
//       K 16q..16q+15 in dwords 0-3 and K 64+16q..64+16q+15 in dwords 4-7
//       (measured on gfx950 with an in-bounds probe of the instruction).
// One instruction multiplies a 16x128 weight tile by 128 K of 16 rows.
//
// Work: a list of (group, 64-row tile) built by the resolve kernel; grid =
// (list bound, output tiles of 128 features).  A workgroup of 4 waves owns
// 64 rows x 128 outputs; each wave 64 rows x 32 outputs (x2 matrices for
// gate/up), i.e. 8 or 16 MFMA per 128-K step.  Epilogues as the decode FFN:
// gate/up -> h = bf16(silu(g) * u); down -> p = bf16(w * y).
#include "common.h"

namespace ftmoe {

namespace {

typedef int intx8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kRowsPerTile = 64;   // activation rows per workgroup tile
constexpr int kTokT = kRowsPerTile / 16;
constexpr int kRowT = 2;           // 16-row weight tiles per wave per matrix
constexpr int kOutPerWG = 4 * kRowT * 16;  // 128

__device__ inline uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return uint16_t((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

template <bool GATEUP, bool ACT_FP4>
__global__ __launch_bounds__(256) void k_mx_gemm(MxGemmArgs a) {
  const int tile = blockIdx.x;
  if (tile >= *a.n_tiles_dev) return;
  const int d = a.tiles[2 * tile], tt0 = a.tiles[2 * tile + 1];
  const GroupDesc g = a.groups[d];
  const int r0 = tt0 * kRowsPerTile;
  if (r0 >= g.row_count) return;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane >> 4, n = lane & 15;
  constexpr int NM = GATEUP ? 2 : 1;
  const MatLayout& m0 = a.lay.m[GATEUP ? 0 : 2];
  const int K = m0.cols;
  const int nkb = K / kTileK;
  const int rb0 = blockIdx.y * (kOutPerWG / 16) + wave * kRowT;  // first 16-row weight tile of this wave
  const uint8_t* W = reinterpret_cast<const uint8_t*>(g.wptr);

  // activation rows of this lane, one per 16-row sub-tile
  int64_t arow[kTokT];
  bool valid[kTokT];
#pragma unroll
  for (int t = 0; t < kTokT; ++t) {
    const int r = r0 + t * 16 + n;
    valid[t] = r < g.row_count;
    const int row = g.row_begin + (valid[t] ? r : 0);
    arow[t] = GATEUP ? int64_t(a.row_tok[row]) : int64_t(row);
  }
  constexpr int CB = 16;  // activation code bytes per lane per 128-K step (FP8: per half)
  const int64_t act_pitch = ACT_FP4 ? K / 2 : K;

  floatx4 acc[NM][kRowT][kTokT];
#pragma unroll
  for (int mi = 0; mi < NM; ++mi)
#pragma unroll
    for (int rt = 0; rt < kRowT; ++rt)
#pragma unroll
      for (int t = 0; t < kTokT; ++t) acc[mi][rt][t] = {0.f, 0.f, 0.f, 0.f};

  for (int kb = 0; kb < nkb; ++kb) {
    intx8 A[NM][kRowT];
    int sa[NM][kRowT];
#pragma unroll
    for (int mi = 0; mi < NM; ++mi) {
      const MatLayout& m = a.lay.m[GATEUP ? mi : 2];
#pragma unroll
      for (int rt = 0; rt < kRowT; ++rt) {
        const int64_t tl = int64_t(rb0 + rt) * nkb + kb;
        const uint4 c = *reinterpret_cast<const uint4*>(W + m.codes_off + (tl * 64 + lane) * 16);
        A[mi][rt] = intx8{int(c.x), int(c.y), int(c.z), int(c.w), 0, 0, 0, 0};
        sa[mi][rt] = W[m.scales_off + tl * 64 + lane];
      }
    }
    intx8 B[kTokT];
    int sb[kTokT];
#pragma unroll
    for (int t = 0; t < kTokT; ++t) {
      if (valid[t]) {
        const uint8_t* p = a.act_codes + arow[t] * act_pitch + int64_t(kb) * (ACT_FP4 ? 64 : 128) + q * CB;
        const uint4 c0 = *reinterpret_cast<const uint4*>(p);
        if (ACT_FP4) {
          B[t] = intx8{int(c0.x), int(c0.y), int(c0.z), int(c0.w), 0, 0, 0, 0};
        } else {
          const uint4 c1 = *reinterpret_cast<const uint4*>(p + 64);
          B[t] = intx8{int(c0.x), int(c0.y), int(c0.z), int(c0.w), int(c1.x), int(c1.y), int(c1.z), int(c1.w)};
        }
        sb[t] = a.act_scales[arow[t] * (K / 32) + kb * 4 + q];
      } else {
        B[t] = intx8{0, 0, 0, 0, 0, 0, 0, 0};
        sb[t] = 127;
      }
    }
#pragma unroll
    for (int mi = 0; mi < NM; ++mi)
#pragma unroll
      for (int rt = 0; rt < kRowT; ++rt)
#pragma unroll
        for (int t = 0; t < kTokT; ++t)
          acc[mi][rt][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              A[mi][rt], B[t], acc[mi][rt][t], 4 /* A: fp4 e2m1 */, ACT_FP4 ? 4 : 0 /* B: fp4 or fp8 e4m3 */,
              0, sa[mi][rt], 0, sb[t]);
  }

  // epilogue: lane holds outputs (rb*16 + 4q + i) of row (r0 + t*16 + n)
#pragma unroll
  for (int t = 0; t < kTokT; ++t) {
    if (!valid[t]) continue;
    const int row = g.row_begin + r0 + t * 16 + n;
#pragma unroll
    for (int rt = 0; rt < kRowT; ++rt) {
      const int o0 = (rb0 + rt) * 16 + 4 * q;
      uint16_t hv[4];
      if constexpr (GATEUP) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float gv = acc[0][rt][t][i], uv = acc[1][rt][t][i];
          hv[i] = f32_to_bf16_rne(gv / (1.0f + expf(-gv)) * uv);
        }
        *reinterpret_cast<uint2*>(a.out + int64_t(row) * a.inter + o0) =
            make_uint2(uint32_t(hv[0]) | (uint32_t(hv[1]) << 16), uint32_t(hv[2]) | (uint32_t(hv[3]) << 16));
      } else {
        const float wr = a.row_w[row];
#pragma unroll
        for (int i = 0; i < 4; ++i) hv[i] = f32_to_bf16_rne(wr * acc[0][rt][t][i]);
        *reinterpret_cast<uint2*>(a.out + int64_t(row) * a.hidden + o0) =
            make_uint2(uint32_t(hv[0]) | (uint32_t(hv[1]) << 16), uint32_t(hv[2]) | (uint32_t(hv[3]) << 16));
      }
    }
  }
}

}  // namespace

int mx_gemm_rows_per_tile() { return kRowsPerTile; }

hipError_t launch_mx_gemm(const MxGemmArgs& a, bool gateup, bool act_fp4, hipStream_t s, Ev ev) {
  const int outs = gateup ? a.inter : a.hidden;
  if (outs % kOutPerWG) return hipErrorInvalidValue;
  const dim3 grid(a.max_tiles, outs / kOutPerWG);
  if (gateup) {
    if (act_fp4)
      ft_launch(k_mx_gemm<true, true>, grid, dim3(256), s, ev, a);
    else
      ft_launch(k_mx_gemm<true, false>, grid, dim3(256), s, ev, a);
  } else {
    if (act_fp4)
      ft_launch(k_mx_gemm<false, true>, grid, dim3(256), s, ev, a);
    else
      ft_launch(k_mx_gemm<false, false>, grid, dim3(256), s, ev, a);
  }
  return hipGetLastError();
}

}  // namespace ftmoe
