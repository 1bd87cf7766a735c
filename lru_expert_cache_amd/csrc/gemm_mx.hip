// Grouped expert GEMM of a prefill chunk on gfx950's block-scaled MFMA,
// v_mfma_scale_f32_16x16x128_f8f6f4, with MXFP4 weights and MX-quantised
// activations (MXFP4 or MXFP8, the prefill activation modes).
//
// Both operands reach the instruction in the form it takes, with no conversion:
//   A = a 16x128 weight tile of the device layout: lane 16q+r holds row r,
//       K 32q..32q+31 as 16 bytes of E2M1 codes, and its E8M0 scale byte;
//   B = 16 activation rows: lane 16q+n holds row n and the row's E8M0 scale of
//       32-block q.  FP4: K 32q..32q+31 as 16 bytes (dwords 0-3).  FP8: the
//       8-bit operand splits K in two halves, K 16q..16q+15 in dwords 0-3 and
//       K 64+16q..64+16q+15 in dwords 4-7 (measured on gfx950 with an
//       in-bounds probe of the instruction).
// One instruction multiplies a 16x128 weight tile by 128 K of 16 rows.
//
// Work: a list of (group, 128-row tile) built by the resolve kernel; grid =
// (list bound, blocks of output features).  A workgroup computes 128 rows x
// 128 features (down) or 128 rows x 64 features of both matrices (gate/up);
// each of its 4 waves owns 64 rows x 64 accumulator columns, i.e. 16 MFMA per
// 128-K step, and eight 16x128 weight tiles are staged per step either way.
// Per K step the workgroup stages
// the weight tiles (in the A-operand layout, 1 KB per 16-row tile) and the
// activation rows (scattered into the B-operand lane layout) in LDS; the next
// step's global loads are in flight in registers while the MFMAs run.
// Activation rows past the group's end read a valid dummy line: they only
// feed output columns that are not written.  Epilogues as the decode FFN:
// gate/up -> h = bf16(silu(g) * u); down -> p = bf16(w * y).
#include "common.h"
#include "gmem.h"

namespace ftmoe {

namespace {

typedef int intx8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRowsPerTile = 128;  // activation rows per workgroup tile
// weight tiles of 16 features per wave and per matrix (64 accumulator columns a wave)
constexpr int feat_tiles(bool gateup) { return gateup ? 2 : 4; }
// output features per workgroup (per matrix)
constexpr int feat_per_wg(bool gateup) { return 2 * feat_tiles(gateup) * 16; }

__device__ inline uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return uint16_t((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

template <bool GATEUP, bool ACT_FP4>
struct MxSmem {
  static constexpr int BB = ACT_FP4 ? 16 : 32;  // B bytes per lane
  u32x4 a[2][8][64];                             // 8 weight tiles, A-operand layout
  uint8_t as[2][8][64];                          // their scale bytes
  u32x4 b[2][8][64 * (BB / 16)];                 // 8 sub-tiles of 16 rows, B-operand layout
  uint8_t bs[2][8][64];                          // row scales: [sub-tile][16q + n]
};

template <bool GATEUP, bool ACT_FP4>
__global__ __launch_bounds__(256, 2) void k_mx_gemm(MxGemmArgs a) {
  constexpr int NM = GATEUP ? 2 : 1;
  constexpr int FT = feat_tiles(GATEUP);
  constexpr int BQ = ACT_FP4 ? 1 : 2;  // u32x4 per lane of a B operand
  __shared__ MxSmem<GATEUP, ACT_FP4> sm;

  const int tile = blockIdx.x;
  if (tile >= *a.n_tiles_dev) return;
  const int d = a.tiles[2 * tile], tt0 = a.tiles[2 * tile + 1];
  const GroupDesc g = a.groups[d];
  const int r0 = tt0 * kRowsPerTile;
  if (r0 >= g.row_count) return;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int q = lane >> 4, n = lane & 15;
  const int th = w & 1, fh = w >> 1;  // this wave: rows th*64.., features fh*64..
  const MatLayout& m0 = a.lay.m[GATEUP ? 0 : 2];
  const int K = m0.cols;
  const int nkb = K / kTileK;
  const int fb = blockIdx.y;  // feature block: weight tiles fb*2*FT .. of each matrix
  const uint8_t* W = reinterpret_cast<const uint8_t*>(g.wptr);
  const int64_t act_pitch = ACT_FP4 ? K / 2 : K;
  const int64_t sc_pitch = K / 32;

  // rows this thread loads: FP4 rounds of 64 rows x 4 chunks, FP8 rounds of 32 rows x 8 chunks
  constexpr int BR = ACT_FP4 ? 2 : 4;  // load rounds for the B codes
  int64_t brow[BR];
#pragma unroll
  for (int r = 0; r < BR; ++r) {
    const int tok = ACT_FP4 ? r * 64 + (tid >> 2) : r * 32 + (tid >> 3);
    const int rr = r0 + tok;
    const bool ok = rr < g.row_count;
    const int row = g.row_begin + (ok ? rr : 0);
    brow[r] = ok ? (GATEUP ? int64_t(a.row_tok[row]) : int64_t(row)) : -1;
  }
  int64_t srow = -1;  // scale row of threads 0..127
  if (tid < kRowsPerTile) {
    const int rr = r0 + tid;
    if (rr < g.row_count) {
      const int row = g.row_begin + rr;
      srow = GATEUP ? int64_t(a.row_tok[row]) : int64_t(row);
    }
  }

  // the 8 staged weight tiles: chunk ci = matrix (ci / (2 FT)), tile fb*2*FT + ci % (2 FT)
  auto chunk_mat = [&](int ci) -> const MatLayout& { return a.lay.m[GATEUP ? ci / (2 * FT) : 2]; };
  auto chunk_tile = [&](int ci, int kb) -> int64_t {
    return int64_t(fb * 2 * FT + ci % (2 * FT)) * nkb + kb;
  };
  // one K step's global reads, held in registers until they go to LDS
  u32x4 ga[2];
  u32x4 gas = {0u, 0u, 0u, 0u};
  u32x4 gb[BR];
  uint32_t gbs = 0;
  auto load = [&](int kb) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int ci = r * 4 + (tid >> 6);
      ga[r] = gload<u32x4>(W + chunk_mat(ci).codes_off + chunk_tile(ci, kb) * 1024 + lane * 16);
    }
    if (tid < 32) {
      const int ci = tid >> 2, part = tid & 3;
      gas = gload<u32x4>(W + chunk_mat(ci).scales_off + chunk_tile(ci, kb) * 64 + part * 16);
    }
#pragma unroll
    for (int r = 0; r < BR; ++r) {
      const int c = ACT_FP4 ? (tid & 3) : (tid & 7);
      const uint8_t* p = brow[r] >= 0
                             ? a.act_codes + brow[r] * act_pitch + int64_t(kb) * (ACT_FP4 ? 64 : 128) + c * 16
                             : a.act_codes;
      gb[r] = *reinterpret_cast<const u32x4*>(p);
    }
    if (tid < kRowsPerTile)
      gbs = *reinterpret_cast<const uint32_t*>(srow >= 0 ? a.act_scales + srow * sc_pitch + kb * 4 : a.act_scales);
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int r = 0; r < 2; ++r) sm.a[buf][r * 4 + (tid >> 6)][lane] = ga[r];
    if (tid < 32) *reinterpret_cast<u32x4*>(&sm.as[buf][tid >> 2][(tid & 3) * 16]) = gas;
#pragma unroll
    for (int r = 0; r < BR; ++r) {
      if constexpr (ACT_FP4) {
        const int tok = r * 64 + (tid >> 2), c = tid & 3;
        sm.b[buf][tok >> 4][16 * c + (tok & 15)] = gb[r];
      } else {
        const int tok = r * 32 + (tid >> 3), c = tid & 7;
        sm.b[buf][tok >> 4][2 * (16 * (c & 3) + (tok & 15)) + (c >> 2)] = gb[r];
      }
    }
    if (tid < kRowsPerTile) {
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) sm.bs[buf][tid >> 4][16 * qq + (tid & 15)] = uint8_t(gbs >> (8 * qq));
    }
  };

  floatx4 acc[NM][FT][4];
#pragma unroll
  for (int mi = 0; mi < NM; ++mi)
#pragma unroll
    for (int ft = 0; ft < FT; ++ft)
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[mi][ft][t] = {0.f, 0.f, 0.f, 0.f};

  load(0);
  store(0);
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < nkb) load(kb + 1);
    intx8 B[4];
    int sb[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int st = th * 4 + t;
      const u32x4 lo = sm.b[buf][st][BQ * lane];
      if constexpr (ACT_FP4) {
        B[t] = intx8{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]), 0, 0, 0, 0};
      } else {
        const u32x4 hi = sm.b[buf][st][BQ * lane + 1];
        B[t] = intx8{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]), int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};
      }
      sb[t] = sm.bs[buf][st][lane];
    }
#pragma unroll
    for (int mi = 0; mi < NM; ++mi)
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) {
        const int ci = mi * 2 * FT + fh * FT + ft;
        const u32x4 c = sm.a[buf][ci][lane];
        const intx8 A = intx8{int(c[0]), int(c[1]), int(c[2]), int(c[3]), 0, 0, 0, 0};
        const int sa = sm.as[buf][ci][lane];
#pragma unroll
        for (int t = 0; t < 4; ++t)
          acc[mi][ft][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              A, B[t], acc[mi][ft][t], 4 /* A: fp4 e2m1 */, ACT_FP4 ? 4 : 0 /* B: fp4 or fp8 e4m3 */, 0, sa, 0,
              sb[t]);
      }
    if (kb + 1 < nkb) store(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds features (fb*2*FT*16 + fh*FT*16 + ft*16 + 4q + i) of row (r0 + th*64 + t*16 + n)
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int r = r0 + th * 64 + t * 16 + n;
    if (r >= g.row_count) continue;
    const int row = g.row_begin + r;
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) {
      const int o0 = fb * feat_per_wg(GATEUP) + fh * FT * 16 + ft * 16 + 4 * q;
      uint16_t hv[4];
      if constexpr (GATEUP) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float gv = acc[0][ft][t][i], uv = acc[1][ft][t][i];
          hv[i] = f32_to_bf16_rne(gv / (1.0f + expf(-gv)) * uv);
        }
        *reinterpret_cast<uint2*>(a.out + int64_t(row) * a.inter + o0) =
            make_uint2(uint32_t(hv[0]) | (uint32_t(hv[1]) << 16), uint32_t(hv[2]) | (uint32_t(hv[3]) << 16));
      } else {
        const float wr = a.row_w[row];
#pragma unroll
        for (int i = 0; i < 4; ++i) hv[i] = f32_to_bf16_rne(wr * acc[0][ft][t][i]);
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
  if (outs % feat_per_wg(gateup)) return hipErrorInvalidValue;
  const dim3 grid(a.max_tiles, outs / feat_per_wg(gateup));
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
