// Grouped expert GEMM of a prefill chunk with MXFP4 weights, on gfx950's
// MFMA: bf16 activations (the default prefill mode) or MX-quantised ones
// (MXFP8 / MXFP4, the prefill activation modes).
//
// Operands, per 16-row sub-tile and 128-K step:
//   A = a 16x128 weight tile of the device layout: lane 16q+r holds row r,
//       K 32q..32q+31 as 16 bytes of E2M1 codes, and its E8M0 scale byte.
//   MX activations reach v_mfma_scale_f32_*_f8f6f4 as stored, with no
//       conversion: lane 16q+n holds activation row n and its E8M0 scale of
//       32-block q.  FP4: K 32q..32q+31 as 16 bytes (dwords 0-3).  FP8: the
//       8-bit operand splits K in two halves, K 16q..16q+15 in dwords 0-3 and
//       K 64+16q..64+16q+15 in dwords 4-7 (measured on gfx950 with an
//       in-bounds probe of the instruction).  FP4 x FP4 runs the 32x32x64 form
//       (operands regathered from the same stage), FP8 the 16x16x128 one.
//   bf16 activations run v_mfma_f32_16x16x32_bf16 four times per step: dword
//       j of a weight lane becomes the A operand after one scaled convert
//       (exact), and the B operand is K 32q+8j..+7 of row n, 16 bytes.
//
// Work: a list of (group, 128-row tile) built by the resolve kernel, times the
// blocks of output features; one workgroup per item, in an XCD-aware order.
// A workgroup of 2 WF waves computes 128 rows x 64 WF FX accumulator columns:
// each wave owns 64 rows x 64 FX columns (gate/up: 32 FX features of each
// matrix; FX = 2 with bf16 activations, else 1), and 4 WF FX weight tiles are
// staged per step.
//
// K steps stream through a ring of LDS stages filled by global-to-LDS loads
// (global_load_lds_dwordx4: lane i of a wave writes 16 bytes at the stage
// address + 16 i, so a 1 KB weight tile lands in the A-operand lane order as it
// is stored; so does a 1 KB activation piece of the MX tile layout that
// the quantiser and launch_mx_tile_gather write, and a quarter sub-tile of bf16
// rows when each lane reads its row's 16 bytes; the 4-byte form writes lane i
// at + 4 i and carries the rows' scale bytes).  Every load reads whole cache
// lines: the MX rows gathered by token (64 bytes of a row per step, and 4
// scale bytes) spread a step over ~3x the lines, which the L1's outstanding
// misses then limit.  Every wave issues the same number of loads
// per stage, so one immediate vmcnt wait plus a barrier makes a stage ready
// while the later stages stay in flight: a step waits for its own data, not a
// whole memory latency.  Steps past the end re-load the last step (never
// used), which keeps the counts exact; the ring is drained before the
// epilogue.  Activation rows past the group's end (zeros, stale codes or the
// group's first row) feed output columns that are not written.  Epilogues as
// the decode FFN: gate/up -> h = bf16(silu(g) * u); down -> p = bf16(w * y);
// the down output and the MX gate/up one are put together as a 128-row tile
// in the freed stage ring and written as whole 128-byte lines of their rows;
// with h tiles given, the MX gate/up output is quantised from that tile into
// the down GEMM's activation tiles instead (no bf16 h).
#include "common.h"
#include "gmem.h"
#include "mxq.h"

namespace ftmoe {

namespace {

typedef int intx8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short bf16x8 __attribute__((ext_vector_type(8)));
typedef short bf16x2 __attribute__((ext_vector_type(2)));

// activation operand (the prefill activation modes, FT_ACT_* >> 4)
constexpr int kActBf16 = 0, kActFp8 = 1, kActFp4 = 2;

constexpr int kRowsPerTile = kMxTileRows;  // activation rows per workgroup tile
// weight tiles of 16 features per wave and per matrix: 64 accumulator columns
// a wave, 64 FX with the feature multiplier FX (2 for bf16 activations)
constexpr int feat_tiles(bool gateup, int fx = 1) { return (gateup ? 2 : 4) * fx; }
// output features per workgroup (per matrix) with WF wave columns of 64 FX
// accumulator columns each (and two wave rows of 64 rows)
constexpr int feat_per_wg(bool gateup, int wf, int fx = 1) { return wf * feat_tiles(gateup, fx) * 16; }

__device__ inline uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return uint16_t((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// silu(g) = g / (1 + e^-g) from the hardware exp2 and reciprocal (each about
// 1 ulp in fp32), far inside the bf16 rounding of h that follows.  For
// g -> -inf, e^-g overflows to inf and the reciprocal gives 0 (silu -> -0).
__device__ inline float silu_fast(float g) {
  const float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
  return g * __builtin_amdgcn_rcpf(1.0f + e);
}

// 1 KB activation pieces of a step: FP4 the 8 sub-tiles of 16 rows, FP8 their
// halves, bf16 the 4 K quarters of each (one 16x16x32 B operand each)
constexpr int mx_pieces(int act) { return act == kActFp4 ? 8 : act == kActFp8 ? 16 : 32; }
// One K step's operands in LDS, in the order the MFMAs read them.
template <int ACT, int WF, int FX>
struct MxStage {
  u32x4 a[4 * WF * FX][64];                   // 4 WF FX weight tiles, A-operand lane order
  u32x4 b[8][mx_pieces(ACT) / 8 * 64];        // 16-row sub-tiles: FP4 [lane]; FP8 [half * 64 + lane];
                                              // bf16 [quarter * 64 + lane]
  uint8_t as[4 * WF * FX][64];                // weight scale bytes [tile][lane]
  uint32_t bs[ACT == kActBf16 ? 1 : kRowsPerTile];  // activation scales: row -> bytes of blocks 0..3
};
// ring depth: 4 with WF 2 FP4, 3 with WF 4 FP4 (two workgroups per CU either
// way); 2 with FP8 at WF 4 (34 KB stages: two workgroups per CU, measured
// 6-8% faster than one 16-wave workgroup with 3 stages) and with FX 2 (bf16,
// 66 KB stages); 3 otherwise
constexpr int mx_stages(int act, int wf, int fx) {
  return fx == 2 || (act == kActFp8 && wf == 4) ? 2 : wf == 2 && act == kActFp4 ? 4 : 3;
}
// waves per SIMD the register allocation must allow: 4 for the two 8-wave
// FP8 workgroups per CU (at most 128 registers a wave)
constexpr int mx_min_waves(int act, int wf) { return act == kActFp8 && wf == 4 ? 4 : 1; }
// loads per wave and stage: 2 FX weight tiles, their scales, the wave's share
// of the activation pieces (half a piece when there are more waves than
// pieces), and its share of the activation scales (none for bf16)
constexpr int mx_loads_per_stage(int act, int wf, int fx) {
  return 2 * fx + 1 + (mx_pieces(act) >= 2 * wf ? mx_pieces(act) / (2 * wf) : 1) + (act == kActBf16 ? 0 : 1);
}

// 8 FP4 codes (element 2i in the low nibble of byte i) x E8M0 scale -> 8 bf16,
// exact (the scaled convert applies the exponent of its scale operand)
__device__ inline bf16x8 fp4x8_to_bf16(uint32_t w, float s) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}
__device__ inline bf16x8 as_bf16x8(u32x4 v) {
  return bf16x8{short(v[0] & 0xFFFF), short(v[0] >> 16), short(v[1] & 0xFFFF), short(v[1] >> 16),
                short(v[2] & 0xFFFF), short(v[2] >> 16), short(v[3] & 0xFFFF), short(v[3] >> 16)};
}

// s_waitcnt immediate for vmcnt(n) (6-bit count: bits 3:0 and 15:14), no other waits
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

#define FT_L3 __attribute__((address_space(3)))
// global -> LDS: lane i writes 16 (or 4) bytes at dst + 16 i (+ 4 i); dst uniform over the wave
__device__ __attribute__((always_inline)) inline void lds_load16(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds((const FT_GLOBAL void*)src, (FT_L3 void*)dst, 16, 0, 0);
}
__device__ __attribute__((always_inline)) inline void lds_load4(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds((const FT_GLOBAL void*)src, (FT_L3 void*)dst, 4, 0, 0);
}

template <bool GATEUP, int ACT, int WF, int FX>
__global__ __launch_bounds__(128 * WF, mx_min_waves(ACT, WF)) void k_mx_gemm(MxGemmArgs a) {
  constexpr bool ACT_FP4 = ACT == kActFp4;
  constexpr int NM = GATEUP ? 2 : 1;
  constexpr int FT = feat_tiles(GATEUP, FX);
  constexpr int NW = 2 * WF;        // waves
  constexpr int TPM = WF * FT;      // weight tiles per matrix and workgroup
  constexpr int S = mx_stages(ACT, WF, FX);
  constexpr int LPS = mx_loads_per_stage(ACT, WF, FX);
  constexpr int TW = 2 * FX;        // weight tiles a wave loads per stage (one matrix)
  static_assert(FX == 1 || ACT == kActBf16, "wider wave tiles with bf16 activations only");
  static_assert(TPM % TW == 0, "a wave's weight tiles belong to one matrix");
  static_assert(ACT != kActBf16 || mx_pieces(ACT) % (4 * NW) == 0, "bf16: whole 16-row sub-tiles per wave");
  __shared__ MxStage<ACT, WF, FX> sm[S];

  // XCD-aware order: items (row tile, feature block) run row-tile-major, and
  // the item list is cut into 8 contiguous ranges, one per XCD (workgroups
  // are dispatched to the XCDs round-robin by linear id): an XCD runs all
  // feature blocks of a row tile (its activations stay in that XCD's L2), then
  // the next row tile of the same expert (whose weight tiles are still there).
  // Any dispatch order gives every item exactly once (the grid holds at least
  // 8 * ceil(items / 8) workgroups).
  const int nfb = (GATEUP ? a.inter : a.hidden) / feat_per_wg(GATEUP, WF, FX);  // feature blocks
  const int items = min(*a.n_tiles_dev, a.max_tiles) * nfb;
  const int lin = int(blockIdx.x), xcd = lin & 7, k = lin >> 3;
  const int p = int(int64_t(items) * xcd / 8) + k;
  if (p >= int(int64_t(items) * (xcd + 1) / 8)) return;
  const int tile = p / nfb;
  const int d = a.tiles[2 * tile], tt0 = a.tiles[2 * tile + 1];
  const GroupDesc g = a.groups[d];
  const int r0 = tt0 * kRowsPerTile;
  if (r0 >= g.row_count) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: layout reads stay scalar
  const int q = lane >> 4, n = lane & 15;
  const int th = w & 1, fh = w >> 1;  // this wave: rows th*64.., features fh*64..
  const MatLayout& m0 = a.lay.m[GATEUP ? 0 : 2];
  const int K = m0.cols;
  const int nkb = K / kTileK;
  const int fb = p - tile * nfb;  // feature block: weight tiles fb*TPM .. of each matrix
  const uint8_t* W = reinterpret_cast<const uint8_t*>(g.wptr);
  // this row tile's activation blocks, one per K step (contiguous sub-tiles
  // in B-operand lane order, then the rows' scales)
  const uint8_t* TB = a.act_codes + int64_t(tile) * nkb * mx_tile_code_bytes(ACT_FP4);
  const uint8_t* TS = a.act_scales + int64_t(tile) * nkb * kMxTileScaleBytes;
  // bf16 activations come straight from their rows (x by token, h by row):
  // this wave loads the 16-row sub-tiles w * SPW .. ; a lane's row start, the
  // group's first row standing in past its end (those outputs are not stored)
  constexpr int SPW = ACT == kActBf16 ? mx_pieces(ACT) / (4 * NW) : 1;
  const uint8_t* brow[SPW];
  if constexpr (ACT == kActBf16) {
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int r = r0 + 16 * (w * SPW + i) + n;
      const int row = g.row_begin + (r < g.row_count ? r : 0);
      const int64_t src = a.row_tok ? int64_t(a.row_tok[row]) : int64_t(row);
      brow[i] = reinterpret_cast<const uint8_t*>(a.act_rows + src * K);
    }
  }

  // the 4 WF FX staged weight tiles: chunk ci = matrix (ci / TPM), tile fb*TPM + ci % TPM
  auto chunk_mat = [&](int ci) -> const MatLayout& { return a.lay.m[GATEUP ? ci / TPM : 2]; };
  auto chunk_tile = [&](int ci, int kb) -> int64_t { return int64_t(fb * TPM + ci % TPM) * nkb + kb; };
  // scale bytes of this wave's TW tiles (one matrix), held before the K loop:
  // indexed by the wave, the layout would be re-read from the kernel
  // arguments at every step
  const uint8_t* const WS = W + chunk_mat(TW * w).scales_off;
  // one K step's loads into a stage: LPS per wave, whatever the wave
  auto issue = [&](int kb, MxStage<ACT, WF, FX>& st) {
#pragma unroll
    for (int j = 0; j < TW; ++j) {
      const int ci = TW * w + j;
      lds_load16(W + chunk_mat(ci).codes_off + chunk_tile(ci, kb) * 1024 + lane * 16, &st.a[ci][0]);
    }
    if (lane < 4 * TW) {
      // all tiles of this wave belong to one matrix: its layout is uniform
      const int ci = TW * w + (lane >> 2), part = lane & 3;
      lds_load16(WS + chunk_tile(ci, kb) * 64 + part * 16, &st.as[TW * w][0]);
    }
    if constexpr (ACT == kActBf16) {
      // quarter j of a sub-tile: lane 16 q + n reads its row's K 128 kb + 32 q + 8 j .. + 7
#pragma unroll
      for (int i = 0; i < SPW; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          lds_load16(brow[i] + (int64_t(kb) * kTileK + 32 * q + 8 * j) * 2, &st.b[w * SPW + i][j * 64]);
    } else {
      // activation piece pc (1 KB) of the tile layout lands at piece pc of st.b
      const uint8_t* tb = TB + int64_t(kb) * mx_tile_code_bytes(ACT_FP4) + lane * 16;
      u32x4* bb = &st.b[0][0];
      constexpr int PC = mx_pieces(ACT);
      if constexpr (PC >= NW) {
#pragma unroll
        for (int j = 0; j < PC / NW; ++j) lds_load16(tb + (w * (PC / NW) + j) * 1024, bb + (w * (PC / NW) + j) * 64);
      } else {
        // two waves per piece, half the lanes each (lane i still writes at + 16 i)
        if ((lane >> 5) == (w & 1)) lds_load16(tb + (w >> 1) * 1024, bb + (w >> 1) * 64);
      }
      constexpr int SL = kRowsPerTile / NW;  // rows of activation scales per wave
      if (lane < SL) lds_load4(TS + int64_t(kb) * kMxTileScaleBytes + (w * SL + lane) * 4, &st.bs[w * SL]);
    }
  };

  // FP8 activations: 16x16x128 MFMAs, bf16: 16x16x32 MFMAs, acc[matrix][16-feature tile][16-row tile];
  // FP4 x FP4: 32x32x64 MFMAs (measured 1.6x the 16x16x128 FP4 rate on gfx950),
  // acc32[matrix][32-feature block][32-row block]
  constexpr int NA = ACT_FP4 ? 1 : NM * FT * 4;
  constexpr int NB32 = ACT_FP4 ? NM * (FT / 2) * 2 : 1;
  floatx4 acc[NA];
  floatx16 acc32[NB32];
#pragma unroll
  for (int i = 0; i < NA; ++i) acc[i] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NB32; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc32[i][j] = 0.f;

#pragma unroll
  for (int s0 = 0; s0 < S - 1; ++s0) issue(min(s0, nkb - 1), sm[s0]);
  for (int kb = 0; kb < nkb; ++kb) {
    // this step's stage is complete for this wave once the S - 2 later stages
    // alone are outstanding; the barrier makes it complete for every wave and
    // ends every wave's reads of the stage the next loads overwrite
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((S - 2) * LPS));
    __builtin_amdgcn_s_barrier();
    issue(min(kb + S - 1, nkb - 1), sm[(kb + S - 1) % S]);
    const MxStage<ACT, WF, FX>& st = sm[kb % S];
    if constexpr (ACT == kActFp4) {
      // 32x32x64 operands gathered from the 16x16x128-ordered stage: lane l
      // takes row (or token) l % 32 -- tile (l % 32) / 16, row l % 16 -- and
      // the 32-K block 2h + l / 32 of the 128-K step (h = 0, 1)
      const int r16 = lane & 15, hi16 = (lane >> 4) & 1, kq = lane >> 5;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int qq = 2 * h + kq;
        intx8 B[2];
        int sb[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const int sti = th * 4 + rb * 2 + hi16;
          const u32x4 v = st.b[sti][16 * qq + r16];
          B[rb] = intx8{int(v[0]), int(v[1]), int(v[2]), int(v[3]), 0, 0, 0, 0};
          sb[rb] = reinterpret_cast<const uint8_t*>(st.bs)[(sti * 16 + r16) * 4 + qq];
        }
#pragma unroll
        for (int mi = 0; mi < NM; ++mi)
#pragma unroll
          for (int f2 = 0; f2 < FT / 2; ++f2) {
            const int ci = mi * TPM + fh * FT + 2 * f2 + hi16;
            const u32x4 c = st.a[ci][16 * qq + r16];
            const intx8 A = intx8{int(c[0]), int(c[1]), int(c[2]), int(c[3]), 0, 0, 0, 0};
            const int sa = st.as[ci][16 * qq + r16];
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
              floatx16& ac = acc32[(mi * (FT / 2) + f2) * 2 + rb];
              ac = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B[rb], ac, 4, 4, 0, sa, 0, sb[rb]);
            }
          }
      }
    } else if constexpr (ACT == kActFp8) {
      intx8 B[4];
      int sb[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int sti = th * 4 + t;
        const u32x4 lo = st.b[sti][lane];
        const u32x4 hi = st.b[sti][64 + lane];
        B[t] = intx8{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]), int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};
        sb[t] = reinterpret_cast<const uint8_t*>(st.bs)[(sti * 16 + n) * 4 + q];
      }
#pragma unroll
      for (int mi = 0; mi < NM; ++mi)
#pragma unroll
        for (int ft = 0; ft < FT; ++ft) {
          const int ci = mi * TPM + fh * FT + ft;
          const u32x4 c = st.a[ci][lane];
          const intx8 A = intx8{int(c[0]), int(c[1]), int(c[2]), int(c[3]), 0, 0, 0, 0};
          const int sa = st.as[ci][lane];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            floatx4& ac = acc[(mi * FT + ft) * 4 + t];
            ac = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B[t], ac, 4 /* A: fp4 e2m1 */,
                                                                 0 /* B: fp8 e4m3 */, 0, sa, 0, sb[t]);
          }
        }
    } else {
      // bf16 activations: 16x16x32 MFMAs.  A = dword j of a weight tile's lane
      // (row r, K 32 q + 8 j .. + 7 for lane 16 q + r) as bf16 with its scale;
      // B = quarter j of a row sub-tile (the same K, token n).  (The 32x32x16
      // form issues 1.4x as fast in a register-only loop, but this kernel ran
      // 3-5% slower with it on N(0,1) activations.)
      u32x4 c[NM * FT];
      float sa[NM * FT];
#pragma unroll
      for (int mi = 0; mi < NM; ++mi)
#pragma unroll
        for (int ft = 0; ft < FT; ++ft) {
          const int ci = mi * TPM + fh * FT + ft;
          c[mi * FT + ft] = st.a[ci][lane];
          sa[mi * FT + ft] = __uint_as_float(uint32_t(st.as[ci][lane]) << 23);  // E8M0: the exponent is used
        }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x8 B[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) B[t] = as_bf16x8(st.b[th * 4 + t][j * 64 + lane]);
#pragma unroll
        for (int i = 0; i < NM * FT; ++i) {
          const bf16x8 A = fp4x8_to_bf16(c[i][j], sa[i]);
#pragma unroll
          for (int t = 0; t < 4; ++t) acc[i * 4 + t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B[t], acc[i * 4 + t], 0, 0, 0);
        }
      }
    }
  }
  // the loads of steps past the end may still be writing LDS
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

  // epilogue: a lane holds 4 consecutive features of one row (gate/up ->
  // h = bf16(silu(g) * u), down -> p = bf16(w * y)).  Stored from there, a
  // store writes 16 (32x32 layout) or 32 bytes (16x16) in each of 32 or 16
  // rows.  The down output (a 4096-byte row of p) and the MX gate/up one go
  // through LDS instead: the workgroup's 128-row output tile is put together
  // in the free stage ring and leaves in 16-byte pieces, 8 lanes per 128-byte
  // line of a row, or, for MX gate/up with h tiles given, as quantised 32-
  // element blocks.  (The bf16-mode gate/up stores, 16x16 layout, measured no
  // slower than the extra barriers.)  The routing weights of the lane's rows
  // are read once, before any output is written.
  constexpr bool TILE_EPI = !GATEUP || ACT != kActBf16;
  constexpr int NF = feat_per_wg(GATEUP, WF, FX);  // output features of the workgroup
  constexpr int PITCH = NF * 2 + 16;           // tile row pitch (bytes): row r starts 4 r banks on
  static_assert(!TILE_EPI || kRowsPerTile * PITCH <= int(sizeof(sm)), "the output tile fits in the stage ring");
  uint8_t* tile_out = reinterpret_cast<uint8_t*>(&sm[0]);
  const int ld = GATEUP ? a.inter : a.hidden;
  uint16_t* ob = a.out + int64_t(g.row_begin + r0) * ld + int64_t(fb) * NF;
  // every wave is past its wait and its last reads of the stage ring
  if constexpr (TILE_EPI) __syncthreads();
  auto row_weight = [&](int rloc) -> float {
    const int r = r0 + rloc;
    return !GATEUP && r < g.row_count ? a.row_w[g.row_begin + r] : 0.0f;
  };
  // rloc: row in the tile, o: feature in the workgroup's block (rows past the
  // group's end are computed from stand-in operands and not stored)
  auto emit = [&](int rloc, int o, const float (&gv)[4], const float (&uv)[4], float wr) {
    uint16_t hv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) hv[i] = f32_to_bf16_rne(GATEUP ? silu_fast(gv[i]) * uv[i] : wr * gv[i]);
    const uint2 v = make_uint2(uint32_t(hv[0]) | (uint32_t(hv[1]) << 16), uint32_t(hv[2]) | (uint32_t(hv[3]) << 16));
    if constexpr (TILE_EPI)
      *reinterpret_cast<uint2*>(tile_out + rloc * PITCH + o * 2) = v;
    else if (r0 + rloc < g.row_count)
      *reinterpret_cast<uint2*>(ob + int64_t(rloc) * ld + o) = v;
  };
  const int fbase = fh * FT * 16;
  if constexpr (ACT_FP4) {
    // 32x32 result: value j of lane l is feature 8*(j/4) + 4*(l/32) + j%4, token l%32
    float wr[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) wr[rb] = row_weight(th * 64 + rb * 32 + (lane & 31));
#pragma unroll
    for (int f2 = 0; f2 < FT / 2; ++f2)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int jg = 0; jg < 4; ++jg) {
          float gv[4], uv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            gv[i] = acc32[(0 * (FT / 2) + f2) * 2 + rb][4 * jg + i];
            uv[i] = GATEUP ? acc32[((NM - 1) * (FT / 2) + f2) * 2 + rb][4 * jg + i] : 0.0f;
          }
          emit(th * 64 + rb * 32 + (lane & 31), fbase + f2 * 32 + 8 * jg + 4 * (lane >> 5), gv, uv, wr[rb]);
        }
  } else {
    // 16x16 result: value i of lane l is feature 4*(l/16) + i, row l%16
    float wr[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) wr[t] = row_weight(th * 64 + t * 16 + n);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) {
        float gv[4], uv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          gv[i] = acc[(0 * FT + ft) * 4 + t][i];
          uv[i] = GATEUP ? acc[((NM - 1) * FT + ft) * 4 + t][i] : 0.0f;
        }
        emit(th * 64 + t * 16 + n, fbase + ft * 16 + 4 * q, gv, uv, wr[t]);
      }
  }
  if constexpr (TILE_EPI) {
    __syncthreads();
    const int nrows = min(kRowsPerTile, g.row_count - r0);
    if constexpr (GATEUP && ACT != kActBf16) {
      if (a.h_codes) {
        // h quantised into the down GEMM's activation tiles: one thread per
        // (row, 32-element block) of the tile (128 rows x NF / 32 blocks =
        // the workgroup's threads), at the row's slot and the block's place in
        // the down GEMM's K steps
        constexpr bool QFP4 = ACT == kActFp4;
        constexpr int NB = NF / 32;
        static_assert(kRowsPerTile * NB == 64 * NW, "one block per thread");
        const int r = tid / NB, b = tid - (tid / NB) * NB;
        if (r < nrows) {
          uint32_t w[16];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(tile_out + r * PITCH + b * 64 + i * 16);
            w[4 * i] = v[0]; w[4 * i + 1] = v[1]; w[4 * i + 2] = v[2]; w[4 * i + 3] = v[3];
          }
          uint32_t q[QFP4 ? 4 : 8];
          const uint8_t sb = mxq::quant_block<QFP4>(w, q);
          const int slot = a.row_slot[g.row_begin + r0 + r];
          const int f0 = fb * NF + 32 * b;  // first feature of the block
          const int tl = slot / kMxTileRows;
          mxq::store_tile_block<QFP4>(a.h_codes, a.h_scales, int64_t(tl) * (a.inter / kTileK) + f0 / kTileK,
                                      slot - tl * kMxTileRows, (f0 % kTileK) / 32, q, sb);
        }
        return;
      }
    }
    constexpr int CH = NF * 2 / 16;    // 16-byte pieces of a tile row
    constexpr int RPP = 64 * NW / CH;  // rows per pass of the workgroup
    static_assert((64 * NW) % CH == 0, "whole rows per pass");
    const int c = tid % CH;
    for (int r = tid / CH; r < nrows; r += RPP)
      gstore<u32x4>(ob + int64_t(r) * ld + c * 8, *reinterpret_cast<const u32x4*>(tile_out + r * PITCH + c * 16));
  }
}

}  // namespace

int mx_gemm_rows_per_tile() { return kRowsPerTile; }

// Widest workgroup tile tried, in wave columns of 64 features (measured on the
// Qwen-A3B prefill layer: FP4 activations 4 -> gate/up 106 us against 122 us
// with 2 and 112 us with 8; FP8 activations 8 -> 125 us against 144 us with 4,
// whose 103 KB of LDS leave one 8-wave workgroup per CU; bf16 activations 4,
// whose 32 KB of activations per stage rule out 8).
constexpr int mx_max_wf(int) { return 4; }

namespace {
template <bool GATEUP, int ACT, int WF, int FX = 1>
hipError_t launch_wf(const MxGemmArgs& a, hipStream_t s, Ev ev) {
  // one workgroup per (row tile, feature block) item, at least 8 * ceil(items / 8)
  const int nfb = (GATEUP ? a.inter : a.hidden) / feat_per_wg(GATEUP, WF, FX);
  const int64_t bound = int64_t(a.max_tiles) * nfb;
  ft_launch(k_mx_gemm<GATEUP, ACT, WF, FX>, dim3(unsigned((bound + 7) / 8 * 8)), dim3(128 * WF), s, ev, a);
  return hipGetLastError();
}
// the widest workgroup tile (up to mx_max_wf, with bf16 the 128-column wave
// tiles first) whose feature block divides the outputs
template <bool GATEUP, int ACT>
hipError_t launch_gf(const MxGemmArgs& a, hipStream_t s, Ev ev) {
  const int outs = GATEUP ? a.inter : a.hidden;
  constexpr int wf = mx_max_wf(ACT);
  if constexpr (ACT == kActBf16) {
    if (outs % feat_per_wg(GATEUP, 4, 2) == 0) return launch_wf<GATEUP, ACT, 4, 2>(a, s, ev);
  }
  if constexpr (wf >= 8) {
    if (outs % feat_per_wg(GATEUP, 8) == 0) return launch_wf<GATEUP, ACT, 8>(a, s, ev);
  }
  if (wf >= 4 && outs % feat_per_wg(GATEUP, 4) == 0) return launch_wf<GATEUP, ACT, 4>(a, s, ev);
  if (outs % feat_per_wg(GATEUP, 2) == 0) return launch_wf<GATEUP, ACT, 2>(a, s, ev);
  return hipErrorInvalidValue;
}
template <bool GATEUP>
hipError_t launch_g(const MxGemmArgs& a, int act, hipStream_t s, Ev ev) {
  switch (act) {
    case kActBf16: return launch_gf<GATEUP, kActBf16>(a, s, ev);
    case kActFp8: return launch_gf<GATEUP, kActFp8>(a, s, ev);
    case kActFp4: return launch_gf<GATEUP, kActFp4>(a, s, ev);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace

hipError_t launch_mx_gemm(const MxGemmArgs& a, bool gateup, int act, hipStream_t s, Ev ev) {
  return gateup ? launch_g<true>(a, act, s, ev) : launch_g<false>(a, act, s, ev);
}

}  // namespace ftmoe
