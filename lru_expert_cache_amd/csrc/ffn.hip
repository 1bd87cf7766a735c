// Grouped SwiGLU expert FFN over the rows of each expert group, and the
// atomic-free weighted combine.
//
// Per group (one expert, M rows):  G = X W_g^T, U = X W_u^T (fp32 accumulate),
// h = bf16(silu(G) * U);  Y = h W_d^T;  p = bf16(w_row * Y).
// out[t] = bf16( sum_j p[row(t,j)] (+ p_shared[t]) ), summed in fp32 in rank
// order.  The pages say only that experts are SwiGLU-free-form MoE experts in
// MXFP4 / NVFP4 / FP8 (devpik article "FreeToken: Run Frontier MoE Models on
// Your Own GPU...", "The Real Requirement Is System RAM"); the rounding points
// are this library's reading and match the oracle's.
//
// gfx950 design.  The weights stream from HBM once per group; a wavefront owns
// a 16-row tile of W and a slice of K.  One 16-byte load per lane brings a
// whole 16x128 tile of FP4 codes in the device layout (see common.h);
// v_cvt_scalef32_pk_bf16_fp4 turns each byte into two bf16 values already
// multiplied by the E8M0 block scale (exact); NVFP4's E4M3 block scales are
// not powers of two and get their mantissa factor in fp32 (still exact),
// and v_mfma_f32_16x16x32_bf16 multiplies the 16x32 weight block by 32 K of
// 16 rows of bf16 activations, which are loaded as-is (they are exactly the B
// operand, 8 consecutive K per lane).  FP8-b128 weights convert with unit
// scale and their fp32 block scale is applied to each 128-K partial sum.
// Split-K slices of one row tile are summed through LDS in a fixed order.
#include <algorithm>
#include <cstdio>
#include <cstring>
#include <utility>

#include "common.h"
#include "gmem.h"

namespace ftmoe {

namespace {

typedef short bf16x8 __attribute__((ext_vector_type(8)));
typedef short bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kMaxWaves = 8;  // 512 threads: up to 256 VGPRs per wave

// name of the kernel behind the latest gate/up [0] and down [1] launch (for
// reports; the host thread that enqueues is the one that reads it back)
char g_ffn_kernel[2][96] = {"", ""};
const char* const kFmtName[4] = {"?", "mxfp4", "nvfp4", "fp8"};
void note_kernel(bool gateup, const char* kern, int fmt, const char* params) {
  std::snprintf(g_ffn_kernel[gateup ? 0 : 1], sizeof(g_ffn_kernel[0]), "%s<%s, %s, %s>", kern,
                kFmtName[fmt & 3], gateup ? "gate/up" : "down", params);
}
constexpr int64_t kFfnMaxGrid = 2048;  // 8 workgroups on each of the 256 CUs

__device__ inline uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return uint16_t((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// An E8M0 scale as the scale operand of the scaled converts, which read only
// its exponent field: the byte itself in bits 23..30 (byte 0 leaves the field
// 0, which those instructions take as 2^-127, the value E8M0 byte 0 encodes).
// No compare, so the conversion of a tile never waits on other tiles' scales.
__device__ inline float e8m0_scale_operand(uint32_t b) { return __uint_as_float(b << 23); }

__device__ inline float e4m3_to_f32(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  const float mag = e == 0 ? float(m) * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (b & 0x80u) ? -mag : mag;
}

// 8 FP4 codes (one dword, element 2i in the low nibble of byte i) -> 8 bf16 x scale
__device__ inline bf16x8 fp4x8_to_bf16(uint32_t w, float s) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

typedef float f32x2 __attribute__((ext_vector_type(2)));

// 8 FP4 codes x an arbitrary positive fp32 scale s -> 8 bf16.  The scaled
// converts of gfx950 take only the exponent of their scale operand (E8M0
// semantics), so s = 2^e * f is applied in two parts: 2^e inside the convert,
// the mantissa factor f in fp32.  For E4M3 block scales the product has at
// most 6 significant bits, so every step is exact and the bf16 pack is a
// truncation of exact values.
__device__ inline bf16x8 fp4x8_to_bf16_anyscale(uint32_t w, float s) {
  const uint32_t sb = __float_as_uint(s);
  const float p2 = __uint_as_float(sb & 0x7F800000u);
  const float f = __uint_as_float((sb & 0x007FFFFFu) | 0x3F800000u);
  bf16x8 r;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    f32x2 v;
    switch (b) {
      case 0: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, p2, 0); break;
      case 1: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, p2, 1); break;
      case 2: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, p2, 2); break;
      default: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, p2, 3); break;
    }
    const uint32_t lo = __float_as_uint(v[0] * f), hi = __float_as_uint(v[1] * f);
    r[2 * b] = short(lo >> 16);
    r[2 * b + 1] = short(hi >> 16);
  }
  return r;
}

// 8 E4M3 codes (two dwords) -> 8 bf16 (exact)
__device__ inline bf16x8 fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

__device__ inline bf16x8 as_bf16x8(uint4 v) {
  bf16x8 r;
  r[0] = short(v.x & 0xFFFF); r[1] = short(v.x >> 16);
  r[2] = short(v.y & 0xFFFF); r[3] = short(v.y >> 16);
  r[4] = short(v.z & 0xFFFF); r[5] = short(v.z >> 16);
  r[6] = short(v.w & 0xFFFF); r[7] = short(v.w >> 16);
  return r;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load (weights are read once per call: do not keep them in cache)
__device__ inline uint4 ld_stream16(const void* p) {
  const u32x4 v = gload_nt<u32x4>(p);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
// the 32 bytes of an FP8 tile lane, as two 16-byte loads.  Plain loads: with
// the non-temporal hint the FP8 stream kernel ran 5-17% slower (GLM-shaped
// gate/up, 12-20 experts), while the 4-bit formats (16 bytes a lane) ran
// 1-12% faster with it, so they keep it.
__device__ inline void ld_fp8_lane(const uint8_t* p, uint4& c0, uint4& c1) {
  const u32x4 a = gload<u32x4>(p), b = gload<u32x4>(p + 16);
  c0 = make_uint4(a[0], a[1], a[2], a[3]);
  c1 = make_uint4(b[0], b[1], b[2], b[3]);
}

typedef float f32x4g __attribute__((ext_vector_type(4)));
// four fp32 values through a global pointer
__device__ inline float4 ld_f4(const void* p) {
  const f32x4g v = gload<f32x4g>(p);
  return make_float4(v[0], v[1], v[2], v[3]);
}

template <int FMT>
struct TileRegs;
template <>
struct TileRegs<FT_FMT_MXFP4> {
  uint4 c;
  uint32_t s;  // scale byte
};
template <>
struct TileRegs<FT_FMT_NVFP4> {
  uint4 c;
  uint32_t s;  // two scale bytes
};
template <>
struct TileRegs<FT_FMT_FP8_B128> {
  uint4 c0, c1;  // block scales are read at use (see tile_mma)
};

template <int FMT>
__device__ inline void load_tile(TileRegs<FMT>& r, const uint8_t* __restrict__ W, const MatLayout& m, int64_t tile,
                                 int lane) {
  if constexpr (FMT == FT_FMT_FP8_B128) {
    const uint8_t* p = W + m.codes_off + (tile * 64 + lane) * 32;
    ld_fp8_lane(p, r.c0, r.c1);
  } else {
    r.c = ld_stream16(W + m.codes_off + (tile * 64 + lane) * 16);
    if constexpr (FMT == FT_FMT_MXFP4)
      r.s = gload<uint8_t>(W + m.scales_off + tile * 64 + lane);
    else
      r.s = gload<uint16_t>(W + m.scales_off + (tile * 64 + lane) * 2);
  }
}

// acc += W_tile(16 x 128) * X(128 x 16)
// For FP8-b128, fp8_scales points at the fp32 scales of the 4 accumulator rows
// this lane holds (rows 4q..4q+3 of the tile).
template <int FMT>
__device__ inline void tile_mma(const TileRegs<FMT>& r, const uint4 xv[4], floatx4& acc,
                                const float* __restrict__ fp8_scales) {
  if constexpr (FMT == FT_FMT_FP8_B128) {
    floatx4 t = {0.f, 0.f, 0.f, 0.f};
    const uint32_t w[8] = {r.c0.x, r.c0.y, r.c0.z, r.c0.w, r.c1.x, r.c1.y, r.c1.z, r.c1.w};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16(w[2 * j], w[2 * j + 1]), as_bf16x8(xv[j]), t, 0, 0,
                                                  0);
    const float4 sc = ld_f4(fp8_scales);
    acc[0] += sc.x * t[0];
    acc[1] += sc.y * t[1];
    acc[2] += sc.z * t[2];
    acc[3] += sc.w * t[3];
  } else {
    const uint32_t w[4] = {r.c.x, r.c.y, r.c.z, r.c.w};
    float s0, s1;
    if constexpr (FMT == FT_FMT_MXFP4) {
      s0 = s1 = e8m0_scale_operand(r.s);
    } else {
      s0 = e4m3_to_f32(r.s & 0xFFu);
      s1 = e4m3_to_f32(r.s >> 8);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x8 av;
      if constexpr (FMT == FT_FMT_MXFP4)
        av = fp4x8_to_bf16(w[j], s0);
      else
        av = fp4x8_to_bf16_anyscale(w[j], j < 2 ? s0 : s1);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, as_bf16x8(xv[j]), acc, 0, 0, 0);
    }
  }
}


// tile_mma with the FP8-b128 row scales of the lane's four accumulator rows
// already in registers
template <int FMT>
__device__ inline void tile_mma_sc(const TileRegs<FMT>& r, const uint4 xv[4], floatx4& acc, float4 sc) {
  static_assert(FMT == FT_FMT_FP8_B128, "FP8-b128 only");
  floatx4 t = {0.f, 0.f, 0.f, 0.f};
  const uint32_t w[8] = {r.c0.x, r.c0.y, r.c0.z, r.c0.w, r.c1.x, r.c1.y, r.c1.z, r.c1.w};
#pragma unroll
  for (int j = 0; j < 4; ++j)
    t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16(w[2 * j], w[2 * j + 1]), as_bf16x8(xv[j]), t, 0, 0, 0);
  acc[0] += sc.x * t[0];
  acc[1] += sc.y * t[1];
  acc[2] += sc.z * t[2];
  acc[3] += sc.w * t[3];
}

// ---------------------------------------------------------------------------
// Decode-sized calls (few rows per expert): a workgroup of four waves owns 64
// output features (four 16-row weight tiles, one per wave) of one expert and
// walks the full K in lockstep.  Each wave streams its weight tiles through a
// ring of D register stages; the 16 x 128 activation tile of each K step is
// loaded by the whole workgroup (one 16-byte piece per thread, queued with the
// weights D steps ahead) and handed to the MFMA B operand through a double-
// buffered LDS tile, XOR-swizzled so that both the writes and the b128 reads
// are free of bank conflicts.  Loads complete in issue order, so the loads of
// a step that are not streamed (tokens, routing weights, tensor scales) are
// made when an item starts, before its first prefetch; a prefetch past the end
// reads one shared line instead of branching.  Groups with more than 16 rows
// (at most 64) multiply each weight tile by every 16-row chunk of their
// activations, so the weights are read once whatever the row count.
// f(integral_constant<0>) ... f(integral_constant<N-1>): ring slots indexed at compile time
template <typename F, int... I>
__device__ __attribute__((always_inline)) inline void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __attribute__((always_inline)) inline void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

typedef long long i64x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kStreamWaves = 4;     // 16-row weight tiles per workgroup
constexpr int kStreamMaxChunks = 4; // row chunks of 16 a group may have (max_rows <= 64)

template <int FMT>
__device__ inline void load_tile_sel(TileRegs<FMT>& r, const uint8_t* __restrict__ W, const MatLayout& m,
                                     int64_t tile, int lane, bool live, const uint8_t* dummy) {
  if constexpr (FMT == FT_FMT_FP8_B128) {
    const uint8_t* p = live ? W + m.codes_off + (tile * 64 + lane) * 32 : dummy;
    ld_fp8_lane(p, r.c0, r.c1);
  } else {
    r.c = ld_stream16(live ? W + m.codes_off + (tile * 64 + lane) * 16 : dummy);
    if constexpr (FMT == FT_FMT_MXFP4)
      r.s = gload<uint8_t>(live ? W + m.scales_off + tile * 64 + lane : dummy);
    else
      r.s = gload<uint16_t>(live ? W + m.scales_off + (tile * 64 + lane) * 2 : dummy);
  }
}

template <int FMT, bool GATEUP, int D, int NC>
__global__ __launch_bounds__(64 * kStreamWaves, 2) void k_ffn_stream(FfnArgs a) {
  constexpr int NM = GATEUP ? 2 : 1;
  constexpr bool F8 = FMT == FT_FMT_FP8_B128;
  // per K step, the activation tile of each row chunk: 16 rows x 128 K bf16, swizzled
  __shared__ uint4 xs[2][NC][256];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int q = lane >> 4, n = lane & 15;
  const MatLayout& m0 = a.lay.m[GATEUP ? 0 : 2];
  const int nkb = m0.cols / kTileK;
  const int nfb = m0.rows / (kTileRows * kStreamWaves);  // feature blocks of one group
  const int n_list = min(a.n_list, *a.n_list_dev);
  const int n_items = n_list * nfb;
  const uint8_t* dummy = reinterpret_cast<const uint8_t*>(a.gdesc);
  // this thread's piece of an activation tile: row xr, 8 K values at chunk xc
  const int xr = tid >> 4, xc = tid & 15;
  const int xslot = xr * 16 + (xc ^ xr);
  int par = 0;  // LDS buffer parity, kept across items

  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int gi = item / nfb;
    const GroupDesc g = a.gdesc[gi];
    if (g.row_count <= 0 || g.wptr == 0) continue;  // uniform over the workgroup
    const int rb = (item - gi * nfb) * kStreamWaves + w;  // this wave's 16-row weight tile
    const uint8_t* W = reinterpret_cast<const uint8_t*>(g.wptr);
    // row chunks of this group (uniform over the workgroup; the launch takes
    // NC = the call's bound on the rows of any group, in chunks of 16)
    const int nrc = min((g.row_count + 15) >> 4, NC);

    // per-item reads, made before the stream starts: per row chunk, this
    // thread's activation row (element offset from x) and, for down, the
    // routing weight of the lane's epilogue row
    int64_t xoff[NC];
    float wr[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int r = c * 16 + xr;
      const bool ok = c < nrc && r < g.row_count;
      const int row = g.row_begin + (ok ? r : 0);
      xoff[c] = GATEUP ? int64_t(a.row_tok[row]) * a.hidden : int64_t(row) * a.inter;
      const int re = c * 16 + n;  // epilogue row of this lane
      wr[c] = GATEUP ? 0.0f : a.row_w[g.row_begin + (c < nrc && re < g.row_count ? re : 0)];
    }
    float tsc[NM];
#pragma unroll
    for (int mi = 0; mi < NM; ++mi)
      tsc[mi] = FMT == FT_FMT_NVFP4 ? gload<float>(W + a.lay.tscale_off + 4 * (GATEUP ? mi : 2)) : 1.0f;

    // the ring: weights and the activation pieces (one per row chunk) of
    // K steps s .. s+D-1; each weight tile is read once and multiplied by
    // every row chunk
    TileRegs<FMT> wring[D][NM];
    float4 sring[D][NM];
    u32x4 xring[D][NC];
    auto fetch = [&](int t_s, auto uc) {
      constexpr int u = decltype(uc)::value;
      const bool live = t_s < nkb;
      const int t = live ? t_s : 0;
      const int64_t tile = int64_t(rb) * nkb + t;
#pragma unroll
      for (int mi = 0; mi < NM; ++mi) {
        const MatLayout& m = a.lay.m[GATEUP ? mi : 2];
        load_tile_sel<FMT>(wring[u][mi], W, m, tile, lane, live, dummy);
        if constexpr (F8)
          sring[u][mi] = ld_f4(live ? W + m.scales_off + (tile * 16 + 4 * q) * 4 : dummy);
      }
#pragma unroll
      for (int c = 0; c < NC; ++c)
        if (c < nrc)
          xring[u][c] = *reinterpret_cast<const u32x4*>(live ? a.x + xoff[c] + t * kTileK + xc * 8 : a.x);
    };
    static_for<D>([&](auto uc) { fetch(decltype(uc)::value, uc); });

    floatx4 acc[NC][NM];
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int mi = 0; mi < NM; ++mi) acc[c][mi] = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < nkb; s0 += D) {
      static_for<D>([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        const int s = s0 + u;
        // activation tiles of step s -> LDS, then the operands of this wave
#pragma unroll
        for (int c = 0; c < NC; ++c)
          if (c < nrc) xs[par][c][xslot] = make_uint4(xring[u][c][0], xring[u][c][1], xring[u][c][2], xring[u][c][3]);
        __syncthreads();
        TileRegs<FMT> wt[NM];
        float4 st[NM];
#pragma unroll
        for (int mi = 0; mi < NM; ++mi) {
          wt[mi] = wring[u][mi];
          st[mi] = sring[u][mi];
        }
        fetch(s + D, uc);  // refill the slot just consumed
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          if (c < nrc) {
            uint4 bx[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) bx[j] = xs[par][c][n * 16 + ((4 * q + j) ^ n)];
#pragma unroll
            for (int mi = 0; mi < NM; ++mi) {
              if constexpr (F8)
                tile_mma_sc<FMT>(wt[mi], bx, acc[c][mi], st[mi]);
              else
                tile_mma<FMT>(wt[mi], bx, acc[c][mi], nullptr);
            }
          }
        }
        par ^= 1;
      });
    }
    // epilogue: lane holds features rb*16+4q+i of row c*16+n of each chunk
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int r = c * 16 + n;
      if (c < nrc && r < g.row_count) {
        const int row = g.row_begin + r;
        const int o0 = rb * 16 + 4 * q;
        uint16_t hv[4];
        if constexpr (GATEUP) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float gv = acc[c][0][i] * tsc[0];
            const float uv = acc[c][1][i] * tsc[1];
            hv[i] = f32_to_bf16_rne(gv / (1.0f + expf(-gv)) * uv);
          }
          *reinterpret_cast<uint2*>(a.out + int64_t(row) * a.inter + o0) =
              make_uint2(uint32_t(hv[0]) | (uint32_t(hv[1]) << 16), uint32_t(hv[2]) | (uint32_t(hv[3]) << 16));
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) hv[i] = f32_to_bf16_rne(wr[c] * (acc[c][0][i] * tsc[0]));
          *reinterpret_cast<uint2*>(a.out + int64_t(row) * a.hidden + o0) =
              make_uint2(uint32_t(hv[0]) | (uint32_t(hv[1]) << 16), uint32_t(hv[2]) | (uint32_t(hv[3]) << 16));
        }
      }
    }
  }
}

// K tiles (of 128) a wavefront holds in registers
constexpr int kpw_max(int fmt, bool gateup) { return (fmt == FT_FMT_FP8_B128 && gateup) ? 6 : 8; }

// GATEUP: rows of matrices 0 (gate) and 1 (up) over K = H, epilogue SwiGLU -> hbuf.
// else:   rows of matrix 2 (down) over K = I, epilogue routing weight -> pbuf.
template <int FMT, bool GATEUP, int KPW>
__global__ __launch_bounds__(64 * kMaxWaves) void k_ffn(FfnArgs a, int SK, int RB) {
  constexpr int kpw = KPW;
  constexpr int NM = GATEUP ? 2 : 1;
  __shared__ floatx4 red[kMaxWaves][NM][64];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int rbl = w / SK, sk = w % SK;
  const MatLayout& m0 = a.lay.m[GATEUP ? 0 : 2];
  const int K = m0.cols;
  const int nkb = K / kTileK;
  const int kb0 = sk * kpw;
  const int nrbb = m0.rows / kTileRows / RB;  // row blocks of one group
  const int n_list = min(a.n_list, *a.n_list_dev);
  const int n_items = n_list * nrbb;

  // items (group, row block), group-major, strided over the grid
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int gi = item / nrbb;
    const GroupDesc g = a.gdesc[gi];
    if (g.row_count <= 0) continue;  // uniform over the workgroup
    const int rb = (item - gi * nrbb) * RB + rbl;
    const uint8_t* W = reinterpret_cast<const uint8_t*>(g.wptr);

    // weights of this wave's (row tile, K slice), loaded once
    TileRegs<FMT> tr[NM][KPW];
#pragma unroll
    for (int mi = 0; mi < NM; ++mi) {
      const MatLayout& m = a.lay.m[GATEUP ? mi : 2];
#pragma unroll
      for (int t = 0; t < KPW; ++t)
        if (t < kpw) load_tile<FMT>(tr[mi][t], W, m, int64_t(rb) * nkb + kb0 + t, lane);
    }
    float tsc[NM];
    {
#pragma unroll
      for (int mi = 0; mi < NM; ++mi)
        tsc[mi] = FMT == FT_FMT_NVFP4 ? gload<float>(W + a.lay.tscale_off + 4 * (GATEUP ? mi : 2)) : 1.0f;
    }

    const int q = lane >> 4, n = lane & 15;
    const int ntiles = (g.row_count + 15) / 16;
    for (int nt = 0; nt < ntiles; ++nt) {
      const int r = nt * 16 + n;
      const bool valid = r < g.row_count;
      const int row = g.row_begin + r;
      int64_t xbase = 0;
      if (valid) xbase = GATEUP ? int64_t(a.row_tok[row]) * a.hidden : int64_t(row) * a.inter;

      floatx4 acc[NM];
#pragma unroll
      for (int mi = 0; mi < NM; ++mi) acc[mi] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < KPW; ++t) {
        if (t < kpw) {
          uint4 xv[4];
          const int64_t off = xbase + int64_t(kb0 + t) * kTileK + 32 * q;
          if (valid) {
            const uint4* xp = reinterpret_cast<const uint4*>(a.x + off);
#pragma unroll
            for (int j = 0; j < 4; ++j) xv[j] = xp[j];
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) xv[j] = make_uint4(0, 0, 0, 0);
          }
#pragma unroll
          for (int mi = 0; mi < NM; ++mi) {
            const float* sp = nullptr;
            if constexpr (FMT == FT_FMT_FP8_B128)
              sp = reinterpret_cast<const float*>(W + a.lay.m[GATEUP ? mi : 2].scales_off) +
                   (int64_t(rb) * nkb + kb0 + t) * 16 + 4 * q;
            tile_mma<FMT>(tr[mi][t], xv, acc[mi], sp);
          }
        }
      }
      if (SK > 1) {
#pragma unroll
        for (int mi = 0; mi < NM; ++mi) red[w][mi][lane] = acc[mi];
        __syncthreads();
        if (sk == 0) {
#pragma unroll
          for (int mi = 0; mi < NM; ++mi) {
            floatx4 s = red[w][mi][lane];
            for (int k2 = 1; k2 < SK; ++k2) {
              const floatx4 v = red[w + k2][mi][lane];
              s[0] += v[0]; s[1] += v[1]; s[2] += v[2]; s[3] += v[3];
            }
            acc[mi] = s;
          }
        }
      }
      if (sk == 0 && valid) {
        // lane holds output features rb*16 + 4q + i of row r
        const int o0 = rb * 16 + 4 * q;
        uint16_t hv[4];
        if constexpr (GATEUP) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float gv = acc[0][i] * tsc[0];
            const float uv = acc[1][i] * tsc[1];
            hv[i] = f32_to_bf16_rne(gv / (1.0f + expf(-gv)) * uv);
          }
          uint2 pk = make_uint2(uint32_t(hv[0]) | (uint32_t(hv[1]) << 16), uint32_t(hv[2]) | (uint32_t(hv[3]) << 16));
          *reinterpret_cast<uint2*>(a.out + int64_t(row) * a.inter + o0) = pk;
        } else {
          const float wr = a.row_w[row];
#pragma unroll
          for (int i = 0; i < 4; ++i) hv[i] = f32_to_bf16_rne(wr * (acc[0][i] * tsc[0]));
          uint2 pk = make_uint2(uint32_t(hv[0]) | (uint32_t(hv[1]) << 16), uint32_t(hv[2]) | (uint32_t(hv[3]) << 16));
          *reinterpret_cast<uint2*>(a.out + int64_t(row) * a.hidden + o0) = pk;
        }
      }
      if (SK > 1) __syncthreads();
    }
  }  // items
}

struct Split {
  int SK, RB, kpw;
};

// K tiles per wave (kpw) and waves per row tile (SK): prefer short K slices
// (more waves, more loads in flight), at most kMaxWaves waves per workgroup.
Split choose_split(int K, int R, int kpwmax) {
  const int nkb = K / kTileK, nrb = R / kTileRows;
  Split s{0, 0, 0};
  for (int pass = 0; pass < 2 && s.SK == 0; ++pass) {
    const int lo = pass == 0 ? 1 : 5, hi = pass == 0 ? 4 : kpwmax;
    for (int kpw = hi; kpw >= lo; --kpw)
      if (nkb % kpw == 0 && nkb / kpw <= kMaxWaves) {
        s.kpw = kpw;
        s.SK = nkb / kpw;
        break;
      }
  }
  if (s.SK == 0) return s;
  const int cap = s.SK > 4 ? s.SK : 4;
  s.RB = 1;
  for (int rb : {4, 2}) {
    if (rb * s.SK <= cap && nrb % rb == 0) {
      s.RB = rb;
      break;
    }
  }
  return s;
}

template <int FMT, bool GATEUP>
hipError_t launch_fmt(const FfnArgs& a, const Split& s, dim3 grid, dim3 block, hipStream_t st, Ev ev) {
  switch (s.kpw) {
#define FT_KPW_CASE(N)                                                                   \
  case N:                                                                                \
    if constexpr (N <= kpw_max(FMT, GATEUP)) {                                           \
      note_kernel(GATEUP, "k_ffn", FMT, "split-K");                                     \
      ft_launch(k_ffn<FMT, GATEUP, N>, grid, block, st, ev, a, s.SK, s.RB);              \
      return hipGetLastError();                                                          \
    }                                                                                    \
    break;
    FT_KPW_CASE(1) FT_KPW_CASE(2) FT_KPW_CASE(3) FT_KPW_CASE(4)
    FT_KPW_CASE(5) FT_KPW_CASE(6) FT_KPW_CASE(7) FT_KPW_CASE(8)
#undef FT_KPW_CASE
    default:
      break;
  }
  return hipErrorInvalidValue;
}

// resident workgroups per CU of a kernel (for persistent grids), computed once
template <typename Kern>
int64_t resident_grid(Kern k, int block) {
  int dev = 0, cus = 0, per_cu = 0;
  (void)hipGetDevice(&dev);
  (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, block, 0) != hipSuccess || per_cu < 1) per_cu = 1;
  return int64_t(per_cu) * std::max(cus, 1);
}

template <int FMT, bool GATEUP, int D, int NC>
hipError_t launch_stream_d(const FfnArgs& a, hipStream_t st, Ev ev) {
  static const int64_t cap = resident_grid(k_ffn_stream<FMT, GATEUP, D, NC>, 64 * kStreamWaves);
  const MatLayout& m = a.lay.m[GATEUP ? 0 : 2];
  const int64_t items = int64_t(a.n_list) * (m.rows / (kTileRows * kStreamWaves));
  char prm[48];
  std::snprintf(prm, sizeof(prm), "depth %d, %d row chunk%s", D, NC, NC > 1 ? "s" : "");
  note_kernel(GATEUP, "k_ffn_stream", FMT, prm);
  ft_launch(k_ffn_stream<FMT, GATEUP, D, NC>, dim3(unsigned(std::min(items, cap))), dim3(64 * kStreamWaves), st, ev,
            a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Split-K decode kernel with an item ring: a persistent workgroup of SK waves
// owns one 16-row weight tile per item (item = expert group x row tile) and
// splits its K over the waves (each wave KPW tiles of 128), like k_ffn; the
// registers of one item's slice (weights plus the lane's 64 bytes of
// activations per K tile) form a ring whose slot t is refilled with the next
// item's tile t as soon as tile t has been multiplied, so the next item
// streams in while the current one finishes, its partial sums meet in LDS and
// its epilogue runs.  Per-item reads the ring depends on (the tokens of the
// rows, routing weights) are made one item earlier, so that waiting for them
// never waits for the ring.  Invalid activation rows read one shared line and
// only feed output columns that are not written.  Every group has at most 16
// rows (calls of up to 16 tokens).
template <int FMT, bool GATEUP, int KPW>
__global__ __launch_bounds__(64 * kMaxWaves) void k_ffn_ring(FfnArgs a, int SK) {
  constexpr int NM = GATEUP ? 2 : 1;
  constexpr bool F8 = FMT == FT_FMT_FP8_B128;
  __shared__ floatx4 red[kMaxWaves][NM][64];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int q = lane >> 4, n = lane & 15;
  const int sk = w;  // one row tile per workgroup: wave = K slice
  const MatLayout& m0 = a.lay.m[GATEUP ? 0 : 2];
  const int nkb = m0.cols / kTileK;
  const int kb0 = sk * KPW;
  const int nrb = m0.rows / kTileRows;
  const int n_list = min(a.n_list, *a.n_list_dev);
  const int n_items = n_list * nrb;
  if (int(blockIdx.x) >= n_items) return;
  const int G = int(gridDim.x);
  const uint8_t* dummy = reinterpret_cast<const uint8_t*>(a.gdesc);

  struct Item {
    uint64_t wptr;
    int row_begin, row_count, rb;
  };
  auto desc = [&](int item) -> Item {
    const bool ok = item < n_items;
    const int it = ok ? item : n_items - 1;
    const int gi = it / nrb;
    const GroupDesc g = a.gdesc[gi];
    Item r;
    r.wptr = g.wptr;
    r.row_begin = g.row_begin;
    r.row_count = ok && g.wptr != 0 ? g.row_count : 0;
    r.rb = it - gi * nrb;
    return r;
  };
  // activation row (GATEUP: by token) of this lane for rows 0..15 of an item;
  // null for a row the group does not have
  auto row_src = [&](const Item& d, int rc) -> const uint16_t* {
    const int r = rc * 16 + n;
    if (r >= d.row_count) return nullptr;
    const int row = d.row_begin + r;
    return GATEUP ? a.x + int64_t(a.row_tok[row]) * a.hidden : a.x + int64_t(row) * a.inter;
  };

  TileRegs<FMT> wring[KPW][NM];
  float4 sring[KPW][NM];
  u32x4 xring[KPW][4];
  auto fetch = [&](const Item& d, const uint16_t* xsrc, auto tc) {
    constexpr int t = decltype(tc)::value;
    const bool live = d.row_count > 0;
    const uint8_t* W = reinterpret_cast<const uint8_t*>(d.wptr);
    const int64_t tile = int64_t(d.rb) * nkb + kb0 + t;
#pragma unroll
    for (int mi = 0; mi < NM; ++mi) {
      const MatLayout& m = a.lay.m[GATEUP ? mi : 2];
      load_tile_sel<FMT>(wring[t][mi], W, m, tile, lane, live, dummy);
      if constexpr (F8)
        sring[t][mi] = ld_f4(live ? W + m.scales_off + (tile * 16 + 4 * q) * 4 : dummy);
    }
    // a missing row reads one shared line (its output column is not written)
    const u32x4* xp = reinterpret_cast<const u32x4*>(xsrc ? xsrc + (kb0 + t) * kTileK + 32 * q : a.x);
#pragma unroll
    for (int j = 0; j < 4; ++j) xring[t][j] = xp[xsrc ? j : 0];
  };
  auto mma = [&](auto tc, floatx4 (&acc)[NM]) {
    constexpr int t = decltype(tc)::value;
    uint4 xv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) xv[j] = make_uint4(xring[t][j][0], xring[t][j][1], xring[t][j][2], xring[t][j][3]);
#pragma unroll
    for (int mi = 0; mi < NM; ++mi) {
      if constexpr (F8)
        tile_mma_sc<FMT>(wring[t][mi], xv, acc[mi], sring[t][mi]);
      else
        tile_mma<FMT>(wring[t][mi], xv, acc[mi], nullptr);
    }
  };
  // partial sums of the SK waves meet in LDS; wave 0 writes rows rc*16 + n
  auto finish = [&](const Item& d, int rc, floatx4 (&acc)[NM], const float (&tsc)[NM], float wr) {
    if (SK > 1) {
#pragma unroll
      for (int mi = 0; mi < NM; ++mi) red[w][mi][lane] = acc[mi];
      __syncthreads();
      if (sk == 0) {
#pragma unroll
        for (int mi = 0; mi < NM; ++mi) {
          floatx4 s = red[0][mi][lane];
          for (int k2 = 1; k2 < SK; ++k2) {
            const floatx4 v = red[k2][mi][lane];
            s[0] += v[0]; s[1] += v[1]; s[2] += v[2]; s[3] += v[3];
          }
          acc[mi] = s;
        }
      }
    }
    const int r = rc * 16 + n;
    if (sk == 0 && r < d.row_count) {
      const int row = d.row_begin + r;
      const int o0 = d.rb * 16 + 4 * q;
      uint16_t hv[4];
      if constexpr (GATEUP) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float gv = acc[0][i] * tsc[0];
          const float uv = acc[1][i] * tsc[1];
          hv[i] = f32_to_bf16_rne(gv / (1.0f + expf(-gv)) * uv);
        }
        *reinterpret_cast<uint2*>(a.out + int64_t(row) * a.inter + o0) =
            make_uint2(uint32_t(hv[0]) | (uint32_t(hv[1]) << 16), uint32_t(hv[2]) | (uint32_t(hv[3]) << 16));
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) hv[i] = f32_to_bf16_rne(wr * (acc[0][i] * tsc[0]));
        *reinterpret_cast<uint2*>(a.out + int64_t(row) * a.hidden + o0) =
            make_uint2(uint32_t(hv[0]) | (uint32_t(hv[1]) << 16), uint32_t(hv[2]) | (uint32_t(hv[3]) << 16));
      }
    }
    if (SK > 1) __syncthreads();
  };
  auto row_weight = [&](const Item& d, int rc) -> float {
    const int r = rc * 16 + n;
    return GATEUP ? 0.0f : a.row_w[d.row_begin + (r < d.row_count ? r : 0)];
  };

  // prologue: the first item in the ring, the row data of the second
  int item = blockIdx.x;
  Item cur = desc(item);
  const uint16_t* xs_cur = row_src(cur, 0);
  float wr_cur = row_weight(cur, 0);
  static_for<KPW>([&](auto tc) { fetch(cur, xs_cur, tc); });
  Item nxt = desc(item + G);
  const uint16_t* xs_nxt = row_src(nxt, 0);
  float wr_nxt = row_weight(nxt, 0);

  for (;;) {
    // row data of the item after next, ahead of this item's refills
    const Item nn = desc(item + 2 * G);
    const uint16_t* xs_nn = row_src(nn, 0);
    const float wr_nn = row_weight(nn, 0);
    float tsc[NM];
#pragma unroll
    for (int mi = 0; mi < NM; ++mi)
      tsc[mi] = FMT == FT_FMT_NVFP4 && cur.row_count > 0
                    ? gload<float>(reinterpret_cast<const uint8_t*>(cur.wptr) + a.lay.tscale_off + 4 * (GATEUP ? mi : 2))
                    : 1.0f;
    floatx4 acc[NM];
#pragma unroll
    for (int mi = 0; mi < NM; ++mi) acc[mi] = {0.f, 0.f, 0.f, 0.f};
    static_for<KPW>([&](auto tc) {
      mma(tc, acc);
      fetch(nxt, xs_nxt, tc);  // the slot just used takes the next item's tile
    });
    if (cur.row_count > 0) {
      finish(cur, 0, acc, tsc, wr_cur);
    }
    item += G;
    if (item >= n_items) break;
    cur = nxt;
    xs_cur = xs_nxt;
    wr_cur = wr_nxt;
    nxt = nn;
    xs_nxt = xs_nn;
    wr_nxt = wr_nn;
  }
}

// ---------------------------------------------------------------------------
// Decode calls of at most 16 rows per group, one pass: a workgroup of SK waves
// owns F 16-row weight tiles (both gate and up for gate/up) of one expert over
// the full K, split into SK slices of KPW K tiles.  Every weight tile of a
// wave's slice is requested at once, so that a single round of loads covers
// the launch: at decode sizes the items fit the resident workgroups, and the
// bytes in flight, not the issue rate, set the bandwidth.  The activation tile
// of each K tile (16 rows x 128 K, one row per lane column) is loaded once
// per wave and serves all F weight tiles.  Loads complete in issue order, so
// the weights of the first K tile go out before the activations (whose row
// addresses wait for the group's token list) and the rest after them; the
// multiplies of K tile t then wait only for what precedes it.  Partial sums of
// the SK slices meet in LDS and are added in slice order; wave v finishes
// weight tiles v, v + SK, ...  Missing rows (beyond the group's count) use
// zero activations and are not written.
constexpr int kWideMaxWaves = 8;
static_assert(kGroupTok >= kTileRows, "the wide kernel reads its rows' tokens from the run-list entry");
static_assert(offsetof(GroupDesc, tok) == 24 && sizeof(GroupDesc) == 64, "descriptor dwords as the wide kernel reads them");
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));

// One wide item: weight tiles rb0 .. rb0 + F - 1 of group g over the full K,
// the calling wave being K slice w of SK; red is the item's LDS area
// ([SK][F][NM][64]); tok (gate/up) is the token of the lane's row.  Every
// thread of the workgroup calls it at the same time (one barrier when SK > 1).
template <int FMT, bool GATEUP, int KPW, int F>
__device__ __attribute__((always_inline)) inline void wide_item(const FfnArgs& a, const GroupDesc& g, int rb0, int w,
                                                                int SK, floatx4* red, int tok) {
  constexpr int NM = GATEUP ? 2 : 1;
  constexpr bool F8 = FMT == FT_FMT_FP8_B128;
  const int lane = threadIdx.x & 63;
  const int q = lane >> 4, n = lane & 15;
  const int nkb = a.lay.m[GATEUP ? 0 : 2].cols / kTileK;
  const uint8_t* W = reinterpret_cast<const uint8_t*>(g.wptr);
  const int kb0 = w * KPW;
  const bool rv = n < g.row_count;
  const int row = g.row_begin + (rv ? n : 0);

  TileRegs<FMT> wt[F][NM][KPW];
  float4 ws[F][NM][KPW];
  uint4 xv[KPW][4];
  auto load_w = [&](auto tc) {
    constexpr int t = decltype(tc)::value;
#pragma unroll
    for (int f = 0; f < F; ++f)
#pragma unroll
      for (int mi = 0; mi < NM; ++mi) {
        const MatLayout& m = a.lay.m[GATEUP ? mi : 2];
        const int64_t tile = int64_t(rb0 + f) * nkb + kb0 + t;
        load_tile<FMT>(wt[f][mi][t], W, m, tile, lane);
        if constexpr (F8) ws[f][mi][t] = ld_f4(W + m.scales_off + (tile * 16 + 4 * q) * 4);
      }
  };
  // K tile 0 first, then the activations of every K tile, then the rest; the
  // scheduling barriers keep the compiler from sinking loads towards their
  // uses (which would leave only a few in flight)
  load_w(std::integral_constant<int, 0>{});
  __builtin_amdgcn_sched_barrier(0);
  {
    const uint16_t* xs = GATEUP ? a.x + int64_t(tok) * a.hidden : a.x + int64_t(row) * a.inter;
#pragma unroll
    for (int t = 0; t < KPW; ++t) {
      const uint4* xp = reinterpret_cast<const uint4*>(xs + (kb0 + t) * kTileK + 32 * q);
#pragma unroll
      for (int j = 0; j < 4; ++j) xv[t][j] = rv ? xp[j] : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  static_for<KPW>([&](auto tc) {
    if constexpr (decltype(tc)::value > 0) {
      load_w(tc);
      __builtin_amdgcn_sched_barrier(0);
    }
  });
  float tsc[NM];
#pragma unroll
  for (int mi = 0; mi < NM; ++mi)
    tsc[mi] = FMT == FT_FMT_NVFP4 ? gload<float>(W + a.lay.tscale_off + 4 * (GATEUP ? mi : 2)) : 1.0f;

  floatx4 acc[F][NM];
#pragma unroll
  for (int f = 0; f < F; ++f)
#pragma unroll
    for (int mi = 0; mi < NM; ++mi) acc[f][mi] = {0.f, 0.f, 0.f, 0.f};
  // one K tile at a time, so that each waits only for its own loads
  static_for<KPW>([&](auto tc) {
    constexpr int t = decltype(tc)::value;
#pragma unroll
    for (int f = 0; f < F; ++f)
#pragma unroll
      for (int mi = 0; mi < NM; ++mi) {
        if constexpr (F8)
          tile_mma_sc<FMT>(wt[f][mi][t], xv[t], acc[f][mi], ws[f][mi][t]);
        else
          tile_mma<FMT>(wt[f][mi][t], xv[t], acc[f][mi], nullptr);
      }
    __builtin_amdgcn_sched_barrier(0);
  });

  // slice sums in LDS, added in slice order
  if (SK > 1) {
#pragma unroll
    for (int f = 0; f < F; ++f)
#pragma unroll
      for (int mi = 0; mi < NM; ++mi) red[((w * F + f) * NM + mi) * 64 + lane] = acc[f][mi];
    __syncthreads();
  }
  const float wr = GATEUP ? 0.0f : a.row_w[row];
#pragma unroll
  for (int f = 0; f < F; ++f) {
    if (f % SK != w) continue;
    floatx4 s[NM];
#pragma unroll
    for (int mi = 0; mi < NM; ++mi) {
      if (SK > 1) {
        s[mi] = red[(f * NM + mi) * 64 + lane];
        for (int k2 = 1; k2 < SK; ++k2) {
          const floatx4 v = red[((k2 * F + f) * NM + mi) * 64 + lane];
          s[mi][0] += v[0]; s[mi][1] += v[1]; s[mi][2] += v[2]; s[mi][3] += v[3];
        }
      } else {
        s[mi] = acc[f][mi];
      }
    }
    if (!rv) continue;
    // lane holds output features (rb0 + f) * 16 + 4q + i of row n
    const int o0 = (rb0 + f) * kTileRows + 4 * q;
    uint16_t hv[4];
    if constexpr (GATEUP) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float gv = s[0][i] * tsc[0];
        const float uv = s[1][i] * tsc[1];
        hv[i] = f32_to_bf16_rne(gv / (1.0f + expf(-gv)) * uv);
      }
      *reinterpret_cast<uint2*>(a.out + int64_t(row) * a.inter + o0) =
          make_uint2(uint32_t(hv[0]) | (uint32_t(hv[1]) << 16), uint32_t(hv[2]) | (uint32_t(hv[3]) << 16));
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) hv[i] = f32_to_bf16_rne(wr * (s[0][i] * tsc[0]));
      *reinterpret_cast<uint2*>(a.out + int64_t(row) * a.hidden + o0) =
          make_uint2(uint32_t(hv[0]) | (uint32_t(hv[1]) << 16), uint32_t(hv[2]) | (uint32_t(hv[3]) << 16));
    }
  }
}

template <int FMT, bool GATEUP, int KPW, int F>
__global__ __launch_bounds__(64 * kWideMaxWaves) void k_ffn_wide(FfnArgs a, int SK) {
  extern __shared__ floatx4 wide_red[];  // [SK][F][NM][64]
  // grid: x = block of F weight tiles, y = run-list entry (consecutive
  // workgroups share a group).  The group is read together with the count
  // (the grid never exceeds the descriptor array), so that one load latency
  // precedes the weight loads.
  const int gi = blockIdx.y;
  const int rb0 = int(blockIdx.x) * F;
  // the descriptor and the tokens of its rows in one 64-byte load, so that
  // the activation addresses are known as soon as the weight addresses (no
  // second load that the descriptor's row offset would feed)
  const i32x16 dv = gload<i32x16>(a.gdesc + gi);
  GroupDesc g{};
  g.wptr = uint64_t(uint32_t(dv[0])) | (uint64_t(uint32_t(dv[1])) << 32);
  g.row_begin = dv[2];
  g.row_count = dv[3];
  const int n_list = min(a.n_list, *a.n_list_dev);
  // whole workgroup: one group
  if (gi >= n_list || g.wptr == 0 || g.row_count <= 0) return;
  int tok = 0;
  if constexpr (GATEUP) {
    // token of row (lane & 15): 16-bit entry of dword 6 + (lane & 15) / 2
    const int n = threadIdx.x & 15;
    uint32_t wd = 0;
#pragma unroll
    for (int j = 0; j < kGroupTok / 2; ++j) wd = (n >> 1) == j ? uint32_t(dv[6 + j]) : wd;
    tok = int((n & 1) ? wd >> 16 : wd & 0xFFFFu);
  }
  wide_item<FMT, GATEUP, KPW, F>(a, g, rb0, threadIdx.x >> 6, SK, wide_red, tok);
}

// The wide kernel's (K tiles per wave, weight tiles per item) for a format and
// matrix, chosen so that a wave's registers stay within 256 (two waves per
// SIMD): per K tile the activations take 16 registers and each weight tile 5
// (FP4) or 12 (FP8, with its scales).
struct WideCfg {
  int kpw, f;
};
constexpr int wide_regs(int fmt, bool gateup, int kpw, int f) {
  return (gateup ? 2 : 1) * f * kpw * (fmt == FT_FMT_FP8_B128 ? 12 : 5) + 16 * kpw + (gateup ? 8 : 4) * f + 28;
}

// Launches the wide kernel unless its items would take more than kWideMaxRounds
// rounds of resident workgroups (large K: one pass per item then loses to the
// item rings, which overlap one item's loads with the previous one's work);
// *done tells which.
constexpr int kWideMaxRounds = 6;

template <int FMT, bool GATEUP, int KPW, int F>
hipError_t launch_wide_k(const FfnArgs& a, hipStream_t st, Ev ev, bool* done) {
  const MatLayout& m = a.lay.m[GATEUP ? 0 : 2];
  const int SK = m.cols / kTileK / KPW;
  constexpr int NM = GATEUP ? 2 : 1;
  const int64_t items = int64_t(a.n_list) * (m.rows / (kTileRows * F));
  const size_t lds = SK > 1 ? size_t(SK) * F * NM * 64 * sizeof(floatx4) : 0;
  static int64_t resident[kWideMaxWaves + 1] = {};
  if (!resident[SK]) {
    int dev = 0, cus = 0, per_cu = 0;
    (void)hipGetDevice(&dev);
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_ffn_wide<FMT, GATEUP, KPW, F>, 64 * SK, lds) !=
            hipSuccess ||
        per_cu < 1)
      per_cu = 1;
    resident[SK] = int64_t(per_cu) * std::max(cus, 1);
  }
  if (items > kWideMaxRounds * resident[SK]) {
    *done = false;
    return hipSuccess;
  }
  *done = true;
  {
    char prm[48];
    std::snprintf(prm, sizeof(prm), "%d K tiles x %d waves, %d weight tiles", KPW, SK, F);
    note_kernel(GATEUP, "k_ffn_wide", FMT, prm);
  }
  ft_launch_lds(k_ffn_wide<FMT, GATEUP, KPW, F>, dim3(unsigned(m.rows / (kTileRows * F)), unsigned(a.n_list)),
                dim3(64 * SK), lds, st, ev, a, SK);
  return hipGetLastError();
}

#ifndef FT_STREAM_MAXD
#define FT_STREAM_MAXD 4
#endif
// Ring depth: the deepest (up to 4: deeper rings cost occupancy and measured
// slower) that divides the K steps and keeps the weight ring within 80
// registers.
// Ring depth for NC row chunks: the registers of a ring slot (weights of
// one K tile of each matrix, plus one activation piece per chunk beyond the
// first) within a fixed budget; the depth must divide the K tiles.
// Gate/up with one or two row chunks, FP8 or MXFP4 weights: a ring of depth 1
// takes fewer registers, so more workgroups are resident at once.  FP8
// gate/up takes it whenever its launch fits one round of those workgroups
// (GLM-shaped, 12-24 experts: 1-9% faster than depth 3 in a standalone
// probe); MXFP4 gate/up only when the deeper ring would need a second round
// and depth 1 would not (20-24 experts: 8-18% faster; up to 16 experts, one
// round either way, depth 4 is 10-24% faster).  Down projections keep the
// deep ring (measured no better, or slower, at depth 1).
template <int FMT, bool GATEUP, int D, int NC>
int64_t stream_resident() {
  static const int64_t cap = resident_grid(k_ffn_stream<FMT, GATEUP, D, NC>, 64 * kStreamWaves);
  return cap;
}

template <int FMT, bool GATEUP, int NC>
hipError_t launch_stream_nc(const FfnArgs& a, hipStream_t st, Ev ev) {
  const int nkb = a.lay.m[GATEUP ? 0 : 2].cols / kTileK;
  constexpr int regs = (GATEUP ? 2 : 1) * (FMT == FT_FMT_FP8_B128 ? 12 : 5) + 4 * (NC - 1);  // per ring slot
  constexpr int dmax = std::min(FT_STREAM_MAXD, (NC > 1 ? 96 : 80) / regs);
  if constexpr (GATEUP && NC <= 2 && (FMT == FT_FMT_FP8_B128 || FMT == FT_FMT_MXFP4)) {
    const int64_t items = int64_t(a.n_list) * (a.lay.m[0].rows / (kTileRows * kStreamWaves));
    const int dd = dmax >= 4 && nkb % 4 == 0 ? 4 : dmax >= 3 && nkb % 3 == 0 ? 3 : dmax >= 2 && nkb % 2 == 0 ? 2 : 1;
    const int64_t res_deep = dd == 4   ? stream_resident<FMT, GATEUP, (dmax >= 4 ? 4 : 1), NC>()
                             : dd == 3 ? stream_resident<FMT, GATEUP, (dmax >= 3 ? 3 : 1), NC>()
                             : dd == 2 ? stream_resident<FMT, GATEUP, (dmax >= 2 ? 2 : 1), NC>()
                                       : stream_resident<FMT, GATEUP, 1, NC>();
    const int64_t res1 = stream_resident<FMT, GATEUP, 1, NC>();
    const bool shallow = FMT == FT_FMT_FP8_B128 ? items <= res1 : items > res_deep && items <= res1;
    if (shallow) return launch_stream_d<FMT, GATEUP, 1, NC>(a, st, ev);
  }
  if (dmax >= 4 && nkb % 4 == 0) return launch_stream_d<FMT, GATEUP, (dmax >= 4 ? 4 : 1), NC>(a, st, ev);
  if (dmax >= 3 && nkb % 3 == 0) return launch_stream_d<FMT, GATEUP, (dmax >= 3 ? 3 : 1), NC>(a, st, ev);
  if (dmax >= 2 && nkb % 2 == 0) return launch_stream_d<FMT, GATEUP, (dmax >= 2 ? 2 : 1), NC>(a, st, ev);
  return launch_stream_d<FMT, GATEUP, 1, NC>(a, st, ev);
}

// Row chunks of 16 the launch carries: enough for the call's bound on the
// rows of any group (at most kStreamMaxChunks), so every group's weights
// are read once whatever its row count.
template <int FMT, bool GATEUP>
hipError_t launch_stream(const FfnArgs& a, hipStream_t st, Ev ev) {
  const int chunks = a.max_rows > 0 ? (a.max_rows + kTileRows - 1) / kTileRows : kStreamMaxChunks;
  if (chunks <= 1) return launch_stream_nc<FMT, GATEUP, 1>(a, st, ev);
  if (chunks <= 2) return launch_stream_nc<FMT, GATEUP, 2>(a, st, ev);
  return launch_stream_nc<FMT, GATEUP, 4>(a, st, ev);
}

// Ring kernel split: the most K tiles per wave (at most 4) that divide K with
// at most kMaxWaves waves and keep one item's slice within 112 registers.
template <int FMT, bool GATEUP>
int ring_kpw(int nkb) {
  constexpr int slot = (GATEUP ? 2 : 1) * (FMT == FT_FMT_FP8_B128 ? 12 : 5) + 16;
  for (int kpw = 4; kpw >= 1; --kpw)
    if (nkb % kpw == 0 && nkb / kpw <= kMaxWaves && kpw * slot <= 112) return kpw;
  return 0;
}

template <int FMT, bool GATEUP, int KPW>
hipError_t launch_ring_k(const FfnArgs& a, int SK, hipStream_t st, Ev ev) {
  static int64_t cap[kMaxWaves + 1] = {};
  if (!cap[SK]) cap[SK] = resident_grid(k_ffn_ring<FMT, GATEUP, KPW>, 64 * SK);
  const int64_t items = int64_t(a.n_list) * (a.lay.m[GATEUP ? 0 : 2].rows / kTileRows);
  {
    char prm[48];
    std::snprintf(prm, sizeof(prm), "%d K tiles x %d waves", KPW, SK);
    note_kernel(GATEUP, "k_ffn_ring", FMT, prm);
  }
  ft_launch(k_ffn_ring<FMT, GATEUP, KPW>, dim3(unsigned(std::min(items, cap[SK]))), dim3(64 * SK), st, ev, a, SK);
  return hipGetLastError();
}

// Wide kernel configurations compiled for each format and matrix, in order of
// preference; a configuration applies when its K tiles per wave divide K into
// at most 8 slices and its weight tiles per item divide the rows.
template <int FMT, bool GATEUP>
hipError_t launch_wide(const FfnArgs& a, hipStream_t st, Ev ev, bool* done) {
  const MatLayout& m = a.lay.m[GATEUP ? 0 : 2];
  const int nkb = m.cols / kTileK, nrb = m.rows / kTileRows;
  *done = false;
  // prefer few weight tiles per item when the call has few groups, so that
  // the items still spread over the chip
  const bool few = int64_t(a.n_list) * nrb < 1024;
#define FT_WIDE_TRY(KPW, F)                                                                        \
  if constexpr (wide_regs(FMT, GATEUP, KPW, F) <= 256) {                                          \
    if (nkb % KPW == 0 && nkb / KPW <= kWideMaxWaves && nrb % F == 0)                             \
      return launch_wide_k<FMT, GATEUP, KPW, F>(a, st, ev, done);                                  \
  }
  // (measured on the Qwen-A3B decode shape: with 8 and 17 groups gate/up
  // 4 x 2 beat 4 x 1 by 10-13%, with 31 and 64 it tied 4 x 3; down 2 x 4 beat
  // 3 x 8 by 7-20% from 8 to 64 groups)
  if (GATEUP) {
    if (!few) { FT_WIDE_TRY(4, 3) }
    FT_WIDE_TRY(4, 2) FT_WIDE_TRY(4, 1) FT_WIDE_TRY(7, 1) FT_WIDE_TRY(6, 1) FT_WIDE_TRY(2, 2) FT_WIDE_TRY(3, 1) FT_WIDE_TRY(1, 2)
  } else {
    if (!few) { FT_WIDE_TRY(2, 4) FT_WIDE_TRY(3, 8) FT_WIDE_TRY(4, 4) FT_WIDE_TRY(2, 8) FT_WIDE_TRY(4, 2) }
    FT_WIDE_TRY(3, 2) FT_WIDE_TRY(4, 1) FT_WIDE_TRY(2, 2) FT_WIDE_TRY(1, 4) FT_WIDE_TRY(7, 1) FT_WIDE_TRY(6, 1)
  }
#undef FT_WIDE_TRY
  return hipSuccess;
}

template <int FMT, bool GATEUP>
hipError_t launch_small(const FfnArgs& a, hipStream_t st, Ev ev) {
  const int nkb = a.lay.m[GATEUP ? 0 : 2].cols / kTileK;
  bool wide = a.max_rows > 0 && a.max_rows <= kTileRows;
  if (wide) {
    bool done = false;
    const hipError_t r = launch_wide<FMT, GATEUP>(a, st, ev, &done);
    if (done) return r;
  }
  // gate/up: the item ring; down (short K, tiny items): the K-streaming kernel
  int kpw = GATEUP && a.max_rows > 0 && a.max_rows <= kTileRows ? ring_kpw<FMT, GATEUP>(nkb) : 0;
  switch (kpw) {
    case 4: return launch_ring_k<FMT, GATEUP, 4>(a, nkb / 4, st, ev);
    case 3: return launch_ring_k<FMT, GATEUP, 3>(a, nkb / 3, st, ev);
    case 2: return launch_ring_k<FMT, GATEUP, 2>(a, nkb / 2, st, ev);
    case 1: return launch_ring_k<FMT, GATEUP, 1>(a, nkb, st, ev);
    default: break;
  }
  if (a.lay.m[GATEUP ? 0 : 2].rows % (kTileRows * kStreamWaves)) return hipErrorInvalidValue;
  return launch_stream<FMT, GATEUP>(a, st, ev);
}

template <bool GATEUP>
hipError_t launch_ffn(const FfnArgs& a, hipStream_t st, Ev ev) {
  if (a.n_list <= 0) return hipSuccess;
  bool small = a.max_rows > 0 && a.max_rows <= kStreamMaxChunks * kTileRows;
  if (small) {
    switch (a.lay.fmt) {
      case FT_FMT_MXFP4: return launch_small<FT_FMT_MXFP4, GATEUP>(a, st, ev);
      case FT_FMT_NVFP4: return launch_small<FT_FMT_NVFP4, GATEUP>(a, st, ev);
      case FT_FMT_FP8_B128: return launch_small<FT_FMT_FP8_B128, GATEUP>(a, st, ev);
      default: return hipErrorInvalidValue;
    }
  }
  const MatLayout& m = a.lay.m[GATEUP ? 0 : 2];
  const int fmt = a.lay.fmt;
  const Split s = choose_split(m.cols, m.rows, kpw_max(fmt, GATEUP));
  if (s.SK == 0) return hipErrorInvalidValue;
  // one workgroup per item up to a chip's worth of resident workgroups; the
  // kernel strides over the rest (and over the unused tail of a bound)
  const int64_t items = int64_t(a.n_list) * (m.rows / kTileRows / s.RB);
  const dim3 grid(unsigned(std::min<int64_t>(items, kFfnMaxGrid)));
  const dim3 block(64 * s.RB * s.SK);
  switch (fmt) {
    case FT_FMT_MXFP4: return launch_fmt<FT_FMT_MXFP4, GATEUP>(a, s, grid, block, st, ev);
    case FT_FMT_NVFP4: return launch_fmt<FT_FMT_NVFP4, GATEUP>(a, s, grid, block, st, ev);
    case FT_FMT_FP8_B128: return launch_fmt<FT_FMT_FP8_B128, GATEUP>(a, s, grid, block, st, ev);
    default: return hipErrorInvalidValue;
  }
}

// out[t][h..h+7] = bf16( sum_j fp32(P[row(t,j)][h..h+7]) (+ fp32(P[shared row])) )
__global__ __launch_bounds__(256) void k_combine(const uint16_t* __restrict__ pbuf,
                                                 const int32_t* __restrict__ pair_row, int t0, int k, int H,
                                                 int shared_row0, uint16_t* __restrict__ out) {
  const int tt = blockIdx.y;
  const int t = t0 + tt;
  const int h = (blockIdx.x * 256 + threadIdx.x) * 8;
  if (h >= H) return;
  float acc[8];
  for (int j = 0; j < k; ++j) {
    const int row = pair_row[int64_t(t) * k + j];
    const uint4 v = *reinterpret_cast<const uint4*>(pbuf + int64_t(row) * H + h);
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = __uint_as_float(u[i] << 16), hi = __uint_as_float(u[i] & 0xFFFF0000u);
      if (j == 0) {
        acc[2 * i] = lo;
        acc[2 * i + 1] = hi;
      } else {
        acc[2 * i] += lo;
        acc[2 * i + 1] += hi;
      }
    }
  }
  if (shared_row0 >= 0) {
    const uint4 v = *reinterpret_cast<const uint4*>(pbuf + int64_t(shared_row0 + tt) * H + h);
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += __uint_as_float(u[i] << 16);
      acc[2 * i + 1] += __uint_as_float(u[i] & 0xFFFF0000u);
    }
  }
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = uint32_t(f32_to_bf16_rne(acc[2 * i])) | (uint32_t(f32_to_bf16_rne(acc[2 * i + 1])) << 16);
  *reinterpret_cast<uint4*>(out + int64_t(t) * H + h) = make_uint4(o[0], o[1], o[2], o[3]);
}

}  // namespace

bool ffn_shape_ok(int fmt, int hidden, int inter) {
  return choose_split(hidden, inter, kpw_max(fmt, true)).SK > 0 &&
         choose_split(inter, hidden, kpw_max(fmt, false)).SK > 0;
}

const char* ffn_last_kernel(bool gateup) { return g_ffn_kernel[gateup ? 0 : 1]; }

hipError_t launch_ffn_gateup(const FfnArgs& a, hipStream_t s, Ev ev) { return launch_ffn<true>(a, s, ev); }
hipError_t launch_ffn_down(const FfnArgs& a, hipStream_t s, Ev ev) { return launch_ffn<false>(a, s, ev); }

hipError_t launch_combine(const uint16_t* pbuf, const int32_t* pair_row, int t0, int T, int k, int H,
                          int shared_row0, uint16_t* out, hipStream_t s, Ev ev) {
  if (T <= t0) return hipSuccess;
  const dim3 grid((H / 8 + 255) / 256, T - t0);
  ft_launch(k_combine, grid, dim3(256), s, ev, pbuf, pair_row, t0, k, H, shared_row0, out);
  return hipGetLastError();
}

}  // namespace ftmoe
