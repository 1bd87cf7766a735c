// Router: logits z = x Wr^T + bias in fp64, then per-token top-k with
// renormalised softmax weights.
//
// The pages fix only that a router sends each token to a few experts (devpik
// article "FreeToken: Run Frontier MoE Models on Your Own GPU...", section
// "Why a Huge MoE Model Fits on One Consumer GPU").  The exact reading used
// here: each bf16 x fp32 product is exact in fp64 and summed in fp64, so the
// selection (logit descending, lower expert index on ties) does not depend on
// the summation order beyond fp64 rounding; weights are the softmax of the
// selected logits rounded to fp32, evaluated in fp64.
#include "common.h"
#include "topk.h"

namespace ftmoe {

namespace {

__device__ inline double bf16_to_f64(uint16_t b) {
  return double(__uint_as_float(uint32_t(b) << 16));
}

// Small batches (decode): one workgroup per expert; its 256 threads stride
// over H four elements at a time (coalesced loads), the expert's router row
// stays in registers while up to 16 tokens stream past.  The per-token sums
// are reduced with a butterfly whose steps are interleaved across the tokens
// of the chunk (independent shuffles overlap), then across the 4 waves in LDS.
constexpr int kSmallThreads = 256;
constexpr int kSmallMaxJ = 8;   // H <= 8 * 1024

template <int kTokChunk>
__global__ __launch_bounds__(kSmallThreads) void k_router_logits_small(
    const uint16_t* __restrict__ x, const float* __restrict__ wr, const float* __restrict__ bias,
    double* __restrict__ z, int T, int H, int E) {
  const int e = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  __shared__ double red[kSmallThreads / 64][kTokChunk];
  float4 wv[kSmallMaxJ];
  const float* wrow = wr + int64_t(e) * H;
#pragma unroll
  for (int j = 0; j < kSmallMaxJ; ++j) {
    const int h = 4 * tid + 1024 * j;
    wv[j] = (h < H) ? *reinterpret_cast<const float4*>(wrow + h) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const double b = bias ? double(bias[e]) : 0.0;
  for (int t0 = 0; t0 < T; t0 += kTokChunk) {
    // all loads of the chunk first (clamped rows, so they can be hoisted), then the math
    uint2 xv[kTokChunk][2];
#pragma unroll
    for (int c = 0; c < kTokChunk; ++c) {
      const uint16_t* xr = x + int64_t(min(t0 + c, T - 1)) * H;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int h = 4 * tid + 1024 * j;
        xv[c][j] = (h < H) ? *reinterpret_cast<const uint2*>(xr + h) : make_uint2(0, 0);
      }
    }
    double acc[kTokChunk];
#pragma unroll
    for (int c = 0; c < kTokChunk; ++c) {
      acc[c] = 0.0;
      const uint16_t* xr = x + int64_t(min(t0 + c, T - 1)) * H;
#pragma unroll
      for (int j = 0; j < kSmallMaxJ; ++j) {
        const int h = 4 * tid + 1024 * j;
        if (h < H && t0 + c < T) {
          const uint2 v = j < 2 ? xv[c][j] : *reinterpret_cast<const uint2*>(xr + h);
          acc[c] = fma(bf16_to_f64(uint16_t(v.x & 0xFFFF)), double(wv[j].x), acc[c]);
          acc[c] = fma(bf16_to_f64(uint16_t(v.x >> 16)), double(wv[j].y), acc[c]);
          acc[c] = fma(bf16_to_f64(uint16_t(v.y & 0xFFFF)), double(wv[j].z), acc[c]);
          acc[c] = fma(bf16_to_f64(uint16_t(v.y >> 16)), double(wv[j].w), acc[c]);
        }
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
#pragma unroll
      for (int c = 0; c < kTokChunk; ++c) acc[c] += __shfl_xor(acc[c], off, 64);
    }
    if (lane == 0) {
#pragma unroll
      for (int c = 0; c < kTokChunk; ++c) red[wid][c] = acc[c];
    }
    __syncthreads();
    if (tid < kTokChunk && t0 + tid < T) {
      double s = 0.0;
#pragma unroll
      for (int w = 0; w < kSmallThreads / 64; ++w) s += red[w][tid];
      z[int64_t(t0 + tid) * E + e] = s + b;
    }
    __syncthreads();
  }
}

// Large batches (prefill), on the fp64 matrix cores: v_mfma_f64_16x16x4_f64
// takes a 16 x 4 block of x (lane l: token l % 16, K index l / 16), a 4 x 16
// block of Wr^T (lane l: K index l / 16, expert l % 16) and accumulates the
// 16 x 16 logits in fp64 (lane l, element i: token 4 i + l / 16, expert l % 16).
// Products of bf16 and fp32 values are exact in fp64 and every sum is fp64,
// as in the scalar kernels; only the summation order differs.  The order of
// K in a sum is free, so in each 64-wide K chunk the four lane groups take
// sixteen consecutive K values each (group g: K 16g .. 16g + 15, one per MFMA
// step): a lane's operands are then two 16-byte loads of its x row and four
// of its router row per expert tile, straight from global memory (the router
// rows are shared by the workgroup's waves through the L1), with the next
// chunk's loads issued before this chunk's MFMAs.  A wave owns 16 tokens x 32
// experts (two MFMA tiles), a workgroup 64 x 32.
constexpr int kMfmaTokW = 16, kMfmaKC = 64;

typedef double f64x4 __attribute__((ext_vector_type(4)));

// One K chunk of a lane's operands: 16 bf16 of its token, 16 fp32 of its
// router row in each of the wave's ET expert tiles.
template <int ET>
struct RouterChunk {
  uint4 xv[2];
  float4 wv[ET][4];
};

template <int ET>
__device__ inline void router_chunk_load(RouterChunk<ET>& c, const uint16_t* xr, const float* const (&wrow)[ET],
                                         int k0) {
  c.xv[0] = *reinterpret_cast<const uint4*>(xr + k0);
  c.xv[1] = *reinterpret_cast<const uint4*>(xr + k0 + 8);
#pragma unroll
  for (int e = 0; e < ET; ++e)
#pragma unroll
    for (int j = 0; j < 4; ++j) c.wv[e][j] = *reinterpret_cast<const float4*>(wrow[e] + k0 + 4 * j);
}

__device__ inline float f4_at(const float4& v, int i) { return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w; }

// A workgroup is TW x KS waves: TW waves of 16 tokens each (a wave owns ET
// tiles of 16 experts), times KS wave groups splitting K: group q takes
// chunks q, q + KS, ...; groups 1 .. KS-1 leave their sums in LDS and group 0
// adds them in group order (a fixed order, so the logits do not depend on
// timing).
template <int TW, int ET, int KS>
__global__ __launch_bounds__(64 * TW * KS) void k_router_logits_mfma(
    const uint16_t* __restrict__ x, const float* __restrict__ wr, const float* __restrict__ bias,
    double* __restrict__ z, int T, int H, int E) {
  __shared__ f64x4 part[KS > 1 ? KS - 1 : 1][TW][ET][64];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wv = wid % TW, q = wid / TW;
  const int g = lane >> 4, n = lane & 15;
  const int t0 = blockIdx.x * (kMfmaTokW * TW) + wv * kMfmaTokW;
  const int e0 = blockIdx.y * (16 * ET);
  // operand rows of this lane (clamped: rows past T or E are computed and not
  // stored); lane group g takes K 16g .. 16g + 15 of every 64-wide chunk
  const uint16_t* xr = x + int64_t(min(t0 + n, T - 1)) * H + 16 * g;
  const float* wrow[ET];
#pragma unroll
  for (int e = 0; e < ET; ++e) wrow[e] = wr + int64_t(min(e0 + 16 * e + n, E - 1)) * H + 16 * g;
  f64x4 acc[ET];
#pragma unroll
  for (int e = 0; e < ET; ++e) acc[e] = {0.0, 0.0, 0.0, 0.0};
  RouterChunk<ET> cur, nxt;
  const int kstep = kMfmaKC * KS;
  if (q * kMfmaKC < H) router_chunk_load<ET>(cur, xr, wrow, q * kMfmaKC);
  for (int k0 = q * kMfmaKC; k0 < H; k0 += kstep) {
    if (k0 + kstep < H) router_chunk_load<ET>(nxt, xr, wrow, k0 + kstep);
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const uint32_t xu = s < 8 ? (s < 4 ? (s < 2 ? cur.xv[0].x : cur.xv[0].y) : (s < 6 ? cur.xv[0].z : cur.xv[0].w))
                                : (s < 12 ? (s < 10 ? cur.xv[1].x : cur.xv[1].y) : (s < 14 ? cur.xv[1].z : cur.xv[1].w));
      const double a = bf16_to_f64(uint16_t(s & 1 ? xu >> 16 : xu & 0xFFFF));
#pragma unroll
      for (int e = 0; e < ET; ++e)
        acc[e] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, double(f4_at(cur.wv[e][s >> 2], s & 3)), acc[e], 0, 0, 0);
    }
    cur = nxt;
  }
  if constexpr (KS > 1) {
    if (q > 0)
#pragma unroll
      for (int e = 0; e < ET; ++e) part[q - 1][wv][e][lane] = acc[e];
    __syncthreads();
    if (q > 0) return;
#pragma unroll
    for (int j = 0; j < KS - 1; ++j)
#pragma unroll
      for (int e = 0; e < ET; ++e) acc[e] += part[j][wv][e][lane];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + 4 * i + g;
    if (t >= T) continue;
#pragma unroll
    for (int e = 0; e < ET; ++e) {
      const int ex = e0 + 16 * e + n;
      if (ex < E) z[int64_t(t) * E + ex] = acc[e][i] + (bias ? double(bias[ex]) : 0.0);
    }
  }
}

}  // namespace

namespace {

constexpr int kTopkWaves = 4;

__global__ __launch_bounds__(64 * kTopkWaves) void k_topk(const double* __restrict__ z, int T, int E,
                                                          int k, int32_t* __restrict__ sel,
                                                          float* __restrict__ w,
                                                          double* __restrict__ gap) {
  const int t = blockIdx.x * kTopkWaves + (threadIdx.x >> 6);
  if (t >= T) return;
  wave_topk(z + int64_t(t) * E, E, k, sel + int64_t(t) * k, w + int64_t(t) * k, gap + t);
}

}  // namespace

// Up to 16 tokens: the scalar kernels (one workgroup per expert; a batch of
// 1 takes 4.4 us on the Qwen-A3B shape, where the matrix-core kernel was
// slower).  17 to 64 tokens: one 16-token wave per 16 experts with K split
// over 16 wave groups, so a layer's few tokens still spread over many
// workgroups (GLM-shaped layer at 32 tokens: 23 us against 67 us scalar).
// More (prefill): four 16-token waves of 32 experts each and two K groups
// (two waves per SIMD: 4096 x 2048 x 128 took 69 us with one group, 54 with
// two, 53.5 with four).
hipError_t launch_router_logits(const uint16_t* x, const float* wr, const float* bias, double* z, int T,
                                int H, int E, hipStream_t s, Ev ev) {
  if (T <= 4) {
    ft_launch(k_router_logits_small<4>, dim3(E), dim3(kSmallThreads), s, ev, x, wr, bias, z, T, H, E);
  } else if (T <= 16) {
    ft_launch(k_router_logits_small<16>, dim3(E), dim3(kSmallThreads), s, ev, x, wr, bias, z, T, H, E);
  } else if (T <= 64) {
    const dim3 grid((T + 15) / 16, (E + 15) / 16);
    ft_launch(k_router_logits_mfma<1, 1, 16>, grid, dim3(64 * 16), s, ev, x, wr, bias, z, T, H, E);
  } else {
    const dim3 grid((T + 63) / 64, (E + 31) / 32);
    ft_launch(k_router_logits_mfma<4, 2, 2>, grid, dim3(64 * 4 * 2), s, ev, x, wr, bias, z, T, H, E);
  }
  return hipGetLastError();
}

hipError_t launch_topk(const double* z, int T, int E, int k, int32_t* sel, float* w, double* gap,
                       hipStream_t s, Ev ev) {
  ft_launch(k_topk, dim3((T + kTopkWaves - 1) / kTopkWaves), dim3(64 * kTopkWaves), s, ev, z, T, E, k, sel, w,
            gap);
  return hipGetLastError();
}

}  // namespace ftmoe
