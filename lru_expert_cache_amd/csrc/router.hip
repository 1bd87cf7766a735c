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

// Large batches (prefill): 32 tokens x 32 experts per workgroup, each thread
// a 2x2 register tile, K staged through LDS in chunks of 64 as fp64.
constexpr int kTT = 32, kTE = 32, kKC = 64;

__global__ __launch_bounds__(256) void k_router_logits_tiled(
    const uint16_t* __restrict__ x, const float* __restrict__ wr, const float* __restrict__ bias,
    double* __restrict__ z, int T, int H, int E) {
  __shared__ double xs[kTT][kKC + 1];
  __shared__ double ws[kTE][kKC + 1];
  const int tid = threadIdx.x;
  const int tt0 = blockIdx.x * kTT, te0 = blockIdx.y * kTE;
  const int ty = tid / 16, tx = tid % 16;  // 16 x 16 threads, 2x2 each
  double acc[2][2] = {{0.0, 0.0}, {0.0, 0.0}};
  for (int k0 = 0; k0 < H; k0 += kKC) {
    // x tile: 32 x 64 bf16 = 2048 values, 8 per thread
    {
      const int r = tid / 8, c = (tid % 8) * 8;
      const int t = tt0 + r;
      if (t < T) {
        const uint4 v = *reinterpret_cast<const uint4*>(x + int64_t(t) * H + k0 + c);
        const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          xs[r][c + 2 * i] = bf16_to_f64(uint16_t(u[i] & 0xFFFF));
          xs[r][c + 2 * i + 1] = bf16_to_f64(uint16_t(u[i] >> 16));
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) xs[r][c + i] = 0.0;
      }
    }
    // w tile: 32 x 64 fp32, 8 per thread
    {
      const int r = tid / 8, c = (tid % 8) * 8;
      const int e = te0 + r;
      if (e < E) {
        const float4 a = *reinterpret_cast<const float4*>(wr + int64_t(e) * H + k0 + c);
        const float4 b = *reinterpret_cast<const float4*>(wr + int64_t(e) * H + k0 + c + 4);
        ws[r][c + 0] = a.x; ws[r][c + 1] = a.y; ws[r][c + 2] = a.z; ws[r][c + 3] = a.w;
        ws[r][c + 4] = b.x; ws[r][c + 5] = b.y; ws[r][c + 6] = b.z; ws[r][c + 7] = b.w;
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) ws[r][c + i] = 0.0;
      }
    }
    __syncthreads();
#pragma unroll 8
    for (int h = 0; h < kKC; ++h) {
      const double a0 = xs[2 * ty][h], a1 = xs[2 * ty + 1][h];
      const double b0 = ws[2 * tx][h], b1 = ws[2 * tx + 1][h];
      acc[0][0] = fma(a0, b0, acc[0][0]);
      acc[0][1] = fma(a0, b1, acc[0][1]);
      acc[1][0] = fma(a1, b0, acc[1][0]);
      acc[1][1] = fma(a1, b1, acc[1][1]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int t = tt0 + 2 * ty + i, e = te0 + 2 * tx + j;
      if (t < T && e < E) z[int64_t(t) * E + e] = acc[i][j] + (bias ? double(bias[e]) : 0.0);
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

hipError_t launch_router_logits(const uint16_t* x, const float* wr, const float* bias, double* z, int T,
                                int H, int E, hipStream_t s, Ev ev) {
  if (T <= 64) {
    if (T <= 4)
      ft_launch(k_router_logits_small<4>, dim3(E), dim3(kSmallThreads), s, ev, x, wr, bias, z, T, H, E);
    else
      ft_launch(k_router_logits_small<16>, dim3(E), dim3(kSmallThreads), s, ev, x, wr, bias, z, T, H, E);
  } else {
    ft_launch(k_router_logits_tiled, dim3((T + kTT - 1) / kTT, (E + kTE - 1) / kTE), dim3(256), s, ev, x, wr,
              bias, z, T, H, E);
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
