// Host (CPU) SwiGLU expert for the hybrid split: the misses a step assigns to
// the host run on CPU threads, reading the expert from the pinned host store
// in the device layout, while the GPU streams and computes the rest.
//
// Same rounding points as the GPU path: g and u accumulate in fp32 from the
// exactly decoded weights and the bf16 inputs, h = bf16(silu(g) * u), y
// accumulates in fp32, p = bf16(w * y).  Only the summation order differs.
//
// The work is bound by host memory bandwidth (a GLM-shaped expert is 20-39
// MB for a few rows), so the weights are read once, tile by tile in storage
// order: a thread owns blocks of 16 output rows and walks their tiles along
// K, decoding each 16 x 128 tile with small tables (E2M1 / E4M3 element
// values, the block scale as a power of two or an E4M3 value) and adding its
// products to the rows' sums.  The portable build's inner products have
// eight independent partial sums, so that the compiler vectorises them without
// reassociating a single sum; on CPUs with AVX2 and FMA (checked at run
// time) an explicitly vectorised build decodes and multiplies 8 weights at a
// time.
#include <cmath>
#include <cstring>
#include <functional>
#include <immintrin.h>
#include <thread>
#include <vector>

#include "common.h"

namespace ftmoe {

namespace {

struct Tables {
  float e2m1[16];
  float e4m3[256];
  Tables() {
    const float mag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
    for (int c = 0; c < 16; ++c) e2m1[c] = (c & 8) ? -mag[c & 7] : mag[c & 7];
    for (int b = 0; b < 256; ++b) {
      // OCP E4M3 ("FN"): bias 7, subnormals e = 0, S.1111.111 = NaN, no infinities
      const int e = (b >> 3) & 15, m = b & 7;
      float v = e == 0 ? std::ldexp(float(m) / 8.0f, -6) : std::ldexp(1.0f + float(m) / 8.0f, e - 7);
      if (e == 15 && m == 7) v = NAN;
      e4m3[b] = (b & 0x80) ? -v : v;
    }
  }
};
const Tables& tables() {
  static const Tables t;
  return t;
}

// E8M0 scale byte -> 2^(b - 127) (b = 0: the subnormal 2^-127; 255, NaN, is never stored)
inline float e8m0_value(uint32_t b) {
  const uint32_t u = b ? b << 23 : 0x00400000u;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

inline float bf16_to_f32(uint16_t b) {
  const uint32_t u = uint32_t(b) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}
inline uint16_t f32_to_bf16(float f) {  // round to nearest even (finite inputs)
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return uint16_t((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// The 32 weights of lane `lane` of tile `tile` of matrix m, i.e. row
// lane % 16 of the tile at K 32 (lane / 16) .. + 31, exact in fp32 (NVFP4:
// the per-matrix scale g is folded in, one rounding).
inline void decode_lane(const Tables& tb, const ExpertLayout& L, const uint8_t* blob, int m, int64_t tile, int lane,
                        float g, float* w) {
  const MatLayout& M = L.m[m];
  if (L.fmt == FT_FMT_FP8_B128) {
    const uint8_t* c = blob + M.codes_off + (tile * 64 + lane) * 32;
    float s;
    std::memcpy(&s, blob + M.scales_off + (tile * 16 + (lane & 15)) * 4, 4);
    for (int j = 0; j < 32; ++j) w[j] = tb.e4m3[c[j]] * s;
    return;
  }
  const uint8_t* c = blob + M.codes_off + (tile * 64 + lane) * 16;
  float s0, s1;
  if (L.fmt == FT_FMT_MXFP4) {
    s0 = s1 = e8m0_value(blob[M.scales_off + tile * 64 + lane]);
  } else {
    const uint8_t* sp = blob + M.scales_off + (tile * 64 + lane) * 2;
    s0 = tb.e4m3[sp[0]] * g;
    s1 = tb.e4m3[sp[1]] * g;
  }
  for (int i = 0; i < 16; ++i) {
    const float s = i < 8 ? s0 : s1;
    w[2 * i] = tb.e2m1[c[i] & 15] * s;
    w[2 * i + 1] = tb.e2m1[c[i] >> 4] * s;
  }
}

// Sums over K of the tiles of row blocks [rb_begin, rb_end) of matrices
// m0 .. m0 + nm - 1 against `rows` input rows xf [rows][K]; acc receives
// [matrix][row][16] per row block and `finish(rb, acc)` consumes it.
template <bool AVX2>
struct RowBlocks;

#define FT_HOST_BODY                                                                                   \
  const Tables& tb = tables();                                                                         \
  const int K = L.m[m0].cols, nkb = K / kTileK;                                                        \
  std::vector<float> acc(size_t(nm) * rows * 16);                                                      \
  float w[32];                                                                                         \
  for (int rb = rb_begin; rb < rb_end; ++rb) {                                                         \
    std::fill(acc.begin(), acc.end(), 0.0f);                                                           \
    for (int mi = 0; mi < nm; ++mi)                                                                    \
      for (int kb = 0; kb < nkb; ++kb) {                                                               \
        const int64_t tile = int64_t(rb) * nkb + kb;                                                   \
        for (int lane = 0; lane < 64; ++lane) {                                                        \
          decode_lane(tb, L, blob, m0 + mi, tile, lane, gsc[mi], w);                                   \
          const int r = lane & 15, k0 = kb * kTileK + 32 * (lane >> 4);                                \
          for (int t = 0; t < rows; ++t) {                                                             \
            const float* xr = xf + size_t(t) * K + k0;                                                 \
            float p[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};                                    \
            for (int j = 0; j < 32; j += 8)                                                            \
              for (int u = 0; u < 8; ++u) p[u] += w[j + u] * xr[j + u];                                \
            acc[(size_t(mi) * rows + t) * 16 + r] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7])); \
          }                                                                                            \
        }                                                                                              \
      }                                                                                                \
    finish(rb, acc.data());                                                                            \
  }

template <>
struct RowBlocks<false> {
  static void run(const ExpertLayout& L, const uint8_t* blob, int m0, int nm, const float* gsc, const float* xf,
                  int rows, int rb_begin, int rb_end, const std::function<void(int, const float*)>& finish) {
    FT_HOST_BODY
  }
};
// AVX2 + FMA: a lane's 32 weights decode as four 8-float vectors (E2M1:
// pshufb on the nibbles with a table of 2 x the element values, widened and
// scaled by half the block scale; E4M3: gathers from the value table), and
// each (lane, input row) keeps an 8-wide partial sum across the K tiles of the
// row block, added up once at its end.
template <>
struct RowBlocks<true> {
  __attribute__((target("avx2,fma"))) static void run(const ExpertLayout& L, const uint8_t* blob, int m0, int nm,
                                                       const float* gsc, const float* xf, int rows, int rb_begin,
                                                       int rb_end,
                                                       const std::function<void(int, const float*)>& finish) {
    const Tables& tb = tables();
    const int K = L.m[m0].cols, nkb = K / kTileK;
    const int fmt = L.fmt;
    std::vector<float> acc(size_t(nm) * rows * 16);
    std::vector<__m256> part(size_t(64) * rows);
    const __m128i lut2 = _mm_setr_epi8(0, 1, 2, 3, 4, 6, 8, 12, 0, -1, -2, -3, -4, -6, -8, -12);
    const __m128i lo4 = _mm_set1_epi8(0x0F);
    for (int rb = rb_begin; rb < rb_end; ++rb) {
      std::fill(acc.begin(), acc.end(), 0.0f);
      for (int mi = 0; mi < nm; ++mi) {
        const MatLayout& M = L.m[m0 + mi];
        for (auto& v : part) v = _mm256_setzero_ps();
        for (int kb = 0; kb < nkb; ++kb) {
          const int64_t tile = int64_t(rb) * nkb + kb;
          for (int lane = 0; lane < 64; ++lane) {
            __m256 w[4];
            if (fmt == FT_FMT_FP8_B128) {
              const uint8_t* c = blob + M.codes_off + (tile * 64 + lane) * 32;
              float sc;
              std::memcpy(&sc, blob + M.scales_off + (tile * 16 + (lane & 15)) * 4, 4);
              const __m256 vs = _mm256_set1_ps(sc);
              for (int v = 0; v < 4; ++v) {
                const __m256i idx = _mm256_cvtepu8_epi32(_mm_loadl_epi64(reinterpret_cast<const __m128i*>(c + 8 * v)));
                w[v] = _mm256_mul_ps(_mm256_i32gather_ps(tb.e4m3, idx, 4), vs);
              }
            } else {
              const uint8_t* c = blob + M.codes_off + (tile * 64 + lane) * 16;
              float s0, s1;
              if (fmt == FT_FMT_MXFP4) {
                s0 = s1 = e8m0_value(blob[M.scales_off + tile * 64 + lane]);
              } else {
                const uint8_t* sp = blob + M.scales_off + (tile * 64 + lane) * 2;
                s0 = tb.e4m3[sp[0]] * gsc[mi];
                s1 = tb.e4m3[sp[1]] * gsc[mi];
              }
              const __m128i b = _mm_loadu_si128(reinterpret_cast<const __m128i*>(c));
              const __m128i lo = _mm_and_si128(b, lo4), hi = _mm_and_si128(_mm_srli_epi16(b, 4), lo4);
              // elements 0..15 and 16..31 (element 2i = low nibble of byte i), as 2 x value
              const __m128i e0 = _mm_shuffle_epi8(lut2, _mm_unpacklo_epi8(lo, hi));
              const __m128i e1 = _mm_shuffle_epi8(lut2, _mm_unpackhi_epi8(lo, hi));
              const __m256 h0 = _mm256_set1_ps(0.5f * s0), h1 = _mm256_set1_ps(0.5f * s1);
              w[0] = _mm256_mul_ps(_mm256_cvtepi32_ps(_mm256_cvtepi8_epi32(e0)), h0);
              w[1] = _mm256_mul_ps(_mm256_cvtepi32_ps(_mm256_cvtepi8_epi32(_mm_srli_si128(e0, 8))), h0);
              w[2] = _mm256_mul_ps(_mm256_cvtepi32_ps(_mm256_cvtepi8_epi32(e1)), h1);
              w[3] = _mm256_mul_ps(_mm256_cvtepi32_ps(_mm256_cvtepi8_epi32(_mm_srli_si128(e1, 8))), h1);
            }
            const int k0 = kb * kTileK + 32 * (lane >> 4);
            for (int t = 0; t < rows; ++t) {
              const float* xr = xf + size_t(t) * K + k0;
              __m256 a = part[size_t(lane) * rows + t];
              a = _mm256_fmadd_ps(w[0], _mm256_loadu_ps(xr), a);
              a = _mm256_fmadd_ps(w[1], _mm256_loadu_ps(xr + 8), a);
              a = _mm256_fmadd_ps(w[2], _mm256_loadu_ps(xr + 16), a);
              a = _mm256_fmadd_ps(w[3], _mm256_loadu_ps(xr + 24), a);
              part[size_t(lane) * rows + t] = a;
            }
          }
        }
        for (int lane = 0; lane < 64; ++lane)
          for (int t = 0; t < rows; ++t) {
            alignas(32) float v[8];
            _mm256_store_ps(v, part[size_t(lane) * rows + t]);
            acc[(size_t(mi) * rows + t) * 16 + (lane & 15)] += ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
          }
      }
      finish(rb, acc.data());
    }
  }
};
#undef FT_HOST_BODY

bool cpu_has_avx2_fma() {
  static const bool ok = __builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma");
  return ok;
}

void parallel_blocks(int n, int threads, const std::function<void(int, int)>& fn) {
  threads = std::max(1, std::min(threads, n));
  if (threads == 1) {
    fn(0, n);
    return;
  }
  std::vector<std::thread> th;
  const int chunk = (n + threads - 1) / threads;
  for (int t = 0; t < threads; ++t) {
    const int b = t * chunk, e = std::min(n, b + chunk);
    if (b >= e) break;
    th.emplace_back(fn, b, e);
  }
  for (auto& x : th) x.join();
}

void row_blocks(const ExpertLayout& L, const uint8_t* blob, int m0, int nm, const float* gsc, const float* xf, int rows,
                int threads, const std::function<void(int, const float*)>& finish) {
  const int nrb = L.m[m0].rows / kTileRows;
  const bool avx2 = cpu_has_avx2_fma();
  parallel_blocks(nrb, threads, [&](int b, int e) {
    if (avx2)
      RowBlocks<true>::run(L, blob, m0, nm, gsc, xf, rows, b, e, finish);
    else
      RowBlocks<false>::run(L, blob, m0, nm, gsc, xf, rows, b, e, finish);
  });
}

}  // namespace

void host_expert(const ExpertLayout& L, const uint8_t* blob, const uint16_t* x, const float* wts, int rows,
                 uint16_t* out, int threads) {
  if (rows <= 0) return;
  const int H = L.hidden, I = L.inter;
  float ts[4];
  std::memcpy(ts, blob + L.tscale_off, 16);
  const float one[2] = {1.0f, 1.0f};
  const bool nv = L.fmt == FT_FMT_NVFP4;
  std::vector<float> xf(size_t(rows) * H), hf(size_t(rows) * I);
  for (size_t i = 0; i < xf.size(); ++i) xf[i] = bf16_to_f32(x[i]);
  // gate and up: h = bf16(silu(g) * u)
  row_blocks(L, blob, 0, 2, nv ? ts : one, xf.data(), rows, threads, [&](int rb, const float* acc) {
    for (int t = 0; t < rows; ++t)
      for (int r = 0; r < kTileRows; ++r) {
        const float g = acc[(0 * size_t(rows) + t) * 16 + r], u = acc[(1 * size_t(rows) + t) * 16 + r];
        hf[size_t(t) * I + rb * kTileRows + r] = bf16_to_f32(f32_to_bf16(g / (1.0f + std::exp(-g)) * u));
      }
  });
  // down: p = bf16(w * y)
  row_blocks(L, blob, 2, 1, nv ? ts + 2 : one, hf.data(), rows, threads, [&](int rb, const float* acc) {
    for (int t = 0; t < rows; ++t)
      for (int r = 0; r < kTileRows; ++r)
        out[size_t(t) * H + rb * kTileRows + r] = f32_to_bf16(wts[t] * acc[size_t(t) * 16 + r]);
  });
}

}  // namespace ftmoe
