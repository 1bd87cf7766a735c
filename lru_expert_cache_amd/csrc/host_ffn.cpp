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
// reassociating a single sum; on CPUs with AVX2 and FMA, or AVX-512 (checked
// at run time), explicitly vectorised builds decode and multiply 8 or 16
// weights at a time.
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <atomic>
#include <condition_variable>
#include <functional>
#include <immintrin.h>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "layout.h"

namespace ftmoe {

namespace {

enum Isa { kPortable = 0, kAvx2 = 1, kAvx512 = 2 };

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

// AVX2: the 32 weights of lane `lane` of tile `tile` of matrix M as four
// 8-float vectors, the same values as decode_lane.  E2M1: pshufb on the
// nibbles with a table of 2 x the element values, widened and scaled by half
// the block scale.  E4M3: the code's bits moved into an fp16, widened to
// fp32 and rescaled by a power of two; the value table only where a lane
// holds a NaN code.
__attribute__((target("avx2,fma,f16c"))) inline void decode_lane_avx2(const MatLayout& M, int fmt, const uint8_t* blob,
                                                                  int64_t tile, int lane, float g, __m256 w[4]) {
  const Tables& tb = tables();
  if (fmt == FT_FMT_FP8_B128) {
    const uint8_t* c = blob + M.codes_off + (tile * 64 + lane) * 32;
    float sc;
    std::memcpy(&sc, blob + M.scales_off + (tile * 16 + (lane & 15)) * 4, 4);
    const __m256 vs = _mm256_set1_ps(sc);
    const __m256i abs7 = _mm256_set1_epi8(0x7F);
    const __m256i cb = _mm256_loadu_si256(reinterpret_cast<const __m256i*>(c));
    if (!_mm256_testz_si256(_mm256_cmpeq_epi8(_mm256_and_si256(cb, abs7), abs7), abs7)) {
      // a NaN code (S.1111.111) among the 32: the table keeps it NaN
      for (int v = 0; v < 4; ++v) {
        const __m256i idx = _mm256_cvtepu8_epi32(_mm_loadl_epi64(reinterpret_cast<const __m128i*>(c + 8 * v)));
        w[v] = _mm256_mul_ps(_mm256_i32gather_ps(tb.e4m3, idx, 4), vs);
      }
      return;
    }
    // S.EEEE.MMM placed as the fp16 bits S.0EEEE.MMM0000000 is 2^-8 times the
    // E4M3 value, subnormals included (fp16 subnormals then, which widen to
    // normal fp32 exactly); times 2^8 is exact, times the block scale rounds
    // once.  No fp32 subnormal is formed (slow on some CPUs).
    const __m128i keep = _mm_set1_epi16(int16_t(0xBF80u));
    const __m256 two8 = _mm256_set1_ps(256.0f);
    for (int v = 0; v < 4; ++v) {
      const __m128i h = _mm_and_si128(
          _mm_slli_epi16(_mm_cvtepi8_epi16(_mm_loadl_epi64(reinterpret_cast<const __m128i*>(c + 8 * v))), 7), keep);
      w[v] = _mm256_mul_ps(_mm256_mul_ps(_mm256_cvtph_ps(h), two8), vs);
    }
    return;
  }
  const uint8_t* c = blob + M.codes_off + (tile * 64 + lane) * 16;
  float s0, s1;
  if (fmt == FT_FMT_MXFP4) {
    s0 = s1 = e8m0_value(blob[M.scales_off + tile * 64 + lane]);
  } else {
    const uint8_t* sp = blob + M.scales_off + (tile * 64 + lane) * 2;
    s0 = tb.e4m3[sp[0]] * g;
    s1 = tb.e4m3[sp[1]] * g;
  }
  const __m128i lut2 = _mm_setr_epi8(0, 1, 2, 3, 4, 6, 8, 12, 0, -1, -2, -3, -4, -6, -8, -12);
  const __m128i lo4 = _mm_set1_epi8(0x0F);
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

__attribute__((target("avx2,fma,f16c"))) void decode_lane_avx2_store(const MatLayout& M, int fmt, const uint8_t* blob,
                                                                 int64_t tile, int lane, float g, float* out) {
  __m256 w[4];
  decode_lane_avx2(M, fmt, blob, tile, lane, g, w);
  for (int v = 0; v < 4; ++v) _mm256_storeu_ps(out + 8 * v, w[v]);
}

// AVX-512: the same 32 weights as two 16-float vectors.  E4M3 by the same
// steps as AVX2 (16 codes widened per step).  E2M1: each byte's two nibbles
// index a 16-entry table of the element values times the block scale (one
// permute per 16 weights), so w[0] holds the even elements 0, 2, .., 30 and
// w[1] the odd ones; the caller pairs them with inputs split the same way.
__attribute__((target("avx512f,avx512bw,avx2,fma,f16c"))) inline void decode_lane_avx512(const MatLayout& M, int fmt,
                                                                                     const uint8_t* blob,
                                                                                     int64_t tile, int lane,
                                                                                     float g, __m512 w[2]) {
  if (fmt == FT_FMT_FP8_B128) {
    const uint8_t* c = blob + M.codes_off + (tile * 64 + lane) * 32;
    float sc;
    std::memcpy(&sc, blob + M.scales_off + (tile * 16 + (lane & 15)) * 4, 4);
    const __m512 vs = _mm512_set1_ps(sc);
    const __m256i abs7 = _mm256_set1_epi8(0x7F);
    const __m256i cb = _mm256_loadu_si256(reinterpret_cast<const __m256i*>(c));
    if (!_mm256_testz_si256(_mm256_cmpeq_epi8(_mm256_and_si256(cb, abs7), abs7), abs7)) {
      const Tables& tb = tables();
      for (int v = 0; v < 2; ++v) {
        const __m512i idx = _mm512_cvtepu8_epi32(_mm_loadu_si128(reinterpret_cast<const __m128i*>(c + 16 * v)));
        w[v] = _mm512_mul_ps(_mm512_i32gather_ps(idx, tb.e4m3, 4), vs);
      }
      return;
    }
    const __m256i keep = _mm256_set1_epi16(int16_t(0xBF80u));
    const __m512 two8 = _mm512_set1_ps(256.0f);
    for (int v = 0; v < 2; ++v) {
      const __m256i h = _mm256_and_si256(
          _mm256_slli_epi16(_mm256_cvtepi8_epi16(_mm_loadu_si128(reinterpret_cast<const __m128i*>(c + 16 * v))), 7),
          keep);
      w[v] = _mm512_mul_ps(_mm512_mul_ps(_mm512_cvtph_ps(h), two8), vs);
    }
    return;
  }
  const uint8_t* c = blob + M.codes_off + (tile * 64 + lane) * 16;
  const __m512 lut = _mm512_setr_ps(0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f, -0.0f, -0.5f, -1.0f, -1.5f,
                                    -2.0f, -3.0f, -4.0f, -6.0f);
  const __m512i v = _mm512_cvtepu8_epi32(_mm_loadu_si128(reinterpret_cast<const __m128i*>(c)));
  const __m512i lo = _mm512_and_si512(v, _mm512_set1_epi32(15)), hi = _mm512_srli_epi32(v, 4);
  if (fmt == FT_FMT_MXFP4) {
    const __m512 ls = _mm512_mul_ps(lut, _mm512_set1_ps(e8m0_value(blob[M.scales_off + tile * 64 + lane])));
    w[0] = _mm512_permutexvar_ps(lo, ls);
    w[1] = _mm512_permutexvar_ps(hi, ls);
    return;
  }
  // NVFP4: bytes 0..7 (elements 0..15) take the first scale, bytes 8..15 the second
  const Tables& tb = tables();
  const uint8_t* sp = blob + M.scales_off + (tile * 64 + lane) * 2;
  const __m512 sv = _mm512_mask_blend_ps(__mmask16(0xFF00), _mm512_set1_ps(tb.e4m3[sp[0]] * g),
                                         _mm512_set1_ps(tb.e4m3[sp[1]] * g));
  w[0] = _mm512_mul_ps(_mm512_permutexvar_ps(lo, lut), sv);
  w[1] = _mm512_mul_ps(_mm512_permutexvar_ps(hi, lut), sv);
}

// MXFP4 on AVX-512, for callers that hold the lane's scale: the 16 lanes of a
// K quarter have their E8M0 bytes side by side, so mx_scales16 turns them into
// 16 floats at once (the same values as e8m0_value) and each lane's decode is
// then the table scaling and two permutes, as in decode_lane_avx512.
__attribute__((target("avx512f,avx512bw,avx2,fma,f16c"))) inline void mx_scales16(const uint8_t* s, float* out) {
  const __m512i b = _mm512_cvtepu8_epi32(_mm_loadu_si128(reinterpret_cast<const __m128i*>(s)));
  const __m512i u = _mm512_mask_blend_epi32(_mm512_cmpeq_epi32_mask(b, _mm512_setzero_si512()),
                                            _mm512_slli_epi32(b, 23), _mm512_set1_epi32(0x00400000));
  _mm512_storeu_ps(out, _mm512_castsi512_ps(u));
}
__attribute__((target("avx512f,avx512bw,avx2,fma,f16c"))) inline void decode_mxfp4_avx512(const uint8_t* c, float s,
                                                                                          __m512 w[2]) {
  const __m512 lut = _mm512_setr_ps(0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f, -0.0f, -0.5f, -1.0f, -1.5f,
                                    -2.0f, -3.0f, -4.0f, -6.0f);
  const __m512i v = _mm512_cvtepu8_epi32(_mm_loadu_si128(reinterpret_cast<const __m128i*>(c)));
  const __m512 ls = _mm512_mul_ps(lut, _mm512_set1_ps(s));
  w[0] = _mm512_permutexvar_ps(_mm512_and_si512(v, _mm512_set1_epi32(15)), ls);
  w[1] = _mm512_permutexvar_ps(_mm512_srli_epi32(v, 4), ls);
}

// FP8-b128 on AVX-512 for callers that hold the lane's block scale: the fp16
// placement of decode_lane_avx512, with lanes holding a NaN code (S.1111.111)
// decoded by table out of line.
__attribute__((target("avx512f,avx512bw,avx2,fma,f16c"), noinline)) void decode_fp8_nan_avx512(const uint8_t* c,
                                                                                                 float sc,
                                                                                                 __m512 w[2]) {
  const Tables& tb = tables();
  for (int v = 0; v < 2; ++v) {
    const __m512i idx = _mm512_cvtepu8_epi32(_mm_loadu_si128(reinterpret_cast<const __m128i*>(c + 16 * v)));
    w[v] = _mm512_mul_ps(_mm512_i32gather_ps(idx, tb.e4m3, 4), _mm512_set1_ps(sc));
  }
}
__attribute__((target("avx512f,avx512bw,avx2,fma,f16c"))) inline void decode_fp8_avx512(const uint8_t* c, float sc,
                                                                                        __m512 w[2]) {
  const __m256i abs7 = _mm256_set1_epi8(0x7F);
  const __m256i cb = _mm256_loadu_si256(reinterpret_cast<const __m256i*>(c));
  if (__builtin_expect(!_mm256_testz_si256(_mm256_cmpeq_epi8(_mm256_and_si256(cb, abs7), abs7), abs7), 0)) {
    decode_fp8_nan_avx512(c, sc, w);
    return;
  }
  const __m256i keep = _mm256_set1_epi16(int16_t(0xBF80u));
  const __m512 vs = _mm512_set1_ps(sc), two8 = _mm512_set1_ps(256.0f);
  const __m128i half[2] = {_mm256_castsi256_si128(cb), _mm256_extracti128_si256(cb, 1)};
  for (int v = 0; v < 2; ++v) {
    const __m256i h = _mm256_and_si256(_mm256_slli_epi16(_mm256_cvtepi8_epi16(half[v]), 7), keep);
    w[v] = _mm512_mul_ps(_mm512_mul_ps(_mm512_cvtph_ps(h), two8), vs);
  }
}

__attribute__((target("avx512f,avx512bw,avx2,fma,f16c"))) void decode_lane_avx512_store(const MatLayout& M, int fmt,
                                                                                    const uint8_t* blob,
                                                                                    int64_t tile, int lane, float g,
                                                                                    float* out) {
  __m512 w[2];
  decode_lane_avx512(M, fmt, blob, tile, lane, g, w);
  if (fmt == FT_FMT_FP8_B128) {
    _mm512_storeu_ps(out, w[0]);
    _mm512_storeu_ps(out + 16, w[1]);
    return;
  }
  alignas(64) float ev[16], od[16];
  _mm512_store_ps(ev, w[0]);
  _mm512_store_ps(od, w[1]);
  for (int i = 0; i < 16; ++i) {
    out[2 * i] = ev[i];
    out[2 * i + 1] = od[i];
  }
}

// Sums over K of the tiles of row blocks [rb_begin, rb_end) of matrices
// m0 .. m0 + nm - 1 against `rows` input rows xf [rows][K]; acc receives
// [matrix][row][16] per row block and `finish(rb, acc)` consumes it.
template <int ISA>
struct RowBlocks;

#define FT_HOST_BODY                                                                                   \
  const Tables& tb = tables();                                                                         \
  const int K = L.m[m0].cols, nkb = K / kTileK;                                                        \
  thread_local std::vector<float> acc;                                                                 \
  acc.resize(size_t(nm) * rows * 16);                                                                  \
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
struct RowBlocks<kPortable> {
  static void run(const ExpertLayout& L, const uint8_t* blob, int m0, int nm, const float* gsc, const float* xf,
                  int rows, int rb_begin, int rb_end, const std::function<void(int, const float*)>& finish) {
    FT_HOST_BODY
  }
};
// AVX2 + FMA: a lane's 32 weights decode as four 8-float vectors
// (decode_lane_avx2), and each (lane, input row) keeps an 8-wide partial sum
// across the K tiles of the row block, added up once at its end.
template <>
struct RowBlocks<kAvx2> {
  __attribute__((target("avx2,fma,f16c"))) static void run(const ExpertLayout& L, const uint8_t* blob, int m0, int nm,
                                                       const float* gsc, const float* xf, int rows, int rb_begin,
                                                       int rb_end,
                                                       const std::function<void(int, const float*)>& finish) {
    const int K = L.m[m0].cols, nkb = K / kTileK;
    const int fmt = L.fmt;
    thread_local std::vector<float> acc, part;  // part: [lane][row][8] (plain floats: unaligned vector access)
    acc.resize(size_t(nm) * rows * 16);
    part.resize(size_t(64) * rows * 8);
    for (int rb = rb_begin; rb < rb_end; ++rb) {
      std::fill(acc.begin(), acc.end(), 0.0f);
      for (int mi = 0; mi < nm; ++mi) {
        const MatLayout& M = L.m[m0 + mi];
        std::fill(part.begin(), part.end(), 0.0f);
        for (int kb = 0; kb < nkb; ++kb) {
          const int64_t tile = int64_t(rb) * nkb + kb;
          for (int lane = 0; lane < 64; ++lane) {
            __m256 w[4];
            decode_lane_avx2(M, fmt, blob, tile, lane, gsc[mi], w);
            const int k0 = kb * kTileK + 32 * (lane >> 4);
            for (int t = 0; t < rows; ++t) {
              const float* xr = xf + size_t(t) * K + k0;
              float* pp = &part[(size_t(lane) * rows + t) * 8];
              __m256 a = _mm256_loadu_ps(pp);
              a = _mm256_fmadd_ps(w[0], _mm256_loadu_ps(xr), a);
              a = _mm256_fmadd_ps(w[1], _mm256_loadu_ps(xr + 8), a);
              a = _mm256_fmadd_ps(w[2], _mm256_loadu_ps(xr + 16), a);
              a = _mm256_fmadd_ps(w[3], _mm256_loadu_ps(xr + 24), a);
              _mm256_storeu_ps(pp, a);
            }
          }
        }
        for (int lane = 0; lane < 64; ++lane)
          for (int t = 0; t < rows; ++t) {
            const float* v = &part[(size_t(lane) * rows + t) * 8];
            acc[(size_t(mi) * rows + t) * 16 + (lane & 15)] += ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
          }
      }
      finish(rb, acc.data());
    }
  }
};
// 32 inputs as two 16-float vectors: in order, or (split) the even positions
// then the odd ones.
__attribute__((target("avx512f,avx512bw,avx2,fma,f16c"))) inline void load_x512(const float* p, bool split,
                                                                                 __m512* o) {
  const __m512 a = _mm512_loadu_ps(p), b = _mm512_loadu_ps(p + 16);
  if (!split) {
    o[0] = a;
    o[1] = b;
    return;
  }
  o[0] = _mm512_permutex2var_ps(a, _mm512_setr_epi32(0, 2, 4, 6, 8, 10, 12, 14, 16, 18, 20, 22, 24, 26, 28, 30), b);
  o[1] = _mm512_permutex2var_ps(a, _mm512_setr_epi32(1, 3, 5, 7, 9, 11, 13, 15, 17, 19, 21, 23, 25, 27, 29, 31), b);
}

// AVX-512: a lane's 32 weights as two 16-float vectors.  Lanes are taken
// K-quarter by K-quarter (lane = 16 q + row), so the 32 inputs of each row
// that a quarter multiplies are loaded once per tile for its 16 lanes (split
// into even and odd positions for the E2M1 formats, as their weights come).
template <>
struct RowBlocks<kAvx512> {
  // Up to four input rows of an MXFP4 or FP8 matrix (the experts the hybrid
  // split sends to the host are the least used ones, mostly one or two rows):
  // the inputs of QG K quarters of a tile stay in registers (all four for one
  // or two rows, two for three or four), and a tile row's lanes of those
  // quarters are summed there, so its partial sums part[r][t] are read and
  // written 4 / QG times per tile instead of once per lane.  The decode is the
  // format's own (no branch on the format in the loop): MXFP4 with the
  // quarter's 16 scales converted at once, FP8 with the tile row's block
  // scale read once and the rare NaN codes decoded out of line.
  template <int RR, int QG, bool MX>
  __attribute__((target("avx512f,avx512bw,avx2,fma,f16c"))) static void few_rows(
      const MatLayout& M, const uint8_t* blob, int64_t rb, int nkb, const float* xf, int K, float* part) {
    for (int kb = 0; kb < nkb; ++kb) {
      const int64_t tile = rb * nkb + kb;
      const uint8_t* codes = blob + M.codes_off + tile * (MX ? 1024 : 2048);
      for (int q0 = 0; q0 < 4; q0 += QG) {
        __m512 xv[RR][QG][2];
        for (int t = 0; t < RR; ++t)
          for (int j = 0; j < QG; ++j) load_x512(xf + size_t(t) * K + kb * kTileK + 32 * (q0 + j), MX, xv[t][j]);
        float msc[16 * QG];
        if constexpr (MX)
          for (int j = 0; j < QG; ++j) mx_scales16(blob + M.scales_off + tile * 64 + 16 * (q0 + j), msc + 16 * j);
        for (int r = 0; r < 16; ++r) {
          __m512 a[RR];
          for (int t = 0; t < RR; ++t) a[t] = _mm512_setzero_ps();
          float sc = 0.0f;
          if constexpr (!MX) std::memcpy(&sc, blob + M.scales_off + (tile * 16 + r) * 4, 4);
          for (int j = 0; j < QG; ++j) {
            __m512 w[2];
            const int lane = 16 * (q0 + j) + r;
            if constexpr (MX)
              decode_mxfp4_avx512(codes + lane * 16, msc[16 * j + r], w);
            else
              decode_fp8_avx512(codes + lane * 32, sc, w);
            for (int t = 0; t < RR; ++t)
              a[t] = _mm512_fmadd_ps(w[1], xv[t][j][1], _mm512_fmadd_ps(w[0], xv[t][j][0], a[t]));
          }
          for (int t = 0; t < RR; ++t) {
            float* pp = part + (r * RR + t) * 16;
            _mm512_storeu_ps(pp, _mm512_add_ps(_mm512_loadu_ps(pp), a[t]));
          }
        }
      }
    }
  }
  template <bool MX>
  __attribute__((target("avx512f,avx512bw,avx2,fma,f16c"))) static void few_rows_any(
      int rows, const MatLayout& M, const uint8_t* blob, int64_t rb, int nkb, const float* xf, int K, float* part) {
    switch (rows) {
      case 1: few_rows<1, 4, MX>(M, blob, rb, nkb, xf, K, part); break;
      case 2: few_rows<2, 4, MX>(M, blob, rb, nkb, xf, K, part); break;
      case 3: few_rows<3, 2, MX>(M, blob, rb, nkb, xf, K, part); break;
      default: few_rows<4, 2, MX>(M, blob, rb, nkb, xf, K, part); break;
    }
  }

  __attribute__((target("avx512f,avx512bw,avx2,fma,f16c"))) static void run(
      const ExpertLayout& L, const uint8_t* blob, int m0, int nm, const float* gsc, const float* xf, int rows,
      int rb_begin, int rb_end, const std::function<void(int, const float*)>& finish) {
    const int K = L.m[m0].cols, nkb = K / kTileK;
    const int fmt = L.fmt;
    thread_local std::vector<float> acc, part;  // part: [lane][row][16]
    acc.resize(size_t(nm) * rows * 16);
    part.resize(size_t(64) * rows * 16);
    constexpr int kRegRows = 8;  // input rows whose quarter stays in registers
    __m512 xv[2 * kRegRows];
    const bool fp4 = fmt != FT_FMT_FP8_B128, mx = fmt == FT_FMT_MXFP4;
    for (int rb = rb_begin; rb < rb_end; ++rb) {
      std::fill(acc.begin(), acc.end(), 0.0f);
      for (int mi = 0; mi < nm; ++mi) {
        const MatLayout& M = L.m[m0 + mi];
        std::fill(part.begin(), part.end(), 0.0f);
        if (rows <= 4 && fmt != FT_FMT_NVFP4) {
          // part: [tile row][input row][16]
          if (mx)
            few_rows_any<true>(rows, M, blob, rb, nkb, xf, K, part.data());
          else
            few_rows_any<false>(rows, M, blob, rb, nkb, xf, K, part.data());
          for (int r = 0; r < 16; ++r)
            for (int t = 0; t < rows; ++t)
              acc[(size_t(mi) * rows + t) * 16 + r] += _mm512_reduce_add_ps(_mm512_loadu_ps(&part[(r * rows + t) * 16]));
          continue;
        }
        for (int kb = 0; kb < nkb; ++kb) {
          const int64_t tile = int64_t(rb) * nkb + kb;
          for (int q = 0; q < 4; ++q) {
            const int k0 = kb * kTileK + 32 * q;
            const int nreg = std::min(rows, kRegRows);
            for (int t = 0; t < nreg; ++t) load_x512(xf + size_t(t) * K + k0, fp4, &xv[2 * t]);
            float msc[16];
            if (mx) mx_scales16(blob + M.scales_off + tile * 64 + 16 * q, msc);
            for (int r = 0; r < 16; ++r) {
              const int lane = 16 * q + r;
              __m512 w[2];
              if (mx)
                decode_mxfp4_avx512(blob + M.codes_off + (tile * 64 + lane) * 16, msc[r], w);
              else
                decode_lane_avx512(M, fmt, blob, tile, lane, gsc[mi], w);
              float* pa = &part[size_t(lane) * rows * 16];
              for (int t = 0; t < nreg; ++t)
                _mm512_storeu_ps(pa + 16 * t, _mm512_fmadd_ps(w[1], xv[2 * t + 1],
                                                              _mm512_fmadd_ps(w[0], xv[2 * t],
                                                                              _mm512_loadu_ps(pa + 16 * t))));
              for (int t = nreg; t < rows; ++t) {
                __m512 xr[2];
                load_x512(xf + size_t(t) * K + k0, fp4, xr);
                _mm512_storeu_ps(pa + 16 * t, _mm512_fmadd_ps(w[1], xr[1],
                                                              _mm512_fmadd_ps(w[0], xr[0],
                                                                              _mm512_loadu_ps(pa + 16 * t))));
              }
            }
          }
        }
        for (int lane = 0; lane < 64; ++lane)
          for (int t = 0; t < rows; ++t)
            acc[(size_t(mi) * rows + t) * 16 + (lane & 15)] +=
                _mm512_reduce_add_ps(_mm512_loadu_ps(&part[(size_t(lane) * rows + t) * 16]));
      }
      finish(rb, acc.data());
    }
  }
};
#undef FT_HOST_BODY

// The widest build the CPU runs (AVX-512 F+BW, else AVX2 with FMA, else
// portable), capped by the environment for tests: FT_MOE_HOST_ISA =
// "portable" | "avx2" | "avx512" (or FT_MOE_HOST_PORTABLE set: portable).
int host_isa() {
  static const int isa = [] {
    int best = kPortable;
    if (__builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma") && __builtin_cpu_supports("f16c")) {
      best = kAvx2;
      if (__builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw")) best = kAvx512;
    }
    if (std::getenv("FT_MOE_HOST_PORTABLE") != nullptr) return int(kPortable);
    if (const char* e = std::getenv("FT_MOE_HOST_ISA")) {
      const std::string v(e);
      const int cap = v == "portable" ? kPortable : v == "avx2" ? kAvx2 : kAvx512;
      best = std::min(best, cap);
    }
    return best;
  }();
  return isa;
}

}  // namespace

// ---- worker pool: threads - 1 background threads plus the calling thread
// take work items from a shared counter; run() returns when every item of
// its task is done.
struct WorkerPool::Impl {
  std::mutex mu;
  std::condition_variable start_cv, done_cv;
  std::vector<std::thread> threads;
  const std::function<void(int64_t)>* fn = nullptr;
  int64_t items = 0;
  std::atomic<int64_t> next{0};
  uint64_t generation = 0;
  int busy = 0;  // background threads still working on the current task
  bool stop = false;

  void work() {
    for (;;) {
      const int64_t i = next.fetch_add(1, std::memory_order_relaxed);
      if (i >= items) return;
      (*fn)(i);
    }
  }
  void loop() {
    uint64_t seen = 0;
    for (;;) {
      {
        std::unique_lock<std::mutex> lk(mu);
        start_cv.wait(lk, [&] { return stop || generation != seen; });
        if (stop) return;
        seen = generation;
      }
      work();
      std::lock_guard<std::mutex> lk(mu);
      if (--busy == 0) done_cv.notify_one();
    }
  }
};

WorkerPool::WorkerPool(int threads) : impl_(new Impl) {
  for (int t = 1; t < std::max(1, threads); ++t) impl_->threads.emplace_back([this] { impl_->loop(); });
}

WorkerPool::~WorkerPool() {
  {
    std::lock_guard<std::mutex> lk(impl_->mu);
    impl_->stop = true;
  }
  impl_->start_cv.notify_all();
  for (auto& t : impl_->threads) t.join();
  delete impl_;
}

int WorkerPool::size() const { return int(impl_->threads.size()) + 1; }

void WorkerPool::run(int64_t items, const std::function<void(int64_t)>& fn) {
  if (items <= 0) return;
  Impl& m = *impl_;
  if (m.threads.empty() || items == 1) {
    for (int64_t i = 0; i < items; ++i) fn(i);
    return;
  }
  {
    std::lock_guard<std::mutex> lk(m.mu);
    m.fn = &fn;
    m.items = items;
    m.next.store(0, std::memory_order_relaxed);
    m.busy = int(m.threads.size());
    ++m.generation;
  }
  m.start_cv.notify_all();
  m.work();
  std::unique_lock<std::mutex> lk(m.mu);
  m.done_cv.wait(lk, [&] { return m.busy == 0; });
  m.fn = nullptr;
}

namespace {

// Row blocks per work item: enough tiles per item to amortise its setup,
// few enough that a layer's host experts spread over every thread.
constexpr int kBlocksPerItem = 4;

void run_blocks(const ExpertLayout& L, const uint8_t* blob, int m0, int nm, const float* gsc, const float* xf,
                int rows, int rb_begin, int rb_end, const std::function<void(int, const float*)>& finish) {
  switch (host_isa()) {
    case kAvx512:
      RowBlocks<kAvx512>::run(L, blob, m0, nm, gsc, xf, rows, rb_begin, rb_end, finish);
      break;
    case kAvx2:
      RowBlocks<kAvx2>::run(L, blob, m0, nm, gsc, xf, rows, rb_begin, rb_end, finish);
      break;
    default:
      RowBlocks<kPortable>::run(L, blob, m0, nm, gsc, xf, rows, rb_begin, rb_end, finish);
  }
}

}  // namespace

void host_experts(const ExpertLayout& L, const HostExpertJob* jobs, int n, WorkerPool& pool) {
  if (n <= 0) return;
  const int H = L.hidden, I = L.inter;
  const bool nv = L.fmt == FT_FMT_NVFP4;
  struct JobState {
    std::vector<float> xf, hf;
    float ts[4];
  };
  std::vector<JobState> js(static_cast<size_t>(n));
  for (int j = 0; j < n; ++j) {
    const HostExpertJob& jb = jobs[j];
    js[j].xf.resize(size_t(std::max(jb.rows, 0)) * H);
    js[j].hf.resize(size_t(std::max(jb.rows, 0)) * I);
    for (size_t i = 0; i < js[j].xf.size(); ++i) js[j].xf[i] = bf16_to_f32(jb.x[i]);
    std::memcpy(js[j].ts, jb.blob + L.tscale_off, 16);
  }
  const float one[2] = {1.0f, 1.0f};
  // phase 1, gate and up: h = bf16(silu(g) * u); items = (expert, group of row blocks)
  const int ngu = (I / kTileRows + kBlocksPerItem - 1) / kBlocksPerItem;
  pool.run(int64_t(n) * ngu, [&](int64_t it) {
    const int j = int(it / ngu), b0 = int(it % ngu) * kBlocksPerItem;
    const int rows = jobs[j].rows;
    if (rows <= 0) return;
    float* hf = js[j].hf.data();
    run_blocks(L, jobs[j].blob, 0, 2, nv ? js[j].ts : one, js[j].xf.data(), rows, b0,
               std::min(b0 + kBlocksPerItem, I / kTileRows), [&](int rb, const float* acc) {
                 for (int t = 0; t < rows; ++t)
                   for (int r = 0; r < kTileRows; ++r) {
                     const float g = acc[(0 * size_t(rows) + t) * 16 + r], u = acc[(1 * size_t(rows) + t) * 16 + r];
                     hf[size_t(t) * I + rb * kTileRows + r] = bf16_to_f32(f32_to_bf16(g / (1.0f + std::exp(-g)) * u));
                   }
               });
  });
  // phase 2, down: p = bf16(w * y)
  const int ndn = (H / kTileRows + kBlocksPerItem - 1) / kBlocksPerItem;
  pool.run(int64_t(n) * ndn, [&](int64_t it) {
    const int j = int(it / ndn), b0 = int(it % ndn) * kBlocksPerItem;
    const HostExpertJob& jb = jobs[j];
    if (jb.rows <= 0) return;
    run_blocks(L, jb.blob, 2, 1, nv ? js[j].ts + 2 : one, js[j].hf.data(), jb.rows, b0,
               std::min(b0 + kBlocksPerItem, H / kTileRows), [&](int rb, const float* acc) {
                 for (int t = 0; t < jb.rows; ++t)
                   for (int r = 0; r < kTileRows; ++r)
                     jb.out[size_t(t) * H + rb * kTileRows + r] = f32_to_bf16(jb.w[t] * acc[size_t(t) * 16 + r]);
               });
  });
}

void host_decode_lane(const ExpertLayout& L, const uint8_t* blob, int m, int64_t tile, int lane, float* w) {
  float g = 1.0f;
  if (L.fmt == FT_FMT_NVFP4) std::memcpy(&g, blob + L.tscale_off + 4 * m, 4);
  if (host_isa() == kAvx512) {
    decode_lane_avx512_store(L.m[m], L.fmt, blob, tile, lane, g, w);
    return;
  }
  if (host_isa() == kAvx2) {
    decode_lane_avx2_store(L.m[m], L.fmt, blob, tile, lane, g, w);
    return;
  }
  decode_lane(tables(), L, blob, m, tile, lane, g, w);
}

void host_expert(const ExpertLayout& L, const uint8_t* blob, const uint16_t* x, const float* wts, int rows,
                 uint16_t* out, int threads) {
  if (rows <= 0) return;
  WorkerPool pool(threads);
  const HostExpertJob job{blob, x, wts, rows, out};
  host_experts(L, &job, 1, pool);
}

}  // namespace ftmoe
