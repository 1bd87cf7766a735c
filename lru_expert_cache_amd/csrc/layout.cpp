// Expert blob layouts: the canonical host format accepted at init, and the
// tiled device format used by the GPU kernels and the pinned host store.
#include <cmath>
#include <cstring>
#include <vector>

#include "layout.h"

namespace ftmoe {

namespace {
inline int64_t align256(int64_t v) { return (v + 255) & ~int64_t(255); }

int64_t code_bytes(int fmt, int64_t r, int64_t c) { return fmt == FT_FMT_FP8_B128 ? r * c : r * c / 2; }
int64_t scale_bytes(int fmt, int64_t r, int64_t c) {
  switch (fmt) {
    case FT_FMT_MXFP4: return r * c / 32;
    case FT_FMT_NVFP4: return r * c / 16;
    default: return r * c / 128 * 4;
  }
}

// E2M1 magnitude by 3-bit code (OCP MX v1.0 FP4 element).
const double kE2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

inline double e2m1(uint32_t c) { return (c & 8) ? -kE2M1[c & 7] : kE2M1[c & 7]; }
inline double e4m3(uint32_t b) {  // OCP E4M3 "FN": bias 7, no inf, S.1111.111 = NaN
  int e = (b >> 3) & 15, m = b & 7;
  double mag = e == 0 ? std::ldexp(m / 8.0, -6) : std::ldexp(1.0 + m / 8.0, e - 7);
  if (e == 15 && m == 7) mag = NAN;
  return (b & 0x80) ? -mag : mag;
}
inline double e8m0(uint32_t b) { return b == 255 ? NAN : std::ldexp(1.0, int(b) - 127); }
}  // namespace

int64_t canonical_bytes(int fmt, int hidden, int inter) {
  int64_t H = hidden, I = inter;
  int64_t n = 2 * (code_bytes(fmt, I, H) + scale_bytes(fmt, I, H)) + code_bytes(fmt, H, I) +
              scale_bytes(fmt, H, I);
  return fmt == FT_FMT_NVFP4 ? n + 12 : n;
}

ExpertLayout make_layout(int fmt, int hidden, int inter) {
  ExpertLayout L;
  L.fmt = fmt;
  L.hidden = hidden;
  L.inter = inter;
  const int rows[3] = {inter, inter, hidden};
  const int cols[3] = {hidden, hidden, inter};
  int64_t off = 0;
  for (int m = 0; m < 3; ++m) {
    L.m[m].rows = rows[m];
    L.m[m].cols = cols[m];
    L.m[m].codes_off = off;
    off = align256(off + code_bytes(fmt, rows[m], cols[m]));
  }
  for (int m = 0; m < 3; ++m) {
    L.m[m].scales_off = off;
    off = align256(off + scale_bytes(fmt, rows[m], cols[m]));
  }
  L.tscale_off = off;
  off = align256(off + 16);
  L.bytes = off;
  return L;
}

void repack_expert(const ExpertLayout& L, const uint8_t* src, uint8_t* dst) {
  const int fmt = L.fmt;
  // canonical offsets
  int64_t coff[3], soff[3];
  int64_t off = 0;
  for (int m = 0; m < 3; ++m) {
    coff[m] = off;
    off += code_bytes(fmt, L.m[m].rows, L.m[m].cols);
  }
  for (int m = 0; m < 3; ++m) {
    soff[m] = off;
    off += scale_bytes(fmt, L.m[m].rows, L.m[m].cols);
  }
  for (int m = 0; m < 3; ++m) {
    const int R = L.m[m].rows, K = L.m[m].cols;
    const int nrb = R / kTileRows, nkb = K / kTileK;
    uint8_t* dc = dst + L.m[m].codes_off;
    uint8_t* ds = dst + L.m[m].scales_off;
    const uint8_t* sc = src + coff[m];
    const uint8_t* ss = src + soff[m];
    for (int rb = 0; rb < nrb; ++rb)
      for (int kb = 0; kb < nkb; ++kb) {
        const int64_t tile = int64_t(rb) * nkb + kb;
        for (int lane = 0; lane < 64; ++lane) {
          const int q = lane >> 4, r = lane & 15;
          const int64_t row = int64_t(rb) * kTileRows + r;
          const int64_t k0 = int64_t(kb) * kTileK + 32 * q;  // first K element of the lane
          if (fmt == FT_FMT_FP8_B128) {
            std::memcpy(dc + (tile * 64 + lane) * 32, sc + row * K + k0, 32);
          } else {
            std::memcpy(dc + (tile * 64 + lane) * 16, sc + row * (K / 2) + k0 / 2, 16);
          }
          if (fmt == FT_FMT_MXFP4) {
            ds[tile * 64 + lane] = ss[row * (K / 32) + k0 / 32];
          } else if (fmt == FT_FMT_NVFP4) {
            ds[(tile * 64 + lane) * 2 + 0] = ss[row * (K / 16) + k0 / 16];
            ds[(tile * 64 + lane) * 2 + 1] = ss[row * (K / 16) + k0 / 16 + 1];
          }
        }
        if (fmt == FT_FMT_FP8_B128) {
          float* dsf = reinterpret_cast<float*>(ds);
          for (int r = 0; r < kTileRows; ++r) {
            const int64_t row = int64_t(rb) * kTileRows + r;
            std::memcpy(&dsf[tile * 16 + r], ss + (row * (K / 128) + kb) * 4, 4);
          }
        }
      }
  }
  float ts[4] = {1.f, 1.f, 1.f, 1.f};
  if (fmt == FT_FMT_NVFP4) std::memcpy(ts, src + off, 12);
  std::memcpy(dst + L.tscale_off, ts, 16);
}

// One row of matrix m as exact fp64 values (the NVFP4 per-tensor scale is
// applied too; e2m1 * e4m3 * fp32 and e4m3 * fp32 products are exact in fp64).
void unpack_row_f64(const ExpertLayout& L, const uint8_t* blob, int m, int row, double* out) {
  const int fmt = L.fmt;
  const int K = L.m[m].cols, nkb = K / kTileK;
  const int rb = row / kTileRows, r = row % kTileRows;
  const uint8_t* dc = blob + L.m[m].codes_off;
  const uint8_t* ds = blob + L.m[m].scales_off;
  float ts[4];
  std::memcpy(ts, blob + L.tscale_off, 16);
  const double g = fmt == FT_FMT_NVFP4 ? double(ts[m]) : 1.0;
  for (int kb = 0; kb < nkb; ++kb) {
    const int64_t tile = int64_t(rb) * nkb + kb;
    for (int q = 0; q < 4; ++q) {
      const int lane = q * 16 + r;
      double* o = out + kb * kTileK + 32 * q;
      if (fmt == FT_FMT_FP8_B128) {
        float s;
        std::memcpy(&s, ds + (tile * 16 + r) * 4, 4);
        const uint8_t* c = dc + (tile * 64 + lane) * 32;
        for (int i = 0; i < 32; ++i) o[i] = e4m3(c[i]) * double(s);
      } else {
        const uint8_t* c = dc + (tile * 64 + lane) * 16;
        for (int i = 0; i < 32; ++i) {
          const uint32_t code = (i & 1) ? (c[i >> 1] >> 4) : (c[i >> 1] & 15);
          double s;
          if (fmt == FT_FMT_MXFP4)
            s = e8m0(ds[tile * 64 + lane]);
          else
            s = e4m3(ds[(tile * 64 + lane) * 2 + (i >> 4)]) * g;
          o[i] = e2m1(code) * s;
        }
      }
    }
  }
}

void unpack_matrix_f32(const ExpertLayout& L, const uint8_t* blob, int m, float* out) {
  std::vector<double> row(L.m[m].cols);
  for (int r = 0; r < L.m[m].rows; ++r) {
    unpack_row_f64(L, blob, m, r, row.data());
    for (int c = 0; c < L.m[m].cols; ++c) out[int64_t(r) * L.m[m].cols + c] = float(row[c]);
  }
}

}  // namespace ftmoe
