// MX activation quantiser: bf16 rows -> element codes + one E8M0 scale per 32
// elements along the row, by the OCP Microscaling Formats v1.0 rule for a
// block of scalars: X = 2^(floor(log2 amax) - emax_elem), each element is
// v / X rounded to nearest-even on the element grid and clamped to +-max, and
// an all-zero block gets scale 2^-127.  Used by the prefill activation modes,
// where both the expert inputs x and the SwiGLU outputs h are fed to the
// block-scaled MFMA as MXFP4 (E2M1, emax 2, max 6) or MXFP8 (E4M3, emax 8,
// max 448).  The inputs are bf16 and X a power of two, so v / X is exact; the
// rounding onto the grid is the hardware convert's (see fp4x8 / fp8x4).
//
// Output: row-major codes and scales; the tile gather copies those rows into
// the MX GEMM's activation tiles (the gate/up input, by token).  The down
// input h is quantised by the gate/up GEMM itself, with the same block code
// (mxq.h).
#include "common.h"
#include "gmem.h"
#include "mxq.h"

namespace ftmoe {

namespace {

using mxq::u32x4;

// One thread per 32-element block of a row: quantise it, then store its
// codes and scale byte row-major.
template <bool FP4>
__global__ __launch_bounds__(256) void k_mx_quant(MxQuantArgs a) {
  const int nblk = a.K / 32;
  const int64_t b = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (b >= int64_t(a.rows) * nblk) return;
  const int64_t row = b / nblk;
  const int kb32 = int(b % nblk);
  const uint4* src = reinterpret_cast<const uint4*>(a.in + row * a.K + int64_t(kb32) * 32);
  uint32_t w[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = src[i];
    w[4 * i] = v.x;
    w[4 * i + 1] = v.y;
    w[4 * i + 2] = v.z;
    w[4 * i + 3] = v.w;
  }
  uint32_t out[FP4 ? 4 : 8];
  const uint8_t sbyte = mxq::quant_block<FP4>(w, out);
  a.out_scales[row * nblk + kb32] = sbyte;
  uint8_t* dst = a.out_codes + row * (FP4 ? a.K / 2 : a.K) + int64_t(kb32) * (FP4 ? 16 : 32);
  gstore<u32x4>(dst, u32x4{out[0], out[1], out[2], out[3]});
  if constexpr (!FP4) gstore<u32x4>(dst + 16, u32x4{out[4], out[5], out[6], out[7]});
}

// One workgroup per (row tile, 128-K step) of the work list: copies the
// tile's 128 rows of that step from row-major quantised rows into the tile
// layout, 16 bytes per thread and piece, and the rows' four scale bytes.
// Pieces are numbered in destination order, so a workgroup's writes are one
// contiguous block (the gate/up input: a token's row feeds k tiles, and
// writing those copies from the quantiser directly scatters 16-byte pieces).
template <bool FP4>
__global__ __launch_bounds__(256) void k_mx_tile_gather(MxTileArgs a) {
  const int nkb = a.K / 128;
  const int tile = int(blockIdx.x) / nkb, kb = int(blockIdx.x) - tile * nkb;
  if (tile >= min(*a.n_tiles_dev, a.max_tiles)) return;
  const int d = a.tiles[2 * tile], tt = a.tiles[2 * tile + 1];
  const GroupDesc g = a.groups[d];
  const int r0 = tt * kMxTileRows;
  const int64_t pitch = FP4 ? a.K / 2 : a.K, spitch = a.K / 32;
  const int64_t blk = int64_t(tile) * nkb + kb;
  uint8_t* dst = a.out_codes + blk * mx_tile_code_bytes(FP4);
  constexpr int kPieces = FP4 ? 512 : 1024;  // 16-byte pieces of a block
  for (int pi = threadIdx.x; pi < kPieces; pi += 256) {
    // FP4: pi = 64 s + 16 q + n; FP8: pi = 128 s + 64 h + 16 q + n
    const int n = pi & 15, q = (pi >> 4) & 3;
    const int h = FP4 ? 0 : (pi >> 6) & 1;
    const int s = FP4 ? pi >> 6 : pi >> 7;
    const int r = r0 + 16 * s + n;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < g.row_count) {
      const int64_t src = a.row_map ? int64_t(a.row_map[g.row_begin + r]) : int64_t(g.row_begin + r);
      const int64_t k = FP4 ? int64_t(kb) * 64 + 16 * q : int64_t(kb) * 128 + 64 * h + 16 * q;
      v = gload<u32x4>(a.codes + src * pitch + k);
    }
    gstore<u32x4>(dst + int64_t(pi) * 16, v);
  }
  if (threadIdx.x < kMxTileRows) {
    const int r = r0 + int(threadIdx.x);
    uint32_t sv = 0;
    if (r < g.row_count) {
      const int64_t src = a.row_map ? int64_t(a.row_map[g.row_begin + r]) : int64_t(g.row_begin + r);
      sv = gload<uint32_t>(a.scales + src * spitch + int64_t(kb) * 4);
    }
    gstore<uint32_t>(a.out_scales + blk * kMxTileScaleBytes + int64_t(threadIdx.x) * 4, sv);
  }
}

}  // namespace

hipError_t launch_mx_quant(const MxQuantArgs& a, bool fp4, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  if (a.K % 128) return hipErrorInvalidValue;
  const int64_t blocks = int64_t(a.rows) * (a.K / 32);
  const dim3 grid(unsigned((blocks + 255) / 256));
  if (fp4)
    hipLaunchKernelGGL(k_mx_quant<true>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_mx_quant<false>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_mx_tile_gather(const MxTileArgs& a, bool fp4, hipStream_t s) {
  if (a.max_tiles <= 0) return hipSuccess;
  if (a.K % 128) return hipErrorInvalidValue;
  const dim3 grid(unsigned(int64_t(a.max_tiles) * (a.K / 128)));
  if (fp4)
    hipLaunchKernelGGL(k_mx_tile_gather<true>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_mx_tile_gather<false>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace ftmoe
