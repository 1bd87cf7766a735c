// Host-side declarations of the expert layout in device memory (and in the
// pinned host store), the repacking from the canonical blob, and the host
// expert path.  No HIP headers: the host runtime pieces that use only these
// (layout.cpp, host_ffn.cpp) also build with a plain C++ compiler, e.g. under
// the address and undefined-behaviour sanitizers.
#pragma once

#include <cstdint>
#include <functional>

#include "../../include/ftmoe.h"

namespace ftmoe {

constexpr int kTileRows = 16;     // rows of one weight tile (MFMA M)
constexpr int kTileK = 128;       // K extent of one weight tile

// ------------------------------------------------------------ device expert layout
// One expert in GPU memory (and in the pinned host store, which holds the same
// bytes so a miss is one contiguous copy):
//   [gate codes][up codes][down codes][gate scales][up scales][down scales][tensor scales]
// each section 256-byte aligned.  A matrix W[R][K] is cut into tiles of
// 16 rows x 128 K, stored tile-major ([R/16][K/128]).  Inside a tile, lane
// l = 16*q + r of a 64-wide wavefront owns row r and K range [32q, 32q+32):
//   FP4 codes: 16 bytes per lane, 1024 per tile (nibble order unchanged)
//   FP8 codes: 32 bytes per lane, 2048 per tile
//   MXFP4 scales: 1 byte per lane per tile ([R/16][K/128][64])
//   NVFP4 scales: 2 bytes per lane per tile ([R/16][K/128][64][2])
//   FP8 scales: 16 fp32 per tile, one per row ([R/16][K/128][16])
// so that one 16-byte load per lane fetches a whole tile of FP4 codes, and
// the lane's 8-element sub-blocks are exactly the A operand of
// v_mfma_f32_16x16x32_bf16 (lane 16q+r holds row r, K 8j..8j+7 of sub-step j).
struct MatLayout {
  int64_t codes_off;
  int64_t scales_off;
  int32_t rows, cols;
};

struct ExpertLayout {
  int32_t fmt = 0, hidden = 0, inter = 0;
  MatLayout m[3];  // 0 gate [I][H], 1 up [I][H], 2 down [H][I]
  int64_t tscale_off = 0;  // 4 fp32 (NVFP4 per-matrix scales; others 1.0)
  int64_t bytes = 0;
};

ExpertLayout make_layout(int fmt, int hidden, int inter);
int64_t canonical_bytes(int fmt, int hidden, int inter);
// canonical blob -> device layout (dst has layout.bytes bytes)
void repack_expert(const ExpertLayout& L, const uint8_t* canonical, uint8_t* dst);
// device layout -> one row of matrix m as exact fp64 values (tensor scale applied)
void unpack_row_f64(const ExpertLayout& L, const uint8_t* dev_blob, int m, int row, double* out);
// device layout -> fp32 row-major matrix m (rows*cols)
void unpack_matrix_f32(const ExpertLayout& L, const uint8_t* dev_blob, int m, float* out);
// host_ffn.cpp: persistent host worker threads.  run() hands items 0 ..
// items - 1 to the threads - 1 background threads and the calling thread
// (each item once) and returns when all are done.  One caller at a time.
class WorkerPool {
 public:
  explicit WorkerPool(int threads);
  ~WorkerPool();
  WorkerPool(const WorkerPool&) = delete;
  WorkerPool& operator=(const WorkerPool&) = delete;
  void run(int64_t items, const std::function<void(int64_t)>& fn);
  int size() const;

 private:
  struct Impl;
  Impl* impl_;
};

// One host-computed expert: weights in the device layout (the pinned host
// store), x bf16 [rows][H] in, p = bf16(w * y) [rows][H] out.
struct HostExpertJob {
  const uint8_t* blob;
  const uint16_t* x;
  const float* w;
  int rows;
  uint16_t* out;
};
// The SwiGLU FFN of n experts of one format on the pool's threads: first the
// gate/up row blocks of every expert, then the down row blocks (one work item
// per few row blocks of one expert).
void host_experts(const ExpertLayout& L, const HostExpertJob* jobs, int n, WorkerPool& pool);
// The 32 fp32 weights that the host FFN decodes for lane `lane` of tile `tile`
// of matrix m (row lane % 16 of the tile, K 32 (lane / 16) .. + 31), in the
// build the CPU runs (the AVX2 one where it can).
void host_decode_lane(const ExpertLayout& L, const uint8_t* blob, int m, int64_t tile, int lane, float* w);
// One expert on a temporary pool of `threads` threads.
void host_expert(const ExpertLayout& L, const uint8_t* blob, const uint16_t* x, const float* wts, int rows,
                 uint16_t* out, int threads);

}  // namespace ftmoe
