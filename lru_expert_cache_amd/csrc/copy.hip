// Miss streaming driven by the GPU: the streamed misses of a decode call are
// copied from the pinned host store into their pool slots by a kernel that
// reads host memory over PCIe, with no host round trip between the resolve
// kernel that chose them and the copy.
//
// Pages: a miss is streamed from system RAM over PCIe into the GPU cache --
// devpik article "FreeToken: Run Frontier MoE Models on Your Own GPU, and the
// RAM It Takes", section "Why a Huge MoE Model Fits on One Consumer GPU"; the
// store is pinned host memory -- same article, "The Real Requirement Is
// System RAM".
//
// gfx950 design.  A few dozen workgroups saturate the PCIe link (each lane
// keeps four 16-byte non-temporal loads in flight), so the copy runs beside
// the FFN of the hit experts on the rest of the chip.  The streamed experts
// are treated as one concatenated byte range that is split evenly over the
// workgroups, so every miss count keeps all of them busy.
#include "common.h"
#include "gmem.h"

namespace ftmoe {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_miss_copy(MissCopyArgs a) {
  const int nh = a.dev_header[2], n = a.dev_header[3];
  const int64_t n16 = a.bytes / 16;
  const int64_t total = int64_t(n) * n16;
  const int64_t per = (total + gridDim.x - 1) / gridDim.x;
  int64_t lo = int64_t(blockIdx.x) * per;
  const int64_t hi = lo + per < total ? lo + per : total;
  while (lo < hi) {
    const int i = int(lo / n16);
    const int64_t off = lo - int64_t(i) * n16;
    const int64_t seg = (int64_t(i) + 1) * n16 < hi ? (int64_t(i) + 1) * n16 - lo : hi - lo;
    const GroupDesc g = a.gdesc[nh + i];
    // the slot address comes from an integer: store through a global pointer
    const u32x4* __restrict__ src =
        reinterpret_cast<const u32x4*>(a.host + a.key_off[int64_t(a.layer) * a.E + g.expert]) + off;
    u32x4* __restrict__ dst = reinterpret_cast<u32x4*>(g.wptr) + off;
    int64_t j = threadIdx.x;
    for (; j + 768 < seg; j += 1024) {
      const u32x4 v0 = gload_nt<u32x4>(src + j);
      const u32x4 v1 = gload_nt<u32x4>(src + j + 256);
      const u32x4 v2 = gload_nt<u32x4>(src + j + 512);
      const u32x4 v3 = gload_nt<u32x4>(src + j + 768);
      gstore<u32x4>(dst + j, v0);
      gstore<u32x4>(dst + j + 256, v1);
      gstore<u32x4>(dst + j + 512, v2);
      gstore<u32x4>(dst + j + 768, v3);
    }
    for (; j < seg; j += 256) gstore<u32x4>(dst + j, gload_nt<u32x4>(src + j));
    lo += seg;
  }
}

}  // namespace

hipError_t launch_miss_copy(const MissCopyArgs& a, int workgroups, hipStream_t s, Ev ev) {
  if (a.bytes <= 0 || a.bytes % 16 || workgroups < 1) return hipErrorInvalidValue;
  ft_launch(k_miss_copy, dim3(workgroups), dim3(256), s, ev, a);
  return hipGetLastError();
}

}  // namespace ftmoe
