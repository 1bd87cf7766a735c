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
#include <cstring>

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
  const bool timed = a.clk != nullptr && total > 0;
  if (timed && threadIdx.x == 0) atomicMin(reinterpret_cast<unsigned long long*>(a.clk), wall_clock64());
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
  if (timed) {
    // the end time is taken once every store of the workgroup has completed
    // (`timed` is the same for the whole grid, so the barrier is uniform)
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
      unsigned long long* c = reinterpret_cast<unsigned long long*>(a.clk);
      atomicMax(c + 1, (unsigned long long)wall_clock64());
      __threadfence();
      if (atomicAdd(c + 2, 1ull) == gridDim.x - 1) {
        // last workgroup: every other one has published its end
        __threadfence();
        const unsigned long long t0 = atomicAdd(c, 0ull), t1 = atomicAdd(c + 1, 0ull);
        atomicAdd(reinterpret_cast<unsigned long long*>(a.ticks), t1 > t0 ? t1 - t0 : 0ull);
        atomicExch(c, ~0ull);
        atomicExch(c + 1, 0ull);
        atomicExch(c + 2, 0ull);
      }
    }
  }
}

// Debug mode (pool created with FT_MOE_POISON set): fill every slot about to
// receive a streamed miss with 0xFF bytes before the copy, so that a reader
// racing the copy sees NaN block scales (E8M0 / E4M3 0xFF, fp32 all ones)
// instead of plausible stale weights.
__global__ __launch_bounds__(256) void k_poison_slots(MissCopyArgs a) {
  const int nh = a.dev_header[2], n = a.dev_header[3];
  const int64_t n16 = a.bytes / 16;
  const int64_t total = int64_t(n) * n16;
  const u32x4 ones = {~0u, ~0u, ~0u, ~0u};
  for (int64_t j = int64_t(blockIdx.x) * 256 + threadIdx.x; j < total; j += int64_t(gridDim.x) * 256) {
    const int i = int(j / n16);
    const GroupDesc g = a.gdesc[nh + i];
    gstore<u32x4>(reinterpret_cast<u32x4*>(g.wptr) + (j - int64_t(i) * n16), ones);
  }
}

// Debug mode (pool created with FT_MOE_DEBUG_CHECKSUM set): one workgroup
// per group recomputes the checksum of the weights its FFN is about to read
// (slot_checksum: the sum of the expert's 32-bit words, each XOR-ed with its
// index times 0x9E3779B1, modulo 2^64) and compares it with the checksum of
// the key's blob in the host store.  The first mismatch is recorded in
// bad[0] = 1 + key, bad[1] = slot.  Groups g0 .. min(g1, *n_dev) - 1 of the
// run list; host-computed groups (slot -1) and the shared expert (-2) are
// skipped.
__global__ __launch_bounds__(256) void k_verify_slots(const GroupDesc* __restrict__ gdesc, int g0, int g1,
                                                      const int32_t* __restrict__ n_dev,
                                                      const uint64_t* __restrict__ key_sum, int key0, int64_t bytes,
                                                      unsigned long long* bad) {
  __shared__ unsigned long long part[4];
  const int n = n_dev != nullptr ? min(g1, *n_dev) : g1;
  const int gi = g0 + int(blockIdx.x);
  if (gi >= n) return;
  const GroupDesc g = gdesc[gi];
  if (g.slot < 0 || g.wptr == 0) return;  // uniform over the workgroup
  const uint32_t* w = reinterpret_cast<const uint32_t*>(g.wptr);
  const int64_t nw = bytes / 4;
  unsigned long long acc = 0;
  for (int64_t i = threadIdx.x; i < nw; i += 256) acc += gload<uint32_t>(w + i) ^ (uint32_t(i) * 0x9E3779B1u);
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_down(acc, off, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned long long sum = part[0] + part[1] + part[2] + part[3];
    if (sum != key_sum[key0 + g.expert] &&
        atomicCAS(bad, 0ull, (unsigned long long)(key0 + g.expert) + 1ull) == 0ull)
      atomicExch(bad + 1, (unsigned long long)g.slot);
  }
}

}  // namespace

uint64_t slot_checksum(const uint8_t* blob, int64_t bytes) {
  uint64_t acc = 0;
  for (int64_t i = 0; i < bytes / 4; ++i) {
    uint32_t v;
    std::memcpy(&v, blob + 4 * i, 4);
    acc += uint64_t(v ^ (uint32_t(i) * 0x9E3779B1u));
  }
  return acc;
}

hipError_t launch_verify_slots(const GroupDesc* gdesc, int g0, int g1, const int32_t* n_dev, const uint64_t* key_sum,
                               int key0, int64_t bytes, uint64_t* bad, hipStream_t s) {
  if (g1 <= g0) return hipSuccess;
  hipLaunchKernelGGL(k_verify_slots, dim3(g1 - g0), dim3(256), 0, s, gdesc, g0, g1, n_dev, key_sum, key0, bytes,
                     reinterpret_cast<unsigned long long*>(bad));
  return hipGetLastError();
}

hipError_t launch_poison_slots(const MissCopyArgs& a, int workgroups, hipStream_t s) {
  if (a.bytes <= 0 || a.bytes % 16 || workgroups < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_poison_slots, dim3(workgroups), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_miss_copy(const MissCopyArgs& a, int workgroups, hipStream_t s, Ev ev) {
  if (a.bytes <= 0 || a.bytes % 16 || workgroups < 1) return hipErrorInvalidValue;
  ft_launch(k_miss_copy, dim3(workgroups), dim3(256), s, ev, a);
  return hipGetLastError();
}

}  // namespace ftmoe
