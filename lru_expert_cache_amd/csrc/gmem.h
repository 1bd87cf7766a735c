// Device loads and stores through global-address-space pointers.
//
// Expert weights are addressed by slot addresses held as integers (the group
// descriptors), so a plain dereference is a generic (flat) access.  A flat
// load counts against both the vector-memory and the LDS/scalar wait counters,
// and the compiler then has to wait for every outstanding access at each use:
// loads no longer overlap the multiplies that consume earlier ones.  Casting
// to address space 1 makes them global loads, which complete in issue order
// and can be waited for one at a time.
#pragma once
#include <hip/hip_runtime.h>

#define FT_GLOBAL __attribute__((address_space(1)))

namespace ftmoe {

template <typename T>
__device__ __attribute__((always_inline)) inline T gload(const void* p) {
  return *(const FT_GLOBAL T*)p;
}

// streaming load (read once: not kept in the caches)
template <typename T>
__device__ __attribute__((always_inline)) inline T gload_nt(const void* p) {
  return __builtin_nontemporal_load((const FT_GLOBAL T*)p);
}

template <typename T>
__device__ __attribute__((always_inline)) inline void gstore(void* p, T v) {
  *(FT_GLOBAL T*)p = v;
}

}  // namespace ftmoe
