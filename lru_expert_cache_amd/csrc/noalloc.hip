// The static device scratch behind ft_moe_layer_forward_noalloc: one
// file-scope array per GPU that holds every per-call work buffer of a
// device-driven decode call, for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is looked up once per device with hipGetSymbolAddress (at
// pool creation, with that device current) and only that address is used.
#include <mutex>

#include "common.h"

namespace ftmoe {

namespace {

constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
uint8_t* g_scratch_ptr[kMaxDevices] = {};
bool g_scratch_tried[kMaxDevices] = {};
hipError_t g_scratch_err[kMaxDevices] = {};

}  // namespace

// Looks up the device address of the scratch array on `device` (the current
// device) once; later calls return the kept address.
int scratch_register_device(int device) {
  if (device < 0 || device >= kMaxDevices) {
    set_error("device %d: no scratch slot (at most %d devices)", device, kMaxDevices);
    return FT_E_INVALID;
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_tried[device]) {
    g_scratch_tried[device] = true;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch_err[device] = e;
    if (e == hipSuccess) g_scratch_ptr[device] = static_cast<uint8_t*>(ptr);
    else (void)hipGetLastError();
  }
  if (g_scratch_ptr[device] == nullptr) {
    set_error("hipGetSymbolAddress of the scratch array failed on device %d: %s", device,
              hipGetErrorString(g_scratch_err[device]));
    return FT_E_HIP;
  }
  return FT_OK;
}

uint8_t* scratch_device_ptr(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  return g_scratch_ptr[device];
}

}  // namespace ftmoe
