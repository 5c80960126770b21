// The scratch memory of ckks_keyswitch_noalloc, the key-switch for callers that
// cannot allocate device memory at call time (code under HIP graph capture,
// serving loops, harnesses that forbid allocation).
//
// The workspace of its launch sequence lives in one file-scope device array,
// `scratch`.  Every GPU the library runs on holds its own copy of the array, at
// its own address, from the first context created there until the process ends.
// In host code the array's name is only a stand-in for the symbol; the device
// address is looked up once per device (hipGetSymbolAddress, with that device
// current) when a context is created there, and only that address is passed to
// kernels.  Calls on one GPU share the array: they must not overlap in time.
#include <hip/hip_runtime.h>

#include <mutex>

#include "ckks_internal.h"

namespace {

static __device__ __align__(256) uint32_t scratch[ckks::kScratchBytes / sizeof(uint32_t)];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
bool g_done[kMaxDevices];
hipError_t g_status[kMaxDevices];
uint32_t* g_ptr[kMaxDevices];

}  // namespace

namespace ckks {

hipError_t scratch_setup(int device) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_done[device]) {
    void* p = nullptr;
    g_status[device] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[device] = g_status[device] == hipSuccess ? static_cast<uint32_t*>(p) : nullptr;
    g_done[device] = true;
  }
  return g_status[device];
}

uint32_t* scratch_ptr(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  return g_ptr[device];
}

const char* scratch_error(int device) {
  if (device < 0 || device >= kMaxDevices) return "device index out of range";
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_done[device]) return "no context was created on this device";
  return hipGetErrorString(g_status[device]);
}

}  // namespace ckks
