// The device scratch of the no-allocation entry point (ag_matmul_run_static): one
// file-scope array per device, holding that entry point's workspace (staging buffer, ready
// flags, counters, schedule tables). Its device address is taken once per device with
// hipGetSymbolAddress and kept; host code passes only that address to kernels and copies,
// never the array's name (which in host code is a host-side stand-in, not device memory).
#include <mutex>

#include "agmm_internal.h"

namespace agmm {
namespace {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

}  // namespace

hipError_t scratch_region(int device, void** ptr) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != device) return hipErrorInvalidDevice;  // the caller makes `device` current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr || ((uintptr_t)p & 255u) != 0) return hipErrorInvalidSymbol;
    g_scratch_ptr[device] = p;
  }
  *ptr = g_scratch_ptr[device];
  return hipSuccess;
}

}  // namespace agmm
