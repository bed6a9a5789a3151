// Library state that lives in device memory, one copy per GPU: the word of
// device-side error flags (MOE_FLAG_* of include/moe.h). Kernels receive its
// address as an argument and set bits with atomicOr; the host reads and
// clears it with moe_device_flags.
#include <hip/hip_runtime.h>
#include <mutex>

#include "internal.h"

namespace moe {

static __device__ __align__(256) uint32_t g_flags[64];  // word 0: MOE_FLAG_* bits

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
uint32_t* g_flag_ptr[kMaxDevices];
}  // namespace

uint32_t* device_flags() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_flag_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_flags)) != hipSuccess) return nullptr;
    g_flag_ptr[dev] = static_cast<uint32_t*>(p);
  }
  return g_flag_ptr[dev];
}

}  // namespace moe
