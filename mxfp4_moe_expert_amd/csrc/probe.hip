// Measurement aid: the HBM read rate a plain streaming kernel reaches on
// this GPU, the denominator that sits beside the published 8 TB/s for the
// decode paths (they only read). A block reads 32 KB chunks of the buffer
// (chunk c, c + gridDim.x, ...): every wave-wide load is 64 lanes x 16
// contiguous bytes (1 KB), eight of them in flight per lane before any is
// used; the loaded words are folded together and stored only when they take
// one particular value, so the loads cannot be dropped and nothing but the
// buffer crosses the memory system.
#include <hip/hip_runtime.h>

#include "device.h"
#include "internal.h"
#include "moe.h"

namespace moe {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;

__global__ __launch_bounds__(kProbeThreads) void k_read_probe(const u32x4_t* p, size_t n16, uint32_t* sink) {
  constexpr size_t kChunk = (size_t)kProbeThreads * kProbeUnroll;  // 16-byte words per chunk
  const size_t nfull = n16 / kChunk * kChunk;
  u32x4_t acc = {0u, 0u, 0u, 0u};
  for (size_t c = (size_t)blockIdx.x * kChunk; c < nfull; c += (size_t)gridDim.x * kChunk) {
    u32x4_t v[kProbeUnroll];
#pragma unroll
    for (int j = 0; j < kProbeUnroll; ++j) v[j] = p[c + j * kProbeThreads + threadIdx.x];
#pragma unroll
    for (int j = 0; j < kProbeUnroll; ++j) acc ^= v[j];
  }
  // the words after the last whole chunk
  for (size_t i = nfull + (size_t)blockIdx.x * kProbeThreads + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * kProbeThreads)
    acc ^= p[i];
  const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (x == 0x9e3779b9u) sink[blockIdx.x] = x;
}

}  // namespace moe

extern "C" int moe_read_probe(const void* buf, size_t bytes, int32_t blocks, uint32_t* sink, void* stream) {
  if (!buf || !sink || blocks <= 0 || bytes == 0) return MOE_EINVAL;
  if ((reinterpret_cast<uintptr_t>(buf) & 15) || (bytes & 15)) return MOE_EINVAL;
  hipLaunchKernelGGL(moe::k_read_probe, dim3((unsigned)blocks), dim3(moe::kProbeThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4_t*>(buf), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}
