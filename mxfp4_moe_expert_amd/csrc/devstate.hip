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

// ---------------------------------------------------------------------------
// moe_forward_noalloc: moe_forward with its workspace in library-owned device
// memory, for callers that cannot allocate (graph capture, tight serving
// loops). The workspace is the file-scope array `scratch`, one copy per GPU,
// kept until the process ends. Host code never passes the array's name to a
// kernel (on the host it is only a stand-in for the symbol): the device
// address comes from hipGetSymbolAddress, once per device, with that device
// current.

#include "moe.h"

namespace moe {

constexpr size_t kScratchBytes = (size_t)16 << 20;  // the full-shape layer needs 9.1 MiB at T = 64
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
void* g_scratch_ptr[kMaxDevices];
// a call on this device failed after it may have launched kernels: counters
// in the scratch may be left non-zero, so the next call zero-fills it again
bool g_scratch_dirty[kMaxDevices];
}  // namespace

// The current device's scratch address, set up on first use: the symbol's
// address, then one zero fill (the workspace contract: zero before its first
// use), queued on `st` and, unless `st` is being captured, waited for. The
// fill is repeated on the first call after a failed one.
static void* scratch_for_current_device(hipStream_t st, int* dev_out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  *dev_out = dev;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch_ptr[dev] && !g_scratch_dirty[dev]) return g_scratch_ptr[dev];
  void* p = g_scratch_ptr[dev];
  if (!p && (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)) return nullptr;
  if (launch_fill_zero(p, kScratchBytes, st) != hipSuccess) return nullptr;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) != hipSuccess) return nullptr;
  if (cs == hipStreamCaptureStatusNone && hipStreamSynchronize(st) != hipSuccess) return nullptr;
  g_scratch_ptr[dev] = p;
  g_scratch_dirty[dev] = false;
  return p;
}

static void mark_scratch_dirty(int dev) {
  std::lock_guard<std::mutex> lock(g_mu);
  g_scratch_dirty[dev] = true;
}

}  // namespace moe

extern "C" size_t moe_noalloc_max_bytes(void) { return moe::kScratchBytes; }

extern "C" int moe_forward_noalloc(const moe_config* cfg, int32_t T, const uint16_t* x, const float* gate_w,
                                   const float* bias, const float* logit_offset, const int32_t* token_ids,
                                   const int32_t* tid2eid, int32_t V, const uint8_t* w13_codes,
                                   const uint8_t* w13_scales, const uint8_t* w2_codes, const uint8_t* w2_scales,
                                   const int8_t* sh_w13, const float* sh_w13_scale, const int8_t* sh_w2,
                                   const float* sh_w2_scale, void* out, int32_t out_is_fp32,
                                   int32_t* topk_ids_out, float* topk_w_out, void* stream) {
  if (!cfg) return MOE_EINVAL;
  if (T < 0) return MOE_EINVAL;
  const size_t need = moe_workspace_size(cfg, T);
  if (need == 0) return MOE_EUNSUPPORTED;
  if (need > moe::kScratchBytes) return MOE_EWORKSPACE;  // beyond the fixed scratch: use moe_forward
  if (T == 0) return MOE_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int dev = 0;
  void* ws = moe::scratch_for_current_device(st, &dev);
  if (!ws) return MOE_EHIP;
  const int rc = moe_forward(cfg, T, x, gate_w, bias, logit_offset, token_ids, tid2eid, V, w13_codes, w13_scales,
                             w2_codes, w2_scales, sh_w13, sh_w13_scale, sh_w2, sh_w2_scale, out, out_is_fp32,
                             topk_ids_out, topk_w_out, ws, moe::kScratchBytes, stream);
  if (rc == MOE_EHIP) moe::mark_scratch_dirty(dev);
  return rc;
}
