// Routed w2 + shared-expert w2 + weighted combine for the smallest batches
// (T*(k+1) <= 16) in one launch: the output-stationary block of w2combine.h
// with 8 waves.
#include "device.h"
#include "internal.h"
#include "w2combine.h"

namespace moe {

template <int MAXU, int MAXS, int MAXA>
__global__ __launch_bounds__(kThreads) void k_w2_combine_small(W2CombineArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  w2_combine_block<kWaves, MAXU, MAXS, MAXA>(a, blockIdx.x, lds);
}

size_t w2_combine_small_lds(int T, int k, int I) { return w2c_lds_bytes(T, k, I, kWaves, false); }

hipError_t launch_w2_combine_small(const W2CombineArgs& a, hipStream_t st) {
  if (a.T <= 0) return hipSuccess;
  const int ncols = a.T * (a.k + 1);
  if (ncols > 16) return hipErrorInvalidValue;
  const size_t lds = w2c_lds_bytes(a.T, a.k, a.I, kWaves, false);
  const int units_per_wave = (a.T * a.k * (a.I / 128) + kWaves - 1) / kWaves;
  auto kern = units_per_wave <= 12 ? &k_w2_combine_small<12, 2, 8> : &k_w2_combine_small<24, 2, 8>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  kern<<<a.H / 16, kThreads, lds, st>>>(a);
  return hipGetLastError();
}

}  // namespace moe
