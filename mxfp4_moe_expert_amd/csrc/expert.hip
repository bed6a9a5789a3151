// Expert-pass launches for gfx950. Each launch runs the skinny expert block
// (skinny.h) for one pass, optionally together with the blocks of another,
// independent pass in the same grid, so short decode passes share one launch
// and fill the chip:
//   w13 launch: routed MXFP4 w13 + SwiGLU, with the shared expert's int8 w2
//               (decode) or int8 w13 (large T);
//   w2 launch:  routed MXFP4 w2 x routing weight, optionally with the shared
//               expert's int8 w2 (large T).
// The final combine adds the k weighted slot outputs of each token in slot
// order and the shared expert's output (page "DeepSeek-V4-Flash-0731",
// section "Checked in its code", row "Shared expert": routed + shared).
#include "device.h"
#include "internal.h"
#include "skinny.h"

namespace moe {

// Pass a (blocks [0, a_blocks)) and pass b in one grid of WAVES-wave blocks;
// NA / NB super-steps per wave are in flight at once.
template <int FA, int SA, int FB, int SB, int WAVES, int NA, int NB>
__global__ __launch_bounds__(WAVES * 64) void k_pair(SkinnyArgs a, int a_blocks, SkinnyArgs b) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int bid = blockIdx.x;
  if (bid < a_blocks) {
    skinny_block<FA, SA, WAVES, NA>(a, bid, lds);
  } else {
    skinny_block<FB, SB, WAVES, NB>(b, bid - a_blocks, lds);
  }
}

template <int FA, int SA, int FB, int SB, int WAVES = kWaves, int NA = 4, int NB = 4>
static hipError_t launch_pair(const SkinnyArgs& a, int a_blocks, const SkinnyArgs* b, int b_blocks,
                              hipStream_t st) {
  SkinnyArgs bb{};
  if (b) bb = *b; else b_blocks = 0;
  const long long nblk = (long long)a_blocks + b_blocks;
  if (nblk <= 0) return hipSuccess;
  if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
  size_t lds = a_blocks > 0 ? skinny_lds_bytes(a.tile_n, a.K, SA, WAVES) : 0;
  if (b_blocks > 0) {
    const size_t lb = skinny_lds_bytes(bb.tile_n, bb.K, SB, WAVES);
    lds = lb > lds ? lb : lds;
  }
  auto kern = &k_pair<FA, SA, FB, SB, WAVES, NA, NB>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  kern<<<(unsigned)nblk, WAVES * 64, lds, st>>>(a, a_blocks, bb);
  return hipGetLastError();
}

hipError_t launch_w13(const SkinnyArgs& a, int a_blocks, const SkinnyArgs* b, int b_blocks, bool b_is_shared_w2,
                      hipStream_t st) {
  // b is the shared expert: its w2 in the decode schedule, its w13 otherwise
  if (b && b_is_shared_w2) return launch_pair<kFmtMx, kW13, kFmtI8, kW2>(a, a_blocks, b, b_blocks, st);
  return launch_pair<kFmtMx, kW13, kFmtI8, kW13>(a, a_blocks, b, b_blocks, st);
}

hipError_t launch_w2(const SkinnyArgs& a, int a_blocks, const SkinnyArgs* b, int b_blocks, hipStream_t st) {
  return launch_pair<kFmtMx, kW2, kFmtI8, kW2>(a, a_blocks, b, b_blocks, st);
}

hipError_t launch_shared_w13(const SkinnyArgs& a, int blocks, hipStream_t st) {
  return launch_pair<kFmtI8, kW13, kFmtI8, kW13>(a, blocks, nullptr, 0, st);
}

// One pass alone (EXACT: K = 128 * NPF * WAVES).
template <int F, int S, int WAVES, int NPF, bool EXACT>
__global__ __launch_bounds__(WAVES * 64) void k_single(SkinnyArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  skinny_block<F, S, WAVES, NPF, EXACT>(a, blockIdx.x, lds);
}

template <int F, int S, int WAVES, int NPF, bool EXACT>
static hipError_t launch_single(const SkinnyArgs& a, int blocks, hipStream_t st) {
  if (blocks <= 0) return hipSuccess;
  const size_t lds = skinny_lds_bytes(a.tile_n, a.K, S, WAVES);
  auto kern = &k_single<F, S, WAVES, NPF, EXACT>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  kern<<<(unsigned)blocks, WAVES * 64, lds, st>>>(a);
  return hipGetLastError();
}

// Routed w13 alone with 4-wave blocks and up to 8 super-steps per wave in
// flight: with K <= 4096 a whole 16-row slice of a slot's expert is requested
// at once and the decode grid (slots x I/16 blocks) is resident in one round.
// K = 512 .. 4096 (powers of two) take the branch-free block.
hipError_t launch_w13_deep(const SkinnyArgs& a, int blocks, hipStream_t st) {
  switch (a.K) {
    case 512: return launch_single<kFmtMx, kW13, 4, 1, true>(a, blocks, st);
    case 1024: return launch_single<kFmtMx, kW13, 4, 2, true>(a, blocks, st);
    case 2048: return launch_single<kFmtMx, kW13, 4, 4, true>(a, blocks, st);
    case 4096: return launch_single<kFmtMx, kW13, 4, 8, true>(a, blocks, st);
    default: return launch_single<kFmtMx, kW13, 4, 8, false>(a, blocks, st);
  }
}

// ---------------------------------------------------------------- combine

// out[t][n] = sum_{j<k} ybuf[t*k+j][n] (+ zbuf[t][n]), slots in order; ybuf
// fp32, or bf16 (y_bf16) as the large-batch GEMMs write it. The slot count
// is a template argument so that a thread requests all of its k slot pieces
// and its shared piece before the first add: with a loop over a run-time k,
// each piece was requested only after the previous one had arrived (seven
// dependent memory round trips per thread at k = 6). The additions keep the
// slot order, then the shared piece, so the sums are unchanged.
template <int KS>
__global__ __launch_bounds__(256) void k_combine(CombineArgs a) {
  const size_t i4 = (size_t)blockIdx.x * 256 + threadIdx.x;  // index of 4 outputs
  const size_t n4 = (size_t)a.T * a.H / 4;
  if (i4 >= n4) return;
  const size_t t = i4 * 4 / a.H, n = i4 * 4 - t * a.H;
  float4 y[KS];
  if (a.y_bf16) {
    uint2 v[KS];
#pragma unroll
    for (int j = 0; j < KS; ++j)
      v[j] = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.ybuf) + (t * KS + j) * a.H + n);
#pragma unroll
    for (int j = 0; j < KS; ++j)
      y[j] = make_float4(bf16_to_f32(v[j].x & 0xffffu), bf16_to_f32(v[j].x >> 16), bf16_to_f32(v[j].y & 0xffffu),
                         bf16_to_f32(v[j].y >> 16));
  } else {
#pragma unroll
    for (int j = 0; j < KS; ++j)
      y[j] = *reinterpret_cast<const float4*>(static_cast<const float*>(a.ybuf) + (t * KS + j) * a.H + n);
  }
  const float4 z = a.zbuf ? *reinterpret_cast<const float4*>(a.zbuf + t * a.H + n) : make_float4(0.f, 0.f, 0.f, 0.f);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int j = 0; j < KS; ++j) {
    acc.x += y[j].x;
    acc.y += y[j].y;
    acc.z += y[j].z;
    acc.w += y[j].w;
  }
  if (a.zbuf) {
    acc.x += z.x;
    acc.y += z.y;
    acc.z += z.z;
    acc.w += z.w;
  }
  if (a.out_is_fp32) {
    *reinterpret_cast<float4*>(static_cast<float*>(a.out) + t * a.H + n) = acc;
  } else {
    uint2 pk;
    pk.x = (uint32_t)f32_to_bf16(acc.x) | ((uint32_t)f32_to_bf16(acc.y) << 16);
    pk.y = (uint32_t)f32_to_bf16(acc.z) | ((uint32_t)f32_to_bf16(acc.w) << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + t * a.H + n) = pk;
  }
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t st) {
  const size_t n4 = (size_t)a.T * a.H / 4;
  if (n4 == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((n4 + 255) / 256);
  switch (a.k) {
    case 1: k_combine<1><<<blocks, 256, 0, st>>>(a); break;
    case 2: k_combine<2><<<blocks, 256, 0, st>>>(a); break;
    case 3: k_combine<3><<<blocks, 256, 0, st>>>(a); break;
    case 4: k_combine<4><<<blocks, 256, 0, st>>>(a); break;
    case 5: k_combine<5><<<blocks, 256, 0, st>>>(a); break;
    case 6: k_combine<6><<<blocks, 256, 0, st>>>(a); break;
    case 7: k_combine<7><<<blocks, 256, 0, st>>>(a); break;
    case 8: k_combine<8><<<blocks, 256, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- zero fill

__global__ __launch_bounds__(256) void k_fill_zero(uint4* p, size_t n16, unsigned char* tail, int ntail) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n16) p[i] = make_uint4(0, 0, 0, 0);
  if (i < (size_t)ntail) tail[i] = 0;
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st) {
  if (bytes == 0) return hipSuccess;
  const size_t n16 = bytes / 16;
  const int ntail = (int)(bytes - n16 * 16);
  const size_t n = n16 > (size_t)ntail ? n16 : (size_t)ntail;
  k_fill_zero<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(
      static_cast<uint4*>(p), n16, static_cast<unsigned char*>(p) + n16 * 16, ntail);
  return hipGetLastError();
}

}  // namespace moe
