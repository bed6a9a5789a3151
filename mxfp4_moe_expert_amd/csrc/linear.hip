// The model's int8 per-channel linear layers ("w8a16": page
// "deepseek-v4-mxfp4-int8 config.json", quantization_config, config group
// linears_w8a16) at decode sizes (T <= 64): y = x W^T, W[n][k] = s[n] q[n][k],
// plain or grouped (block-diagonal, as wo_a with o_groups).
//
// A projection has few output rows for the chip at decode sizes (the
// compressor's 256, fused_wqa_wkv's 1536), so K is split too: block (rb, s)
// owns 64 weight rows (4 waves x 16) and the K slice [s ks, (s+1) ks).
//   - Each lane requests all of its weights for the slice at once (16 bytes
//     of its row per 64-K step, at most 16 steps), then the block stages the
//     slice of every token's activations in LDS (rows padded by 16 bytes).
//   - Per 64-K step a wave converts its two int8 fragments to bf16 once (exact)
//     and runs two MFMA 16x16x32 per 16-token column tile.
//   - One slice (split = 1): the epilogue scales by the row's fp32 scale and
//     writes the output. Otherwise each block writes its fp32 partial sums
//     with coherent stores, waits for them and counts itself in its row
//     block's arrival word; the last block of the row block (which resets
//     the word for the next call) reads the split partials with coherent
//     loads, adds them in slice order (deterministic), scales and writes.
#include "device.h"
#include "internal.h"

namespace moe {

constexpr int kLinThreads = 256;  // 4 waves x 16 weight rows
constexpr int kLinRows = 64;
constexpr int kLinMaxSteps = 16;  // 64-K steps per block: ks <= 1024
constexpr size_t kLinMaxLds = 140 * 1024;

template <int CT>
__global__ __launch_bounds__(kLinThreads) void k_linear_dec(LinearDecArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];  // [T][2 ks + 16] bf16 activations
  __shared__ int is_last;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r = lane & 15, g = lane >> 4;
  const int rb = blockIdx.x, s = blockIdx.y;
  const int GN = a.G * a.N;
  const int grp = (rb * kLinRows) / a.N;  // N % 64 == 0: a row block lies in one group
  const int k0 = s * a.ks;
  const int nst = a.ks >> 6;
  const int row0 = rb * kLinRows + wave * 16;

  // 1. the wave's weights for the whole slice
  const int8_t* wrow = a.q + (size_t)(row0 + r) * a.K + k0 + g * 16;
  uint4 w[kLinMaxSteps];
#pragma unroll
  for (int i = 0; i < kLinMaxSteps; ++i)
    if (i < nst) w[i] = *reinterpret_cast<const uint4*>(wrow + i * 64);
  asm volatile("" ::: "memory");

  // 2. the slice of every token's activations
  const int rowb = 2 * a.ks + 16;
  const int n16 = a.ks >> 3;
  const size_t ldx = (size_t)a.G * a.K;
  for (int i = tid; i < a.T * n16; i += kLinThreads) {
    const int t = i / n16, o = i - t * n16;
    *reinterpret_cast<uint4*>(lds + (size_t)t * rowb + o * 16) =
        *reinterpret_cast<const uint4*>(a.x + t * ldx + (size_t)grp * a.K + k0 + o * 8);
  }
  __syncthreads();

  // 3. MFMAs: lane (r, g) holds K-values 16g .. 16g+15 of each 64-K step of
  //    row r; column tile c takes tokens 16c .. 16c+15 (past T: the last
  //    token again, never stored)
  f32x4_t acc[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) acc[c] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  const unsigned char* bcol[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) bcol[c] = lds + (size_t)min(16 * c + r, a.T - 1) * rowb + g * 32;
#pragma unroll
  for (int i = 0; i < kLinMaxSteps; ++i) {
    if (i < nst) {
      const bf16x8_t wa = i8x8_to_bf16x8(w[i].x, w[i].y), wb = i8x8_to_bf16x8(w[i].z, w[i].w);
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        acc[c] = mfma_16x16x32(wa, *reinterpret_cast<const bf16x8_t*>(bcol[c] + i * 128), acc[c]);
        acc[c] = mfma_16x16x32(wb, *reinterpret_cast<const bf16x8_t*>(bcol[c] + i * 128 + 16), acc[c]);
      }
    }
  }

  // 4. lane (j = r, g) holds D[rows 4g .. 4g+3][token 16c + j]
  const int n = row0 + 4 * g;
  if (a.split == 1) {
    const float4 sc = *reinterpret_cast<const float4*>(a.scale + n);
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      const int t = 16 * c + r;
      if (t >= a.T) continue;
      const float4 o = make_float4(acc[c][0] * sc.x, acc[c][1] * sc.y, acc[c][2] * sc.z, acc[c][3] * sc.w);
      if (a.out_is_fp32) {
        *reinterpret_cast<float4*>(static_cast<float*>(a.out) + (size_t)t * GN + n) = o;
      } else {
        uint2 pk;
        pk.x = (uint32_t)f32_to_bf16(o.x) | ((uint32_t)f32_to_bf16(o.y) << 16);
        pk.y = (uint32_t)f32_to_bf16(o.z) | ((uint32_t)f32_to_bf16(o.w) << 16);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + (size_t)t * GN + n) = pk;
      }
    }
    return;
  }
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    const int t = 16 * c + r;
    if (t >= a.T) continue;
    uint64_t* d = reinterpret_cast<uint64_t*>(a.part + ((size_t)s * a.T + t) * GN + n);
    __hip_atomic_store(d, (uint64_t)__float_as_uint(acc[c][0]) | ((uint64_t)__float_as_uint(acc[c][1]) << 32),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(d + 1, (uint64_t)__float_as_uint(acc[c][2]) | ((uint64_t)__float_as_uint(acc[c][3]) << 32),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt((15 << 8) | (7 << 4));  // vmcnt(0): this wave's partials are written
  __syncthreads();
  if (tid == 0) is_last = atomicAdd(a.count + rb, 1) == a.split - 1;
  __syncthreads();
  if (!is_last) return;
  // thread: 4 consecutive rows of one token; the slices' partials are
  // requested 8 at a time (coherent 16-byte loads), then added in slice order
  for (int i = tid; i < a.T * (kLinRows / 4); i += kLinThreads) {
    const int t = i / (kLinRows / 4), nn = rb * kLinRows + 4 * (i - t * (kLinRows / 4));
    f32x4_t v = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < a.split; s0 += 8) {
      u32x4_t pv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        pv[j] = load_agent_u32x4(a.part + ((size_t)min(s0 + j, a.split - 1) * a.T + t) * GN + nn);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (s0 + j < a.split) v += __builtin_bit_cast(f32x4_t, pv[j]);
    }
    const float4 sc = *reinterpret_cast<const float4*>(a.scale + nn);
    const float4 o = make_float4(v[0] * sc.x, v[1] * sc.y, v[2] * sc.z, v[3] * sc.w);
    if (a.out_is_fp32) {
      *reinterpret_cast<float4*>(static_cast<float*>(a.out) + (size_t)t * GN + nn) = o;
    } else {
      uint2 pk;
      pk.x = (uint32_t)f32_to_bf16(o.x) | ((uint32_t)f32_to_bf16(o.y) << 16);
      pk.y = (uint32_t)f32_to_bf16(o.z) | ((uint32_t)f32_to_bf16(o.w) << 16);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + (size_t)t * GN + nn) = pk;
    }
  }
  if (tid == 0) a.count[rb] = 0;  // ready for the next call
}

// K per block: a multiple of 128 that divides K, at most 1024, whose
// activations fit the LDS budget. Up to 16 tokens: the largest slice that
// still gives at least one block per CU (256), else the smallest. Above 16
// tokens the partial sums (4 split T bytes per weight row, against K bytes
// of weights) and the activations each block stages (2 T bytes per K-value)
// grow with T: the smallest slice whose partials stay within a quarter of
// the weight bytes, else the largest.
int linear_dec_ks(int T, int K, int N, int G) {
  if (T <= 0 || T > kSmallT || K % 128 || N % kLinRows) return 0;
  const long long rbs = (long long)G * N / kLinRows;
  const int m = K / 128;
  int best = 0;
  for (int c = 1; c <= m && 128 * c <= 1024; ++c) {
    if (m % c) continue;
    const int ks = 128 * c;
    if ((size_t)T * (2 * ks + 16) > kLinMaxLds) continue;
    const long long split = K / ks;
    if (T <= 16) {
      if (best == 0 || rbs * split >= 256) best = ks;
    } else {
      const bool cheap = 16LL * split * T <= K;
      if (cheap) return ks;
      best = ks;
    }
  }
  return best;
}

hipError_t launch_linear_dec(const LinearDecArgs& a, hipStream_t st) {
  if (a.T <= 0) return hipSuccess;
  if (a.ks != linear_dec_ks(a.T, a.K, a.N, a.G) || a.ks <= 0 || a.split != a.K / a.ks || !a.x || !a.q ||
      !a.scale || !a.out || (a.split > 1 && (!a.part || !a.count)))
    return hipErrorInvalidValue;
  const size_t lds = (size_t)a.T * (2 * a.ks + 16);
  const dim3 grid((unsigned)((long long)a.G * a.N / kLinRows), (unsigned)a.split);
  auto go = [&](auto kern) -> hipError_t {
    if (lds > 64 * 1024) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    kern<<<grid, kLinThreads, lds, st>>>(a);
    return hipGetLastError();
  };
  if (a.T <= 16) return go(&k_linear_dec<1>);
  if (a.T <= 32) return go(&k_linear_dec<2>);
  return go(&k_linear_dec<4>);
}

}  // namespace moe
