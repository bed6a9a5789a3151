// Device-side helpers shared by the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

namespace moe {

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16 bits, round to nearest even (Inf/NaN kept).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// E8M0 byte -> an fp32 whose exponent field is that byte. The gfx950 scaled
// FP4 conversion uses only the exponent of its scale operand, so this encodes
// 2^(b-127) for every byte 0..254 (byte 0 included).
__device__ __forceinline__ float e8m0_scale_operand(uint32_t b) { return __uint_as_float(b << 23); }

// Eight E2M1 codes (one dword, element 2i in the low nibble of byte i) times
// 2^(scale) -> eight bf16 in element order. Exact: an E2M1 value times a
// power of two has at most two significant bits.
__device__ __forceinline__ bf16x8_t fp4x8_to_bf16x8(uint32_t codes, float scale) {
  bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0);
  bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1);
  bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2);
  bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3);
  return (bf16x8_t){p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Eight int8 (two dwords, little-endian) -> eight bf16. Exact: |q| <= 128 has
// at most eight significant bits, so dropping the low half of the fp32 is exact.
__device__ __forceinline__ uint32_t i8pair_to_bf16x2(uint32_t d, int sh) {
  float f0 = (float)(int8_t)(d >> sh);
  float f1 = (float)(int8_t)(d >> (sh + 8));
  return (__float_as_uint(f0) >> 16) | (__float_as_uint(f1) & 0xffff0000u);
}

__device__ __forceinline__ bf16x8_t i8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  uint4 u;
  u.x = i8pair_to_bf16x2(lo, 0);
  u.y = i8pair_to_bf16x2(lo, 16);
  u.z = i8pair_to_bf16x2(hi, 0);
  u.w = i8pair_to_bf16x2(hi, 16);
  return __builtin_bit_cast(bf16x8_t, u);
}

// D[16x16] += A[16x32] * B[32x16], bf16 in, fp32 accumulate.
// Lane l holds A[l%16][8*(l/16) .. +8], B[8*(l/16) .. +8][l%16] and
// D[4*(l/16) .. +4][l%16] (checked on gfx950).
__device__ __forceinline__ f32x4_t mfma_16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float softplus(float z) { return fmaxf(z, 0.0f) + log1pf(expf(-fabsf(z))); }

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// h = silu(min(g, L)) * clamp(u, -L, L)
__device__ __forceinline__ float swiglu_clamped(float g, float u, float L) {
  float gc = fminf(g, L);
  float uc = fminf(fmaxf(u, -L), L);
  return silu(gc) * uc;
}

// Coherent (L1-bypassing) load of a value another block wrote in this launch.
__device__ __forceinline__ float load_acquire_f32(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Returns true in exactly one block of a grid of `nblocks`: the last to get
// here. Each block's global writes made before the call are visible to that
// block after it returns true. The counter wraps back to 0 after the last
// arrival (atomicInc with limit nblocks-1), so it is ready for the next launch.
// Every thread of the block must call it.
__device__ __forceinline__ bool last_block_arrives(unsigned* counter, unsigned nblocks, int* flag_lds) {
  __threadfence();  // release this thread's writes at agent scope
  __syncthreads();
  if (threadIdx.x == 0) *flag_lds = (atomicInc(counter, nblocks - 1) == nblocks - 1) ? 1 : 0;
  __syncthreads();
  bool last = *flag_lds != 0;
  if (last) __threadfence();  // acquire: see every other block's writes
  return last;
}

// Exclusive scan of n <= 256 ints held one per thread (threads >= n hold 0).
// Returns the exclusive prefix for this thread; *total gets the sum.
__device__ __forceinline__ int block_exclusive_scan_256(int v, int* tmp, int* total) {
  const int tid = threadIdx.x;
  tmp[tid] = v;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    int add = tid >= o ? tmp[tid - o] : 0;
    __syncthreads();
    tmp[tid] += add;
    __syncthreads();
  }
  int incl = tmp[tid];
  *total = tmp[255];
  __syncthreads();
  return incl - v;
}

}  // namespace moe
