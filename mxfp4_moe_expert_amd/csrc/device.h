// Device-side helpers shared by the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

namespace moe {

constexpr int kWave = 64;
constexpr int kTopKMax = 8;

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

// 3-bit down-expert blocks: 32 weights along K in 12 code bytes (three
// dwords D0, D1, D2) and a binary16 scale d; weight = d * level[code], with
// 8 levels per table (the uniform book is code - 4). Code bits: byte j of
// dword q (j < 4, q < 3) holds the code of weight 8q + j in bits 0..2 and of
// weight 8q + 4 + j in bits 3..5; weight 24 + j has its bits 0..1 in bits
// 6..7 of D0's byte j and bit 2 in bit 6 of D2's byte j; weight 28 + j the
// same from D1's byte j and bit 7 of D2's byte j. The layout lets a mask
// turn four codes into the byte selectors of one v_perm_b32.
//
// A lane's scaled code book for one block: level[c] * d rounded to bf16
// (nearest even), split into byte planes so that one perm looks up the low
// bytes of four weights and one the high bytes.
struct Q3Book {
  uint32_t lo0, lo1, hi0, hi1;  // lo0: low bytes of entries 0..3, lo1: of 4..7; hi*: high bytes
};

typedef __attribute__((ext_vector_type(2))) float f32x2_t;

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

__device__ __forceinline__ Q3Book q3_book(const float (&lv)[8], float d) {
  const uint32_t p0 = bf16x2_rne(lv[0] * d, lv[1] * d), p1 = bf16x2_rne(lv[2] * d, lv[3] * d);
  const uint32_t p2 = bf16x2_rne(lv[4] * d, lv[5] * d), p3 = bf16x2_rne(lv[6] * d, lv[7] * d);
  Q3Book b;
  b.lo0 = __builtin_amdgcn_perm(p1, p0, 0x06040200u);  // bytes 0, 2 of p0, then of p1
  b.hi0 = __builtin_amdgcn_perm(p1, p0, 0x07050301u);
  b.lo1 = __builtin_amdgcn_perm(p3, p2, 0x06040200u);
  b.hi1 = __builtin_amdgcn_perm(p3, p2, 0x07050301u);
  return b;
}

// Four codes (selector bytes 0..7) -> four bf16 of the book, as two dwords.
__device__ __forceinline__ uint2 q3_look4(const Q3Book& b, uint32_t sel) {
  const uint32_t lo = __builtin_amdgcn_perm(b.lo1, b.lo0, sel);
  const uint32_t hi = __builtin_amdgcn_perm(b.hi1, b.hi0, sel);
  return make_uint2(__builtin_amdgcn_perm(hi, lo, 0x05010400u), __builtin_amdgcn_perm(hi, lo, 0x07030602u));
}

// Weights 8kk .. 8kk+7 of a block as bf16, in order.
__device__ __forceinline__ bf16x8_t q3_frag(uint32_t d0, uint32_t d1, uint32_t d2, int kk, const Q3Book& b) {
  uint32_t sa, sb;
  if (kk == 0) {
    sa = d0 & 0x07070707u;
    sb = (d0 >> 3) & 0x07070707u;
  } else if (kk == 1) {
    sa = d1 & 0x07070707u;
    sb = (d1 >> 3) & 0x07070707u;
  } else if (kk == 2) {
    sa = d2 & 0x07070707u;
    sb = (d2 >> 3) & 0x07070707u;
  } else {
    sa = ((d0 >> 6) & 0x03030303u) | ((d2 >> 4) & 0x04040404u);
    sb = ((d1 >> 6) & 0x03030303u) | ((d2 >> 5) & 0x04040404u);
  }
  const uint2 x = q3_look4(b, sa), y = q3_look4(b, sb);
  const uint4 u = make_uint4(x.x, x.y, y.x, y.y);
  return __builtin_bit_cast(bf16x8_t, u);
}

// The 8 levels of a table (expert e's row of `table`), or the uniform book
// when table is null. e is uniform across the wave.
__device__ __forceinline__ void q3_levels(const float* table, int e, float (&lv)[8]) {
  if (table) {
#pragma unroll
    for (int c = 0; c < 8; ++c) lv[c] = table[(size_t)e * 8 + c];
  } else {
#pragma unroll
    for (int c = 0; c < 8; ++c) lv[c] = (float)(c - 4);
  }
}

// D[16x16] += A[16x32] * B[32x16], bf16 in, fp32 accumulate.
// Lane l holds A[l%16][8*(l/16) .. +8], B[8*(l/16) .. +8][l%16] and
// D[4*(l/16) .. +4][l%16] (checked on gfx950).
__device__ __forceinline__ f32x4_t mfma_16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float softplus(float z) { return fmaxf(z, 0.0f) + log1pf(expf(-fabsf(z))); }

// silu(z) = z / (1 + e^-z) with the hardware base-2 exponential and
// reciprocal (about 1 ulp each; h is rounded to bf16 right after). For very
// negative z, e^-z overflows to +inf and the reciprocal gives 0: silu -> -0.
__device__ __forceinline__ float silu(float z) {
  const float e = __builtin_amdgcn_exp2f(-z * 1.4426950408889634f);
  return z * __builtin_amdgcn_rcpf(1.0f + e);
}

// h = silu(min(g, L)) * clamp(u, -L, L)
__device__ __forceinline__ float swiglu_clamped(float g, float u, float L) {
  float gc = fminf(g, L);
  float uc = fminf(fmaxf(u, -L), L);
  return silu(gc) * uc;
}

// Top-k keys: the fp32 selection value b mapped to an unsigned integer of the
// same order in the high word, the inverted expert id in the low word, so
// that one unsigned 64-bit comparison orders by b and then by the lower id.
// Every valid key is above 0, which marks "no candidate".
__device__ __forceinline__ uint64_t topk_key(float b, int e) {
  const uint32_t u = __float_as_uint(b);
  const uint32_t hi = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)hi << 32) | (uint32_t)~e;
}

// One step of a wave-wide max of 64-bit keys: the key DPP brings in replaces
// the lane's if larger. Lanes the pattern leaves without a source see 0.
template <int CTRL, int ROW_MASK = 0xf, int BANK_MASK = 0xf>
__device__ __forceinline__ uint64_t keymax_dpp_step(uint64_t key) {
  const uint32_t hi = __builtin_amdgcn_update_dpp(0, (int)(key >> 32), CTRL, ROW_MASK, BANK_MASK, false);
  const uint32_t lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)key, CTRL, ROW_MASK, BANK_MASK, false);
  const uint64_t other = ((uint64_t)hi << 32) | lo;
  return other > key ? other : key;
}

// Wave-wide max of 64-bit keys, returned to every lane: quad swaps, row
// rotations by 4 and 8 (each 16-lane row then holds its row maximum), row
// broadcasts 15 and 31 (lane 63 holds the wave maximum), read from lane 63.
__device__ __forceinline__ uint64_t wave_keymax(uint64_t key) {
  key = keymax_dpp_step<0xB1>(key);        // quad_perm [1,0,3,2]
  key = keymax_dpp_step<0x4E>(key);        // quad_perm [2,3,0,1]
  key = keymax_dpp_step<0x124>(key);       // row_ror:4
  key = keymax_dpp_step<0x128>(key);       // row_ror:8
  key = keymax_dpp_step<0x142, 0xA>(key);  // row_bcast:15 -> rows 1, 3
  key = keymax_dpp_step<0x143, 0xC>(key);  // row_bcast:31 -> rows 2, 3
  const uint32_t hi = __builtin_amdgcn_readlane((int)(key >> 32), 63);
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)key, 63);
  return ((uint64_t)hi << 32) | lo;
}

// One wave selects the top-k experts of one token from its E <= 256 scores
// s (fp32 sqrt(softplus(logit))) and selection values b = fp32(s + bias):
// the k largest b, ties to the lower expert id; weights scale * s / sum(s)
// over the chosen, summed in slot order. Lane l owns experts l, l+64, l+128,
// l+192; each of the k rounds is one branch-free DPP wave max of 64-bit keys.
// Lane 0 writes ids/weights for slots j = 0..k-1 and, if ids_lds is given,
// the ids there too.
struct TopkRow {
  float s[4];
  float b[4];
};

// The lane's four (score, selection value) pairs of one token.
// Device-wide coherent (agent-scope) 32-bit load and store: they bypass the
// per-XCD L2 copies, for data handed between blocks of one launch.
__device__ __forceinline__ float load_agent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16 bytes as two coherent 64-bit loads.
__device__ __forceinline__ u32x4_t load_agent_u32x4(const void* p) {
  const uint64_t* q = reinterpret_cast<const uint64_t*>(p);
  const uint64_t lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return (u32x4_t){(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)};
}

// COH: the scores were written by other blocks of the same launch.
template <bool COH = false>
__device__ __forceinline__ TopkRow topk_load(const float* s_row, const float* b_row, int E) {
  const int lane = threadIdx.x & 63;
  TopkRow t;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = min(lane + 64 * q, E - 1);  // loads stay in bounds; surplus lanes get key 0 below
    t.s[q] = COH ? load_agent(s_row + e) : s_row[e];
    t.b[q] = COH ? load_agent(b_row + e) : b_row[e];
  }
  return t;
}

// COH: ids and weights are written through to memory (agent-scope stores),
// for other blocks of the same launch.
template <bool COH = false>
__device__ __forceinline__ void wave_topk_row(const TopkRow& row, int E, int k, float scale, int32_t* ids_out,
                                              float* w_out, int32_t* ids_lds) {
  const int lane = threadIdx.x & 63;
  float s[4];
  uint64_t key[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane + 64 * q;
    s[q] = row.s[q];
    key[q] = e < E ? topk_key(row.b[q], e) : 0;
  }
  float sel_s[kTopKMax];
  int sel_id[kTopKMax];
#pragma unroll
  for (int j = 0; j < kTopKMax; ++j) {
    sel_s[j] = 0.0f;
    sel_id[j] = 0;
    if (j >= k) continue;  // uniform
    uint64_t m = key[0] > key[1] ? key[0] : key[1];
    const uint64_t m2 = key[2] > key[3] ? key[2] : key[3];
    m = m > m2 ? m : m2;
    m = wave_keymax(m);
    const int e = (int)~(uint32_t)m;
    const int owner = e & 63, q_of = e >> 6;
    const float mys = (q_of == 0) ? s[0] : (q_of == 1) ? s[1] : (q_of == 2) ? s[2] : s[3];
    sel_s[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mys), owner));
    sel_id[j] = e;
#pragma unroll
    for (int q = 0; q < 4; ++q) key[q] = (lane == owner && q == q_of) ? 0 : key[q];
  }
  if (lane == 0) {
    float sum = 0.0f;
#pragma unroll
    for (int j = 0; j < kTopKMax; ++j)
      if (j < k) sum += sel_s[j];
#pragma unroll
    for (int j = 0; j < kTopKMax; ++j) {
      if (j >= k) continue;
      const float wj = scale * sel_s[j] / sum;
      if constexpr (COH) {
        store_agent(reinterpret_cast<uint32_t*>(ids_out) + j, (uint32_t)sel_id[j]);
        store_agent(reinterpret_cast<uint32_t*>(w_out) + j, __float_as_uint(wj));
      } else {
        ids_out[j] = sel_id[j];
        w_out[j] = wj;
      }
      if (ids_lds) ids_lds[j] = sel_id[j];
    }
  }
}

// Hash-layer routing of one token by a wave (page "Tidalluna/DeepSeek-V4-
// Flash-0731-Tina-CQ4KM", section "Compatibility", item 2: the first layers
// take their experts from a token-id table): the k experts of the token's
// table row, in table order, weighted by their renormalised scores x scale.
// row.s holds the scores of experts lane + 64 q. trow is the token's table
// row, or null for a token id out of range (the caller flags it): then the
// weights are NaN and the experts 0. A table entry outside [0, E) is taken
// as expert 0, with NaN weights for the token and kFlagTableEntry set. COH:
// ids and weights are written through to memory, as wave_topk_row.
template <bool COH = false>
__device__ __forceinline__ void wave_hash_row(const TopkRow& row, const int32_t* trow, int E, int k, float scale,
                                              int32_t* ids_out, float* w_out, int32_t* ids_lds, uint32_t* flags) {
  const int lane = threadIdx.x & 63;
  float sel_s[kTopKMax];
  int sel_id[kTopKMax];
  bool ok = trow != nullptr, ent_ok = true;
#pragma unroll
  for (int j = 0; j < kTopKMax; ++j) {
    sel_s[j] = 0.0f;
    sel_id[j] = 0;
    if (j >= k) continue;  // uniform
    int e = ok ? __builtin_amdgcn_readfirstlane(trow[j]) : 0;
    if ((unsigned)e >= (unsigned)E) {
      ent_ok = false;
      e = 0;
    }
    const int owner = e & 63, q_of = e >> 6;
    const float mys = (q_of == 0) ? row.s[0] : (q_of == 1) ? row.s[1] : (q_of == 2) ? row.s[2] : row.s[3];
    sel_s[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mys), owner));
    sel_id[j] = e;
  }
  ok = ok && ent_ok;
  if (lane == 0) {
    if (!ent_ok && flags) atomicOr(flags, 2u);  // kFlagTableEntry
    float sum = 0.0f;
#pragma unroll
    for (int j = 0; j < kTopKMax; ++j)
      if (j < k) sum += sel_s[j];
#pragma unroll
    for (int j = 0; j < kTopKMax; ++j) {
      if (j >= k) continue;
      const float wj = ok ? scale * sel_s[j] / sum : __builtin_nanf("");
      if constexpr (COH) {
        store_agent(reinterpret_cast<uint32_t*>(ids_out) + j, (uint32_t)sel_id[j]);
        store_agent(reinterpret_cast<uint32_t*>(w_out) + j, __float_as_uint(wj));
      } else {
        ids_out[j] = sel_id[j];
        w_out[j] = wj;
      }
      if (ids_lds) ids_lds[j] = sel_id[j];
    }
  }
}

template <bool COH = false>
__device__ __forceinline__ void wave_topk(const float* s_row, const float* b_row, int E, int k, float scale,
                                          int32_t* ids_out, float* w_out, int32_t* ids_lds) {
  wave_topk_row<COH>(topk_load(s_row, b_row, E), E, k, scale, ids_out, w_out, ids_lds);
}

// Exclusive scan over the block of one int per thread (blockDim a multiple
// of 64, at most 1024; tmp: at least blockDim/64 ints of LDS). Each wave
// scans its lanes with shuffles, the waves' totals meet in LDS. Returns this
// thread's exclusive prefix; *total gets the sum.
__device__ __forceinline__ int block_exclusive_scan(int v, int* tmp, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  int base = 0, tot = 0;
  for (int w = 0; w < nw; ++w) {
    const int t = tmp[w];
    base += w < wave ? t : 0;
    tot += t;
  }
  *total = tot;
  __syncthreads();  // tmp is free again
  return base + x - v;
}

}  // namespace moe
