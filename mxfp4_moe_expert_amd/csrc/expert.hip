// Expert feed-forward kernels for gfx950: MXFP4 routed experts ("w4a16") and
// the int8 per-channel shared expert ("w8a16"), page "deepseek-v4-mxfp4-int8
// config.json", quantization_config.config_groups; clamped SwiGLU, page
// "DeepSeek-V4-Flash-0731", section "Checked in its code", row "SwiGLU
// feed-forward"; weighted combine plus the shared expert, same section, row
// "Shared expert".
//
// k_skinny: one block = 16 weight rows (for w13: 16 gate rows and the 16
// matching up rows, so the SwiGLU is local) x one tile of <= 16 activation
// columns (tokens). K is split over the 4 waves, interleaved by 128-wide
// super-steps, so the 4 waves of a block read 256 contiguous bytes of each
// MXFP4 row per round. Lane (r = l%16, g = l/16) streams 16 bytes (32 codes,
// exactly one E8M0 group) of row r per super-step, converts them to bf16 with
// the hardware scaled FP4 conversion (exact) and feeds 4 MFMA 16x16x32 bf16;
// the matching activation fragments come from an LDS copy of the tile's
// columns. Weights of up to NPF super-steps are in flight per wave before the
// first MFMA. The 4 wave partials are summed in LDS in a fixed order.
#include "device.h"
#include "internal.h"

namespace moe {

enum { kFmtMx = 0, kFmtI8 = 1 };
enum { kW13 = 0, kW2 = 1 };

template <int FMT, int QV, int NPF>
__device__ __forceinline__ void prefetch_rows(const uint8_t* q, const uint8_t* sc, int s0, int S,
                                              uint4 (&qv)[NPF * QV], uint32_t (&sv)[NPF]) {
#pragma unroll
  for (int i = 0; i < NPF; ++i) {
    const int s = s0 + 4 * i;
    if (s < S) {
      if (FMT == kFmtMx) {
        qv[i] = *reinterpret_cast<const uint4*>(q + (size_t)s * 64);
        sv[i] = sc[(size_t)s * 4];
      } else {
        qv[2 * i] = *reinterpret_cast<const uint4*>(q + (size_t)s * 128);
        qv[2 * i + 1] = *reinterpret_cast<const uint4*>(q + (size_t)s * 128 + 16);
      }
    }
  }
}

// Weight fragment j (k = 8j .. 8j+7 of this lane's 32) as bf16.
template <int FMT, int QV>
__device__ __forceinline__ bf16x8_t weight_frag(const uint4* qv, float scale, int j) {
  if (FMT == kFmtMx) {
    const uint32_t d = j == 0 ? qv[0].x : j == 1 ? qv[0].y : j == 2 ? qv[0].z : qv[0].w;
    return fp4x8_to_bf16x8(d, scale);
  } else {
    const uint4 u = qv[j >> 1];
    const uint32_t lo = (j & 1) ? u.z : u.x;
    const uint32_t hi = (j & 1) ? u.w : u.y;
    return i8x8_to_bf16x8(lo, hi);
  }
}

template <int FMT, int STAGE, int NPF>
__global__ __launch_bounds__(256) void k_skinny(SkinnyArgs p) {
  constexpr int QV = (FMT == kFmtMx) ? 1 : 2;
  constexpr int NACC = (STAGE == kW13) ? 2 : 1;
  extern __shared__ __align__(16) unsigned char lds_act[];
  __shared__ f32x4_t red[4][NACC][64];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, g = lane >> 4;
  const int tg = blockIdx.x % p.n_tiles_grid;  // tiles fastest: the blocks of one row
  const int rb = blockIdx.x / p.n_tiles_grid;  // block run close together in time

  int e = 0, pos0, ncols;
  if (p.routed) {
    const int ntiles = p.tile_off[p.E];
    if (tg >= ntiles) return;  // uniform over the block, before any barrier
    int lo = 0, hi = p.E - 1;  // largest e with tile_off[e] <= tg
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.tile_off[mid] <= tg) lo = mid; else hi = mid - 1;
    }
    e = lo;
    pos0 = p.offsets[e] + (tg - p.tile_off[e]) * p.tile_n;
    ncols = min(p.tile_n, p.offsets[e + 1] - pos0);
  } else {
    pos0 = tg * p.tile_n;
    ncols = min(p.tile_n, p.T - pos0);
  }

  const int K = p.K;
  const int S = K >> 7;
  const int rowA = rb * 16 + r;
  const int rowB = p.half + rb * 16 + r;
  const uint8_t *qA, *qB = nullptr, *sA = nullptr, *sB = nullptr;
  if (FMT == kFmtMx) {
    const uint8_t* qe = p.wq + (long long)e * p.q_expert_stride;
    const uint8_t* se = p.wsc + (long long)e * p.s_expert_stride;
    qA = qe + (size_t)rowA * (K / 2) + g * 16;
    sA = se + (size_t)rowA * (K / 32) + g;
    if (STAGE == kW13) {
      qB = qe + (size_t)rowB * (K / 2) + g * 16;
      sB = se + (size_t)rowB * (K / 32) + g;
    }
  } else {
    qA = p.wq + (size_t)rowA * K + g * 32;
    if (STAGE == kW13) qB = p.wq + (size_t)rowB * K + g * 32;
  }

  uint4 qa[NPF * QV], qb[NPF * QV];
  uint32_t sa[NPF], sb[NPF];
#pragma unroll
  for (int i = 0; i < NPF; ++i) sa[i] = sb[i] = 0;
  int s0 = wave;
  prefetch_rows<FMT, QV, NPF>(qA, sA, s0, S, qa, sa);
  if (STAGE == kW13) prefetch_rows<FMT, QV, NPF>(qB, sB, s0, S, qb, sb);

  // the tile's activation columns -> LDS, rows padded by 16 bytes
  const int row_bytes = K * 2 + 16;
  const int n16 = K >> 3;
  for (int i = tid; i < ncols * n16; i += 256) {
    const int c = i / n16, o = i - c * n16;
    size_t row;
    if (p.act_is_x) row = (size_t)(p.sorted_slots[pos0 + c] / p.topk);
    else row = (size_t)(pos0 + c);
    const uint4 v = reinterpret_cast<const uint4*>(p.act + row * p.act_ld)[o];
    *reinterpret_cast<uint4*>(lds_act + c * row_bytes + o * 16) = v;
  }
  __syncthreads();

  f32x4_t accA = {0.f, 0.f, 0.f, 0.f}, accB = {0.f, 0.f, 0.f, 0.f};
  const bf16x8_t zero8 = {};
  const unsigned char* bcol = lds_act + r * row_bytes + g * 64;
  while (s0 < S) {
#pragma unroll
    for (int i = 0; i < NPF; ++i) {
      const int s = s0 + 4 * i;
      if (s < S) {
        bf16x8_t bj[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          bj[j] = (r < ncols) ? *reinterpret_cast<const bf16x8_t*>(bcol + s * 256 + j * 16) : zero8;
        const float scA = e8m0_scale_operand(sa[i]);
#pragma unroll
        for (int j = 0; j < 4; ++j) accA = mfma_16x16x32(weight_frag<FMT, QV>(&qa[i * QV], scA, j), bj[j], accA);
        if (STAGE == kW13) {
          const float scB = e8m0_scale_operand(sb[i]);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            accB = mfma_16x16x32(weight_frag<FMT, QV>(&qb[i * QV], scB, j), bj[j], accB);
        }
      }
    }
    s0 += 4 * NPF;
    if (s0 < S) {
      prefetch_rows<FMT, QV, NPF>(qA, sA, s0, S, qa, sa);
      if (STAGE == kW13) prefetch_rows<FMT, QV, NPF>(qB, sB, s0, S, qb, sb);
    }
  }

  red[wave][0][lane] = accA;
  if (STAGE == kW13) red[wave][NACC - 1][lane] = accB;
  __syncthreads();
  if (wave != 0 || r >= ncols) return;

  const f32x4_t A = (red[0][0][lane] + red[1][0][lane]) + (red[2][0][lane] + red[3][0][lane]);
  const int row0 = rb * 16 + 4 * g;  // this lane holds rows row0 .. row0+3 of column r
  if (STAGE == kW13) {
    const f32x4_t B = (red[0][NACC - 1][lane] + red[1][NACC - 1][lane]) +
                      (red[2][NACC - 1][lane] + red[3][NACC - 1][lane]);
    uint16_t h[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float gv = A[i], uv = B[i];
      if (FMT == kFmtI8) {
        gv *= p.row_scale[row0 + i];
        uv *= p.row_scale[p.half + row0 + i];
      }
      h[i] = f32_to_bf16(swiglu_clamped(gv, uv, p.limit));
    }
    uint2 packed;
    packed.x = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
    packed.y = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
    *reinterpret_cast<uint2*>(p.hout + (size_t)(pos0 + r) * p.hout_ld + row0) = packed;
  } else {
    float4 y;
    size_t orow;
    if (FMT == kFmtMx) {
      const int slot = p.sorted_slots[pos0 + r];
      const float wv = p.slot_w[slot];
      y = make_float4(A[0] * wv, A[1] * wv, A[2] * wv, A[3] * wv);
      orow = (size_t)slot;
    } else {
      y = make_float4(A[0] * p.row_scale[row0], A[1] * p.row_scale[row0 + 1], A[2] * p.row_scale[row0 + 2],
                      A[3] * p.row_scale[row0 + 3]);
      orow = (size_t)(pos0 + r);
    }
    *reinterpret_cast<float4*>(p.yout + orow * p.yout_ld + row0) = y;
  }
}

template <int FMT, int STAGE, int NPF>
static hipError_t launch_skinny(const SkinnyArgs& a, int max_tiles, hipStream_t st) {
  if (max_tiles <= 0 || a.n_rowblocks <= 0) return hipSuccess;
  const size_t lds = (size_t)a.tile_n * (size_t)(a.K * 2 + 16);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_skinny<FMT, STAGE, NPF>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, 144 * 1024);
    if (err != hipSuccess) return err;
    attr_set = true;
  }
  const long long nblk = (long long)max_tiles * a.n_rowblocks;
  if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
  k_skinny<FMT, STAGE, NPF><<<(unsigned)nblk, 256, lds, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_skinny_w13_mxfp4(const SkinnyArgs& a, int max_tiles, hipStream_t st) {
  return launch_skinny<kFmtMx, kW13, 8>(a, max_tiles, st);
}
hipError_t launch_skinny_w2_mxfp4(const SkinnyArgs& a, int max_tiles, hipStream_t st) {
  return launch_skinny<kFmtMx, kW2, 8>(a, max_tiles, st);
}
hipError_t launch_skinny_w13_int8(const SkinnyArgs& a, int max_tiles, hipStream_t st) {
  return launch_skinny<kFmtI8, kW13, 4>(a, max_tiles, st);
}
hipError_t launch_skinny_w2_int8(const SkinnyArgs& a, int max_tiles, hipStream_t st) {
  return launch_skinny<kFmtI8, kW2, 8>(a, max_tiles, st);
}

// ---------------------------------------------------------------- combine

// out[t][n] = sum_{j<k} ybuf[t*k+j][n] (+ zbuf[t][n]), slots in order.
__global__ __launch_bounds__(256) void k_combine(CombineArgs a) {
  const size_t i4 = (size_t)blockIdx.x * 256 + threadIdx.x;  // index of 4 outputs
  const size_t n4 = (size_t)a.T * a.H / 4;
  if (i4 >= n4) return;
  const size_t t = i4 * 4 / a.H, n = i4 * 4 - t * a.H;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < a.k; ++j) {
    const float4 y = *reinterpret_cast<const float4*>(a.ybuf + (t * a.k + j) * a.H + n);
    acc.x += y.x;
    acc.y += y.y;
    acc.z += y.z;
    acc.w += y.w;
  }
  if (a.zbuf) {
    const float4 z = *reinterpret_cast<const float4*>(a.zbuf + t * a.H + n);
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
  k_combine<<<(unsigned)((n4 + 255) / 256), 256, 0, st>>>(a);
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
