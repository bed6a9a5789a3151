// Router kernels for gfx950: learned router (sqrt-softplus scores, bias-
// assisted top-k, renormalised weights) and the token-id hash router.
//
// Method: page "DeepSeek-V4-Flash-0731", section "Checked in its code", rows
// "Mixture of experts" and "Auxiliary-loss-free load balancing (selection
// bias)": the bias is added to the scores for the top-k choice only and the
// combine weights are gathered from the unbiased scores. Scores are
// sqrt(softplus(logit)) and the weights are renormalised and scaled by 1.5
// (page "deepseek-v4-mxfp4-int8 config.json": scoring_func sqrtsoftplus,
// norm_topk_prob, routed_scaling_factor). Hash layers take the experts from
// a token-id table (page "Tidalluna/DeepSeek-V4-Flash-0731-Tina-CQ4KM",
// section "Compatibility").
//
// Logits are fp32 sums of bf16 x times fp32 Wg. The selection compares the
// fp32 values s + bias; equal values go to the lower expert id.
#include "device.h"
#include "internal.h"

namespace moe {

// ---------------------------------------------------------------- top-k

// One wave selects the top-k experts of one token from its E <= 256 logits.
// Lane l owns experts l, l+64, l+128, l+192. Writes ids/weights for slots
// j = 0..k-1 (by biased score descending, ties to the lower id); if ids_lds is
// given, lane 0 also stores the ids there.
__device__ void wave_topk(const float* logits_row, const float* bias, int E, int k, float scale,
                          int32_t* ids_out, float* w_out, int32_t* ids_lds) {
  const int lane = threadIdx.x & 63;
  float s[4], b[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    int e = lane + 64 * q;
    if (e < E) {
      float l = load_acquire_f32(logits_row + e);
      s[q] = sqrtf(softplus(l));
      b[q] = s[q] + bias[e];
    } else {
      s[q] = 0.0f;
      b[q] = -INFINITY;
    }
  }
  unsigned taken = 0;
  float sel_s[8];
  int sel_id[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    sel_s[j] = 0.0f;
    sel_id[j] = 0;
    if (j >= k) continue;
    // lane-local best among the not-yet-taken entries (lower id first on ties)
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int e = lane + 64 * q;
      bool ok = e < E && !(taken & (1u << q));
      if (ok && (b[q] > bv || (b[q] == bv && e < bi))) {
        bv = b[q];
        bi = e;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      float ov = __shfl_xor(bv, o);
      int oi = __shfl_xor(bi, o);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    // every lane now holds the winner bi; its owner marks it taken
    const int owner = bi & 63, q_of = bi >> 6;
    float mys = (q_of == 0) ? s[0] : (q_of == 1) ? s[1] : (q_of == 2) ? s[2] : s[3];
    float ws = __shfl(mys, owner);
    if (lane == owner) taken |= 1u << q_of;
    sel_s[j] = ws;
    sel_id[j] = bi;
  }
  if (lane == 0) {
    float sum = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < k) sum += sel_s[j];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j >= k) continue;
      ids_out[j] = sel_id[j];
      w_out[j] = scale * sel_s[j] / sum;
      if (ids_lds) ids_lds[j] = sel_id[j];
    }
  }
}

// ---------------------------------------------------------------- block helpers

// Stable counting sort of n <= kSmallSlots slots held in LDS (ids_lds) by one
// block of 256 threads; writes offsets[E+1], sorted_slots, slot_pos and the
// tile prefix tile_off[E+1] (tiles of tile_n slots per expert).
__device__ void block_small_permute(const int32_t* ids_lds, int n, int E, int tile_n,
                                    int32_t* offsets, int32_t* sorted_slots, int32_t* slot_pos,
                                    int32_t* tile_off, int* cnt_lds, int* scan_tmp) {
  const int tid = threadIdx.x;
  if (tid < 256) cnt_lds[tid] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += 256) atomicAdd(&cnt_lds[ids_lds[i]], 1);
  __syncthreads();
  int c = tid < E ? cnt_lds[tid] : 0;
  int total;
  int off = block_exclusive_scan_256(c, scan_tmp, &total);
  int nt = (c + tile_n - 1) / tile_n;
  int ttotal;
  int toff = block_exclusive_scan_256(nt, scan_tmp, &ttotal);
  if (tid < E) {
    offsets[tid] = off;
    tile_off[tid] = toff;
    cnt_lds[tid] = off;  // reuse as the expert's first position
  }
  if (tid == 0) {
    offsets[E] = total;
    tile_off[E] = ttotal;
  }
  __syncthreads();
  for (int i = tid; i < n; i += 256) {
    int e = ids_lds[i];
    int rank = 0;
    for (int j = 0; j < i; ++j) rank += (ids_lds[j] == e);
    int pos = cnt_lds[e] + rank;
    sorted_slots[pos] = i;
    slot_pos[i] = pos;
  }
}

// ---------------------------------------------------------------- small-T router

// Grid: E blocks of 256 threads, block e computes logit[t][e] for all T <=
// kSmallT tokens (thread i covers k = 8i + 2048 j). The last block to finish
// then selects the top-k of every token and, if perm != 0, builds the
// permutation and tile list.
__global__ __launch_bounds__(256) void k_router_small(RouterArgs a) {
  __shared__ float red[4][kSmallT];
  __shared__ int32_t ids_lds[kSmallT * 8];
  __shared__ int cnt_lds[256];
  __shared__ int scan_tmp[256];
  __shared__ int flag;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int e = blockIdx.x;
  const int H = a.H;
  const float* we = a.gate_w + (size_t)e * H;
  for (int t0 = 0; t0 < a.T; t0 += 8) {
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
    for (int k0 = tid * 8; k0 < H; k0 += 2048) {
      float4 w0 = *reinterpret_cast<const float4*>(we + k0);
      float4 w1 = *reinterpret_cast<const float4*>(we + k0 + 4);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (t0 + q < a.T) {
          uint4 xv = *reinterpret_cast<const uint4*>(a.x + (size_t)(t0 + q) * H + k0);
          float sacc = acc[q];
          sacc += bf16_to_f32(xv.x & 0xffff) * w0.x;
          sacc += bf16_to_f32(xv.x >> 16) * w0.y;
          sacc += bf16_to_f32(xv.y & 0xffff) * w0.z;
          sacc += bf16_to_f32(xv.y >> 16) * w0.w;
          sacc += bf16_to_f32(xv.z & 0xffff) * w1.x;
          sacc += bf16_to_f32(xv.z >> 16) * w1.y;
          sacc += bf16_to_f32(xv.w & 0xffff) * w1.z;
          sacc += bf16_to_f32(xv.w >> 16) * w1.w;
          acc[q] = sacc;
        }
      }
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      float v = wave_sum(acc[q]);
      if (lane == 0 && t0 + q < a.T) red[wave][t0 + q] = v;
    }
  }
  __syncthreads();
  const float off = a.logit_offset ? a.logit_offset[e] : 0.0f;
  for (int t = tid; t < a.T; t += 256)
    a.logits[(size_t)t * a.E + e] = ((red[0][t] + red[1][t]) + (red[2][t] + red[3][t])) + off;

  if (!last_block_arrives(a.counter, gridDim.x, &flag)) return;

  for (int t = wave; t < a.T; t += 4)
    wave_topk(a.logits + (size_t)t * a.E, a.bias, a.E, a.k, a.scale, a.ids + (size_t)t * a.k,
              a.w + (size_t)t * a.k, ids_lds + t * a.k);
  if (!a.perm) return;
  __syncthreads();
  block_small_permute(ids_lds, a.T * a.k, a.E, a.tile_n, a.offsets, a.sorted_slots, a.slot_pos,
                      a.tile_off, cnt_lds, scan_tmp);
}

// ---------------------------------------------------------------- large-T router

// logits[T][E] = x[T][H] * Wg[E][H]^T (+ offset): 64x64 output tile per block,
// 256 threads with 4x4 outputs each, K staged through LDS 32 at a time.
__global__ __launch_bounds__(256) void k_router_tiled(RouterArgs a) {
  constexpr int BT = 64, BE = 64, BK = 32;
  __shared__ float xs[BK][BT + 4];
  __shared__ float gs[BK][BE + 4];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * BT, e0 = blockIdx.y * BE;
  const int ty = tid / 16, tx = tid % 16;
  float acc[4][4] = {};
  const int lr = tid / 4, lk = (tid % 4) * 8;  // loader: row lr, k offset lk
  for (int k0 = 0; k0 < a.H; k0 += BK) {
    {
      int t = t0 + lr;
      uint4 xv = make_uint4(0, 0, 0, 0);
      if (t < a.T) xv = *reinterpret_cast<const uint4*>(a.x + (size_t)t * a.H + k0 + lk);
      xs[lk + 0][lr] = bf16_to_f32(xv.x & 0xffff);
      xs[lk + 1][lr] = bf16_to_f32(xv.x >> 16);
      xs[lk + 2][lr] = bf16_to_f32(xv.y & 0xffff);
      xs[lk + 3][lr] = bf16_to_f32(xv.y >> 16);
      xs[lk + 4][lr] = bf16_to_f32(xv.z & 0xffff);
      xs[lk + 5][lr] = bf16_to_f32(xv.z >> 16);
      xs[lk + 6][lr] = bf16_to_f32(xv.w & 0xffff);
      xs[lk + 7][lr] = bf16_to_f32(xv.w >> 16);
      int e = e0 + lr;
      float4 g0 = make_float4(0, 0, 0, 0), g1 = make_float4(0, 0, 0, 0);
      if (e < a.E) {
        g0 = *reinterpret_cast<const float4*>(a.gate_w + (size_t)e * a.H + k0 + lk);
        g1 = *reinterpret_cast<const float4*>(a.gate_w + (size_t)e * a.H + k0 + lk + 4);
      }
      gs[lk + 0][lr] = g0.x;
      gs[lk + 1][lr] = g0.y;
      gs[lk + 2][lr] = g0.z;
      gs[lk + 3][lr] = g0.w;
      gs[lk + 4][lr] = g1.x;
      gs[lk + 5][lr] = g1.y;
      gs[lk + 6][lr] = g1.z;
      gs[lk + 7][lr] = g1.w;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < BK; ++kk) {
      float xa[4], gb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xa[i] = xs[kk][ty * 4 + i];
        gb[i] = gs[kk][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += xa[i] * gb[j];
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int t = t0 + ty * 4 + i;
    if (t >= a.T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int e = e0 + tx * 4 + j;
      if (e < a.E) a.logits[(size_t)t * a.E + e] = acc[i][j] + (a.logit_offset ? a.logit_offset[e] : 0.0f);
    }
  }
}

// One wave per token: top-k of the logits written by k_router_tiled.
__global__ __launch_bounds__(256) void k_topk(RouterArgs a) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  wave_topk(a.logits + (size_t)t * a.E, a.bias, a.E, a.k, a.scale, a.ids + (size_t)t * a.k,
            a.w + (size_t)t * a.k, nullptr);
}

// ---------------------------------------------------------------- hash router

// One wave per token: ids from the table row, scores of those experts only.
__global__ __launch_bounds__(256) void k_hash_route(HashArgs a) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= a.T) return;
  const int32_t* row = a.tid2eid + (size_t)a.token_ids[t] * a.k;
  const uint16_t* xt = a.x + (size_t)t * a.H;
  float s[8];
  float sum = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    s[j] = 0.0f;
    if (j >= a.k) continue;
    const float* we = a.gate_w + (size_t)row[j] * a.H;
    float acc = 0.0f;
    for (int k0 = lane * 8; k0 < a.H; k0 += 512) {
      uint4 xv = *reinterpret_cast<const uint4*>(xt + k0);
      float4 w0 = *reinterpret_cast<const float4*>(we + k0);
      float4 w1 = *reinterpret_cast<const float4*>(we + k0 + 4);
      acc += bf16_to_f32(xv.x & 0xffff) * w0.x;
      acc += bf16_to_f32(xv.x >> 16) * w0.y;
      acc += bf16_to_f32(xv.y & 0xffff) * w0.z;
      acc += bf16_to_f32(xv.y >> 16) * w0.w;
      acc += bf16_to_f32(xv.z & 0xffff) * w1.x;
      acc += bf16_to_f32(xv.z >> 16) * w1.y;
      acc += bf16_to_f32(xv.w & 0xffff) * w1.z;
      acc += bf16_to_f32(xv.w >> 16) * w1.w;
    }
    s[j] = sqrtf(softplus(wave_sum(acc)));
    sum += s[j];
  }
  if (lane < a.k) {
    float sj = s[0];
#pragma unroll
    for (int j = 1; j < 8; ++j)
      if (j == lane) sj = s[j];
    a.ids[(size_t)t * a.k + lane] = row[lane];
    a.w[(size_t)t * a.k + lane] = a.scale * sj / sum;
  }
}

// ---------------------------------------------------------------- launchers

hipError_t launch_router(const RouterArgs& a, hipStream_t st) {
  if (a.T <= 0) return hipSuccess;
  if (a.T <= kSmallT) {
    k_router_small<<<a.E, 256, 0, st>>>(a);
    return hipGetLastError();
  }
  dim3 g((a.T + 63) / 64, (a.E + 63) / 64);
  k_router_tiled<<<g, 256, 0, st>>>(a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  k_topk<<<(a.T + 3) / 4, 256, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_hash_route(const HashArgs& a, hipStream_t st) {
  if (a.T <= 0) return hipSuccess;
  k_hash_route<<<(a.T + 3) / 4, 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace moe
