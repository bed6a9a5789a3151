// The "skinny" expert GEMM block for gfx950: 16 weight rows against a tile
// of at most 16 activation columns, for MXFP4 routed experts ("w4a16") and
// the int8 per-channel shared expert ("w8a16"): page "deepseek-v4-mxfp4-int8
// config.json", quantization_config.config_groups. The w13 pass applies the
// clamped SwiGLU (page "DeepSeek-V4-Flash-0731", section "Checked in its
// code", row "SwiGLU feed-forward"); the w2 pass scales each routed slot by
// its routing weight.
//
// Mapping (block of WAVES waves):
//   - K is cut into 128-wide super-steps; wave w takes super-steps w,
//     w+WAVES, ... so the waves of a block read WAVES*64 contiguous bytes of
//     each MXFP4 row (WAVES*128 of each int8 row) per round.
//   - Lane (r = l%16, g = l/16) reads, per super-step, 16 bytes of MXFP4 row r
//     (32 codes = exactly one E8M0 group) or 32 bytes of int8 row r, for the
//     K range 128s + 32g .. +32. These are decoded to bf16 in registers (the
//     hardware scaled FP4 convert is exact) and feed four MFMA 16x16x32 bf16.
//     The activation fragments for the same K range come from an LDS copy of
//     the tile's columns (rows padded by 16 bytes). Any fixed permutation of K
//     shared by both operands leaves the dot products unchanged.
//   - All NPF super-steps of a wave are requested before its first MFMA; with
//     NPF * WAVES * 128 >= K a wave's whole weight slice is in flight.
//   - The wave partials are summed in LDS in wave order (deterministic).
#pragma once

#include "device.h"
#include "internal.h"

namespace moe {


// LDS layout of a skinny block: [activation tile: tile_n rows of 2K+16 bytes]
// [E8M0 scales of the block's rows: NACC x 16 rows of K/32+4 bytes]
// [wave partials: WAVES x NACC x 64 lanes x 16 bytes] [top-k: 64 bytes].
__host__ __device__ inline size_t skinny_scale_off(int tile_n, int K) { return (size_t)tile_n * (size_t)(K * 2 + 16); }
__host__ __device__ inline size_t skinny_red_off(int tile_n, int K, int stage) {
  return skinny_scale_off(tile_n, K) + (size_t)(stage == 0 ? 2 : 1) * 16 * (size_t)(K / 32 + 4);
}
inline size_t skinny_lds_bytes(int tile_n, int K, int stage, int waves) {
  return skinny_red_off(tile_n, K, stage) + (size_t)waves * (stage == 0 ? 2 : 1) * 64 * 16 + 64;
}

template <int FMT, int QV, int NPF, int WAVES>
__device__ __forceinline__ void prefetch_rows(const uint8_t* q, int s0, int S, uint4 (&qv)[NPF * QV]) {
#pragma unroll
  for (int i = 0; i < NPF; ++i) {
    const int s = s0 + WAVES * i;
    if (s < S) {
      if (FMT == kFmtMx) {
        qv[i] = *reinterpret_cast<const uint4*>(q + (size_t)s * 64);
      } else {
        qv[2 * i] = *reinterpret_cast<const uint4*>(q + (size_t)s * 128);
        qv[2 * i + 1] = *reinterpret_cast<const uint4*>(q + (size_t)s * 128 + 16);
      }
    }
  }
}

// Weight fragment j (K = 8j .. 8j+7 of this lane's 32) as bf16.
template <int FMT>
__device__ __forceinline__ bf16x8_t weight_frag(const uint4* qv, float scale, int j) {
  if (FMT == kFmtMx) {
    const uint32_t d = j == 0 ? qv[0].x : j == 1 ? qv[0].y : j == 2 ? qv[0].z : qv[0].w;
    return fp4x8_to_bf16x8(d, scale);
  } else {
    const uint4 u = qv[j >> 1];
    return i8x8_to_bf16x8((j & 1) ? u.z : u.x, (j & 1) ? u.w : u.y);
  }
}

// Piece ii (16 bytes) of a block's E8M0 scales: run ii / pieces_per_run (0:
// the 16 rows at rb*16, 1: the 16 rows at half + rb*16), byte offset
// (ii % pieces_per_run) * 16 in that contiguous 16-row run.
__device__ __forceinline__ const uint4* scale_ptr(const uint8_t* se, int ii, int pieces_per_run, int rb, int half) {
  const int run = ii / pieces_per_run, off = (ii - run * pieces_per_run) * 16;
  const int row = run == 0 ? rb * 16 : half + rb * 16;
  return reinterpret_cast<const uint4*>(se + (size_t)row * pieces_per_run + off);
}

// Stores piece ii to LDS rows of `srow` bytes, dword by dword (a piece may span
// two rows when a row has fewer than 16 bytes, i.e. K < 512).
__device__ __forceinline__ void store_scales16(unsigned char* lds_sc, int srow, int pieces_per_run, int ii,
                                               const uint4& v) {
  const int rowlen = pieces_per_run;  // bytes per row = K / 32 = pieces per 16-row run
  const int run = ii / pieces_per_run, off = (ii - run * pieces_per_run) * 16;
  const uint32_t w0 = v.x, w1 = v.y, w2 = v.z, w3 = v.w;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int o = off + 4 * d, rr = o / rowlen, cc = o - rr * rowlen;
    *reinterpret_cast<uint32_t*>(lds_sc + (size_t)(run * 16 + rr) * srow + cc) =
        d == 0 ? w0 : d == 1 ? w1 : d == 2 ? w2 : w3;
  }
}

// Source of activation piece i (16 bytes) of a tile: column i / n16.
__device__ __forceinline__ const uint4* act_ptr(const SkinnyArgs& p, int pos0, int i, int n16, int act_div) {
  const int c = i / n16, o = i - c * n16;
  const size_t row = (p.act_row ? (size_t)p.act_row[pos0 + c] : (size_t)(pos0 + c)) / act_div;
  return reinterpret_cast<const uint4*>(p.act + row * p.act_ld) + o;
}

// EXACT: K = 128 * NPF * WAVES, so every wave takes exactly NPF super-steps,
// all requested at once, and the code has no per-step guards (the compiler's
// load waits then count exactly and the MFMAs consume each super-step as it
// arrives). SLIM (int8 w13 only): the block's 16 MFMA rows are 8 gate rows
// (r < 8) and the matching 8 up rows (r >= 8), so the block reads half as
// many bytes and twice as many blocks spread a pass over the chip.
template <int FMT, int STAGE, int WAVES, int NPF, bool EXACT = false, bool SLIM = false>
__device__ __forceinline__ void skinny_block(const SkinnyArgs& p, int bid, unsigned char* lds) {
  static_assert(!SLIM || (FMT == kFmtI8 && STAGE == kW13), "slim blocks are int8 w13 only");
  constexpr int THREADS = WAVES * 64;
  constexpr int QV = (FMT == kFmtMx) ? 1 : 2;
  constexpr int NACC = (STAGE == kW13 && !SLIM) ? 2 : 1;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, g = lane >> 4;
  const int tg = bid % p.n_tiles_grid;  // tiles fastest: the blocks of one row block
  const int rb = bid / p.n_tiles_grid;  // run close together in time

  const int K = p.K;
  const int S = K >> 7;
  const int row_bytes = K * 2 + 16;
  const int n16 = K >> 3;
  const int srow = K / 32 + 4;  // padded LDS row of scales
  unsigned char* lds_sc = lds + skinny_scale_off(p.tile_n, K);
  unsigned char* lds_red = lds + skinny_red_off(p.tile_n, K, STAGE);

  // 1. the tile: expert, first sorted position, columns
  int e = 0, pos0, ncols, act_div = 1;
  if (p.routed == 2) {
    pos0 = tg;  // one slot per tile: token tg / k, choice tg % k
    ncols = 1;
    act_div = p.topk;
  } else if (p.routed) {
    if (tg >= *p.n_tiles) return;  // uniform over the block, before any barrier
    const int4 ti = p.tile_info[tg];
    e = ti.x;
    pos0 = ti.y;
    ncols = ti.z;
  } else {
    pos0 = tg * p.tile_n;
    ncols = min(p.tile_n, p.T - pos0);
  }

  // 2. activation columns: small tiles (<= 2 uint4 per thread) are loaded into
  //    registers right away, before the top-k and the weights
  const int nact = ncols * n16;
  const bool act_in_regs = nact <= 2 * THREADS;
  uint4 act0 = make_uint4(0, 0, 0, 0), act1 = make_uint4(0, 0, 0, 0);
  if (act_in_regs) {  // indices clamped so that the loads are unconditional; surplus values are unused
    act0 = *act_ptr(p, pos0, min(tid, nact - 1), n16, act_div);
    act1 = *act_ptr(p, pos0, min(tid + THREADS, nact - 1), n16, act_div);
  }

  // 3. slot tiles: the expert is the top-k choice tg % k of token tg / k
  if (p.routed == 2) {
    int32_t* sel = reinterpret_cast<int32_t*>(lds_red + (size_t)WAVES * NACC * 64 * 16);
    float* selw = reinterpret_cast<float*>(sel + kTopKMax);
    const int t = tg / p.topk, j = tg - t * p.topk;
    if (wave == 0)
      wave_topk(p.scores + (size_t)t * p.E, p.keys + (size_t)t * p.E, p.E, p.topk, p.scale, sel, selw, nullptr);
    __syncthreads();
    e = sel[j];
    if (rb == 0 && tid == 0) {
      p.ids_out[tg] = e;
      p.w_out[tg] = selw[j];
    }
  }

  // 4. the block's E8M0 scales (two contiguous 16-row runs, 16-byte pieces),
  //    then its weights: every wave requests its NPF super-steps. The scales
  //    go first so that waiting for them does not wait for the weights.
  const int rowA = SLIM ? (r < 8 ? rb * 8 + r : p.half + rb * 8 + (r - 8)) : rb * 16 + r;
  const int rowB = p.half + rb * 16 + r;
  const uint8_t *qA, *qB = nullptr;
  const uint8_t* se = nullptr;
  if (FMT == kFmtMx) {
    const uint8_t* qe = p.wq + (long long)e * p.q_expert_stride;
    se = p.wsc + (long long)e * p.s_expert_stride;
    qA = qe + (size_t)rowA * (K / 2) + g * 16;
    if (STAGE == kW13) qB = qe + (size_t)rowB * (K / 2) + g * 16;
  } else {
    qA = p.wq + (size_t)rowA * K + g * 32;
    if (STAGE == kW13 && !SLIM) qB = p.wq + (size_t)rowB * K + g * 32;
  }
  const int nsc16 = NACC * K / 32;  // 16-byte pieces of the block's scales (16 rows x K/32 per run)
  const int pieces_per_run = K / 32;
  uint4 sc0 = make_uint4(0, 0, 0, 0), sc1 = make_uint4(0, 0, 0, 0);
  if (FMT == kFmtMx) {
    sc0 = *scale_ptr(se, min(tid, nsc16 - 1), pieces_per_run, rb, p.half);
    sc1 = *scale_ptr(se, min(tid + THREADS, nsc16 - 1), pieces_per_run, rb, p.half);
  }
  uint4 qa[NPF * QV], qb[NPF * QV];
  int s0 = wave;
  if (EXACT) {
#pragma unroll
    for (int i = 0; i < NPF; ++i) {
      const int s = s0 + WAVES * i;
      if (FMT == kFmtMx) {
        qa[i] = *reinterpret_cast<const uint4*>(qA + (size_t)s * 64);
        if (STAGE == kW13) qb[i] = *reinterpret_cast<const uint4*>(qB + (size_t)s * 64);
      } else {
        qa[2 * i] = *reinterpret_cast<const uint4*>(qA + (size_t)s * 128);
        qa[2 * i + 1] = *reinterpret_cast<const uint4*>(qA + (size_t)s * 128 + 16);
        if (STAGE == kW13 && !SLIM) {
          qb[2 * i] = *reinterpret_cast<const uint4*>(qB + (size_t)s * 128);
          qb[2 * i + 1] = *reinterpret_cast<const uint4*>(qB + (size_t)s * 128 + 16);
        }
      }
    }
  } else {
    prefetch_rows<FMT, QV, NPF, WAVES>(qA, s0, S, qa);
    if (STAGE == kW13 && !SLIM) prefetch_rows<FMT, QV, NPF, WAVES>(qB, s0, S, qb);
  }

  // 5. activations and scales -> LDS
  if (act_in_regs) {
    if (tid < nact) *reinterpret_cast<uint4*>(lds + (tid / n16) * row_bytes + (tid % n16) * 16) = act0;
    if (tid + THREADS < nact) {
      const int ii = tid + THREADS;
      *reinterpret_cast<uint4*>(lds + (ii / n16) * row_bytes + (ii % n16) * 16) = act1;
    }
  } else {  // batches of 8 pieces per thread in flight (clamped loads, guarded stores)
    for (int base = 0; base < nact; base += 8 * THREADS) {
      uint4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = *act_ptr(p, pos0, min(base + tid + j * THREADS, nact - 1), n16, act_div);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = base + tid + j * THREADS;
        if (i < nact) *reinterpret_cast<uint4*>(lds + (i / n16) * row_bytes + (i % n16) * 16) = v[j];
      }
    }
  }
  if (FMT == kFmtMx) {
    if (tid < nsc16) store_scales16(lds_sc, srow, pieces_per_run, tid, sc0);
    if (tid + THREADS < nsc16) store_scales16(lds_sc, srow, pieces_per_run, tid + THREADS, sc1);
    for (int ii = tid + 2 * THREADS; ii < nsc16; ii += THREADS)  // only when K > 64 * THREADS
      store_scales16(lds_sc, srow, pieces_per_run, ii, *scale_ptr(se, ii, pieces_per_run, rb, p.half));
  }
  __syncthreads();

  // 6. MFMA over the wave's super-steps
  f32x4_t accA = {0.f, 0.f, 0.f, 0.f}, accB = {0.f, 0.f, 0.f, 0.f};
  const bf16x8_t zero8 = {};
  const unsigned char* bcol = lds + r * row_bytes + g * 64;
  const unsigned char* scA = lds_sc + (size_t)r * srow + g;
  const unsigned char* scB = lds_sc + (size_t)(16 + r) * srow + g;
  while (s0 < S) {
#pragma unroll
    for (int i = 0; i < NPF; ++i) {
      const int s = s0 + WAVES * i;
      if (EXACT || s < S) {
        bf16x8_t bj[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          bj[j] = (r < ncols) ? *reinterpret_cast<const bf16x8_t*>(bcol + s * 256 + j * 16) : zero8;
        const float sA = FMT == kFmtMx ? e8m0_scale_operand(scA[s * 4]) : 1.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) accA = mfma_16x16x32(weight_frag<FMT>(&qa[i * QV], sA, j), bj[j], accA);
        if (STAGE == kW13 && !SLIM) {
          const float sB = FMT == kFmtMx ? e8m0_scale_operand(scB[s * 4]) : 1.0f;
#pragma unroll
          for (int j = 0; j < 4; ++j) accB = mfma_16x16x32(weight_frag<FMT>(&qb[i * QV], sB, j), bj[j], accB);
        }
      }
    }
    if (EXACT) break;
    s0 += WAVES * NPF;
    if (s0 < S) {
      prefetch_rows<FMT, QV, NPF, WAVES>(qA, s0, S, qa);
      if (STAGE == kW13 && !SLIM) prefetch_rows<FMT, QV, NPF, WAVES>(qB, s0, S, qb);
    }
  }

  f32x4_t* red = reinterpret_cast<f32x4_t*>(lds_red);
  red[(wave * NACC) * 64 + lane] = accA;
  if (STAGE == kW13 && !SLIM) red[(wave * NACC + 1) * 64 + lane] = accB;
  __syncthreads();
  if (SLIM) {
    // lanes (r, g < 2) hold gate rows rb*8 + 4g + i of column r; the up rows
    // of the same outputs sit at lane + 32
    if (wave != 0 || r >= ncols || g >= 2) return;
    f32x4_t G = red[lane], U = red[lane + 32];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) {
      G += red[w * 64 + lane];
      U += red[w * 64 + lane + 32];
    }
    const int hc = rb * 8 + 4 * g;
    uint16_t h[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      h[i] = f32_to_bf16(swiglu_clamped(G[i] * p.row_scale[hc + i], U[i] * p.row_scale[p.half + hc + i], p.limit));
    uint2 packed;
    packed.x = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
    packed.y = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
    *reinterpret_cast<uint2*>(p.hout + (size_t)(pos0 + r) * p.hout_ld + hc) = packed;
    return;
  }
  if (wave != 0 || r >= ncols) return;

  auto wsum = [&](int q) {
    const f32x4_t* v = red + q * 64 + lane;
    f32x4_t sum = v[0];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) sum += v[w * NACC * 64];
    return sum;
  };
  const f32x4_t A = wsum(0);
  const int row0 = rb * 16 + 4 * g;  // this lane holds rows row0 .. row0+3 of column r
  if (STAGE == kW13) {
    const f32x4_t B = wsum(NACC - 1);
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

}  // namespace moe
