// Routed w2 + shared-expert w2 + weighted combine for the smallest batches
// (T*(k+1) <= 16, e.g. single-token decode) on gfx950: one block per 16
// output rows.
//
// The combine of the MoE block (page "DeepSeek-V4-Flash-0731", section
// "Checked in its code", row "Shared expert": the routed output plus the
// shared expert's) is output-stationary here: block b owns output rows
// [16b, 16b+16) of every token. MFMA columns are the activation vectors:
// column j < T*k is slot j's bf16 h (token j / k, choice j % k), column
// T*k + t is token t's shared-expert h. A routed unit (slot j, super-step s)
// multiplies the 16 MXFP4 w2 rows of slot j's expert with column j only (the
// other columns of its B fragment are zero); a shared unit (super-step s)
// multiplies the 16 int8 rows of the shared w2 with all T shared columns at
// once. One 16x16 accumulator per wave thus collects every y. K = I is cut
// into 128-wide super-steps; units are dealt to the waves round-robin and up
// to MAXU routed units per wave are requested up front. The wave partials
// are summed in LDS in wave order, then
//   out[t][n] = sum_j w[t,j] * y_{t,j}[n] (j = 0..k-1 in order) + s2[n] * zraw_t[n].
#pragma once

#include "device.h"
#include "internal.h"

namespace moe {

__host__ __device__ inline size_t w2c_lds_bytes(int T, int k, int I, int waves, bool ext_shared) {
  const int ncols = T * k + (ext_shared ? 0 : T);
  return (size_t)ncols * (I * 2 + 16) + (size_t)T * k * 16 * (I / 32 + 4) + (size_t)waves * 64 * 16 + 256 * 4 +
         16 * 4 + 16 * 4 + 16;
}

template <int WAVES, int MAXU, int MAXS, int MAXA>
__device__ __forceinline__ void w2_combine_block(const W2CombineArgs& a, int rb, unsigned char* lds) {
  constexpr int THREADS = WAVES * 64;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, g = lane >> 4;
  const int I = a.I, H = a.H;
  const int nslots = a.T * a.k, ncols = nslots + a.T;
  const int S = I >> 7;
  const int nunits = nslots * S;
  const int row_bytes = I * 2 + 16;
  const int srow = I / 32 + 4;                                                 // padded scale row
  unsigned char* lds_sc = lds + (size_t)ncols * row_bytes;                      // [nslots][16][srow]
  f32x4_t* red = reinterpret_cast<f32x4_t*>(lds_sc + (size_t)nslots * 16 * srow);  // [WAVES][64]
  float* ycol = reinterpret_cast<float*>(red + WAVES * 64);                     // [16 rows][16 columns]
  int32_t* sid = reinterpret_cast<int32_t*>(ycol + 256);                         // [16] expert of each slot

  // Loads are issued in the order they are needed, since a wait for one load
  // also waits for every load issued before it. (Indices past the end are
  // clamped, not skipped: the loads stay unconditional, so the compiler's
  // waits count them exactly; what a clamped load returns is never used.)
  const int n16 = I >> 3;
  const int nact = ncols * n16;
  auto act_src = [&](int i) {
    const int c = i / n16, o = i - c * n16;
    const uint16_t* src = c < nslots ? a.hbuf + (size_t)c * I : a.hs + (size_t)(c - nslots) * I;
    return reinterpret_cast<const u32x4_t*>(src) + o;
  };
  auto act_dst = [&](int i) {
    const int c = i / n16, o = i - c * n16;
    return reinterpret_cast<u32x4_t*>(lds + c * row_bytes + o * 16);
  };
  const int row = rb * 16 + r;

  // 1. the slots' experts; the shared w2 rows and the activation columns,
  //    which do not depend on them
  const int my_id = *(a.ids + min(tid, nslots - 1));
  u32x4_t av[MAXA];
#pragma unroll
  for (int i = 0; i < MAXA; ++i) av[i] = *act_src(min(tid + i * THREADS, nact - 1));
  uint4 qs[2 * MAXS];
  const uint8_t* shrow = reinterpret_cast<const uint8_t*>(a.sh_w2) + (size_t)row * I + g * 32;
#pragma unroll
  for (int i = 0; i < MAXS; ++i) {
    const int s = min(wave + WAVES * i, S - 1);
    qs[2 * i] = *reinterpret_cast<const uint4*>(shrow + s * 128);
    qs[2 * i + 1] = *reinterpret_cast<const uint4*>(shrow + s * 128 + 16);
  }
  if (tid < nslots) sid[tid] = my_id;
  __syncthreads();

  // 2. the E8M0 scales of every slot's 16 rows (a contiguous run of 16 * I/32
  //    bytes per slot) in 16-byte pieces, then every routed unit's weights
  const long long qstride = (long long)H * (I / 2), sstride = (long long)H * (I / 32);
  const int ppr = I / 32;  // 16-byte pieces per run = scale bytes per row
  const int npieces = nslots * ppr;
  auto sc_src = [&](int ii) {
    const int j = ii / ppr, off = (ii - j * ppr) * 16;
    return reinterpret_cast<const uint4*>(a.w2s + sid[j] * sstride + (size_t)(rb * 16) * ppr + off);
  };
  const uint4 sc0 = *sc_src(min(tid, npieces - 1));
  const uint4 sc1 = *sc_src(min(tid + THREADS, npieces - 1));
  auto q_load = [&](int u) {
    const int j = u / S, s = u - j * S;
    return *reinterpret_cast<const uint4*>(a.w2c + sid[j] * qstride + (size_t)row * (I / 2) + s * 64 + g * 16);
  };
  uint4 q[MAXU];
#pragma unroll
  for (int i = 0; i < MAXU; ++i) q[i] = q_load(min(wave + WAVES * i, nunits - 1));

  // 3. activation columns -> LDS: slots' h, then the tokens' shared h
#pragma unroll
  for (int i = 0; i < MAXA; ++i) {
    const int ii = tid + i * THREADS;
    if (ii < nact) *act_dst(ii) = av[i];
  }
  for (int ii = tid + MAXA * THREADS; ii < nact; ii += THREADS) *act_dst(ii) = *act_src(ii);
  auto sc_store = [&](int ii, const uint4& v) {
    const int j = ii / ppr, off = (ii - j * ppr) * 16;
    const uint32_t w0 = v.x, w1 = v.y, w2 = v.z, w3 = v.w;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int o = off + 4 * d, rr = o / ppr, cc = o - rr * ppr;
      *reinterpret_cast<uint32_t*>(lds_sc + (size_t)(j * 16 + rr) * srow + cc) = d == 0 ? w0 : d == 1 ? w1 : d == 2 ? w2 : w3;
    }
  };
  if (tid < npieces) sc_store(tid, sc0);
  if (tid + THREADS < npieces) sc_store(tid + THREADS, sc1);
  for (int ii = tid + 2 * THREADS; ii < npieces; ii += THREADS) sc_store(ii, *sc_src(ii));
  __syncthreads();

  // 4. MFMA over the wave's units: shared first (requested first), then routed
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  const bf16x8_t zero8 = {};
  auto shared_unit = [&](const uint4& lo, const uint4& hi, int s) {
    const bool mine = r >= nslots && r < ncols;
    const unsigned char* bsrc = lds + (mine ? r : 0) * row_bytes + s * 256 + g * 64;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const uint4 u = (jj >> 1) ? hi : lo;
      const bf16x8_t w = i8x8_to_bf16x8((jj & 1) ? u.z : u.x, (jj & 1) ? u.w : u.y);
      const bf16x8_t b = mine ? *reinterpret_cast<const bf16x8_t*>(bsrc + jj * 16) : zero8;
      acc = mfma_16x16x32(w, b, acc);
    }
  };
#pragma unroll
  for (int i = 0; i < MAXS; ++i) {
    const int s = wave + WAVES * i;
    if (s < S) shared_unit(qs[2 * i], qs[2 * i + 1], s);
  }
  for (int s = wave + WAVES * MAXS; s < S; s += WAVES) {
    shared_unit(*reinterpret_cast<const uint4*>(shrow + s * 128), *reinterpret_cast<const uint4*>(shrow + s * 128 + 16),
                s);
  }
  auto routed_unit = [&](const uint4& qq, int u) {
    const int j = u / S, s = u - j * S;
    const float scale = e8m0_scale_operand(lds_sc[(size_t)(j * 16 + r) * srow + s * 4 + g]);
    const unsigned char* bsrc = lds + j * row_bytes + s * 256 + g * 64;
    const uint32_t d[4] = {qq.x, qq.y, qq.z, qq.w};
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const bf16x8_t b = (r == j) ? *reinterpret_cast<const bf16x8_t*>(bsrc + jj * 16) : zero8;
      acc = mfma_16x16x32(fp4x8_to_bf16x8(d[jj], scale), b, acc);
    }
  };
  // units beyond the first MAXU: each register is reloaded (clamped, so
  // unconditionally) with the unit MAXU further on as soon as it is consumed
  for (int u0 = wave; u0 < nunits; u0 += WAVES * MAXU) {
#pragma unroll
    for (int i = 0; i < MAXU; ++i) {
      const int u = u0 + WAVES * i;
      if (u < nunits) routed_unit(q[i], u);
      q[i] = q_load(min(u + WAVES * MAXU, nunits - 1));
    }
  }

  // 5. wave partials summed in wave order, then the combine
  red[wave * 64 + lane] = acc;
  __syncthreads();
  if (wave == 0) {
    const f32x4_t* v = red + lane;
    f32x4_t y = v[0];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) y += v[w * 64];
    // lane (r, g) holds column r, rows 4g .. 4g+3
#pragma unroll
    for (int i = 0; i < 4; ++i) ycol[(4 * g + i) * 16 + r] = y[i];
  }
  __syncthreads();
  if (tid < a.T * 16) {  // thread (t, rr): output row rb*16 + rr of token t
    const int t = tid >> 4, rr = tid & 15;
    const int n = rb * 16 + rr;
    float o = 0.0f;
    for (int j = 0; j < a.k; ++j) o += a.w[t * a.k + j] * ycol[rr * 16 + t * a.k + j];
    o += a.sh_w2_scale[n] * ycol[rr * 16 + nslots + t];
    if (a.out_is_fp32) static_cast<float*>(a.out)[(size_t)t * H + n] = o;
    else static_cast<uint16_t*>(a.out)[(size_t)t * H + n] = f32_to_bf16(o);
  }
}

}  // namespace moe
