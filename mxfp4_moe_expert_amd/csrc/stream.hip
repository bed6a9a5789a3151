// Streaming expert pass for batched decode (2 < T <= 64) on gfx950: each
// wave owns its weight rows over the whole of K, so a block needs no
// cross-wave reduction, and every wave keeps D stages of its rows in flight
// through a branch-free register pipeline. MXFP4 routed experts ("w4a16")
// and the int8 per-channel shared expert ("w8a16"): page
// "deepseek-v4-mxfp4-int8 config.json", quantization_config. The w13 pass
// applies the clamped SwiGLU (page "DeepSeek-V4-Flash-0731", section
// "Checked in its code", row "SwiGLU feed-forward"); the routed w2 pass
// scales each slot by its routing weight, the shared w2 pass by the output
// channel's int8 scale.
//
// Block (4 waves) = one tile of at most 16 activation columns (an expert's
// sorted positions, or consecutive tokens for the shared expert) x one row
// group: w13 = 64 h columns (wave w: gate rows and up rows of columns
// 16w .. 16w+15), w2 = 128 output rows (wave w: rows 32w .. 32w+31).
//   - K runs in stages of 128. Lane (r = l%16, g = l/16) reads, per stage and
//     row block, the K range 128 st + 32g .. +32 of row r: 16 bytes of E2M1
//     pairs (exactly one E8M0 group, whose byte the block staged in LDS with
//     all its rows' scales) or 32 int8 bytes. Converted to bf16 in registers,
//     they feed four MFMA 16x16x32 bf16 per row block; the activation
//     fragments for the same K range come from the tile's columns in LDS.
//     Any permutation of K shared by both operands leaves the sums unchanged.
//   - Loads for stage st + D are issued right after stage st is consumed;
//     the last D stages are a second copy of the loop body without loads, so
//     neither loop has branches (the compiler's waits count exactly) and no
//     load is spent on a stage past the end.
//   - The first D stages of weights are requested as soon as the tile's
//     expert is known; the activation columns' round trips (row ids, then
//     rows) overlap them.
#include "device.h"
#include "internal.h"
#include "skinny.h"

namespace moe {

constexpr int kStreamThreads = 256;

template <int FMT>
struct StreamStage {
  uint4 q[FMT == kFmtMx ? 1 : 2];
};

template <int FMT>
__device__ __forceinline__ void stream_load(const uint8_t* q, int st, StreamStage<FMT>& d) {
  if constexpr (FMT == kFmtMx) {
    d.q[0] = *reinterpret_cast<const uint4*>(q + (size_t)st * 64);
  } else {
    d.q[0] = *reinterpret_cast<const uint4*>(q + (size_t)st * 128);
    d.q[1] = *reinterpret_cast<const uint4*>(q + (size_t)st * 128 + 16);
  }
}

// scale: the E8M0 byte of the lane's group (MXFP4), unused for int8
template <int FMT>
__device__ __forceinline__ bf16x8_t stream_frag(const StreamStage<FMT>& d, int kk, uint32_t scale) {
  if constexpr (FMT == kFmtMx) {
    const uint32_t w = kk == 0 ? d.q[0].x : kk == 1 ? d.q[0].y : kk == 2 ? d.q[0].z : d.q[0].w;
    return fp4x8_to_bf16x8(w, e8m0_scale_operand(scale));
  } else {
    const uint4 u = d.q[kk >> 1];
    return i8x8_to_bf16x8((kk & 1) ? u.z : u.x, (kk & 1) ? u.w : u.y);
  }
}

// Pieces base + tid + 256 j (j < 4, clamped to the last) of a tile's
// activation columns (16 bytes each; column = piece / n16): the row of every
// piece first, then every piece, so that no load waits for another. The
// empty asm keeps the loads where they are issued (ahead of the weights).
__device__ __forceinline__ void stream_act_batch(const SkinnyArgs& p, int pos0, int base, int nact, int n16,
                                                 u32x4_t (&av)[4]) {
  const int tid = threadIdx.x;
  int src[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = min(base + tid + j * kStreamThreads, nact - 1);
    const int c = i / n16;
    src[j] = p.act_row ? p.act_row[pos0 + c] : pos0 + c;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = min(base + tid + j * kStreamThreads, nact - 1);
    const int c = i / n16, o = i - c * n16;
    av[j] = *reinterpret_cast<const u32x4_t*>(p.act + (size_t)src[j] * p.act_ld + o * 8);
  }
  asm volatile("" ::: "memory");
}

template <int FMT, int MODE, int D>
__device__ __forceinline__ void stream_block(const SkinnyArgs& p, int bid, unsigned char* lds) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, g = lane >> 4;
  const int tg = bid % p.n_tiles_grid;  // tiles fastest: neighbouring blocks stream different experts
  const int rg = bid / p.n_tiles_grid;

  int e = 0, pos0, ncols;
  if (p.routed) {
    if (tg >= *p.n_tiles) return;  // uniform over the block, before any barrier
    const int4 ti = p.tile_info[tg];
    e = ti.x;
    pos0 = ti.y;
    ncols = ti.z;
  } else {
    pos0 = tg * p.tile_n;
    ncols = min(p.tile_n, p.T - pos0);
  }
  const int K = p.K, S = K >> 7, n16 = K >> 3, row_bytes = 2 * K + 16;

  // 2. the wave's two row blocks and the first D stages of their weights
  //    (they depend only on the tile's expert)
  int rowA, rowB;
  if (MODE == kW13) {
    rowA = rg * 64 + wave * 16 + r;
    rowB = p.half + rowA;
  } else {
    rowA = rg * 128 + wave * 32 + r;
    rowB = rowA + 16;
  }
  const uint8_t *qA, *qB, *se = nullptr;
  if (FMT == kFmtMx) {
    const uint8_t* qe = p.wq + (long long)e * p.q_expert_stride;
    se = p.wsc + (long long)e * p.s_expert_stride;
    qA = qe + (size_t)rowA * (K / 2) + g * 16;
    qB = qe + (size_t)rowB * (K / 2) + g * 16;
  } else {
    qA = p.wq + (size_t)rowA * K + g * 32;
    qB = p.wq + (size_t)rowB * K + g * 32;
  }
  StreamStage<FMT> wA[D], wB[D];
#pragma unroll
  for (int i = 0; i < D; ++i) {
    const int st = min(i, S - 1);
    stream_load<FMT>(qA, st, wA[i]);
    stream_load<FMT>(qB, st, wB[i]);
  }

  // 2b. the E8M0 scales of the block's 128 rows (MXFP4: two runs of 64 rows
  //    for w13, gate and up; one run of 128 for w2), 16 bytes per thread and
  //    step, then the activation columns' first batch (up to 4 pieces per
  //    thread: the source rows of all pieces, then the pieces); all of these
  //    round trips overlap the first weight stages already in flight
  const int srow = K / 32;  // scale bytes per row (a multiple of 4)
  unsigned char* lds_sc = lds + (size_t)p.tile_n * row_bytes;  // [128 rows][srow]
  const bool sc16 = srow % 16 == 0;                            // rows of whole 16-byte pieces
  const int nsc = FMT == kFmtMx ? 128 * srow / (sc16 ? 16 : 4) : 0;
  auto sc_off = [&](int i, int piece) {  // global byte offset of piece i
    const int row = (i * piece) / srow;  // block row 0..127
    const int grow = MODE == kW13 ? (row < 64 ? rg * 64 + row : p.half + rg * 64 + (row - 64)) : rg * 128 + row;
    return (size_t)grow * srow + (i * piece - row * srow);
  };
  u32x4_t sv[4];
  if (FMT == kFmtMx && sc16) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      sv[j] = *reinterpret_cast<const u32x4_t*>(se + sc_off(min(tid + j * kStreamThreads, nsc - 1), 16));
  }
  const int nact = ncols * n16;
  u32x4_t av[4];
  stream_act_batch(p, pos0, 0, nact, n16, av);

  // 3. scales and activation columns -> LDS (activation rows padded by 16
  //    bytes), remaining batches
  if (FMT == kFmtMx && sc16) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = tid + j * kStreamThreads;
      if (i < nsc) *reinterpret_cast<u32x4_t*>(lds_sc + i * 16) = sv[j];
    }
    for (int i = tid + 4 * kStreamThreads; i < nsc; i += kStreamThreads)
      *reinterpret_cast<u32x4_t*>(lds_sc + i * 16) = *reinterpret_cast<const u32x4_t*>(se + sc_off(i, 16));
  } else if (FMT == kFmtMx) {  // rows of K/32 bytes not a multiple of 16: dword pieces
    for (int i = tid; i < nsc; i += kStreamThreads)
      *reinterpret_cast<uint32_t*>(lds_sc + i * 4) = *reinterpret_cast<const uint32_t*>(se + sc_off(i, 4));
  }
  auto act_dst = [&](int i) { return reinterpret_cast<u32x4_t*>(lds + (i / n16) * row_bytes + (i % n16) * 16); };
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = tid + j * kStreamThreads;
    if (i < nact) *act_dst(i) = av[j];
  }
  for (int base = 4 * kStreamThreads; base < nact; base += 4 * kStreamThreads) {
    stream_act_batch(p, pos0, base, nact, n16, av);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = base + tid + j * kStreamThreads;
      if (i < nact) *act_dst(i) = av[j];
    }
  }
  __syncthreads();

  // 4. the K loop
  f32x4_t accA = {0.f, 0.f, 0.f, 0.f}, accB = {0.f, 0.f, 0.f, 0.f};
  const bf16x8_t zero8 = {};
  const bool live = r < ncols;
  const unsigned char* bcol = lds + (live ? r : 0) * row_bytes + g * 64;
  // this lane's scale bytes: block rows of its two row blocks, group 4 st + g
  const int brA = MODE == kW13 ? wave * 16 + r : wave * 32 + r;
  const int brB = MODE == kW13 ? 64 + wave * 16 + r : wave * 32 + 16 + r;
  const unsigned char* scA = lds_sc + (size_t)brA * srow + g;
  const unsigned char* scB = lds_sc + (size_t)brB * srow + g;
  auto stage = [&](int i, int st) __attribute__((always_inline)) {
    bf16x8_t b[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      b[kk] = live ? *reinterpret_cast<const bf16x8_t*>(bcol + st * 256 + kk * 16) : zero8;
    const uint32_t scaleA = FMT == kFmtMx ? scA[st * 4] : 0u;
    const uint32_t scaleB = FMT == kFmtMx ? scB[st * 4] : 0u;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      accA = mfma_16x16x32(stream_frag<FMT>(wA[i], kk, scaleA), b[kk], accA);
      accB = mfma_16x16x32(stream_frag<FMT>(wB[i], kk, scaleB), b[kk], accB);
    }
  };
  int st0 = 0;
  for (; st0 + D < S; st0 += D) {  // S is a multiple of D
#pragma unroll
    for (int i = 0; i < D; ++i) {
      stage(i, st0 + i);
      stream_load<FMT>(qA, st0 + i + D, wA[i]);
      stream_load<FMT>(qB, st0 + i + D, wB[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < D; ++i) stage(i, st0 + i);  // the last D stages: nothing left to request
  if (!live) return;

  // 5. epilogue: lane (r, g) holds rows 4g .. 4g+3 of each row block, column r
  if (MODE == kW13) {
    const int hc = rg * 64 + wave * 16 + 4 * g;
    uint16_t h[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float gv = accA[i], uv = accB[i];
      if (FMT == kFmtI8) {
        gv *= p.row_scale[hc + i];
        uv *= p.row_scale[p.half + hc + i];
      }
      h[i] = f32_to_bf16(swiglu_clamped(gv, uv, p.limit));
    }
    uint2 packed;
    packed.x = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
    packed.y = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
    *reinterpret_cast<uint2*>(p.hout + (size_t)(pos0 + r) * p.hout_ld + hc) = packed;
  } else {
    const int n0 = rg * 128 + wave * 32 + 4 * g;
    float* dst;
    float4 ya, yb;
    if (FMT == kFmtMx) {
      const int slot = p.sorted_slots[pos0 + r];
      const float wv = p.slot_w[slot];
      ya = make_float4(accA[0] * wv, accA[1] * wv, accA[2] * wv, accA[3] * wv);
      yb = make_float4(accB[0] * wv, accB[1] * wv, accB[2] * wv, accB[3] * wv);
      dst = p.yout + (size_t)slot * p.yout_ld;
    } else {
      const float* rs = p.row_scale;
      ya = make_float4(accA[0] * rs[n0], accA[1] * rs[n0 + 1], accA[2] * rs[n0 + 2], accA[3] * rs[n0 + 3]);
      yb = make_float4(accB[0] * rs[n0 + 16], accB[1] * rs[n0 + 17], accB[2] * rs[n0 + 18], accB[3] * rs[n0 + 19]);
      dst = p.yout + (size_t)(pos0 + r) * p.yout_ld;
    }
    *reinterpret_cast<float4*>(dst + n0) = ya;
    *reinterpret_cast<float4*>(dst + n0 + 16) = yb;
  }
}

// Pass b (int8 shared, blocks [0, b_blocks)) and pass a (MXFP4 routed) of
// the same stage in one grid; the shared blocks go first so that they do not
// form the tail.
template <int MODE, int DA, int DB>
__global__ __launch_bounds__(kStreamThreads) void k_stream(SkinnyArgs a, int b_blocks, SkinnyArgs b) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int bid = blockIdx.x;
  if (bid < b_blocks) {
    stream_block<kFmtI8, MODE, DB>(b, bid, lds);
  } else {
    stream_block<kFmtMx, MODE, DA>(a, bid - b_blocks, lds);
  }
}

template <int MODE, int DA, int DB>
static hipError_t launch_stream_t(const SkinnyArgs& a, int a_blocks, const SkinnyArgs& b, int b_blocks,
                                  hipStream_t st) {
  const long long nblk = (long long)a_blocks + b_blocks;
  if (nblk <= 0) return hipSuccess;
  if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
  size_t lds = 0;
  if (a_blocks > 0) lds = (size_t)a.tile_n * (2 * (size_t)a.K + 16) + 128 * (size_t)(a.K / 32);
  if (b_blocks > 0) {
    const size_t lb = (size_t)b.tile_n * (2 * (size_t)b.K + 16);
    lds = lb > lds ? lb : lds;
  }
  auto kern = &k_stream<MODE, DA, DB>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  kern<<<(unsigned)nblk, kStreamThreads, lds, st>>>(a, b_blocks, b);
  return hipGetLastError();
}

// Row groups: w13 I/64 (64 h columns each), w2 H/128 (128 rows each); the
// caller sets n_rowblocks to that count. Stage depth D: 8 (MXFP4) and 4
// (int8) when the stage count is a multiple of 8, else the largest that
// divides it of 4 and 1.
hipError_t launch_stream(int mode, const SkinnyArgs& a, int a_blocks, const SkinnyArgs* b, int b_blocks,
                         hipStream_t st) {
  SkinnyArgs bb{};
  if (b) bb = *b; else b_blocks = 0;
  const int K = a_blocks > 0 ? a.K : bb.K;
  if (K % 128 || (a_blocks > 0 && b_blocks > 0 && a.K != bb.K)) return hipErrorInvalidValue;
  const int S = K / 128;
  if (mode == kW13) {
    if (S % 8 == 0) return launch_stream_t<kW13, 8, 4>(a, a_blocks, bb, b_blocks, st);
    if (S % 4 == 0) return launch_stream_t<kW13, 4, 4>(a, a_blocks, bb, b_blocks, st);
    return launch_stream_t<kW13, 1, 1>(a, a_blocks, bb, b_blocks, st);
  }
  if (S % 8 == 0) return launch_stream_t<kW2, 8, 4>(a, a_blocks, bb, b_blocks, st);
  if (S % 4 == 0) return launch_stream_t<kW2, 4, 4>(a, a_blocks, bb, b_blocks, st);
  return launch_stream_t<kW2, 1, 1>(a, a_blocks, bb, b_blocks, st);
}

}  // namespace moe
