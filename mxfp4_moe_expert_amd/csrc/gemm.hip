// Grouped expert GEMM for large token counts on gfx950 (prefill): MXFP4
// routed experts ("w4a16") and the int8 per-channel shared expert ("w8a16"),
// page "deepseek-v4-mxfp4-int8 config.json", quantization_config; clamped
// SwiGLU epilogue on w13 (page "DeepSeek-V4-Flash-0731", section "Checked in
// its code", row "SwiGLU feed-forward"); the shared expert's w2 epilogue adds
// the k weighted routed outputs of the token in slot order (row "Shared
// expert": routed + shared).
//
// Tile: 256 weight rows x 128 token positions, one block of 8 waves.
// Wave w owns 32 weight rows (2 blocks of 16) x all 128 positions (8 blocks
// of 16): 16 MFMA 16x16x32 accumulators, so each weight fragment converted
// to bf16 feeds 8 MFMAs (on gfx950 VALU work and MFMAs share a SIMD's issue
// time, so converts per MFMA matter). For w13 the wave's 2 row blocks are 16
// gate rows and the matching 16 up rows, so the SwiGLU is computed in
// registers.
//   - K runs in stages of 128 (MXFP4) or 64 (int8): each lane reads, per
//     stage and row block, 16 bytes of its row (the quarter g of the stage's
//     K-values) straight into registers, two stages ahead. For MXFP4 these 32
//     values are exactly one group, so one E8M0 byte per row block and stage;
//     MXFP4 is converted to bf16 with the exact scaled FP4 convert. The E8M0
//     bytes of the block's 256 rows are copied to LDS once, at the start
//     (rows padded to K/32 + 4 bytes: 16 consecutive rows hit 16 banks): a
//     one-byte global load per lane and stage costs as much of the memory
//     pipeline as a 16-byte one.
//   - tokens: the 128 gathered activation rows of a stage go global ->
//     registers -> LDS, double-buffered, one stage ahead. LDS holds them
//     fragment-major: for each (16-token block m, k-step kk) the 64 lanes'
//     16-byte B fragments lie contiguously in lane order, so every MFMA
//     operand read, and every store of a wave, is one contiguous 1 KB
//     (padded token rows leave 16-byte reads with bank conflicts on gfx950).
//   - MFMA k-step kk of a stage takes the lane's K-values 8kk .. +8 of its
//     quarter on both operands (a fixed permutation of K, so the dot products
//     are unchanged).
//   - persistent: one block per CU walks tiles. Each XCD (block % 8) owns a
//     contiguous run of the tiles with the N tiles of one token tile
//     adjacent (L2 reuse of tokens), handed out by a counter per XCD; a
//     block knows its next tile while the current one computes and requests
//     that tile's record and gathered row ids meanwhile (with one block per
//     tile, that chain of two dependent loads ran before every tile's first
//     MFMA).
#include <type_traits>

#include "device.h"
#include "internal.h"
#include "skinny.h"

namespace moe {

constexpr int kBM = 128;  // token positions per tile
constexpr int kBN = 256;  // weight rows per tile (w13: 128 gate + 128 up)
constexpr int kGemmThreads = 512;  // 8 waves
constexpr int kMB = kBM / 16;       // token blocks per wave (the whole tile)
constexpr int kRB = 2;              // 16-row weight blocks per wave

// Per format: K per stage (each lane's 16 weight bytes per row block are 32
// E2M1 values or 16 int8 values, a quarter of the stage), MFMA k-steps per
// stage, LDS bytes per stage and 16-byte activation pieces per thread (the
// thread's quarter of one token row: pieces kk = 0 .. kKK-1 of quarter g).
template <int FMT>
struct GemmCfg {
  static constexpr int kBK = FMT != kFmtI8 ? 128 : 64;
  static constexpr int kKK = kBK / 32;
  static constexpr int kStage = kBM * kBK * 2;
  static constexpr int kAVec = kBK / 32;
  static_assert(kAVec == kKK, "a thread's pieces are the k-steps of one quarter");
};

// A lane's weight bytes for one row block and stage, converted to bf16
// eight K-values at a time (MXFP4: scaled FP4 convert; 3-bit: look-ups in
// the block's scaled code book; int8: exact).
template <int FMT>
__device__ __forceinline__ bf16x8_t gemm_conv(const u32x4_t& q, int kk, uint32_t sc, const Q3Book& book) {
  if constexpr (FMT == kFmtMx) {
    const uint32_t d = kk == 0 ? q.x : kk == 1 ? q.y : kk == 2 ? q.z : q.w;
    return fp4x8_to_bf16x8(d, e8m0_scale_operand(sc));
  } else if constexpr (FMT == kFmtQ3) {
    return q3_frag(q.x, q.y, q.z, kk, book);
  } else {
    return i8x8_to_bf16x8(kk == 0 ? q.x : q.z, kk == 0 ? q.y : q.w);
  }
}

// Weights of the wave's row blocks for stage st: 16 bytes per lane and row
// block (MXFP4, int8) or one 12-byte 3-bit block.
template <int FMT>
__device__ __forceinline__ void gemm_load_w(const uint8_t* qe, const uint32_t (&qoff)[kRB], int st,
                                            u32x4_t (&w)[kRB]) {
#pragma unroll
  for (int b = 0; b < kRB; ++b) {
    if constexpr (FMT == kFmtQ3) {
      const uint32_t* s = reinterpret_cast<const uint32_t*>(qe + (qoff[b] + (uint32_t)st * 48));
      w[b] = (u32x4_t){s[0], s[1], s[2], 0u};
    } else {
      w[b] = *reinterpret_cast<const u32x4_t*>(qe + (qoff[b] + (uint32_t)st * 64));
    }
  }
}

// The scale of the lane's 32 K-values of stage st in each row block (block
// 4 st + g of the row: those 32 values are exactly one group), from the
// block's scales in LDS: an E8M0 byte (MXFP4) or binary16 bits (3-bit).
template <int FMT>
__device__ __forceinline__ void gemm_scales(const unsigned char* lds_s, const uint32_t (&soff)[kRB], int st,
                                            uint32_t (&sc)[kRB]) {
#pragma unroll
  for (int b = 0; b < kRB; ++b) {
    if constexpr (FMT == kFmtMx) sc[b] = lds_s[soff[b] + (uint32_t)st * 4];
    else if constexpr (FMT == kFmtQ3) sc[b] = *reinterpret_cast<const uint16_t*>(lds_s + soff[b] + (uint32_t)st * 8);
    else sc[b] = 0u;
  }
}


// The thread's quarter of one gathered token row for stage st.
template <int FMT>
struct GemmA {
  static constexpr int N = GemmCfg<FMT>::kAVec;
  u32x4_t v[N];
  // The empty asm with a memory clobber keeps the loads where they are
  // issued: otherwise they are sunk past the MFMA work to their LDS store and
  // their latency is no longer hidden.
  __device__ __forceinline__ void load(const uint16_t* asrc, int st) {
    const u32x4_t* s = reinterpret_cast<const u32x4_t*>(asrc + st * GemmCfg<FMT>::kBK);
#pragma unroll
    for (int j = 0; j < N; ++j) v[j] = s[j];
    asm volatile("" ::: "memory");
  }
  // dst: the thread's piece for k-step 0; k-step j lies 64 pieces further.
  __device__ __forceinline__ void store(u32x4_t* dst) const {
#pragma unroll
    for (int j = 0; j < N; ++j) dst[j * 64] = v[j];
  }
};

// For each MFMA k-step: the wave's weight fragments converted once, each
// activation fragment used for kRB MFMAs. The activation fragments of k-step
// kk+1 are read from LDS before the MFMAs of k-step kk (a scheduling barrier
// keeps the reads there: left alone, the compiler issues each read right
// before its MFMAs and every MFMA pair waits for the LDS latency).
template <int FMT, int MB>
__device__ __forceinline__ void gemm_compute(f32x4_t (&acc)[kRB][MB], const u32x4_t (&w)[kRB],
                                             const unsigned char* lds_s, const uint32_t (&soff)[kRB], int st,
                                             const unsigned char* abase, const float* lv_lds) {
  constexpr int kKK = GemmCfg<FMT>::kKK;
  uint32_t sc[kRB];
  gemm_scales<FMT>(lds_s, soff, st, sc);
  Q3Book book[kRB] = {};
  if constexpr (FMT == kFmtQ3) {
    {
      float lv[8];  // the tile's expert's levels, from LDS (broadcast reads)
#pragma unroll
      for (int c = 0; c < 8; ++c) lv[c] = lv_lds[c];
#pragma unroll
      for (int b = 0; b < kRB; ++b) book[b] = q3_book(lv, f16_bits_to_f32(sc[b]));
    }
  }
  // int8 weights are unpacked here, in their stage: without the empty asm
  // the compiler starts unpacking them right after their load, a stage
  // ahead, which waits for that load and holds the unpacked bytes meanwhile
  // (the shared expert's GEMMs ran 2-8 % slower).
  u32x4_t wv[kRB];
#pragma unroll
  for (int b = 0; b < kRB; ++b) {
    wv[b] = w[b];
    if constexpr (FMT == kFmtI8) asm volatile("" : "+v"(wv[b]));
  }
  bf16x8_t bt[2][MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) bt[0][m] = *reinterpret_cast<const bf16x8_t*>(abase + (m * kKK) * 1024);
#pragma unroll
  for (int kk = 0; kk < kKK; ++kk) {
    if (kk + 1 < kKK) {
#pragma unroll
      for (int m = 0; m < MB; ++m)
        bt[(kk + 1) & 1][m] = *reinterpret_cast<const bf16x8_t*>(abase + (m * kKK + kk + 1) * 1024);
    }
    __builtin_amdgcn_sched_barrier(0);
    bf16x8_t wa[kRB];
#pragma unroll
    for (int b = 0; b < kRB; ++b) wa[b] = gemm_conv<FMT>(wv[b], kk, sc[b], book[b]);
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int b = 0; b < kRB; ++b) acc[b][m] = mfma_16x16x32(wa[b], bt[kk & 1][m], acc[b][m]);
  }
}

// Shared w2 + combine epilogue: out[t][n] = sum_j ybuf[t k + j][n] (slot
// order) + s2[n] acc[n][t]. The matrix cores are idle here, and the k bf16
// slot rows of a token dominate the tile's bytes (at k = 6, 393 KB against
// the K loop's 0.5 MB of weights), so they are requested as a batch: all k
// rows of both row blocks for a column block of 16 tokens, the next column
// block's batch before the current one is added. At 8192 tokens this took
// the launch from 339 to 268 us (the loop over the slots had kept one load
// per wave in flight); three column blocks in flight measured no better.
template <int MB>
__device__ __forceinline__ void gemm_combine(const GemmArgs& p, const f32x4_t (&acc)[kRB][MB], int ncols, int pos0,
                                             int nt, int wn, int g, int r) {
  const int k = p.topk;
  int n[kRB];
  float s2[kRB][4];
#pragma unroll
  for (int b = 0; b < kRB; ++b) {
    n[b] = nt * kBN + wn * 32 + b * 16 + 4 * g;
#pragma unroll
    for (int i = 0; i < 4; ++i) s2[b][i] = p.row_scale[n[b] + i];
  }
  uint2 y[2][kRB][kMaxTopK];
  auto fetch = [&](int m, uint2 (&d)[kRB][kMaxTopK]) __attribute__((always_inline)) {
    const int tok = m * 16 + r;
    const uint16_t* row = p.ybuf + (size_t)(pos0 + (tok < ncols ? tok : 0)) * k * p.out_ld;
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j)
      if (j < k) {
#pragma unroll
        for (int b = 0; b < kRB; ++b) d[b][j] = *reinterpret_cast<const uint2*>(row + (size_t)j * p.out_ld + n[b]);
      }
  };
  fetch(0, y[0]);
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    if (m + 1 < MB) fetch(m + 1, y[(m + 1) & 1]);
    const int tok = m * 16 + r;
    if (tok >= ncols) continue;
    const size_t orow = (size_t)(pos0 + tok) * p.out_ld;
#pragma unroll
    for (int b = 0; b < kRB; ++b) {
      float o[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j)
        if (j < k) {
          const uint2 v = y[m & 1][b][j];
          o[0] += bf16_to_f32(v.x & 0xffffu);
          o[1] += bf16_to_f32(v.x >> 16);
          o[2] += bf16_to_f32(v.y & 0xffffu);
          o[3] += bf16_to_f32(v.y >> 16);
        }
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] += s2[b][i] * acc[b][m][i];
      if (p.out_is_fp32) {
        *reinterpret_cast<float4*>(static_cast<float*>(p.out) + orow + n[b]) = make_float4(o[0], o[1], o[2], o[3]);
      } else {
        uint2 pk;
        pk.x = (uint32_t)f32_to_bf16(o[0]) | ((uint32_t)f32_to_bf16(o[1]) << 16);
        pk.y = (uint32_t)f32_to_bf16(o[2]) | ((uint32_t)f32_to_bf16(o[3]) << 16);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + orow + n[b]) = pk;
      }
    }
  }
}

// The K loop and epilogue of one block over its first MB*16 positions.
template <int FMT, int MODE, int MB, class StoreScales>
__device__ __forceinline__ void gemm_main(const GemmArgs& p, const uint8_t* qe, const unsigned char* lds_s,
                                          const uint32_t (&qoff)[kRB], const uint32_t (&soff)[kRB],
                                          const uint16_t* asrc, u32x4_t* adst0, u32x4_t* adst1,
                                          const unsigned char* abase0, const unsigned char* abase1, int nst,
                                          int ncols, int pos0, int nt, int wn, int g, int r,
                                          const StoreScales& store_scales, const int (&slot_r)[kMB],
                                          const float* lv) {
  f32x4_t acc[kRB][MB];
#pragma unroll
  for (int b = 0; b < kRB; ++b)
#pragma unroll
    for (int m = 0; m < MB; ++m) acc[b][m] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

  // Software pipeline, branch-free so that every wait counts exactly: stage
  // st computes from LDS buffer st%2 and weight registers st%2; the
  // activations of stages st+1 and st+2 are in registers (set s%2 holds
  // stage s) or in flight, and the weights of st+2 are in flight. Loads past
  // the last stage re-read it (clamped, never used).
  u32x4_t w0[kRB], w1[kRB];
  GemmA<FMT> av0, av1;
  const int last = nst - 1;
  gemm_load_w<FMT>(qe, qoff, 0, w0);
  av0.load(asrc, 0);
  store_scales();  // the block's scales, requested before these first loads
  // routed w2: the routing weights of the lane's columns (their slots came
  // before the scales, so they are in), in flight during the K loop
  float wv_r[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) wv_r[m] = MODE == kGemmW2 ? p.slot_w[slot_r[m]] : 0.0f;
  asm volatile("" ::: "memory");
  av0.store(adst0);
  av1.load(asrc, min(1, last));
  av0.load(asrc, min(2, last));
  gemm_load_w<FMT>(qe, qoff, min(1, last), w1);
  for (int st = 0; st + 1 < nst; st += 2) {
    __syncthreads();
    av1.store(adst1);  // stage st+1
    av1.load(asrc, min(st + 3, last));
    gemm_compute<FMT, MB>(acc, w0, lds_s, soff, st, abase0, lv);
    gemm_load_w<FMT>(qe, qoff, min(st + 2, last), w0);
    __syncthreads();
    av0.store(adst0);  // stage st+2
    av0.load(asrc, min(st + 4, last));
    gemm_compute<FMT, MB>(acc, w1, lds_s, soff, st + 1, abase1, lv);
    gemm_load_w<FMT>(qe, qoff, min(st + 3, last), w1);
  }
  if (nst & 1) {  // the last stage (buffer 0, w0)
    __syncthreads();
    gemm_compute<FMT, MB>(acc, w0, lds_s, soff, last, abase0, lv);
  }

  // epilogue: lane holds acc[b][m][i] = D[row 4g+i of block b][token r of block m]
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    const int tok = m * 16 + r;  // position within the tile
    if (tok >= ncols) continue;
    const int pos = pos0 + tok;
    if (MODE == kGemmW13) {  // block 0: gate rows, block 1: the matching up rows
      const int hc = nt * (kBN / 2) + wn * 16 + 4 * g;
      uint16_t h[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float gv = acc[0][m][i], uv = acc[1][m][i];
        if (FMT == kFmtI8) {
          gv *= p.row_scale[hc + i];
          uv *= p.row_scale[p.half + hc + i];
        }
        h[i] = f32_to_bf16(swiglu_clamped(gv, uv, p.limit));
      }
      uint2 pk;
      pk.x = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
      pk.y = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
      *reinterpret_cast<uint2*>(p.hout + (size_t)pos * p.hout_ld + hc) = pk;
    } else if (MODE == kGemmW2) {  // routed: y * w -> yout[slot], bf16
      const int slot = slot_r[m];
      const float wv = wv_r[m];
#pragma unroll
      for (int b = 0; b < kRB; ++b) {
        const int n = nt * kBN + wn * 32 + b * 16 + 4 * g;
        uint2 pk;
        pk.x = (uint32_t)f32_to_bf16(acc[b][m][0] * wv) | ((uint32_t)f32_to_bf16(acc[b][m][1] * wv) << 16);
        pk.y = (uint32_t)f32_to_bf16(acc[b][m][2] * wv) | ((uint32_t)f32_to_bf16(acc[b][m][3] * wv) << 16);
        *reinterpret_cast<uint2*>(p.yout + (size_t)slot * p.yout_ld + n) = pk;
      }
    }
  }
  if constexpr (MODE == kGemmW2Combine) gemm_combine<MB>(p, acc, ncols, pos0, nt, wn, g, r);
}

template <int FMT, int MODE>
__global__ __launch_bounds__(kGemmThreads) void k_gemm(GemmArgs p) {
  constexpr int kBK = GemmCfg<FMT>::kBK, kKK = GemmCfg<FMT>::kKK;
  __shared__ __align__(16) unsigned char lds_a[2][GemmCfg<FMT>::kStage];
  // MXFP4: [256 local rows][K/32 + 4] E8M0 bytes; 3-bit: [256][K/16 + 4] bytes of binary16 scales
  extern __shared__ __align__(16) unsigned char lds_s[];
  __shared__ int grabbed;
  __shared__ float lds_lv[8];

  // Persistent: at most the blocks that fit at once, each walking tiles.
  // XCD-aware order: XCD x (blocks b with b % 8 == x) owns a contiguous run
  // of the logical tiles (N tiles fastest), handed out in order: a block's
  // first two tiles are fixed, then it grabs from its XCD's counter, two
  // tiles ahead, so that while a tile computes the block already knows the
  // next one and requests its record and gathered row ids. Once its XCD's
  // run is handed out, a block takes tiles from the run of the XCD with the
  // most left (equal runs of tiles are not equal work: at prefill the last
  // XCD finished 90-130 us after the median one).
  const int nblk = p.routed ? *p.n_tiles * p.n_ntiles : ((p.T + kBM - 1) / kBM) * p.n_ntiles;
  if (nblk <= 0) return;  // no tiles (a rejected permutation): the whole grid leaves, the queue untouched
  const int kNone = nblk;  // no tile
  constexpr bool kSteal = FMT != kFmtI8;  // the shared expert's tiles (int8) are all alike: no stealing
  const int G = gridDim.x;
  const int xcd = blockIdx.x & 7, inx = blockIdx.x >> 3;
  const int per = nblk >> 3, extra = nblk & 7;
  // XCD y's run [lo, hi) and its blocks; tiles past the first two per block go through its counter
  auto run_of = [&](int y, int& ylo, int& yhi, int& yq0) __attribute__((always_inline)) {
    ylo = y * per + min(y, extra);
    yhi = ylo + per + (y < extra ? 1 : 0);
    yq0 = ylo + 2 * ((G - y + 7) >> 3);
  };
  int lo, hi, q0;
  run_of(xcd, lo, hi, q0);
  const int nx = (G - xcd + 7) >> 3;  // blocks on this XCD
  int* const q = p.queue;  // [8] tiles handed out per XCD, [8] blocks done
  // another XCD's tile (thread 0, once this XCD's run is handed out): the
  // counters are read, the run with the most tiles left is chosen and one
  // tile taken from it with its counter; kNone when no run has any left
  auto steal = [&]() -> int {
    for (int attempt = 0; attempt < 8; ++attempt) {
      int best = -1, best_left = 0, bhi = 0, bq0 = 0;
#pragma unroll 1
      for (int y = 0; y < 8; ++y) {
        int ylo, yhi, yq0;
        run_of(y, ylo, yhi, yq0);
        const int left = yhi - (yq0 + (int)load_agent(reinterpret_cast<const uint32_t*>(q + y)));
        if (y != xcd && left > best_left && left >= 2) {
          best = y;
          best_left = left;
          bhi = yhi;
          bq0 = yq0;
        }
      }
      if (best < 0) return kNone;
      const int t = bq0 + atomicAdd(q + best, 1);
      if (t < bhi) return t;
    }
    return kNone;
  };

  const int K = p.K;
  const int nst = K / kBK;
  const int rowlen = FMT == kFmtQ3 ? K / 16 : K / 32;  // scale bytes per weight row
  const int srow = rowlen + 4;                          // padded LDS row of scales
  const int npieces = FMT != kFmtI8 ? 2 * 128 * rowlen / 16 : 0;
  const int hpieces = npieces > 1 ? npieces / 2 : 1;  // pieces per run of 128 rows
  constexpr int kScalePieces = 4;

  // a tile's record (uniform): expert, first sorted position, positions
  auto record = [&](int lg) -> int4 {
    const int tg = min(lg, nblk - 1) / p.n_ntiles;
    int4 t = p.routed ? p.tile_info[tg] : make_int4(0, tg * kBM, min(kBM, p.T - tg * kBM), 0);
    t.x = __builtin_amdgcn_readfirstlane(t.x);
    t.y = __builtin_amdgcn_readfirstlane(t.y);
    t.z = __builtin_amdgcn_readfirstlane(t.z);
    t.w = 0;
    return t;
  };
  // the gathered activation row of this lane's token (16*wave + lane%16 of
  // the tile; rows past the tile re-read its first row, never stored)
  auto act_row_of = [&](const int4& rec, int arow) -> int {
    const int apos = rec.y + (arow < rec.z ? arow : 0);
    return p.act_row ? p.act_row[apos] : apos;
  };

  int cur = lo + inx < hi ? lo + inx : kNone;
  int nxt = lo + nx + inx < hi ? lo + nx + inx : kNone;
  int4 rec = record(cur);
  int atrow = act_row_of(rec, (threadIdx.x >> 6) * 16 + (threadIdx.x & 15));
  while (cur < kNone) {
    // Per-lane values come from an opaque copy of the thread index, so that
    // they are recomputed per tile: hoisted out of the loop they stayed live
    // across it and spilled.
    int tid;
    asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"((int)threadIdx.x));
    const int wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, g = lane >> 4;
    const int wn = wave;  // the wave's 32 weight rows; every wave covers all 128 positions
    // the tile after next: its index is only needed at the end of this tile
    int grab = 0;
    if (tid == 0) grab = atomicAdd(q + xcd, 1);
    const int4 rec_n = record(nxt);  // the next tile's record; its row ids once the scales are in
    int atrow_n = atrow;

    const int nt = cur % p.n_ntiles;
    const int e = rec.x, pos0 = rec.y, ncols = rec.z;
    // weight rows of the wave's 2 row blocks (w13: 16 gate rows and the
    // matching 16 up rows), as 32-bit offsets from the expert's (uniform) bases
    const uint8_t* qe = p.wq + (long long)e * p.q_expert_stride;
    // 3-bit: the expert's levels to LDS (read after the K loop's first
    // barrier; the previous tile's readers passed the barrier that ends it)
    if constexpr (FMT == kFmtQ3) {
      if (tid < 8) lds_lv[tid] = p.table ? p.table[(size_t)e * 8 + tid] : (float)(tid - 4);
    }
    const float* lv = lds_lv;
    uint32_t qoff[kRB], soff[kRB];
#pragma unroll
    for (int b = 0; b < kRB; ++b) {
      int wrow;
      if (MODE == kGemmW13) wrow = (b == 0 ? 0 : p.half) + nt * (kBN / 2) + wn * 16 + r;
      else wrow = nt * kBN + wn * 32 + b * 16 + r;
      qoff[b] = FMT == kFmtQ3 ? (uint32_t)wrow * (K / 32 * 12) + g * 12
                              : (uint32_t)wrow * (FMT == kFmtMx ? K / 2 : K) + g * 16;
      // local row: gate rows (w13) or the first 128 rows (w2) at 0 .., the rest at 128 ..
      const int lrow = MODE == kGemmW13 ? (b == 0 ? 0 : 128) + wn * 16 + r : wn * 32 + b * 16 + r;
      soff[b] = (uint32_t)lrow * srow + g * (FMT == kFmtQ3 ? 2 : 1);
    }
    // the tile's scales: two runs of 128 rows (w13: gate rows, up rows; w2:
    // the tile's 256 rows), K/32 bytes per row, in 16-byte pieces. Up to
    // kScalePieces per thread are requested now, ahead of the pipeline's
    // first loads, and written to LDS after those are issued (any more are
    // copied then, for K above 4096).
    const uint8_t* se = p.wsc + (long long)e * p.s_expert_stride;
    auto piece_src = [&](int i) {
      const int run = i / hpieces, o = (i - run * hpieces) * 16;
      const int grow0 = MODE == kGemmW13 ? (run == 0 ? 0 : p.half) + nt * (kBN / 2) : nt * kBN + run * 128;
      return reinterpret_cast<const uint4*>(se + (size_t)grow0 * rowlen + o);
    };
    auto piece_store = [&](int i, const uint4& v) {
      const int run = i / hpieces, o = (i - run * hpieces) * 16;
      const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int oq = o + 4 * qq, row = oq / rowlen, col = oq - row * rowlen;
        *reinterpret_cast<uint32_t*>(lds_s + (size_t)(run * 128 + row) * srow + col) = d[qq];
      }
    };
    // routed w2: the slots of the lane's columns, requested first (the
    // epilogue scatters by slot and scales by its routing weight: loaded
    // there, slot then weight, two memory round trips ended every tile)
    int slot_r[kMB];
#pragma unroll
    for (int m = 0; m < kMB; ++m) {
      const int tok = m * 16 + r;
      slot_r[m] = MODE == kGemmW2 ? p.sorted_slots[pos0 + (tok < ncols ? tok : 0)] : 0;
    }
    uint4 scv[kScalePieces];
    if (FMT != kFmtI8) {
#pragma unroll
      for (int j = 0; j < kScalePieces; ++j) scv[j] = *piece_src(min(tid + j * kGemmThreads, npieces - 1));
    }
    const int arow = wave * 16 + r;
    auto store_scales = [&]() __attribute__((always_inline)) {
      if (FMT != kFmtI8) {
#pragma unroll
        for (int j = 0; j < kScalePieces; ++j) {
          const int i = tid + j * kGemmThreads;
          if (i < npieces) piece_store(i, scv[j]);
        }
        for (int i = tid + kScalePieces * kGemmThreads; i < npieces; i += kGemmThreads)
          piece_store(i, *piece_src(i));
      }
      atrow_n = act_row_of(rec_n, arow);  // the next tile's record came before these scales
    };
    // this thread's activation loads: token row arow, quarter lane/16 of
    // the row's stage (so that a wave's LDS stores are contiguous)
    const uint16_t* asrc = p.act + (size_t)atrow * p.act_ld + g * (kBK / 4);
    // fragment-major LDS: piece (token t, quarter q, k-step j) at 16 bytes x
    // ((t/16 * kKK + j) * 64 + q * 16 + t%16), i.e. where lane (r = t%16, g =
    // q) of the MFMAs of token block t/16 reads it
    const int aslot = ((arow >> 4) * kKK) * 64 + g * 16 + (arow & 15);
    u32x4_t* adst0 = reinterpret_cast<u32x4_t*>(&lds_a[0][aslot * 16]);
    u32x4_t* adst1 = reinterpret_cast<u32x4_t*>(&lds_a[1][aslot * 16]);
    const unsigned char* abase0 = &lds_a[0][lane * 16];
    const unsigned char* abase1 = &lds_a[1][lane * 16];

    // a tile runs the MFMAs of its positions rounded up to 32 (uniform
    // branch: partly filled last tiles of the experts would otherwise waste
    // about a sixth of the work at prefill)
    switch ((ncols + 31) >> 5) {
      case 1:
        gemm_main<FMT, MODE, 2>(p, qe, lds_s, qoff, soff, asrc, adst0, adst1, abase0, abase1, nst, ncols, pos0, nt,
                                wn, g, r, store_scales, slot_r, lv);
        break;
      case 2:
        gemm_main<FMT, MODE, 4>(p, qe, lds_s, qoff, soff, asrc, adst0, adst1, abase0, abase1, nst, ncols, pos0, nt,
                                wn, g, r, store_scales, slot_r, lv);
        break;
      case 3:
        gemm_main<FMT, MODE, 6>(p, qe, lds_s, qoff, soff, asrc, adst0, adst1, abase0, abase1, nst, ncols, pos0, nt,
                                wn, g, r, store_scales, slot_r, lv);
        break;
      default:
        gemm_main<FMT, MODE, kMB>(p, qe, lds_s, qoff, soff, asrc, adst0, adst1, abase0, abase1, nst, ncols, pos0,
                                  nt, wn, g, r, store_scales, slot_r, lv);
    }
    if (tid == 0) {
      int t = q0 + grab;
      if (t >= hi) t = kSteal && p.routed ? steal() : kNone;
      grabbed = t;
    }
    __syncthreads();  // every wave is done with this tile's LDS; the grab is visible
    const int got = __builtin_amdgcn_readfirstlane(grabbed);
    if (kSteal && nxt == kNone) {
      // no next tile was known (a run shorter than two tiles per block): a
      // stolen tile is taken now, its record loaded here
      cur = got;
      if (cur < kNone) {
        rec = record(cur);
        atrow = act_row_of(rec, (threadIdx.x >> 6) * 16 + (threadIdx.x & 15));
      }
    } else {
      cur = nxt;
      nxt = got;
      rec = rec_n;
      atrow = atrow_n;
    }
  }
  // the last block out sets the counters back to zero for the next launch
  if (threadIdx.x == 0 && atomicAdd(q + 8, 1) == G - 1) {
#pragma unroll
    for (int i = 0; i < 9; ++i) q[i] = 0;
  }
}

template <int FMT, int MODE>
static hipError_t launch_gemm_t(const GemmArgs& p, int tiles, hipStream_t st) {
  const long long nblk = (long long)tiles * p.n_ntiles;
  if (nblk <= 0) return hipSuccess;
  if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
  const size_t dyn = FMT != kFmtI8 ? (size_t)2 * 128 * (p.K / (FMT == kFmtQ3 ? 16 : 32) + 4) : 0;
  if (dyn + 2 * GemmCfg<FMT>::kStage > 160 * 1024) return hipErrorInvalidValue;
  static size_t raised = 0;  // dynamic LDS limit set so far for this kernel
  if (dyn > raised) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm<FMT, MODE>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
    if (e != hipSuccess) return e;
    raised = dyn;
  }
  // persistent: at most the blocks that fit on the chip at once
  static int resident = 0;  // per kernel: blocks per CU x CUs
  if (resident == 0) {
    int per_cu = 0, dev = 0, cus = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_gemm<FMT, MODE>, kGemmThreads, dyn);
    if (e == hipSuccess) e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    resident = per_cu * cus > 0 ? per_cu * cus : 1;
  }
  const long long grid = nblk < resident ? nblk : resident;
  k_gemm<FMT, MODE><<<(unsigned)grid, kGemmThreads, dyn, st>>>(p);
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& p, int tiles, hipStream_t st) {
  if (p.K % 128 || p.K <= 0 || !p.queue) return hipErrorInvalidValue;
  if (p.fmt == kFmtMx) {
    if (p.mode == kGemmW13) return launch_gemm_t<kFmtMx, kGemmW13>(p, tiles, st);
    return launch_gemm_t<kFmtMx, kGemmW2>(p, tiles, st);
  }
  if (p.fmt == kFmtQ3) {  // routed w2 only
    if (p.mode != kGemmW2) return hipErrorInvalidValue;
    return launch_gemm_t<kFmtQ3, kGemmW2>(p, tiles, st);
  }
  if (p.mode == kGemmW13) return launch_gemm_t<kFmtI8, kGemmW13>(p, tiles, st);
  return launch_gemm_t<kFmtI8, kGemmW2Combine>(p, tiles, st);
}

}  // namespace moe
