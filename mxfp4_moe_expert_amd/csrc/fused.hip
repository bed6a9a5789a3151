// The whole MoE layer for the smallest batches (T <= 2, T*(k+1) <= 16, e.g.
// single-token decode) in one launch on gfx950, one block of 8 waves per CU.
//
// Every block b does a slice of every step, in this order:
//   1. router: the logit of expert b for every token, then its score
//      sqrt(softplus(logit)) (page "DeepSeek-V4-Flash-0731", section
//      "Checked in its code", row "Mixture of experts");
//   2. shared expert, int8 w13 (page "deepseek-v4-mxfp4-int8 config.json",
//      linears_w8a16): gate rows 8b..8b+7 and the matching up rows, so the
//      block owns h_shared[8b .. 8b+7] (clamped SwiGLU, first page, row
//      "SwiGLU feed-forward");
//   3. the top-k of every token over score + bias (row "Auxiliary-loss-free
//      load balancing"), computed by the block itself from every block's
//      published score; then routed MXFP4 w13 for every slot on the same 8
//      gate + 8 up rows of the slot's expert: h_slot[8b .. 8b+7];
//   4. routed MXFP4 w2 + shared int8 w2 + weighted combine for output rows
//      16b .. 16b+15 of every token (row "Shared expert"), once every block's
//      h slices are published.
// Each 16-row MFMA job is split along K over the 8 waves (wave w takes the
// w-th eighth of K) and the wave partials are summed in LDS in wave order.
//
// The weight stream of a block is one in-order sequence: shared w13 (with
// the router row), shared w2 once the block's score is published, the
// routed w13 jobs with two in flight per wave, the first three routed w2 jobs
// (they arrive while the block reduces and publishes its h slices, when the
// CU's loads would otherwise pause), then, once the block's h slices are
// published, the other routed w2 jobs, which stream while the other blocks'
// h slices arrive. A CU queues its loads in order, so a load requested early
// delays whatever the CU requests after it: each hand-off store goes out
// before the bulk loads that follow it. (Requesting the w2 jobs before the
// w13 jobs moves the end of the w13 stream, and with it every h slice, to
// the end of the whole routed stream; measured slower. Requesting 2 to 4 w2
// jobs before the h publish took the layer at one token from 30.0 to
// 28.5 us; 5 or 6 delay the publish and lose it again.)
//
// Hand-offs: a producer stores each 32-bit word (a score, or a pair of bf16
// h values) XORed with a tag that no computed word equals, so that no
// published word is zero, with device-wide coherent stores; a consumer polls
// the words themselves with coherent loads until none is zero. The buffers
// are zero before a layer: each block counts the layers it has run in a word
// of its own (every block runs every layer, so all counts agree), layers
// alternate between two buffers by that count's parity, and each block
// zeroes its slices of the other buffer, which no block reads during this
// layer, once its h slices are published (see layer_tail). Every poll is
// bounded: past the limit the output is NaN, never a silent wrong value. The
// waits are for every block of the grid, so the launch checks with the
// occupancy calculator that the whole grid is resident at once.
#include <algorithm>

#include "device.h"
#include "internal.h"

namespace moe {

constexpr int kLayerWaves = 8;
constexpr int kLayerThreads = kLayerWaves * 64;
constexpr uint32_t kScoreTag = 0x7F800001u;  // an fp32 signalling NaN: no computed score
constexpr uint32_t kHTag = 0x7F817F81u;      // two bf16 signalling NaNs: no rounded h pair
constexpr uint32_t kNaNPair = 0x7FC07FC0u;   // h of a block whose routing timed out
constexpr int kPollLimit = 1 << 20;          // polls (each followed by a short sleep)
constexpr int kEarlyW2 = 3;                  // routed w2 jobs requested before the h publish

template <int NH, int NI, int TT, int KK>
struct LayerShape {
  static constexpr int H = 1024 * NH, I = 1024 * NI;
  static constexpr int NS = TT * KK, NCOL = NS + TT;
  static constexpr int XPT = H / kLayerThreads;  // x / router elements per thread
  static constexpr int P = 2;                    // routed w13 jobs in flight per wave (1: 27.1 us, 3: 27.6)
  static constexpr int HROW = I * 2 + 16;        // LDS row of an h column
  static constexpr int ZROW = (H > I ? H : I) * 2;  // LDS zero row: the B operand of inactive lanes
  static constexpr size_t off_zero = (size_t)TT * H * 2;
  static constexpr size_t off_red13 = off_zero + ZROW;
  static constexpr size_t off_hl = off_red13 + (size_t)(1 + NS) * kLayerWaves * TT * 16 * 4;
  static constexpr size_t off_red2 = off_hl + (size_t)NCOL * HROW;
  static constexpr size_t off_ycol = off_red2 + (size_t)kLayerWaves * 64 * 16;
  static constexpr size_t off_rred = off_ycol + 16 * 16 * 4;
  static constexpr size_t off_sel = off_rred + (size_t)kLayerWaves * TT * 4;
  static constexpr size_t off_lv = off_sel + 16 * 4 + 16 * 4 + 16;  // 3-bit w2: 8 levels per slot
  static constexpr size_t lds_bytes = off_lv + 16 * 8 * 4;
  static_assert(NCOL <= kXferCols && TT <= kXferTokens && I <= kXferMaxI, "hand-off buffers too small");
  static_assert(NCOL <= 16, "one 16-column MFMA tile holds every slot and the shared columns");
  static_assert(XPT == 4 || XPT == 8, "H / 512 elements per thread");
};

// The hand-off buffers of one layer (parity p) and of the next (1 - p).
struct Xfer {
  uint32_t* epoch;                         // [kXferBlocks] layers run by each block
  uint32_t *scores, *h, *x;                // [2 tokens][256], [16 columns][1024 pairs], [2 tokens][2048 pairs]
  uint32_t *scores_next, *h_next, *x_next;  // the other parity: zeroed for the next layer
  __device__ __forceinline__ Xfer(uint32_t* base, uint32_t p) {
    epoch = base;
    uint32_t* s0 = base + kXferBlocks;
    uint32_t* h0 = s0 + 2 * kXferScoreWords;
    uint32_t* x0 = h0 + 2 * kXferHWords;
    scores = s0 + p * kXferScoreWords;
    scores_next = s0 + (1 - p) * kXferScoreWords;
    h = h0 + p * kXferHWords;
    h_next = h0 + (1 - p) * kXferHWords;
    x = x0 + p * kXferXWords;
    x_next = x0 + (1 - p) * kXferXWords;
  }
};

// The E8M0 bytes a lane needs for N super-steps of one row: groups 4i + g
// for i < N (lane group g), i.e. 4N consecutive bytes; byte 4i + g is byte g
// of word i.
template <int N>
__device__ __forceinline__ void load_scale_words(const uint8_t* p, uint32_t (&s)[N]) {
  if constexpr (N == 4) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    s[0] = v.x; s[1] = v.y; s[2] = v.z; s[3] = v.w;
  } else if constexpr (N == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    s[0] = v.x; s[1] = v.y;
  } else {
    s[0] = *reinterpret_cast<const uint32_t*>(p);
  }
}

// 16 bytes of MXFP4 (32 elements of one row, one E8M0 group) against 64
// bytes of bf16 B at bsrc: 4 MFMAs.
__device__ __forceinline__ void mx16_mfma(const uint4& q, uint32_t sbyte, const unsigned char* bsrc, f32x4_t& acc) {
  const float sc = e8m0_scale_operand(sbyte);
  const uint32_t d[4] = {q.x, q.y, q.z, q.w};
  bf16x8_t b[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) b[m] = *reinterpret_cast<const bf16x8_t*>(bsrc + m * 16);
#pragma unroll
  for (int m = 0; m < 4; ++m) acc = mfma_16x16x32(fp4x8_to_bf16x8(d[m], sc), b[m], acc);
}

// 16 bytes of int8 (16 elements of one row) against 32 bytes of bf16 B: 2 MFMAs.
__device__ __forceinline__ void i816_mfma(const uint4& q, const unsigned char* bsrc, f32x4_t& acc) {
  const bf16x8_t b0 = *reinterpret_cast<const bf16x8_t*>(bsrc);
  const bf16x8_t b1 = *reinterpret_cast<const bf16x8_t*>(bsrc + 16);
  acc = mfma_16x16x32(i8x8_to_bf16x8(q.x, q.y), b0, acc);
  acc = mfma_16x16x32(i8x8_to_bf16x8(q.z, q.w), b1, acc);
}

// One 3-bit block (32 elements of one row: 12 code bytes in q.x .. q.z and
// the binary16 scale h16) against 64 bytes of bf16 B at bsrc: 4 MFMAs.
__device__ __forceinline__ void q3_16_mfma(const uint4& q, uint32_t h16, const float (&lv)[8],
                                           const unsigned char* bsrc, f32x4_t& acc) {
  const Q3Book bk = q3_book(lv, f16_bits_to_f32(h16));
  bf16x8_t b[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) b[m] = *reinterpret_cast<const bf16x8_t*>(bsrc + m * 16);
#pragma unroll
  for (int m = 0; m < 4; ++m) acc = mfma_16x16x32(q3_frag(q.x, q.y, q.z, m, bk), b[m], acc);
}

// Indices and LDS carve-up of a block.
template <int NH, int NI, int TT, int KK>
struct LayerBlock {
  using S = LayerShape<NH, NI, TT, KK>;
  int b, tid, w, lane, r, g, E, NB, gb, ob, row13, n2;
  uint16_t* xs;         // [TT][H] the tokens
  unsigned char* zero;  // [ZROW] zeros
  float* red13;         // [1+NS][8 waves][TT][16 rows]
  unsigned char* hl;    // [NCOL][HROW] h columns
  f32x4_t* red2;        // [8 waves][64 lanes]
  float* ycol;          // [16 rows][16 columns]
  float* rred;          // [8 waves][TT]
  int32_t* sid;         // [16]
  float* sw;            // [16]
  int* flag;            // [4]: 0 router hand-off failed, 1 h hand-off failed
  float* lv;            // [16 slots][8] levels of each slot's expert (3-bit w2)
  __device__ __forceinline__ LayerBlock(const LayerArgs& a, unsigned char* lds, int thread = threadIdx.x) {
    b = blockIdx.x;
    tid = thread;
    w = tid >> 6;
    lane = tid & 63;
    r = lane & 15;
    g = lane >> 4;
    E = a.E;
    NB = gridDim.x;
    gb = min(b, S::I / 8 - 1);   // h rows 8gb .. 8gb+7 (blocks past I/8 repeat the last, unstored)
    ob = min(b, S::H / 16 - 1);  // output rows 16ob .. 16ob+15
    row13 = r < 8 ? 8 * gb + r : S::I + 8 * gb + (r - 8);
    n2 = 16 * ob + r;
    xs = reinterpret_cast<uint16_t*>(lds);
    zero = lds + S::off_zero;
    red13 = reinterpret_cast<float*>(lds + S::off_red13);
    hl = lds + S::off_hl;
    red2 = reinterpret_cast<f32x4_t*>(lds + S::off_red2);
    ycol = reinterpret_cast<float*>(lds + S::off_ycol);
    rred = reinterpret_cast<float*>(lds + S::off_rred);
    sid = reinterpret_cast<int32_t*>(lds + S::off_sel);
    sw = reinterpret_cast<float*>(sid + 16);
    flag = reinterpret_cast<int*>(sw + 16);
    lv = reinterpret_cast<float*>(lds + S::off_lv);
  }
};

// Steps 1-4, the same for every wave: router slice, shared w13, top-k.
// Returns the wave's shared w13 partial; qs2 gets the shared w2 weights.
// xin: the layer's input rows come from the previous layer of the same
// launch through X.x (its blocks publish them as tagged bf16 pairs), not
// from a.x.
template <int NH, int NI, int TT, int KK>
__device__ __forceinline__ f32x4_t layer_head(const LayerArgs& a, const LayerBlock<NH, NI, TT, KK>& L,
                                              const Xfer& X, uint4 (&qs2)[2 * NI], bool xin = false) {
  using S = LayerShape<NH, NI, TT, KK>;
  constexpr int H = S::H, I = S::I, XPT = S::XPT, N13I = 2 * NH, N2I = 2 * NI;
  const int b = L.b, tid = L.tid, w = L.w, lane = L.lane, r = L.r, g = L.g, E = L.E;

  // 1. loads, in the order they are needed: this thread's x slice (K =
  //    tid*XPT ..), the router row slice of expert b, the shared w13 weights
  //    of the wave's K range
  uint32_t xr[TT][XPT / 2];
  if (!xin) {
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      const uint16_t* src = a.x + (size_t)t * H + tid * XPT;
      if constexpr (XPT == 8) {
        const uint4 v = *reinterpret_cast<const uint4*>(src);
        xr[t][0] = v.x; xr[t][1] = v.y; xr[t][2] = v.z; xr[t][3] = v.w;
      } else {
        const uint2 v = *reinterpret_cast<const uint2*>(src);
        xr[t][0] = v.x; xr[t][1] = v.y;
      }
    }
  }
  const int er = min(b, E - 1);
  const float off_e = a.logit_offset ? a.logit_offset[er] : 0.0f;  // uniform: scalar loads
  float4 rw[XPT / 4];
#pragma unroll
  for (int i = 0; i < XPT / 4; ++i)
    rw[i] = *reinterpret_cast<const float4*>(a.gate_w + (size_t)er * H + tid * XPT + 4 * i);
  bool xbad = false;  // the previous layer's rows did not all arrive
  if (xin) {  // poll this thread's words of every token's row until none is zero
    bool got[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) got[t] = false;
    int spins = 0;
    while (true) {
      bool rdy = true;
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        if (!got[t]) {
          const uint32_t* src = X.x + (size_t)t * (kXferMaxH / 2) + tid * (XPT / 2);
          if constexpr (XPT == 8) {
            const u32x4_t v = load_agent_u32x4(src);
#pragma unroll
            for (int i = 0; i < 4; ++i) xr[t][i] = v[i];
          } else {
#pragma unroll
            for (int i = 0; i < 2; ++i) xr[t][i] = load_agent(src + i);
          }
          bool all = true;
#pragma unroll
          for (int i = 0; i < XPT / 2; ++i) all = all && xr[t][i] != 0u;
          got[t] = all;
        }
        rdy = rdy && got[t];
      }
      if (rdy) break;
      if (++spins >= kPollLimit) {
        xbad = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
      for (int i = 0; i < XPT / 2; ++i) xr[t][i] ^= kHTag;
  }
  // every wave's x and router slices are requested before any wave's shared
  // expert weights (the logit needs all eight slices: with each wave
  // requesting its three kinds back to back, the last slices queued behind
  // up to 56 KB of other waves' shared weights; 0.7 us at one token)
  asm volatile("" ::: "memory");
  __syncthreads();
  uint4 qsh[N13I];
  {
    const int8_t* base = a.sh13 + (size_t)L.row13 * H + w * (H / 8) + g * 16;
#pragma unroll
    for (int i = 0; i < N13I; ++i) qsh[i] = *reinterpret_cast<const uint4*>(base + i * 64);
  }
  asm volatile("" ::: "memory");

  // x -> LDS (the B columns of every w13 job); the zero row; the flags
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    uint32_t* dst = reinterpret_cast<uint32_t*>(L.xs + (size_t)t * H + tid * XPT);
#pragma unroll
    for (int i = 0; i < XPT / 2; ++i) dst[i] = xr[t][i];
  }
  for (int i = tid; i < S::ZROW / 16; i += kLayerThreads)
    reinterpret_cast<u32x4_t*>(L.zero)[i] = (u32x4_t){0u, 0u, 0u, 0u};
  if (tid < 4) L.flag[tid] = 0;

  // 2. router logit of expert b -> its published score
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < XPT / 4; ++i) {
      const uint32_t x01 = xr[t][2 * i], x23 = xr[t][2 * i + 1];
      acc += bf16_to_f32(x01 & 0xffff) * rw[i].x;
      acc += bf16_to_f32(x01 >> 16) * rw[i].y;
      acc += bf16_to_f32(x23 & 0xffff) * rw[i].z;
      acc += bf16_to_f32(x23 >> 16) * rw[i].w;
    }
    acc = wave_sum(acc);
    if (lane == 0) L.rred[w * TT + t] = acc;
  }
  __syncthreads();
  if (xbad) L.flag[1] = 1;  // the layer's output becomes NaN
  if (tid < TT && b < E) {
    float logit = 0.0f;
#pragma unroll
    for (int v = 0; v < kLayerWaves; ++v) logit += L.rred[v * TT + tid];
    logit += off_e;
    const float sc = sqrtf(softplus(logit));
    store_agent(X.scores + tid * kXferBlocks + b, __float_as_uint(sc) ^ kScoreTag);
  }
  {  // the shared w2 weights, needed last
    const int8_t* base = a.sh2 + (size_t)L.n2 * I + w * (I / 8) + g * 16;
#pragma unroll
    for (int i = 0; i < N2I; ++i) qs2[i] = *reinterpret_cast<const uint4*>(base + i * 64);
  }
  asm volatile("" ::: "memory");

  // 3. shared w13 (its weights came before anything that waits)
  f32x4_t acc_sh = {0.f, 0.f, 0.f, 0.f};
  {
    const unsigned char* bsrc = (r < TT ? reinterpret_cast<const unsigned char*>(L.xs + (size_t)r * H) : L.zero) +
                                (size_t)(w * (H / 8) + g * 16) * 2;
#pragma unroll
    for (int i = 0; i < N13I; ++i) i816_mfma(qsh[i], bsrc + i * 128, acc_sh);
  }

  // 4. the top-k of each token (wave t) from every block's published score
  if (w < TT) {
    float bq[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) bq[q] = a.bias ? a.bias[min(lane + 64 * q, E - 1)] : 0.0f;
    const uint32_t* srow = X.scores + w * kXferBlocks;
    uint32_t v[4];
    int spins = 0;
    while (true) {
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = load_agent(srow + min(lane + 64 * q, E - 1));
      const bool rdy = v[0] != 0 && v[1] != 0 && v[2] != 0 && v[3] != 0;
      if (__all(rdy)) break;
      if (++spins >= kPollLimit) {
        if (lane == 0) L.flag[0] = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    TopkRow row;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      row.s[q] = __uint_as_float(v[q] ^ kScoreTag);
      row.b[q] = row.s[q] + bq[q];
    }
    if (a.tid2eid) {  // hash layer: the token's table row (page "Tidalluna/...Tina-CQ4KM", "Compatibility")
      const int tok = __builtin_amdgcn_readfirstlane(a.token_ids[w]);
      const bool tok_ok = (unsigned)tok < (unsigned)a.V;
      if (!tok_ok && lane == 0 && b == 0 && a.flags) atomicOr(a.flags, kFlagTokenId);
      wave_hash_row(row, tok_ok ? a.tid2eid + (size_t)tok * KK : nullptr, E, KK, a.scale, L.sid + w * KK,
                    L.sw + w * KK, nullptr, b == 0 ? a.flags : nullptr);
    } else {
      wave_topk_row(row, E, KK, a.scale, L.sid + w * KK, L.sw + w * KK, nullptr);
    }
  }
  __syncthreads();
  if (b == 0 && tid < S::NS) {
    a.ids_out[tid] = L.sid[tid];
    a.w_out[tid] = L.sw[tid];
  }
  return acc_sh;
}

// Steps 5-9. Q3: the routed w2 in 3-bit blocks (a.w2c codes [E][H][I/32][12],
// a.w2s binary16 scales [E][H][I/32], a.w2tab levels [E][8] or null).
// The next layer's (or call's) hand-off buffers are zeroed before the h
// slices are awaited. STACK: one of several layers in one launch; every
// zeroing store is complete before this block publishes its output rows
// (every block enters the next layer only once it has all of this layer's
// rows, so none can read a stale word there), and the layer count is kept by
// the launch. publish: the output rows go to the next layer through X.x_next
// (and to a.out, bf16).
template <int NH, int NI, int TT, int KK, bool Q3, bool STACK = false>
__device__ __forceinline__ void layer_tail(const LayerArgs& a, const LayerBlock<NH, NI, TT, KK>& L, const Xfer& X,
                                           uint32_t ep, f32x4_t acc_sh, const uint4 (&qs2)[2 * NI],
                                           bool publish = false) {
  using S = LayerShape<NH, NI, TT, KK>;
  constexpr int H = S::H, I = S::I, NS = S::NS, NCOL = S::NCOL, P = S::P, HROW = S::HROW;
  constexpr int N13 = NH, N2 = NI, N2I = 2 * NI;
  const int b = L.b, tid = L.tid, w = L.w, lane = L.lane, r = L.r, g = L.g, NB = L.NB;
  const int gb = L.gb, ob = L.ob, row13 = L.row13, n2 = L.n2;
  const bool ok_route = L.flag[0] == 0;
  if (Q3 && tid < NS * 8) {  // the levels of each slot's expert, read from LDS before each use
    const int u = tid >> 3, c = tid & 7;
    L.lv[tid] = a.w2tab ? a.w2tab[(size_t)L.sid[u] * 8 + c] : (float)(c - 4);
  }
  auto slot_levels = [&](int u, float (&lv)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < 8; ++c) lv[c] = L.lv[u * 8 + c];
  };

  // preloaded for wave 0's reduction and the combine
  float shs[4] = {0.f, 0.f, 0.f, 0.f};  // shared w13 scales: gate rows 8gb+2p, +1; up rows
  if (w == 0) {
    const int p4 = lane & 3;
    shs[0] = a.sh13s[8 * gb + 2 * p4];
    shs[1] = a.sh13s[8 * gb + 2 * p4 + 1];
    shs[2] = a.sh13s[I + 8 * gb + 2 * p4];
    shs[3] = a.sh13s[I + 8 * gb + 2 * p4 + 1];
  }
  const float s2n = a.sh2s[16 * ob + (tid & 15)];
  float s2p[2] = {0.f, 0.f};  // publish: the shared w2 scales of output rows 2q, 2q + 1 (thread (t, q))
  if (STACK && publish) {
    s2p[0] = a.sh2s[16 * ob + 2 * (tid & 7)];
    s2p[1] = a.sh2s[16 * ob + 2 * (tid & 7) + 1];
  }

  // this block's slices of the next layer's (or call's) hand-off buffers:
  // scores of experts b, b+NB, ..; h pieces b, b+NB, .. of all columns;
  // (stack) its output pairs of every token
  auto zero_next = [&]() __attribute__((always_inline)) {
    constexpr int kPieces = kXferMaxI / 8;
    for (int i = tid; i < kXferCols * ((kPieces + NB - 1) / NB); i += kLayerThreads) {
      const int c = i % kXferCols, o = b + NB * (i / kXferCols);
      if (o < kPieces) {
        uint64_t* d = reinterpret_cast<uint64_t*>(X.h_next + c * (kXferMaxI / 2) + 4 * o);
        __hip_atomic_store(d, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(d + 1, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    for (int i = tid; i < kXferTokens * ((kXferBlocks + NB - 1) / NB); i += kLayerThreads) {
      const int t = i % kXferTokens, e = b + NB * (i / kXferTokens);
      if (e < kXferBlocks) store_agent(X.scores_next + t * kXferBlocks + e, 0u);
    }
    if (STACK && b < H / 16 && tid < kXferTokens * 4) {  // 8 words of each token's row
      uint64_t* d = reinterpret_cast<uint64_t*>(X.x_next + (size_t)(tid >> 2) * (kXferMaxH / 2) + 8 * b + 2 * (tid & 3));
      __hip_atomic_store(d, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };

  f32x4_t acc13[1 + NS];
  acc13[0] = acc_sh;
#pragma unroll
  for (int q = 1; q <= NS; ++q) acc13[q] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

  // 5. routed w13 jobs (slot j: 8 gate + 8 up rows of expert sid[j]) with P
  //    in flight; the routed w2 jobs (slot u: 16 rows of expert sid[u])
  //    follow the h slices
  uint4 q13[NS][N13];
  uint32_t s13[NS][N13];
  auto issue13 = [&](int j) __attribute__((always_inline)) {
    const long long e = L.sid[j];
    const uint8_t* sb = a.w13s + e * (2LL * I * (H / 32)) + (size_t)row13 * (H / 32) + w * (H / 256);
    load_scale_words<N13>(sb, s13[j]);
    const uint8_t* qb = a.w13c + e * (2LL * I * (H / 2)) + (size_t)row13 * (H / 2) + w * (H / 16) + g * 16;
#pragma unroll
    for (int i = 0; i < N13; ++i) q13[j][i] = *reinterpret_cast<const uint4*>(qb + i * 64);
  };
  uint4 q2[NS][N2];
  uint32_t s2[NS][N2];
  auto issue2 = [&](int u) __attribute__((always_inline)) {
    const long long e = L.sid[u];
    if constexpr (Q3) {  // piece i: block w*(I/256) + 4i + g of row n2 (12 bytes) and its scale
      const long long row = e * H + n2;
      const uint8_t* qb = a.w2c + row * (I / 32) * 12 + (size_t)(w * (I / 256) + g) * 12;
      const uint16_t* sb = reinterpret_cast<const uint16_t*>(a.w2s) + row * (I / 32) + w * (I / 256) + g;
#pragma unroll
      for (int i = 0; i < N2; ++i) {
        const uint32_t* c = reinterpret_cast<const uint32_t*>(qb + i * 48);
        q2[u][i] = make_uint4(c[0], c[1], c[2], 0u);
        s2[u][i] = sb[4 * i];
      }
    } else {
      const uint8_t* sb = a.w2s + e * ((long long)H * (I / 32)) + (size_t)n2 * (I / 32) + w * (I / 256);
      load_scale_words<N2>(sb, s2[u]);
      const uint8_t* qb = a.w2c + e * ((long long)H * (I / 2)) + (size_t)n2 * (I / 2) + w * (I / 16) + g * 16;
#pragma unroll
      for (int i = 0; i < N2; ++i) q2[u][i] = *reinterpret_cast<const uint4*>(qb + i * 64);
    }
  };
#pragma unroll
  for (int j = 0; j < P && j < NS; ++j) issue13(j);
  asm volatile("" ::: "memory");
  const unsigned char* bx = (r < TT ? reinterpret_cast<const unsigned char*>(L.xs + (size_t)r * H) : L.zero) +
                            (size_t)(w * (H / 8) + g * 32) * 2;
#pragma unroll
  for (int j = 0; j < NS; ++j) {
#pragma unroll
    for (int i = 0; i < N13; ++i) mx16_mfma(q13[j][i], (s13[j][i] >> (8 * g)) & 0xff, bx + i * 256, acc13[1 + j]);
    if (j + P < NS) issue13(j + P);
    asm volatile("" ::: "memory");
  }
  // the first routed w2 jobs, requested behind every w13 load: they arrive
  // while the block reduces and publishes its h slices, when the CU's loads
  // would otherwise pause
  constexpr int kEarly = NS < kEarlyW2 ? NS : kEarlyW2;
#pragma unroll
  for (int u = 0; u < kEarly; ++u) issue2(u);
  asm volatile("" ::: "memory");

  // 6. h slices: wave partials (the TT useful columns) -> LDS; wave 0 sums
  //    them in wave order, applies the clamped SwiGLU and publishes; then
  //    every wave requests its routed w2 weights
  if (r < TT) {
#pragma unroll
    for (int q = 0; q <= NS; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) L.red13[((q * kLayerWaves + w) * TT + r) * 16 + 4 * g + i] = acc13[q][i];
  }
  __syncthreads();
  if (w == 0) {
    for (int u = lane; u < (1 + NS) * TT * 4; u += 64) {
      const int q = u / (TT * 4), t = (u >> 2) % TT, p4 = u & 3;
      if (q > 0 && t != (q - 1) / KK) continue;  // slot q-1 belongs to one token
      float h2[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int i = 2 * p4 + hh;
        float gs = 0.0f, us = 0.0f;
#pragma unroll
        for (int v = 0; v < kLayerWaves; ++v) {
          gs += L.red13[((q * kLayerWaves + v) * TT + t) * 16 + i];
          us += L.red13[((q * kLayerWaves + v) * TT + t) * 16 + 8 + i];
        }
        if (q == 0) {
          gs *= shs[hh];
          us *= shs[2 + hh];
        }
        h2[hh] = swiglu_clamped(gs, us, a.limit);
      }
      uint32_t packed = (uint32_t)f32_to_bf16(h2[0]) | ((uint32_t)f32_to_bf16(h2[1]) << 16);
      if (!ok_route) packed = kNaNPair;
      const int col = q == 0 ? NS + t : q - 1;
      if (b < I / 8) store_agent(X.h + col * (kXferMaxI / 2) + 4 * gb + p4, packed ^ kHTag);
    }
  }
  __syncthreads();  // the h stores are requested before the other routed w2 loads of this CU
#pragma unroll
  for (int u = kEarly; u < NS; ++u) issue2(u);
  asm volatile("" ::: "memory");
  // the other buffers and the layer count are nobody's in this layer: done
  // here, off the tail (at the end they held up the last block's exit)
  zero_next();
  if constexpr (!STACK) {
    for (int i = tid; i < (kXferBlocks + NB - 1) / NB; i += kLayerThreads) {
      const int bb = b + NB * i;
      if (bb < kXferBlocks) store_agent(X.epoch + bb, ep + 1);
    }
  }

  // the early routed w2 jobs' weights, converted to bf16 while the other
  // blocks' h slices are awaited (they arrived before the h publish; the
  // w2 MFMAs after the wait are bound by these converts, four per MFMA)
  constexpr int kPre = NS <= 6 ? kEarly : 0;  // registers allow it for one token
  bf16x8_t c2[kPre > 0 ? kPre : 1][N2][4];
#pragma unroll
  for (int u = 0; u < kPre; ++u)
#pragma unroll
    for (int i = 0; i < N2; ++i) {
      if constexpr (Q3) {
        float lv[8];
        slot_levels(u, lv);
        const Q3Book bk = q3_book(lv, f16_bits_to_f32(s2[u][i]));
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          c2[u][i][m] = q3_frag(q2[u][i].x, q2[u][i].y, q2[u][i].z, m, bk);
          asm volatile("" : "+v"(c2[u][i][m]));
        }
      } else {
        const float sc = e8m0_scale_operand((s2[u][i] >> (8 * g)) & 0xff);
        const uint32_t d[4] = {q2[u][i].x, q2[u][i].y, q2[u][i].z, q2[u][i].w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          c2[u][i][m] = fp4x8_to_bf16x8(d[m], sc);
          asm volatile("" : "+v"(c2[u][i][m]));
        }
      }
    }

  // the shared w2 weights too (int8, in registers since the start)
  bf16x8_t cs2[kPre > 0 ? N2I : 1][2];
  if constexpr (kPre > 0) {
#pragma unroll
    for (int i = 0; i < N2I; ++i) {
      cs2[i][0] = i8x8_to_bf16x8(qs2[i].x, qs2[i].y);
      cs2[i][1] = i8x8_to_bf16x8(qs2[i].z, qs2[i].w);
      asm volatile("" : "+v"(cs2[i][0]), "+v"(cs2[i][1]));
    }
  }

  // 7. every block's h slices: poll the columns into LDS. A piece whose four
  //    words are all in is kept and not read again (the polls of 256 blocks
  //    compete with the w2 weight stream for the memory system)
  {
    constexpr int n16 = I / 8;
    constexpr int nact = NCOL * n16;
    constexpr int PER = (nact + kLayerThreads - 1) / kLayerThreads;
    u32x4_t v[PER];
    bool got[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) got[i] = false;
    int spins = 0;
    while (true) {
      bool rdy = true;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        if (!got[i]) {
          const int ii = min(tid + i * kLayerThreads, nact - 1);
          const int c = ii / n16, o = ii - c * n16;
          v[i] = load_agent_u32x4(X.h + c * (kXferMaxI / 2) + 4 * o);
          got[i] = v[i][0] != 0 && v[i][1] != 0 && v[i][2] != 0 && v[i][3] != 0;
        }
        rdy = rdy && got[i];
      }
      if (rdy) break;
      if (++spins >= kPollLimit) {
        L.flag[1] = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int ii = tid + i * kLayerThreads;
      if (ii < nact) {
        const int c = ii / n16, o = ii - c * n16;
        *reinterpret_cast<u32x4_t*>(L.hl + (size_t)c * HROW + o * 16) = v[i] ^ kHTag;
      }
    }
  }
  // stack: this thread's zeroing stores are complete (the w2 weights, needed
  // next, are in too) before the barrier that precedes the output
  if constexpr (STACK) __builtin_amdgcn_s_waitcnt((15 << 8) | (7 << 4));  // vmcnt(0)
  __syncthreads();
  const bool ok = ok_route && L.flag[1] == 0;

  // 8. w2: column u < NS is slot u's h, column NS + t token t's shared h;
  //    four accumulators, so that the MFMAs do not wait for each other
  f32x4_t acc2[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc2[c] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    const unsigned char* bsrc = (r == u ? L.hl + (size_t)u * HROW : L.zero) + (size_t)(w * (I / 8) + g * 32) * 2;
#pragma unroll
    for (int i = 0; i < N2; ++i) {
      if (u < kPre) {
#pragma unroll
        for (int m = 0; m < 4; ++m)
          acc2[(u * N2 + i) & 3] = mfma_16x16x32(c2[u][i][m], *reinterpret_cast<const bf16x8_t*>(bsrc + i * 256 + m * 16),
                                                 acc2[(u * N2 + i) & 3]);
      } else {
        if constexpr (Q3) {
          float lv[8];
          slot_levels(u, lv);
          q3_16_mfma(q2[u][i], s2[u][i], lv, bsrc + i * 256, acc2[(u * N2 + i) & 3]);
        } else {
          mx16_mfma(q2[u][i], (s2[u][i] >> (8 * g)) & 0xff, bsrc + i * 256, acc2[(u * N2 + i) & 3]);
        }
      }
    }
  }
  {
    const unsigned char* bsrc = (r >= NS && r < NCOL ? L.hl + (size_t)r * HROW : L.zero) +
                                (size_t)(w * (I / 8) + g * 16) * 2;
#pragma unroll
    for (int i = 0; i < N2I; ++i) {
      if constexpr (kPre > 0) {
        acc2[i & 3] = mfma_16x16x32(cs2[i][0], *reinterpret_cast<const bf16x8_t*>(bsrc + i * 128), acc2[i & 3]);
        acc2[i & 3] = mfma_16x16x32(cs2[i][1], *reinterpret_cast<const bf16x8_t*>(bsrc + i * 128 + 16), acc2[i & 3]);
      } else {
        i816_mfma(qs2[i], bsrc + i * 128, acc2[i & 3]);
      }
    }
  }
  L.red2[w * 64 + lane] = (acc2[0] + acc2[1]) + (acc2[2] + acc2[3]);
  __syncthreads();
  if (tid < NCOL * 16) {  // y[rr][c] summed over the waves in wave order
    const int c = tid >> 4, rr = tid & 15;
    float s = 0.0f;
#pragma unroll
    for (int v = 0; v < kLayerWaves; ++v) s += L.red2[v * 64 + c + 16 * (rr >> 2)][rr & 3];
    L.ycol[rr * 16 + c] = s;
  }
  __syncthreads();
  if (STACK && publish) {
    if (tid < TT * 8) {  // thread (t, q): output rows 16ob + 2q, + 1 of token t, as one tagged pair
      const int t = tid >> 3, q = tid & 7;
      float o2[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int rr = 2 * q + hh;
        float o = 0.0f;
#pragma unroll
        for (int j = 0; j < KK; ++j) o += L.sw[t * KK + j] * L.ycol[rr * 16 + t * KK + j];
        o += s2p[hh] * L.ycol[rr * 16 + NS + t];
        o2[hh] = o;
      }
      uint32_t packed = (uint32_t)f32_to_bf16(o2[0]) | ((uint32_t)f32_to_bf16(o2[1]) << 16);
      if (!ok) packed = kNaNPair;  // a hand-off timed out: never a silent wrong value
      if (!ok && tid == 0 && a.flags) atomicOr(a.flags, kFlagWaitExpired);
      if (b < H / 16) {
        store_agent(X.x_next + (size_t)t * (kXferMaxH / 2) + 8 * ob + q, packed ^ kHTag);
        reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.out) + (size_t)t * H + 16 * ob)[q] = packed;
      }
    }
  } else if (tid < TT * 16) {  // thread (t, rr): output row 16ob + rr of token t
    const int t = tid >> 4, rr = tid & 15;
    const int n = 16 * ob + rr;
    float o = 0.0f;
#pragma unroll
    for (int j = 0; j < KK; ++j) o += L.sw[t * KK + j] * L.ycol[rr * 16 + t * KK + j];
    o += s2n * L.ycol[rr * 16 + NS + t];
    if (!ok) o = __builtin_nanf("");  // a hand-off timed out: never a silent wrong value
    if (!ok && tid == 0 && a.flags) atomicOr(a.flags, kFlagWaitExpired);
    if (b < H / 16) {
      if (a.out_is_fp32) static_cast<float*>(a.out)[(size_t)t * H + n] = o;
      else static_cast<uint16_t*>(a.out)[(size_t)t * H + n] = f32_to_bf16(o);
    }
  }
}

template <int NH, int NI, int TT, int KK, bool Q3>
__global__ __launch_bounds__(kLayerThreads) void k_layer_small(LayerArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  const LayerBlock<NH, NI, TT, KK> L(a, lds);
  const uint32_t ep = load_agent(a.xfer + blockIdx.x);  // this block's calls so far
  const Xfer X(a.xfer, ep & 1);
  uint4 qs2[2 * NI];
  const f32x4_t acc_sh = layer_head(a, L, X, qs2);
  layer_tail<NH, NI, TT, KK, Q3>(a, L, X, ep, acc_sh, qs2);
}

// Layers run back to back in one launch (a stack at T <= 2): layer j of the
// launch uses the hand-off buffers of parity (layers so far + j) & 1, takes
// its input rows from the previous layer through them (the first from its
// x) and publishes its output rows the same way (the last one only writes
// its out).
template <int NH, int NI, int TT, int KK>
__global__ __launch_bounds__(kLayerThreads) void k_layer_stack(StackArgs sa) {
  extern __shared__ __align__(16) unsigned char lds[];
  const uint32_t* xfer = sa.layer[0].xfer;
  const uint32_t ep = load_agent(xfer + blockIdx.x);  // this block's layers so far
  const int n = sa.n;
  for (int j = 0; j < n; ++j) {
    const LayerArgs& a = sa.layer[j];
    // per-lane values from an opaque copy of the thread index, recomputed per
    // layer: hoisted out of the loop they stay live across it and spill
    int thread;
    asm volatile("v_mov_b32 %0, %1" : "=v"(thread) : "v"((int)threadIdx.x));
    const LayerBlock<NH, NI, TT, KK> L(a, lds, thread);
    const Xfer X(a.xfer, (ep + j) & 1);
    uint4 qs2[2 * NI];
    const f32x4_t acc_sh = layer_head(a, L, X, qs2, j > 0);
    layer_tail<NH, NI, TT, KK, false, true>(a, L, X, ep + j, acc_sh, qs2, j + 1 < n);
    __syncthreads();  // the next layer reuses the LDS
  }
  // count the layers for blocks b, b+NB, .. (every count in step)
  const Xfer X(sa.layer[0].xfer, 0);
  for (int i = threadIdx.x; i < (kXferBlocks + (int)gridDim.x - 1) / (int)gridDim.x; i += kLayerThreads) {
    const int bb = blockIdx.x + gridDim.x * i;
    if (bb < kXferBlocks) store_agent(X.epoch + bb, ep + n);
  }
}

namespace {

using LayerKernel = void (*)(LayerArgs);
using StackKernel = void (*)(StackArgs);

// LDS asked for: at least 81 KB of the CU's 160 KB, so that one block holds
// a CU (the design is one block per CU; two on one CU would leave another
// idle).
template <int NH, int NI, int TT, int KK>
LayerKernel pick(size_t* lds, bool q3) {
  *lds = std::max(LayerShape<NH, NI, TT, KK>::lds_bytes, (size_t)81 * 1024);
  return q3 ? &k_layer_small<NH, NI, TT, KK, true> : &k_layer_small<NH, NI, TT, KK, false>;
}

LayerKernel layer_kernel(int H, int I, int T, int k, size_t* lds, bool q3) {
  if (k != 6) return nullptr;
  if (H == 4096 && I == 2048)
    return T == 1 ? pick<4, 2, 1, 6>(lds, q3) : T == 2 ? pick<4, 2, 2, 6>(lds, q3) : nullptr;
  if (H == 2048 && I == 1024)
    return T == 1 ? pick<2, 1, 1, 6>(lds, q3) : T == 2 ? pick<2, 1, 2, 6>(lds, q3) : nullptr;
  return nullptr;
}

// Blocks of kernel k that the current device holds at once (0 if unknown),
// cached per device and kernel.
int resident_blocks(const void* k, size_t lds) {
  constexpr int kDev = 16, kKern = 16;
  static const void* seen[kDev][kKern];
  static int count[kDev][kKern];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDev) return 0;
  for (int i = 0; i < kKern; ++i)
    if (seen[dev][i] == k) return count[dev][i];
  if (lds > 64 * 1024 && hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
    return 0;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, kLayerThreads, lds) !=
          hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  for (int i = 0; i < kKern; ++i)
    if (!seen[dev][i]) {
      seen[dev][i] = k;
      count[dev][i] = per_cu * cus;
      break;
    }
  return per_cu * cus;
}

int layer_grid(int H, int I, int E) { return std::max(E, std::max(I / 8, H / 16)); }

template <int NH, int NI, int TT, int KK>
StackKernel pick_stack(size_t* lds) {
  *lds = std::max(LayerShape<NH, NI, TT, KK>::lds_bytes, (size_t)81 * 1024);
  return &k_layer_stack<NH, NI, TT, KK>;
}

StackKernel stack_kernel(int H, int I, int T, int k, size_t* lds) {
  if (k != 6) return nullptr;
  if (H == 4096 && I == 2048)
    return T == 1 ? pick_stack<4, 2, 1, 6>(lds) : T == 2 ? pick_stack<4, 2, 2, 6>(lds) : nullptr;
  if (H == 2048 && I == 1024)
    return T == 1 ? pick_stack<2, 1, 1, 6>(lds) : T == 2 ? pick_stack<2, 1, 2, 6>(lds) : nullptr;
  return nullptr;
}

}  // namespace

bool layer_small_supported(int H, int I, int E, int T, int k, bool w2q3) {
  size_t lds = 0;
  LayerKernel kern = layer_kernel(H, I, T, k, &lds, w2q3);
  if (!kern || E < k || E > 256) return false;
  const int grid = layer_grid(H, I, E);
  return grid <= kXferBlocks && resident_blocks(reinterpret_cast<const void*>(kern), lds) >= grid;
}

hipError_t launch_layer_small(const LayerArgs& a, hipStream_t st) {
  size_t lds = 0;
  LayerKernel kern = layer_kernel(a.H, a.I, a.T, a.k, &lds, a.w2q3 != 0);
  if (!kern) return hipErrorInvalidValue;
  const int grid = layer_grid(a.H, a.I, a.E);
  if (grid > kXferBlocks || resident_blocks(reinterpret_cast<const void*>(kern), lds) < grid) return hipErrorInvalidValue;
  kern<<<grid, kLayerThreads, lds, st>>>(a);
  return hipGetLastError();
}

bool layer_stack_supported(int H, int I, int E, int T, int k) {
  size_t lds = 0;
  StackKernel kern = stack_kernel(H, I, T, k, &lds);
  if (!kern || E < k || E > 256) return false;
  const int grid = layer_grid(H, I, E);
  return grid <= kXferBlocks && resident_blocks(reinterpret_cast<const void*>(kern), lds) >= grid;
}

hipError_t launch_layer_stack(const StackArgs& sa, hipStream_t st) {
  if (sa.n < 1 || sa.n > kStackChunk) return hipErrorInvalidValue;
  const LayerArgs& a = sa.layer[0];
  for (int j = 1; j < sa.n; ++j)  // one shape and one hand-off region for every layer of the launch
    if (sa.layer[j].T != a.T || sa.layer[j].H != a.H || sa.layer[j].I != a.I || sa.layer[j].E != a.E ||
        sa.layer[j].k != a.k || sa.layer[j].xfer != a.xfer || sa.layer[j].w2q3)
      return hipErrorInvalidValue;
  size_t lds = 0;
  StackKernel kern = stack_kernel(a.H, a.I, a.T, a.k, &lds);
  if (!kern || a.w2q3) return hipErrorInvalidValue;
  const int grid = layer_grid(a.H, a.I, a.E);
  if (grid > kXferBlocks || resident_blocks(reinterpret_cast<const void*>(kern), lds) < grid)
    return hipErrorInvalidValue;
  kern<<<grid, kLayerThreads, lds, st>>>(sa);
  return hipGetLastError();
}

}  // namespace moe
