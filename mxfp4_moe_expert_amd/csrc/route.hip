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
//
// Decode sizes (T <= kSmallT) use two launches. The logits, scores and
// selection values come from k_router_dec (blocks of 4 experts x 8 tokens,
// the tokens staged in LDS) or, for one or two tokens, from k_router_small
// (one block per expert, sharing its launch with the shared expert's w13
// blocks, which do not depend on the routing). Then k_topk_dec selects the
// experts of every token, one wave per token over many blocks, and the last
// block to finish builds the permutation and the expert tile table.
#include "device.h"
#include "internal.h"
#include "skinny.h"

namespace moe {

// ---------------------------------------------------------------- small-T router

// Score and selection value of (token t, expert e) from its logit, computed
// once here so that every top-k reader only compares.
__device__ __forceinline__ void store_score(const RouterArgs& a, int t, int e, float logit) {
  const float sc = sqrtf(softplus(logit));
  a.scores[(size_t)t * a.E + e] = sc;
  a.keys[(size_t)t * a.E + e] = sc + (a.bias ? a.bias[e] : 0.0f);  // no bias on hash layers
}

// Logits of expert e for 8 < T <= kSmallT tokens, H <= 4096: wave w takes
// tokens w, w + 8, ...; lane l holds elements 512 c + 8 l .. +8 (c < H/512)
// of the expert's router row in registers and reduces one token at a time.
__device__ __forceinline__ void router_logits_waves(const RouterArgs& a, int e) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int H = a.H;
  const float* we = a.gate_w + (size_t)e * H;
  float4 w[16];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int k0 = c * 512 + lane * 8;
    const bool ok = k0 < H;
    w[2 * c] = ok ? *reinterpret_cast<const float4*>(we + k0) : make_float4(0.f, 0.f, 0.f, 0.f);
    w[2 * c + 1] = ok ? *reinterpret_cast<const float4*>(we + k0 + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const float off = a.logit_offset ? a.logit_offset[e] : 0.0f;
  for (int t = wave; t < a.T; t += kWaves) {
    const uint16_t* xt = a.x + (size_t)t * H;
    float acc = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int k0 = c * 512 + lane * 8;
      if (k0 < H) {
        const uint4 xv = *reinterpret_cast<const uint4*>(xt + k0);
        const float4 w0 = w[2 * c], w1 = w[2 * c + 1];
        acc += bf16_to_f32(xv.x & 0xffff) * w0.x;
        acc += bf16_to_f32(xv.x >> 16) * w0.y;
        acc += bf16_to_f32(xv.y & 0xffff) * w0.z;
        acc += bf16_to_f32(xv.y >> 16) * w0.w;
        acc += bf16_to_f32(xv.z & 0xffff) * w1.x;
        acc += bf16_to_f32(xv.z >> 16) * w1.y;
        acc += bf16_to_f32(xv.w & 0xffff) * w1.z;
        acc += bf16_to_f32(xv.w >> 16) * w1.w;
      }
    }
    const float v = wave_sum(acc);
    if (lane == 0) store_score(a, t, e, v + off);
  }
}

__device__ __forceinline__ void router_logits_block(const RouterArgs& a, int e, unsigned char* lds) {
  if (a.T > 8 && a.H <= 4096) {
    router_logits_waves(a, e);
    return;
  }
  float* red = reinterpret_cast<float*>(lds);  // [kWaves][kSmallT]
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int H = a.H;
  const float* we = a.gate_w + (size_t)e * H;
  for (int t0 = 0; t0 < a.T; t0 += 8) {
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
    for (int k0 = tid * 8; k0 < H; k0 += kThreads * 8) {
      const float4 w0 = *reinterpret_cast<const float4*>(we + k0);
      const float4 w1 = *reinterpret_cast<const float4*>(we + k0 + 4);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (t0 + q < a.T) {
          const uint4 xv = *reinterpret_cast<const uint4*>(a.x + (size_t)(t0 + q) * H + k0);
          float s = acc[q];
          s += bf16_to_f32(xv.x & 0xffff) * w0.x;
          s += bf16_to_f32(xv.x >> 16) * w0.y;
          s += bf16_to_f32(xv.y & 0xffff) * w0.z;
          s += bf16_to_f32(xv.y >> 16) * w0.w;
          s += bf16_to_f32(xv.z & 0xffff) * w1.x;
          s += bf16_to_f32(xv.z >> 16) * w1.y;
          s += bf16_to_f32(xv.w & 0xffff) * w1.z;
          s += bf16_to_f32(xv.w >> 16) * w1.w;
          acc[q] = s;
        }
      }
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (t0 + q < a.T) {
        const float v = wave_sum(acc[q]);
        if (lane == 0) red[wave * kSmallT + t0 + q] = v;
      }
    }
  }
  __syncthreads();
  const float off = a.logit_offset ? a.logit_offset[e] : 0.0f;
  for (int t = tid; t < a.T; t += kThreads) {
    const float* v = red + t;
    const float sum = ((v[0] + v[kSmallT]) + (v[2 * kSmallT] + v[3 * kSmallT])) +
                      ((v[4 * kSmallT] + v[5 * kSmallT]) + (v[6 * kSmallT] + v[7 * kSmallT]));
    store_score(a, t, e, sum + off);
  }
}

// Blocks [0, E): router logits of expert blockIdx.x for all T <= kSmallT
// tokens; blocks [E, E + shared_blocks): shared-expert w13 + SwiGLU in slim
// blocks (8 gate + 8 up rows), so that with E = 256 every CU gets about the
// same bytes. NS super-steps per wave; EXACT when K = 128 * NS * kWaves.
template <int NS, bool EXACT>
__global__ __launch_bounds__(kThreads) void k_router_small(RouterArgs a, SkinnyArgs sh, int has_shared) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int b = blockIdx.x;
  if (b < a.E) {
    router_logits_block(a, b, lds);
  } else if (has_shared) {
    skinny_block<kFmtI8, kW13, kWaves, NS, EXACT, true>(sh, b - a.E, lds);
  }
}

// Logits of experts 8 bx .. 8 bx + 7 (one per wave) for tokens 8 by .. +7,
// H = 512 NC (NC = 2, 4 or 8): the block stages the token rows in LDS in one
// round of loads; each wave keeps its expert's router row in registers
// (lane l: elements 512 c + 8 l .. +8), forms the lane partials of all 8
// tokens at once (the products of a token in the order of
// router_logits_waves), reduces them over the wave, and lane q then takes
// the score of token q.
constexpr int kDecExperts = 8, kDecTokens = 8;

template <int NC>
__global__ __launch_bounds__(kDecExperts * 64) void k_router_dec(RouterArgs a) {
  constexpr int H = NC * 512;
  __shared__ __align__(16) uint16_t xs[kDecTokens * H];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int e = blockIdx.x * kDecExperts + wave;  // surplus waves compute, never store
  const int t0 = blockIdx.y * kDecTokens, nt = min(kDecTokens, a.T - t0);
  const float* we = a.gate_w + (size_t)min(e, a.E - 1) * H;
  float4 w[2 * NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    w[2 * c] = *reinterpret_cast<const float4*>(we + c * 512 + lane * 8);
    w[2 * c + 1] = *reinterpret_cast<const float4*>(we + c * 512 + lane * 8 + 4);
  }
  constexpr int n16 = H / 8, npieces = kDecTokens * n16;  // 16-byte pieces of the 8 rows
  constexpr int per = npieces / (kDecExperts * 64);
  uint4 v[per];
#pragma unroll
  for (int j = 0; j < per; ++j) {  // rows past the batch repeat its last one (never used)
    const int i = tid + kDecExperts * 64 * j;
    v[j] = *reinterpret_cast<const uint4*>(a.x + (size_t)(t0 + min(i / n16, nt - 1)) * H + (i % n16) * 8);
  }
#pragma unroll
  for (int j = 0; j < per; ++j) *reinterpret_cast<uint4*>(xs + (size_t)(tid + kDecExperts * 64 * j) * 8) = v[j];
  __syncthreads();
  // token t's row pieces are read from LDS while token t-1's products are
  // formed (a scheduling barrier keeps the reads there: left alone, the
  // compiler requested two pieces at a time and waited for each pair)
  float acc[kDecTokens];
  uint4 xb[2][NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) xb[0][c] = *reinterpret_cast<const uint4*>(xs + c * 512 + lane * 8);
#pragma unroll
  for (int t = 0; t < kDecTokens; ++t) {
    if (t + 1 < kDecTokens) {
#pragma unroll
      for (int c = 0; c < NC; ++c)
        xb[(t + 1) & 1][c] = *reinterpret_cast<const uint4*>(xs + (t + 1) * H + c * 512 + lane * 8);
    }
    __builtin_amdgcn_sched_barrier(0);
    acc[t] = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const uint4 xv = xb[t & 1][c];
      const float4 w0 = w[2 * c], w1 = w[2 * c + 1];
      float s = acc[t];
      s += bf16_to_f32(xv.x & 0xffff) * w0.x;
      s += bf16_to_f32(xv.x >> 16) * w0.y;
      s += bf16_to_f32(xv.y & 0xffff) * w0.z;
      s += bf16_to_f32(xv.y >> 16) * w0.w;
      s += bf16_to_f32(xv.z & 0xffff) * w1.x;
      s += bf16_to_f32(xv.z >> 16) * w1.y;
      s += bf16_to_f32(xv.w & 0xffff) * w1.z;
      s += bf16_to_f32(xv.w >> 16) * w1.w;
      acc[t] = s;
    }
  }
  // transposed reduction of the 8 token partials over the wave: each
  // exchange halves the values a lane holds (8 -> 4 -> 2 -> 1 at lane
  // distances 32, 16, 8), then 4, 2, 1 finish one token per group of 8
  // lanes (11 shuffles in place of 8 x 6)
  const bool h32 = lane & 32, h16 = lane & 16, h8 = lane & 8;
  float b4[4], b2[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float keep = h32 ? acc[i + 4] : acc[i], send = h32 ? acc[i] : acc[i + 4];
    b4[i] = keep + __shfl_xor(send, 32);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float keep = h16 ? b4[i + 2] : b4[i], send = h16 ? b4[i] : b4[i + 2];
    b2[i] = keep + __shfl_xor(send, 16);
  }
  float b1 = (h8 ? b2[1] : b2[0]) + __shfl_xor(h8 ? b2[0] : b2[1], 8);
  b1 += __shfl_xor(b1, 4);
  b1 += __shfl_xor(b1, 2);
  b1 += __shfl_xor(b1, 1);
  // lane l holds token (l >> 3) & 7; lane q < 8 takes token q from lane 8q
  const float mine = __shfl(b1, (lane & 7) * 8);
  if (e < a.E && lane < nt) store_score(a, t0 + lane, e, mine + (a.logit_offset ? a.logit_offset[e] : 0.0f));
}

// Top-k of every token, one wave per token (4 per block); then the last
// block to finish (an arrival count in the workspace, which it sets back to
// zero) makes the stable counting sort of the T*k <= 512 slots, the expert
// tile table and the tile records of the streaming passes, and zeroes their
// counters. Stable ranks come from per-expert slot bitmasks: the
// rank of slot i among the slots of its expert is the number of set bits
// below bit i of that expert's mask.
constexpr int kTopkThreads = 256;
constexpr int kMaskWords = kSmallT * kMaxTopK / 64;  // 64-bit words per expert mask

__global__ __launch_bounds__(kTopkThreads) void k_topk_dec(RouterArgs a, Perm p, int* arrivals) {
  __shared__ unsigned long long mask[kMaxExperts][kMaskWords];
  __shared__ int first[kMaxExperts], count[kMaxExperts], tile0[kMaxExperts];
  __shared__ int scan_tmp[kTopkThreads];
  __shared__ int is_last;
  const int tid = threadIdx.x;
  const int t = blockIdx.x * (kTopkThreads / 64) + (tid >> 6);
  // ids and weights are written through to memory; each wave waits for its
  // stores before the block is counted, and the last block reads them with
  // coherent loads (no cache write-back or invalidation: the fences that
  // did this cost about 1.5 us)
  if (t < a.T) {
    if (a.tid2eid) {  // hash layer: the token's table row instead of the top-k
      const int tok = __builtin_amdgcn_readfirstlane(a.token_ids[t]);
      const bool tok_ok = (unsigned)tok < (unsigned)a.V;
      if (!tok_ok && (tid & 63) == 0 && a.flags) atomicOr(a.flags, kFlagTokenId);
      const float* srow = a.scores + (size_t)t * a.E;
      wave_hash_row<true>(topk_load(srow, srow, a.E), tok_ok ? a.tid2eid + (size_t)tok * a.k : nullptr, a.E, a.k,
                          a.scale, a.ids + (size_t)t * a.k, a.w + (size_t)t * a.k, nullptr, a.flags);
    } else {
      wave_topk<true>(a.scores + (size_t)t * a.E, a.keys + (size_t)t * a.E, a.E, a.k, a.scale,
                      a.ids + (size_t)t * a.k, a.w + (size_t)t * a.k, nullptr);
    }
  }
  __builtin_amdgcn_s_waitcnt((15 << 8) | (7 << 4));  // vmcnt(0): this wave's stores are done
  __syncthreads();
  if (tid == 0) is_last = atomicAdd(arrivals, 1) == (int)gridDim.x - 1;
  __syncthreads();
  if (!is_last) return;

  // the thread's slots (tid, tid + 256; T*k <= 512): expert and weight, read once
  constexpr int kPer = kSmallT * kMaxTopK / kTopkThreads;
  const int n = a.T * a.k;
  int es[kPer];
  float ws[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = min(tid + j * kTopkThreads, n - 1);
    es[j] = (int)load_agent(reinterpret_cast<const uint32_t*>(a.ids) + i);
    ws[j] = __uint_as_float(load_agent(reinterpret_cast<const uint32_t*>(a.w) + i));
  }
  unsigned long long* mflat = &mask[0][0];
  for (int i = tid; i < kMaxExperts * kMaskWords; i += kTopkThreads) mflat[i] = 0ull;
  __syncthreads();
  const int words = (n + 63) >> 6;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = tid + j * kTopkThreads;
    if (i < n) atomicOr(&mask[es[j]][i >> 6], 1ull << (i & 63));
  }
  __syncthreads();
  int c = 0;
  if (tid < a.E)
    for (int w = 0; w < words; ++w) c += __popcll(mask[tid][w]);
  // one scan for both prefixes: slots in the low 16 bits, tiles in the high
  // (at most 512 of either); expert e's tiles are at most tile_n consecutive
  // sorted positions each, in expert order
  const int nt = (c + p.tile_n - 1) / p.tile_n;
  int total;
  const int both = block_exclusive_scan(c | (nt << 16), scan_tmp, &total);
  const int off = both & 0xffff, toff = both >> 16;
  if (tid < a.E) {
    p.offsets[tid] = off;
    first[tid] = off;
    count[tid] = c;
    tile0[tid] = toff;
    for (int i = 0; i < nt; ++i) {
      const int f = i * p.tile_n;
      p.tile_info[toff + i] = make_int4(tid, off + f, min(p.tile_n, c - f), 0);
    }
  }
  if (tid == 0) {
    p.offsets[a.E] = total & 0xffff;
    *p.n_tiles = total >> 16;
  }
  __syncthreads();
  // every slot: its sorted position, and its column of its tile's record
  // (the tile's first column also writes the record's head)
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = tid + j * kTopkThreads;
    if (i >= n) continue;
    const int e_i = es[j];
    const float wv = ws[j];
    const int wi = i >> 6;
    int rank = __popcll(mask[e_i][wi] & ((1ull << (i & 63)) - 1ull));
    for (int w = 0; w < wi; ++w) rank += __popcll(mask[e_i][w]);
    const int pos = first[e_i] + rank;
    p.sorted_slots[pos] = i;
    p.slot_pos[i] = pos;
    p.sorted_tok[pos] = i / a.k;
    const int tl = rank / p.tile_n, col = rank - tl * p.tile_n;
    const int ncols = min(p.tile_n, count[e_i] - tl * p.tile_n);
    int* rec = p.tile_rec + (size_t)(tile0[e_i] + tl) * kRecInts;
    if (col == 0) {
      rec[0] = e_i;
      rec[1] = pos;
      rec[2] = ncols;
      rec[3] = 0;
    }
    rec[4 + col] = i / a.k;
    rec[20 + col] = i;
    rec[36 + col] = __float_as_int(wv);
  }
  for (int i = tid; i < p.max_tiles + kSmallT; i += kTopkThreads) p.done[i] = 0;
  if (tid == 0) {
    *arrivals = 0;  // ready for the next call
    p.queues[0] = 0;
    p.queues[1] = 0;
  }
}

// The large-T learned router is in router_mfma.hip.

// ---------------------------------------------------------------- hash router

// One wave per token: ids from the table row, scores of those experts only.
// NC = ceil(H / 512): lane l holds elements 512 c + 8 l .. +8 (c < NC) of the
// token row and of one expert's router row. The k table entries come in one
// load (lane j < k reads entry j), and each expert's row pieces are requested
// together, the next expert's before this one's products are formed (one
// expert at a time when NC > 8: two rows of 16 pieces would not fit the
// registers). Before, the loop over a run-time H and the per-expert table
// loads made about 50 dependent memory round trips per wave (47 us at 4096
// tokens). The products are added in the same order as before; lanes past H
// add zeros.
template <int NC>
__global__ __launch_bounds__(256) void k_hash_route(HashArgs a) {
  constexpr int NB = NC <= 8 ? 2 : 1;  // router rows in flight
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= a.T) return;
  const int H = a.H, k = a.k;
  // a token id outside [0, V) or a table entry outside [0, E) is flagged;
  // the token then reads table row 0 / router row 0 (nothing is indexed out
  // of range), keeps in-range ids and gets NaN weights
  const int tok = a.token_ids[t];
  const bool tok_ok = (unsigned)tok < (unsigned)a.V;
  const int32_t* row = a.tid2eid + (size_t)(tok_ok ? tok : 0) * k;
  const int my_e = lane < k ? row[lane] : 0;
  const uint16_t* xt = a.x + (size_t)t * H;
  // pieces past H (H a multiple of 128, not of 512) read in-range addresses
  // and take zero activations, so every load is unconditional (per-lane
  // branches around them made the compiler wait for every load at each one)
  // and the extra products add zeros
  uint4 xv[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int k0 = c * 512 + lane * 8;
    const uint4 v = *reinterpret_cast<const uint4*>(xt + min(k0, H - 8));
    xv[c] = k0 < H ? v : make_uint4(0u, 0u, 0u, 0u);
  }
  int ids[kMaxTopK];
  bool ent_ok = true;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    ids[j] = 0;
    if (j >= k) continue;  // uniform
    const int e = __builtin_amdgcn_readlane(my_e, j);
    const bool e_ok = (unsigned)e < (unsigned)a.E;
    ent_ok = ent_ok && e_ok;
    ids[j] = e_ok ? e : 0;
  }
  float4 wr[NB][NC][2];
  auto request = [&](int j, float4 (&w)[NC][2]) __attribute__((always_inline)) {
    const float* we = a.gate_w + (size_t)ids[j] * H;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int k0 = min(c * 512 + lane * 8, H - 8);
      w[c][0] = *reinterpret_cast<const float4*>(we + k0);
      w[c][1] = *reinterpret_cast<const float4*>(we + k0 + 4);
    }
  };
  request(0, wr[0]);
  float s[kMaxTopK];
  float sum = 0.0f;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    s[j] = 0.0f;
    if (j >= k) continue;
    if (NB == 2 && j + 1 < k) request(j + 1, wr[(j + 1) % NB]);
    __builtin_amdgcn_sched_barrier(0);
    float acc = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const uint4 x = xv[c];
      const float4 w0 = wr[j % NB][c][0], w1 = wr[j % NB][c][1];
      acc += bf16_to_f32(x.x & 0xffff) * w0.x;
      acc += bf16_to_f32(x.x >> 16) * w0.y;
      acc += bf16_to_f32(x.y & 0xffff) * w0.z;
      acc += bf16_to_f32(x.y >> 16) * w0.w;
      acc += bf16_to_f32(x.z & 0xffff) * w1.x;
      acc += bf16_to_f32(x.z >> 16) * w1.y;
      acc += bf16_to_f32(x.w & 0xffff) * w1.z;
      acc += bf16_to_f32(x.w >> 16) * w1.w;
    }
    if (NB == 1 && j + 1 < k) request(j + 1, wr[0]);
    s[j] = sqrtf(softplus(wave_sum(acc)));
    sum += s[j];
  }
  const bool ok = tok_ok && ent_ok;
  if (!ok && lane == 0 && a.flags) atomicOr(a.flags, (tok_ok ? 0u : kFlagTokenId) | (ent_ok ? 0u : kFlagTableEntry));
  if (lane < k) {
    float sj = s[0];
    int ej = ids[0];
#pragma unroll
    for (int j = 1; j < kMaxTopK; ++j)
      if (j == lane) {
        sj = s[j];
        ej = ids[j];
      }
    a.ids[(size_t)t * k + lane] = ej;
    a.w[(size_t)t * k + lane] = ok ? a.scale * sj / sum : __builtin_nanf("");
  }
}

// ---------------------------------------------------------------- launchers

template <class K>
static hipError_t allow_lds(K kernel, size_t bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)bytes);
}

hipError_t launch_router_small(const RouterArgs& r, const SkinnyArgs* sh, int shared_blocks, hipStream_t st) {
  if (r.T <= 0) return hipSuccess;
  size_t lds = (size_t)kWaves * kSmallT * sizeof(float);
  SkinnyArgs s{};
  if (sh) {
    s = *sh;
    const size_t l2 = skinny_lds_bytes(s.tile_n, s.K, kW13, kWaves);
    lds = l2 > lds ? l2 : lds;
  } else {
    shared_blocks = 0;
  }
  auto kern = s.K == 1024   ? &k_router_small<1, true>
              : s.K == 2048 ? &k_router_small<2, true>
              : s.K == 4096 ? &k_router_small<4, true>
                            : &k_router_small<4, false>;
  hipError_t e = allow_lds(kern, lds);
  if (e != hipSuccess) return e;
  kern<<<r.E + shared_blocks, kThreads, lds, st>>>(r, s, sh ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_router_dec(const RouterArgs& r, hipStream_t st) {
  if (r.T <= 0) return hipSuccess;
  const dim3 grid((r.E + kDecExperts - 1) / kDecExperts, (r.T + kDecTokens - 1) / kDecTokens);
  const dim3 block(kDecExperts * 64);
  if (r.H == 1024) k_router_dec<2><<<grid, block, 0, st>>>(r);
  else if (r.H == 2048) k_router_dec<4><<<grid, block, 0, st>>>(r);
  else if (r.H == 4096) k_router_dec<8><<<grid, block, 0, st>>>(r);
  else return launch_router_small(r, nullptr, 0, st);
  return hipGetLastError();
}

hipError_t launch_topk_permute_small(const RouterArgs& r, const Perm& p, int* arrivals, hipStream_t st) {
  if (r.T <= 0) return hipSuccess;
  if (r.T > kSmallT || r.k > kMaxTopK || r.E > kMaxExperts) return hipErrorInvalidValue;
  const int per = kTopkThreads / 64;
  k_topk_dec<<<(r.T + per - 1) / per, kTopkThreads, 0, st>>>(r, p, arrivals);
  return hipGetLastError();
}

hipError_t launch_hash_route(const HashArgs& a, hipStream_t st) {
  if (a.T <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)((a.T + 3) / 4);
  switch ((a.H + 511) / 512) {
    case 1: k_hash_route<1><<<blocks, 256, 0, st>>>(a); break;
    case 2: k_hash_route<2><<<blocks, 256, 0, st>>>(a); break;
    case 3: k_hash_route<3><<<blocks, 256, 0, st>>>(a); break;
    case 4: k_hash_route<4><<<blocks, 256, 0, st>>>(a); break;
    case 5: k_hash_route<5><<<blocks, 256, 0, st>>>(a); break;
    case 6: k_hash_route<6><<<blocks, 256, 0, st>>>(a); break;
    case 7: k_hash_route<7><<<blocks, 256, 0, st>>>(a); break;
    case 8: k_hash_route<8><<<blocks, 256, 0, st>>>(a); break;
    case 9: k_hash_route<9><<<blocks, 256, 0, st>>>(a); break;
    case 10: k_hash_route<10><<<blocks, 256, 0, st>>>(a); break;
    case 11: k_hash_route<11><<<blocks, 256, 0, st>>>(a); break;
    case 12: k_hash_route<12><<<blocks, 256, 0, st>>>(a); break;
    case 13: k_hash_route<13><<<blocks, 256, 0, st>>>(a); break;
    case 14: k_hash_route<14><<<blocks, 256, 0, st>>>(a); break;
    case 15: k_hash_route<15><<<blocks, 256, 0, st>>>(a); break;
    case 16: k_hash_route<16><<<blocks, 256, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
