// Learned router for large token counts on gfx950, on bf16 MFMA: the logits
// of page "DeepSeek-V4-Flash-0731", section "Checked in its code", row
// "Mixture of experts" are x (bf16) times the fp32 router rows. Each fp32
// weight w is split exactly enough into three bf16 parts, w = hi + mid + lo
// (hi = bf16(w), mid = bf16(w - hi), lo = bf16(w - hi - mid); the remainder
// is below 2^-24 |w|), so x . w = x . hi + x . mid + x . lo with every
// product exact in fp32 and the sums accumulated in fp32 by the MFMAs: the
// same precision as an fp32 dot product, at bf16 matrix-core speed.
//
// k_router_split writes the three planes (per call; 1.5x the fp32 bytes).
// k_router_mfma: block = 8 waves = 256 expert rows x 128 tokens x one K
// slice (K split KS ways so that a large batch fills the chip); wave w owns
// expert rows 32w .. 32w+31 (2 row blocks) x all 128 tokens (8 MFMA column
// blocks), each of its 3x2 weight fragments per k-step feeding 8 MFMAs. K
// runs in stages of 32: the weight fragments are loaded from global memory
// two stages ahead, the tokens go global -> registers -> LDS (fragment-
// major: lane l of the MFMAs of token block m reads the 16 bytes at slot
// 64 m + l), double-buffered. The partial logits of the block's K slice go
// to plog[slice][token][expert].
// k_topk_sum: one wave per token sums the KS partial logits in slice order,
// adds the per-expert offset, takes the score sqrt(softplus(logit)) and the
// selection value score + bias (row "Auxiliary-loss-free load balancing"),
// and selects the top-k (ties to the lower expert id).
#include "device.h"
#include "internal.h"

namespace moe {

constexpr int kRmThreads = 512;
constexpr int kRmTok = 128;   // tokens per block
constexpr int kRmRows = 256;  // expert rows per block (the most experts supported)

__global__ __launch_bounds__(256) void k_router_split(const float* __restrict__ w, uint16_t* __restrict__ out,
                                                      long long n) {
  const long long i = ((long long)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;  // n is a multiple of 4 (H is)
  const float4 v = *reinterpret_cast<const float4*>(w + i);
  const float f[4] = {v.x, v.y, v.z, v.w};
  uint16_t hi[4], mid[4], lo[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    hi[j] = f32_to_bf16(f[j]);
    const float r1 = f[j] - bf16_to_f32(hi[j]);
    mid[j] = f32_to_bf16(r1);
    lo[j] = f32_to_bf16(r1 - bf16_to_f32(mid[j]));
  }
  auto pack = [](const uint16_t (&h)[4]) {
    return make_uint2((uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16));
  };
  *reinterpret_cast<uint2*>(out + i) = pack(hi);
  *reinterpret_cast<uint2*>(out + n + i) = pack(mid);
  *reinterpret_cast<uint2*>(out + 2 * n + i) = pack(lo);
}

__device__ __forceinline__ void rm_compute(f32x4_t (&acc)[2][8], const u32x4_t (&wa)[3][2],
                                           const unsigned char* buf, int lane) {
  bf16x8_t bt[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) bt[m] = *reinterpret_cast<const bf16x8_t*>(buf + (m * 64 + lane) * 16);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int p = 0; p < 3; ++p)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const bf16x8_t av = __builtin_bit_cast(bf16x8_t, wa[p][b]);
#pragma unroll
      for (int m = 0; m < 8; ++m) acc[b][m] = mfma_16x16x32(av, bt[m], acc[b][m]);
    }
}

__global__ __launch_bounds__(kRmThreads) void k_router_mfma(RouterMfmaArgs a) {
  __shared__ __align__(16) unsigned char lds[2][kRmTok * 32 * 2];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, g = lane >> 4;
  const int tile = blockIdx.x / a.KS, ks = blockIdx.x - tile * a.KS;
  const int pos0 = tile * kRmTok;
  const int H = a.H, E = a.E, T = a.T;
  const int Kc = H / a.KS, k0 = ks * Kc, nst = Kc / 32;

  // weight fragments: plane p, row block b: expert row 32 wave + 16 b + r
  // (clamped to the last expert: surplus rows are computed, never stored),
  // the lane's 8 K-values g*8 .. of each 32-wide stage
  const size_t plane = (size_t)E * H;
  uint32_t woff[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) woff[b] = (uint32_t)(min(32 * wave + 16 * b + r, E - 1) * H + k0 + g * 8);
  auto load_w = [&](int st, u32x4_t (&wa)[3][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < 3; ++p)
#pragma unroll
      for (int b = 0; b < 2; ++b)
        wa[p][b] = *reinterpret_cast<const u32x4_t*>(a.wsplit + p * plane + woff[b] + st * 32);
  };
  // this thread's token piece: token 16 wave + r, chunk g (8 K-values) of the
  // stage; LDS slot 64 wave + lane (token block wave, lane r + 16 g)
  const int tk = 16 * wave + r;
  const uint16_t* asrc = a.x + (size_t)min(pos0 + tk, T - 1) * H + k0 + g * 8;
  u32x4_t* adst0 = reinterpret_cast<u32x4_t*>(&lds[0][(wave * 64 + lane) * 16]);
  u32x4_t* adst1 = reinterpret_cast<u32x4_t*>(&lds[1][(wave * 64 + lane) * 16]);
  auto load_a = [&](int st) __attribute__((always_inline)) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(asrc + st * 32);
    asm volatile("" ::: "memory");
    return v;
  };

  f32x4_t acc[2][8];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int m = 0; m < 8; ++m) acc[b][m] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  // branch-free pipeline: stage st computes from LDS buffer st%2 and weight
  // set st%2; the tokens of st+1 wait in registers, the weights of st+2 are
  // in flight; loads past the last stage re-read it (clamped, never used)
  const int last = nst - 1;
  u32x4_t w0[3][2], w1[3][2];
  load_w(0, w0);
  u32x4_t av = load_a(0);
  *adst0 = av;
  av = load_a(min(1, last));
  load_w(min(1, last), w1);
  for (int st = 0; st + 1 < nst; st += 2) {
    __syncthreads();
    *adst1 = av;  // stage st+1
    av = load_a(min(st + 2, last));
    rm_compute(acc, w0, lds[0], lane);
    load_w(min(st + 2, last), w0);
    __syncthreads();
    *adst0 = av;  // stage st+2
    av = load_a(min(st + 3, last));
    rm_compute(acc, w1, lds[1], lane);
    load_w(min(st + 3, last), w1);
  }
  if (nst & 1) {
    __syncthreads();
    rm_compute(acc, w0, lds[0], lane);
  }

  // lane holds acc[b][m][i] = logit part of (expert 32 wave + 16 b + 4 g + i,
  // token pos0 + 16 m + r)
  float* out = a.plog + (size_t)ks * T * E;
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const int t = pos0 + 16 * m + r;
    if (t >= T) continue;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int e0 = 32 * wave + 16 * b + 4 * g;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (e0 + i < E) out[(size_t)t * E + e0 + i] = acc[b][m][i];
    }
  }
}

// One wave per token: logits from the partial sums, then scores, selection
// values and the top-k. The slice count is a template argument so that a
// lane requests all of its partial logits, offsets and biases before the
// first add: with a loop over a run-time count each load was issued only
// after the previous one had arrived (20 dependent round trips per wave at
// four slices). The sums keep the slice order, then the offset.
template <int KS>
__global__ __launch_bounds__(256) void k_topk_sum(RouterArgs a, const float* __restrict__ plog) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  const int lane = threadIdx.x & 63;
  float part[4][KS], off[4], bias[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = min(lane + 64 * q, a.E - 1);  // surplus lanes get key 0 inside the selection
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) part[q][ks] = plog[((size_t)ks * a.T + t) * a.E + e];
    off[q] = a.logit_offset ? a.logit_offset[e] : 0.0f;
    bias[q] = a.bias[e];
  }
  TopkRow row;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float logit = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) logit += part[q][ks];
    if (a.logit_offset) logit += off[q];
    row.s[q] = sqrtf(softplus(logit));
    row.b[q] = row.s[q] + bias[q];
  }
  wave_topk_row(row, a.E, a.k, a.scale, a.ids + (size_t)t * a.k, a.w + (size_t)t * a.k, nullptr);
}

int router_mfma_splits(int T, int H) {
  const int tiles = (T + kRmTok - 1) / kRmTok;
  int ks = 1;
  while (ks < 8 && tiles * ks < 256 && H % (ks * 2 * 32) == 0) ks *= 2;
  return ks;
}

hipError_t launch_router_mfma(const RouterArgs& r, uint16_t* wsplit, float* plog, hipStream_t st) {
  if (r.T <= 0) return hipSuccess;
  if (r.E > kRmRows || r.E < 1 || r.H % 32) return hipErrorInvalidValue;
  const long long n = (long long)r.E * r.H;
  k_router_split<<<(unsigned)((n / 4 + 255) / 256), 256, 0, st>>>(r.gate_w, wsplit, n);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  RouterMfmaArgs a;
  a.T = r.T;
  a.H = r.H;
  a.E = r.E;
  a.KS = router_mfma_splits(r.T, r.H);
  a.x = r.x;
  a.wsplit = wsplit;
  a.plog = plog;
  const int tiles = (r.T + kRmTok - 1) / kRmTok;
  k_router_mfma<<<(unsigned)(tiles * a.KS), kRmThreads, 0, st>>>(a);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const unsigned blocks = (unsigned)((r.T + 3) / 4);
  switch (a.KS) {
    case 1: k_topk_sum<1><<<blocks, 256, 0, st>>>(r, plog); break;
    case 2: k_topk_sum<2><<<blocks, 256, 0, st>>>(r, plog); break;
    case 4: k_topk_sum<4><<<blocks, 256, 0, st>>>(r, plog); break;
    case 8: k_topk_sum<8><<<blocks, 256, 0, st>>>(r, plog); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
