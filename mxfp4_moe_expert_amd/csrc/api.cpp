// Host entry points of the C ABI declared in include/moe.h: argument checks,
// workspace carving and kernel dispatch on the caller's stream. Nothing here
// allocates device memory or synchronises with the device.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "internal.h"
#include "moe.h"

namespace {

using namespace moe;

constexpr int kMaxT = 65536;
constexpr int kMaxDim = 8192;  // H and I: the largest whose activation and scale tiles fit a block's LDS
constexpr size_t kActLdsBudget = 128 * 1024;  // activation tile bytes per block

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct Layout {
  size_t counters, xfer, wsplit, plog, scores, ids, w, offsets, sorted, slot_pos, sorted_tok, tile_info, tile_rec,
      done, blk_counts, hbuf, hs, ybuf, zbuf, xsplit, hscale, total;
  int tile_n, max_tiles;
  bool mx;  // routed GEMMs on the block-scaled MFMA (activations split into fp8 hi/lo)
};

bool cfg_ok(const moe_config* c) {
  if (!c) return false;
  const int H = c->hidden_size, E = c->n_routed_experts, k = c->top_k, I = c->moe_intermediate;
  if (H < 128 || H % 128 || H > kMaxDim) return false;
  if (I < 128 || I % 128 || I > kMaxDim) return false;
  if (k < 1 || k > kMaxTopK || E < k || E > kMaxExperts) return false;
  if (!(c->routed_scaling_factor == c->routed_scaling_factor)) return false;
  if (!(c->swiglu_limit == c->swiglu_limit)) return false;
  if (c->norm_topk_prob != 1) return false;  // the weights are always renormalised over the top-k
  return true;
}

// Largest power-of-two tile width <= want whose activation tile fits the LDS budget.
int fit_tile(int want, int K) {
  int tn = 1;
  while (tn * 2 <= want && (size_t)(tn * 2) * (2 * (size_t)K + 16) <= kActLdsBudget) tn *= 2;
  return tn;
}

// Tokens per shared-expert tile of the streaming passes: each tile streams
// the whole shared expert, so wide tiles read it fewer times; up to 16 (one
// MFMA's columns), with the tile's bf16 rows at most 140 KB of LDS (the
// streaming blocks run one per CU).
int shared_stream_tile(int T, int K) {
  int tn = T < 16 ? T : 16;
  while (tn > 1 && (size_t)tn * (2 * (size_t)K + 16) > 140 * 1024) --tn;
  return tn;
}

// Columns per routed expert tile at decode sizes: a few times the expected
// tokens per expert (1.5 at 64 tokens, 6 of 256 experts), so that an expert
// seldom needs a second tile, which would stream its weights again, while
// the LDS activation tile stays no larger than the shared expert's.
// Batches above kSmallT run the grouped GEMMs (256-row output tiles along H).
bool use_gemm(const moe_config& c, int T) { return T > kSmallT && c.hidden_size % 256 == 0; }
// Process-wide options (moe_set_option).
int g_opt_prefill_block_scaled = 0;

// the routed grouped GEMMs run on the block-scaled MFMA when that option is on and the shapes fit
// its tiles
bool use_gemm_mx(const moe_config& c, int T) {
  return g_opt_prefill_block_scaled && use_gemm(c, T) && gemm_mx_supported(c.hidden_size, c.moe_intermediate);
}

int routed_tile_n(const moe_config& c, int T) {
  if (use_gemm_mx(c, T)) return kGemmMxTokens;
  if (use_gemm(c, T)) return kGemmTokens;
  const int K = c.hidden_size > c.moe_intermediate ? c.hidden_size : c.moe_intermediate;
  int tn = T <= 1 ? 1 : 6;
  // the streaming unit holds the tile's rows and its 256 weight rows' scales
  while (tn > 1 &&
         ((size_t)tn * (2 * (size_t)K + 16) > kActLdsBudget || stream_unit_lds(tn, K, false) > kLdsBlockMax))
    --tn;
  return tn;
}

int routed_max_tiles(const moe_config& c, int T, int tile_n) {
  const long long slots = (long long)T * c.top_k;
  const long long by_width = (slots + tile_n - 1) / tile_n + (slots < c.n_routed_experts ? slots : c.n_routed_experts);
  return (int)(by_width < slots ? by_width : slots);
}

Layout layout(const moe_config& c, int T) {
  const size_t H = c.hidden_size, E = c.n_routed_experts, k = c.top_k, I = c.moe_intermediate;
  const size_t slots = (size_t)T * k;
  const size_t nblk = (slots + kPermBlock - 1) / kPermBlock;
  Layout L;
  L.tile_n = routed_tile_n(c, T);
  L.max_tiles = routed_max_tiles(c, T, L.tile_n);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  L.counters = take(256);
  L.xfer = take(kXferBytes);
  // large-T router: bf16 planes of the router rows, partial logits per K slice
  const bool big = T > kSmallT;
  L.wsplit = take(big ? (size_t)3 * E * H * 2 : 0);
  L.plog = take(big ? (size_t)router_mfma_splits(T, (int)H) * T * E * 4 : 0);
  L.scores = take((size_t)2 * T * E * 4);  // scores, then selection values
  L.ids = take(slots * 4);
  L.w = take(slots * 4);
  L.offsets = take((E + 1) * 4);
  L.sorted = take(slots * 4);
  L.slot_pos = take(slots * 4);
  L.sorted_tok = take(slots * 4);
  L.tile_info = take((size_t)L.max_tiles * 16);
  L.tile_rec = take((size_t)L.max_tiles * kRecInts * 4);
  L.done = take((size_t)(L.max_tiles + kSmallT) * 4);
  L.blk_counts = take(nblk * E * 4);
  L.hbuf = take(slots * I * 2);
  L.hs = take((size_t)T * I * 2);
  L.ybuf = take(slots * H * 4);
  L.zbuf = take((size_t)T * H * 4);
  // block-scaled routed GEMMs: x split into hi/lo fp8 [T][H] + E8M0 [T][H/32] each; the h split
  // lives in hbuf (hi [slots][I], lo [slots][I]), its E8M0 bytes here ([slots][I/32] each)
  L.mx = use_gemm_mx(c, T);
  L.xsplit = take(L.mx ? (size_t)T * H * 2 + (size_t)T * (H / 32) * 2 : 0);
  L.hscale = take(L.mx ? slots * (I / 32) * 2 : 0);
  L.total = o;
  return L;
}

template <class P>
inline P* at(void* ws, size_t off) {
  return reinterpret_cast<P*>(static_cast<char*>(ws) + off);
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Tile queue of one grouped-GEMM launch (9 ints in the counters region,
// zero on first use and left zero by every launch).
inline int* gemm_queue(void* ws, const Layout& L, int which) {
  return at<int32_t>(ws, L.counters) + kGemmQueueInts + 9 * which;
}

// A failed launch or runtime call: HIP's error state is cleared so that it
// does not surface in the caller's next HIP call.
int status(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  (void)hipGetLastError();
  return MOE_EHIP;
}

// Measurement hook (moe_set_kernel_events): events recorded around one kernel.
int g_prof_kernel = MOE_KERNEL_NONE;
hipEvent_t g_prof_start = nullptr, g_prof_stop = nullptr;

// Launch `fn` bracketed by the measurement events if `kernel_id` is selected.
template <class F>
hipError_t timed(int kernel_id, hipStream_t st, F&& fn) {
  const bool on = g_prof_kernel == kernel_id && g_prof_start && g_prof_stop;
  if (on) {
    hipError_t e = hipEventRecord(g_prof_start, st);
    if (e != hipSuccess) return e;
  }
  hipError_t err = fn();
  if (err != hipSuccess) return err;
  if (on) return hipEventRecord(g_prof_stop, st);
  return hipSuccess;
}

Perm perm_of(void* ws, const Layout& L, int32_t* offsets, int32_t* sorted, int32_t* slot_pos) {
  Perm p;
  p.offsets = offsets;
  p.sorted_slots = sorted;
  p.slot_pos = slot_pos;
  p.sorted_tok = at<int32_t>(ws, L.sorted_tok);
  p.tile_info = at<int4>(ws, L.tile_info);
  p.n_tiles = at<int32_t>(ws, L.counters);
  p.tile_rec = at<int32_t>(ws, L.tile_rec);
  p.queues = at<int32_t>(ws, L.counters) + kQueueInts;
  p.done = at<int32_t>(ws, L.done);
  p.tile_n = L.tile_n;
  p.max_tiles = L.max_tiles;
  p.flags = device_flags();
  return p;
}

SkinnyArgs skinny_common(const moe_config& c, int T) {
  SkinnyArgs a;
  memset(&a, 0, sizeof(a));
  a.T = T;
  a.limit = c.swiglu_limit;
  a.flags = device_flags();
  return a;
}

// Routed w13 + SwiGLU: h [sorted position][I] bf16.
SkinnyArgs routed_w13_args(const moe_config& c, int T, const uint16_t* x, const Perm& p, const uint8_t* w13c,
                           const uint8_t* w13s, uint16_t* hbuf) {
  const int H = c.hidden_size, I = c.moe_intermediate;
  SkinnyArgs a = skinny_common(c, T);
  a.routed = 1;
  a.tile_info = p.tile_info;
  a.n_tiles = p.n_tiles;
  a.tile_n = p.tile_n;
  a.n_tiles_grid = p.max_tiles;
  a.wq = w13c;
  a.wsc = w13s;
  a.q_expert_stride = (long long)2 * I * (H / 2);
  a.s_expert_stride = (long long)2 * I * (H / 32);
  a.K = H;
  a.half = I;
  a.rows = 2 * I;
  a.n_rowblocks = I / 16;
  a.act = x;
  a.act_ld = H;
  a.act_row = p.sorted_tok;
  a.hout = hbuf;
  a.hout_ld = I;
  a.tile_rec = p.tile_rec;
  return a;
}

// Routed w2 x routing weight: ybuf [slot][H] fp32.
SkinnyArgs routed_w2_args(const moe_config& c, int T, const Perm& p, const float* slot_w, const uint8_t* w2c,
                          const uint8_t* w2s, const uint16_t* hbuf, float* ybuf) {
  const int H = c.hidden_size, I = c.moe_intermediate;
  SkinnyArgs a = skinny_common(c, T);
  a.routed = 1;
  a.tile_info = p.tile_info;
  a.n_tiles = p.n_tiles;
  a.tile_n = p.tile_n;
  a.n_tiles_grid = p.max_tiles;
  a.wq = w2c;
  a.wsc = w2s;
  a.q_expert_stride = (long long)H * (I / 2);
  a.s_expert_stride = (long long)H * (I / 32);
  a.K = I;
  a.half = 0;
  a.rows = H;
  a.n_rowblocks = H / 16;
  a.act = hbuf;
  a.act_ld = I;
  a.act_row = nullptr;
  a.yout = ybuf;
  a.yout_ld = H;
  a.sorted_slots = p.sorted_slots;
  a.slot_w = slot_w;
  a.tile_rec = p.tile_rec;
  return a;
}

// Shared expert w13 + SwiGLU: hs [T][I] bf16.
// slim: blocks of 8 gate + 8 up rows (the router launch); else 16 + 16.
SkinnyArgs shared_w13_args(const moe_config& c, int T, const uint16_t* x, const int8_t* q13, const float* s13,
                           uint16_t* hs, int* blocks, bool slim) {
  const int H = c.hidden_size, I = c.moe_intermediate;
  SkinnyArgs a = skinny_common(c, T);
  a.routed = 0;
  a.tile_n = fit_tile(T < 16 ? T : 16, H);
  a.n_tiles_grid = (T + a.tile_n - 1) / a.tile_n;
  a.wq = reinterpret_cast<const uint8_t*>(q13);
  a.row_scale = s13;
  a.K = H;
  a.half = I;
  a.rows = 2 * I;
  a.n_rowblocks = slim ? I / 8 : I / 16;
  a.act = x;
  a.act_ld = H;
  a.hout = hs;
  a.hout_ld = I;
  *blocks = a.n_tiles_grid * a.n_rowblocks;
  return a;
}

// Shared expert w2: zbuf [T][H] fp32.
SkinnyArgs shared_w2_args(const moe_config& c, int T, const int8_t* q2, const float* s2, const uint16_t* hs,
                          float* zbuf, int* blocks) {
  const int H = c.hidden_size, I = c.moe_intermediate;
  SkinnyArgs a = skinny_common(c, T);
  a.routed = 0;
  a.tile_n = fit_tile(T < 16 ? T : 16, I);
  a.n_tiles_grid = (T + a.tile_n - 1) / a.tile_n;
  a.wq = reinterpret_cast<const uint8_t*>(q2);
  a.row_scale = s2;
  a.K = I;
  a.half = 0;
  a.rows = H;
  a.n_rowblocks = H / 16;
  a.act = hs;
  a.act_ld = I;
  a.yout = zbuf;
  a.yout_ld = H;
  *blocks = a.n_tiles_grid * a.n_rowblocks;
  return a;
}

GemmArgs gemm_common(const moe_config& c, int T) {
  GemmArgs g;
  memset(&g, 0, sizeof(g));
  g.T = T;
  g.topk = c.top_k;
  g.limit = c.swiglu_limit;
  return g;
}

// Routed w13 (+ SwiGLU) as a grouped GEMM: h [sorted position][I].
GemmArgs gemm_routed_w13(const moe_config& c, int T, const uint16_t* x, const Perm& p, const uint8_t* w13c,
                         const uint8_t* w13s, uint16_t* hbuf) {
  const int H = c.hidden_size, I = c.moe_intermediate;
  GemmArgs g = gemm_common(c, T);
  g.fmt = 0;
  g.mode = kGemmW13;
  g.wq = w13c;
  g.wsc = w13s;
  g.q_expert_stride = (long long)2 * I * (H / 2);
  g.s_expert_stride = (long long)2 * I * (H / 32);
  g.K = H;
  g.half = I;
  g.routed = 1;
  g.tile_info = p.tile_info;
  g.n_tiles = p.n_tiles;
  g.n_ntiles = I / 128;
  g.act = x;
  g.act_ld = H;
  g.act_row = p.sorted_tok;
  g.hout = hbuf;
  g.hout_ld = I;
  return g;
}

// Routed w2 x routing weight: ybuf [slot][H], bf16 (the combine sums the k
// rounded slot outputs of a token in fp32).
GemmArgs gemm_routed_w2(const moe_config& c, int T, const Perm& p, const float* slot_w, const uint8_t* w2c,
                        const uint8_t* w2s, const uint16_t* hbuf, uint16_t* ybuf) {
  const int H = c.hidden_size, I = c.moe_intermediate;
  GemmArgs g = gemm_common(c, T);
  g.fmt = 0;
  g.mode = kGemmW2;
  g.wq = w2c;
  g.wsc = w2s;
  g.q_expert_stride = (long long)H * (I / 2);
  g.s_expert_stride = (long long)H * (I / 32);
  g.K = I;
  g.routed = 1;
  g.tile_info = p.tile_info;
  g.n_tiles = p.n_tiles;
  g.n_ntiles = H / 256;
  g.act = hbuf;
  g.act_ld = I;
  g.yout = ybuf;
  g.yout_ld = H;
  g.sorted_slots = p.sorted_slots;
  g.slot_w = slot_w;
  return g;
}

// Shared w13 (+ SwiGLU): hs [T][I].
GemmArgs gemm_shared_w13(const moe_config& c, int T, const uint16_t* x, const int8_t* q13, const float* s13,
                         uint16_t* hs) {
  const int H = c.hidden_size, I = c.moe_intermediate;
  GemmArgs g = gemm_common(c, T);
  g.fmt = 1;
  g.mode = kGemmW13;
  g.wq = reinterpret_cast<const uint8_t*>(q13);
  g.row_scale = s13;
  g.K = H;
  g.half = I;
  g.routed = 0;
  g.n_ntiles = I / 128;
  g.act = x;
  g.act_ld = H;
  g.hout = hs;
  g.hout_ld = I;
  return g;
}

// Shared w2 + the final combine: out[t] = sum_j ybuf[t*k+j] + s2 * (Q2 hs_t).
GemmArgs gemm_shared_w2_combine(const moe_config& c, int T, const int8_t* q2, const float* s2, const uint16_t* hs,
                                const uint16_t* ybuf, void* out, int out_is_fp32) {
  const int H = c.hidden_size, I = c.moe_intermediate;
  GemmArgs g = gemm_common(c, T);
  g.fmt = 1;
  g.mode = kGemmW2Combine;
  g.wq = reinterpret_cast<const uint8_t*>(q2);
  g.row_scale = s2;
  g.K = I;
  g.routed = 0;
  g.n_ntiles = H / 256;
  g.act = hs;
  g.act_ld = I;
  g.ybuf = ybuf;
  g.out = out;
  g.out_ld = H;
  g.out_is_fp32 = out_is_fp32;
  return g;
}

// Routed w13 + SwiGLU and w2 x routing weight on the block-scaled MFMA: x is
// split into hi/lo fp8 first, the w13 epilogue writes h split the same way,
// and w2 writes the weighted slot outputs in bf16 (ybuf, by slot).
hipError_t routed_gemms_mx(const moe_config& c, int T, const uint16_t* x, const Perm& p, const float* slot_w,
                           const uint8_t* w13c, const uint8_t* w13s, const uint8_t* w2c, const uint8_t* w2s,
                           void* ws, const Layout& L, uint16_t* ybf, hipStream_t st) {
  const int H = c.hidden_size, I = c.moe_intermediate;
  const size_t slots = (size_t)T * c.top_k;
  uint8_t* xh = at<uint8_t>(ws, L.xsplit);
  uint8_t* xl = xh + (size_t)T * H;
  uint8_t* xsh = xl + (size_t)T * H;
  uint8_t* xsl = xsh + (size_t)T * (H / 32);
  uint8_t* hh = at<uint8_t>(ws, L.hbuf);
  uint8_t* hl = hh + slots * I;
  uint8_t* hsh = at<uint8_t>(ws, L.hscale);
  uint8_t* hsl = hsh + slots * (I / 32);
  hipError_t e = launch_quant_rows(x, T, H, xh, xl, xsh, xsl, st);
  if (e != hipSuccess) return e;
  MxGemmArgs a;
  memset(&a, 0, sizeof(a));
  a.mode = kGemmW13;
  a.wq = w13c;
  a.wsc = w13s;
  a.q_expert_stride = (long long)2 * I * (H / 2);
  a.s_expert_stride = (long long)2 * I * (H / 32);
  a.K = H;
  a.half = I;
  a.N = I;
  a.I = I;
  a.tile_info = p.tile_info;
  a.n_tiles = p.n_tiles;
  a.n_ntiles = I / 128;
  a.a_hi = xh;
  a.a_lo = xl;
  a.as_hi = xsh;
  a.as_lo = xsl;
  a.act_row = p.sorted_tok;
  a.h_hi = hh;
  a.h_lo = hl;
  a.hs_hi = hsh;
  a.hs_lo = hsl;
  a.limit = c.swiglu_limit;
  a.order = 0;
  a.queue = at<int32_t>(ws, L.counters) + kGemmQueueInts + 9 * kQRoutedW13;
  e = timed(MOE_KERNEL_ROUTED_W13, st, [&] { return launch_gemm_mx(a, p.max_tiles, st); });
  if (e != hipSuccess) return e;
  MxGemmArgs b;
  memset(&b, 0, sizeof(b));
  b.mode = kGemmW2;
  b.wq = w2c;
  b.wsc = w2s;
  b.q_expert_stride = (long long)H * (I / 2);
  b.s_expert_stride = (long long)H * (I / 32);
  b.K = I;
  b.N = H;
  b.tile_info = p.tile_info;
  b.n_tiles = p.n_tiles;
  b.n_ntiles = H / 256;
  b.a_hi = hh;
  b.a_lo = hl;
  b.as_hi = hsh;
  b.as_lo = hsl;
  b.act_row = nullptr;
  b.yout = ybf;
  b.yout_ld = H;
  b.sorted_slots = p.sorted_slots;
  b.slot_w = slot_w;
  b.limit = c.swiglu_limit;
  b.order = 0;
  b.queue = at<int32_t>(ws, L.counters) + kGemmQueueInts + 9 * kQRoutedW2;
  return timed(MOE_KERNEL_ROUTED_W2, st, [&] { return launch_gemm_mx(b, p.max_tiles, st); });
}

// The single-launch layer's arguments (MXFP4 w2; the caller sets the 3-bit
// fields). Hash layers (tid2eid) take no selection bias or logit offset.
LayerArgs single_layer_args(const moe_config& c, int T, const uint16_t* x, const float* gate_w, const float* bias,
                            const float* logit_offset, const int32_t* token_ids, const int32_t* tid2eid, int V,
                            const uint8_t* w13c, const uint8_t* w13s, const uint8_t* w2c, const uint8_t* w2s,
                            const int8_t* sh13, const float* sh13s, const int8_t* sh2, const float* sh2s, void* out,
                            int out_is_fp32, int32_t* ids, float* w, uint32_t* xfer) {
  const bool hash = tid2eid != nullptr;
  LayerArgs la;
  memset(&la, 0, sizeof(la));
  la.T = T;
  la.H = c.hidden_size;
  la.I = c.moe_intermediate;
  la.E = c.n_routed_experts;
  la.k = c.top_k;
  la.scale = c.routed_scaling_factor;
  la.limit = c.swiglu_limit;
  la.x = x;
  la.gate_w = gate_w;
  la.bias = hash ? nullptr : bias;
  la.logit_offset = hash ? nullptr : logit_offset;
  la.w13c = w13c;
  la.w13s = w13s;
  la.w2c = w2c;
  la.w2s = w2s;
  la.sh13 = sh13;
  la.sh13s = sh13s;
  la.sh2 = sh2;
  la.sh2s = sh2s;
  la.out = out;
  la.out_is_fp32 = out_is_fp32 ? 1 : 0;
  la.ids_out = ids;
  la.w_out = w;
  la.xfer = xfer;
  la.flags = device_flags();
  la.token_ids = hash ? token_ids : nullptr;
  la.tid2eid = tid2eid;
  la.V = hash ? V : 0;
  return la;
}

int check_ws(const moe_config& c, int T, const void* ws, size_t bytes) {
  if (!ws) return MOE_EINVAL;
  if (reinterpret_cast<uintptr_t>(ws) & 255) return MOE_EINVAL;
  if (bytes < layout(c, T).total) return MOE_EWORKSPACE;
  return MOE_OK;
}

RouterArgs router_args(const moe_config& c, int T, const uint16_t* x, const float* gate_w, const float* bias,
                       const float* logit_offset, float* scores, int32_t* ids, float* w) {
  RouterArgs a;
  a.T = T;
  a.H = c.hidden_size;
  a.E = c.n_routed_experts;
  a.k = c.top_k;
  a.scale = c.routed_scaling_factor;
  a.x = x;
  a.gate_w = gate_w;
  a.bias = bias;
  a.logit_offset = logit_offset;
  a.scores = scores;
  a.keys = scores + (size_t)T * c.n_routed_experts;
  a.ids = ids;
  a.w = w;
  a.token_ids = nullptr;
  a.tid2eid = nullptr;
  a.V = 0;
  a.flags = device_flags();
  return a;
}

// The launch sequence of moe_forward (MOE_SCHED_*).
// Hash layers take the same schedules, with the token's table row in place
// of the top-k, except the three-launch tiny schedule (its routed w13 blocks
// redo the top-k themselves): there they take the decode schedule.
// Routed w2 in 3-bit blocks runs in the fused streaming launch (T <= 64; both
// stages' K multiples of 1024) or the grouped GEMM (T > 64; H a multiple of 256).
bool w2q3_supported(const moe_config& c, int T) {
  if (T <= kSmallT)  // the fused streaming launch, whose w2 units hold binary16 scale rows
    return c.hidden_size % 1024 == 0 && c.moe_intermediate % 1024 == 0 &&
           stream_unit_lds(routed_tile_n(c, T), c.moe_intermediate, true) <= kLdsBlockMax;
  return use_gemm(c, T);
}

// The routed experts' w2: MXFP4 (codes + E8M0 bytes) or 3-bit blocks (codes
// + binary16 scales + optional per-expert levels).
struct W2Weights {
  int fmt;  // kFmtMx or kFmtQ3
  const uint8_t* codes;
  const uint8_t* scales;
  const float* table;
};

// Points a routed w2 pass (streaming or GEMM) at 3-bit blocks: codes
// [E][H][I/32][12], binary16 scales [E][H][I/32], levels [E][8] or null.
template <class Args>
void set_w2q3(const moe_config& c, const W2Weights& w, Args& a) {
  const long long H = c.hidden_size, I = c.moe_intermediate;
  a.fmt = kFmtQ3;
  a.wq = w.codes;
  a.wsc = w.scales;
  a.table = w.table;
  a.q_expert_stride = H * (I / 32) * 12;
  a.s_expert_stride = H * (I / 32) * 2;
}

int schedule(const moe_config& c, int T, bool hash) {
  if (T * (c.top_k + 1) <= 16) {
    if (layer_small_supported(c.hidden_size, c.moe_intermediate, c.n_routed_experts, T, c.top_k))
      return MOE_SCHED_SINGLE;
    // the tiny schedule's last launch holds every column's h (T k slots + T tokens)
    if (!hash && w2_combine_small_lds(T, c.top_k, c.moe_intermediate) <= kLdsBlockMax) return MOE_SCHED_TINY;
  }
  if (T <= kSmallT) return MOE_SCHED_DECODE;
  return MOE_SCHED_LARGE;
}

}  // namespace

extern "C" {

const char* moe_status_string(int s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument (null, negative or misaligned)";
    case MOE_EUNSUPPORTED: return "unsupported shape";
    case MOE_EWORKSPACE: return "workspace too small";
    case MOE_EHIP: return "HIP launch or runtime error";
    default: return "unknown status";
  }
}

const char* moe_version(void) { return "0.2.0"; }

int moe_device_flags(uint32_t* flags, int32_t clear, void* stream) {
  uint32_t* f = device_flags();
  if (!f) return MOE_EHIP;
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint32_t v = 0;
  hipError_t e = hipMemcpyAsync(&v, f, sizeof(v), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess && clear) e = launch_fill_zero(f, sizeof(uint32_t), st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return MOE_EHIP;
  if (flags) *flags = v;
  return MOE_OK;
}

int moe_set_option(int32_t option, int32_t value) {
  switch (option) {
    case MOE_OPTION_PREFILL_BLOCK_SCALED:
      if (value != 0 && value != 1) return MOE_EINVAL;
      g_opt_prefill_block_scaled = value;
      return MOE_OK;
    default:
      return MOE_EINVAL;
  }
}

int moe_get_option(int32_t option) {
  switch (option) {
    case MOE_OPTION_PREFILL_BLOCK_SCALED: return g_opt_prefill_block_scaled;
    default: return MOE_EINVAL;
  }
}

int moe_set_kernel_events(int32_t kernel_id, void* start_event, void* stop_event) {
  if (kernel_id < MOE_KERNEL_NONE || kernel_id > MOE_KERNEL_COMBINE) return MOE_EINVAL;
  g_prof_kernel = kernel_id;
  g_prof_start = static_cast<hipEvent_t>(start_event);
  g_prof_stop = static_cast<hipEvent_t>(stop_event);
  return MOE_OK;
}

size_t moe_workspace_size(const moe_config* cfg, int32_t T) {
  if (!cfg_ok(cfg) || T < 0 || T > kMaxT) return 0;
  return layout(*cfg, T).total;
}

int moe_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace && workspace_bytes) return MOE_EINVAL;
  return status(launch_fill_zero(workspace, workspace_bytes, static_cast<hipStream_t>(stream)));
}

int moe_route(const moe_config* cfg, int32_t T, const uint16_t* x, const float* gate_w, const float* bias,
              const float* logit_offset, int32_t* topk_ids, float* topk_w, void* workspace,
              size_t workspace_bytes, void* stream) {
  if (!cfg) return MOE_EINVAL;
  if (!cfg_ok(cfg) || T > kMaxT) return MOE_EUNSUPPORTED;
  if (T < 0) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!x || !gate_w || !bias || !topk_ids || !topk_w) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(gate_w) || !aligned16(topk_ids) || !aligned16(topk_w)) return MOE_EINVAL;
  int rc = check_ws(*cfg, T, workspace, workspace_bytes);
  if (rc) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const Layout L = layout(*cfg, T);
  RouterArgs a = router_args(*cfg, T, x, gate_w, bias, logit_offset, at<float>(workspace, L.scores), topk_ids,
                             topk_w);
  if (T <= kSmallT) {
    Perm p = perm_of(workspace, L, at<int32_t>(workspace, L.offsets), at<int32_t>(workspace, L.sorted),
                     at<int32_t>(workspace, L.slot_pos));
    rc = status(launch_router_dec(a, st));
    if (rc) return rc;
    return status(launch_topk_permute_small(a, p, at<int32_t>(workspace, L.counters) + kArrivalsInt, st));
  }
  return status(launch_router_mfma(a, at<uint16_t>(workspace, L.wsplit), at<float>(workspace, L.plog), st));
}

int moe_hash_route(const moe_config* cfg, int32_t T, const uint16_t* x, const int32_t* token_ids,
                   const int32_t* tid2eid, int32_t V, const float* gate_w, int32_t* topk_ids, float* topk_w,
                   void* stream) {
  if (!cfg) return MOE_EINVAL;
  if (!cfg_ok(cfg) || T > kMaxT) return MOE_EUNSUPPORTED;
  if (T < 0 || V <= 0) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!x || !token_ids || !tid2eid || !gate_w || !topk_ids || !topk_w) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(gate_w)) return MOE_EINVAL;
  HashArgs a;
  a.T = T;
  a.H = cfg->hidden_size;
  a.E = cfg->n_routed_experts;
  a.k = cfg->top_k;
  a.V = V;
  a.scale = cfg->routed_scaling_factor;
  a.x = x;
  a.token_ids = token_ids;
  a.tid2eid = tid2eid;
  a.gate_w = gate_w;
  a.ids = topk_ids;
  a.w = topk_w;
  a.flags = device_flags();
  return status(launch_hash_route(a, static_cast<hipStream_t>(stream)));
}

int moe_permute(const moe_config* cfg, int32_t T, const int32_t* topk_ids, int32_t* expert_offsets,
                int32_t* sorted_slots, int32_t* slot_pos, void* workspace, size_t workspace_bytes,
                void* stream) {
  if (!cfg) return MOE_EINVAL;
  if (!cfg_ok(cfg) || T > kMaxT) return MOE_EUNSUPPORTED;
  if (T < 0) return MOE_EINVAL;
  if (!expert_offsets) return MOE_EINVAL;
  if (T > 0 && (!topk_ids || !sorted_slots || !slot_pos)) return MOE_EINVAL;
  int rc = check_ws(*cfg, T, workspace, workspace_bytes);
  if (rc) return rc;
  const Layout L = layout(*cfg, T);
  Perm p = perm_of(workspace, L, expert_offsets, sorted_slots, slot_pos);
  return status(launch_permute(T, cfg->n_routed_experts, cfg->top_k, topk_ids, p,
                               at<int32_t>(workspace, L.blk_counts), static_cast<hipStream_t>(stream)));
}

int moe_expert_ffn(const moe_config* cfg, int32_t T, const uint16_t* x, const int32_t* expert_offsets,
                   const int32_t* sorted_slots, const float* topk_w, const uint8_t* w13_codes,
                   const uint8_t* w13_scales, const uint8_t* w2_codes, const uint8_t* w2_scales,
                   float* routed_out, void* workspace, size_t workspace_bytes, void* stream) {
  if (!cfg) return MOE_EINVAL;
  if (!cfg_ok(cfg) || T > kMaxT) return MOE_EUNSUPPORTED;
  if (T < 0) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!x || !expert_offsets || !sorted_slots || !topk_w || !w13_codes || !w13_scales || !w2_codes ||
      !w2_scales || !routed_out)
    return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(w13_codes) || !aligned16(w2_codes) || !aligned16(w13_scales) ||
      !aligned16(w2_scales) || !aligned16(routed_out))
    return MOE_EINVAL;
  int rc = check_ws(*cfg, T, workspace, workspace_bytes);
  if (rc) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const Layout L = layout(*cfg, T);
  // the caller's permutation is checked and copied into the workspace
  Perm p = perm_of(workspace, L, at<int32_t>(workspace, L.offsets), at<int32_t>(workspace, L.sorted),
                   at<int32_t>(workspace, L.slot_pos));
  rc = status(launch_tiles_from_offsets(T, cfg->n_routed_experts, cfg->top_k, expert_offsets, sorted_slots, p, st));
  if (rc) return rc;
  uint16_t* hbuf = at<uint16_t>(workspace, L.hbuf);
  float* ybuf = at<float>(workspace, L.ybuf);
  if (L.mx) {
    rc = status(routed_gemms_mx(*cfg, T, x, p, topk_w, w13_codes, w13_scales, w2_codes, w2_scales, workspace, L,
                                reinterpret_cast<uint16_t*>(ybuf), st));
    if (rc) return rc;
  } else if (use_gemm(*cfg, T)) {
    GemmArgs g13 = gemm_routed_w13(*cfg, T, x, p, w13_codes, w13_scales, hbuf);
    GemmArgs g2 = gemm_routed_w2(*cfg, T, p, topk_w, w2_codes, w2_scales, hbuf, reinterpret_cast<uint16_t*>(ybuf));
    g13.queue = gemm_queue(workspace, L, kQRoutedW13);
    g2.queue = gemm_queue(workspace, L, kQRoutedW2);
    rc = status(timed(MOE_KERNEL_ROUTED_W13, st, [&] { return launch_gemm(g13, p.max_tiles, st); }));
    if (rc) return rc;
    rc = status(timed(MOE_KERNEL_ROUTED_W2, st, [&] { return launch_gemm(g2, p.max_tiles, st); }));
    if (rc) return rc;
  } else if (T <= kSmallT) {
    SkinnyArgs r13 = routed_w13_args(*cfg, T, x, p, w13_codes, w13_scales, hbuf);
    SkinnyArgs r2 = routed_w2_args(*cfg, T, p, topk_w, w2_codes, w2_scales, hbuf, ybuf);
    r13.n_rowblocks = cfg->moe_intermediate / 128;
    r2.n_rowblocks = (cfg->hidden_size + 255) / 256;
    rc = status(launch_tile_records(p, topk_w, st));
    if (rc) return rc;
    rc = status(timed(MOE_KERNEL_ROUTED_W13, st, [&] {
      return launch_stream(kW13, r13, p.max_tiles * r13.n_rowblocks, nullptr, 0, p.queues, st);
    }));
    if (rc) return rc;
    rc = status(timed(MOE_KERNEL_ROUTED_W2, st, [&] {
      return launch_stream(kW2, r2, p.max_tiles * r2.n_rowblocks, nullptr, 0, p.queues + 1, st);
    }));
    if (rc) return rc;
  } else {
    const SkinnyArgs r13 = routed_w13_args(*cfg, T, x, p, w13_codes, w13_scales, hbuf);
    const SkinnyArgs r2 = routed_w2_args(*cfg, T, p, topk_w, w2_codes, w2_scales, hbuf, ybuf);
    rc = status(timed(MOE_KERNEL_ROUTED_W13, st, [&] {
      return launch_w13(r13, p.max_tiles * r13.n_rowblocks, nullptr, 0, false, st);
    }));
    if (rc) return rc;
    rc = status(timed(MOE_KERNEL_ROUTED_W2, st,
                      [&] { return launch_w2(r2, p.max_tiles * r2.n_rowblocks, nullptr, 0, st); }));
    if (rc) return rc;
  }
  CombineArgs cb{T, cfg->hidden_size, cfg->top_k, ybuf, nullptr, routed_out, 1, use_gemm(*cfg, T) ? 1 : 0};
  return status(timed(MOE_KERNEL_COMBINE, st, [&] { return launch_combine(cb, st); }));
}

int moe_forward_stack(const moe_config* cfg, int32_t n_layers, const moe_layer_weights* layers, int32_t T,
                      const uint16_t* x, const int32_t* token_ids, uint16_t* act, void* out, int32_t out_is_fp32,
                      void* workspace, size_t workspace_bytes, void* stream) {
  if (!cfg || n_layers < 0 || T < 0) return MOE_EINVAL;
  if (!cfg_ok(cfg) || T > kMaxT) return MOE_EUNSUPPORTED;
  if (n_layers == 0 || T == 0) return MOE_OK;
  if (!layers || !x || !out || (n_layers > 1 && !act)) return MOE_EINVAL;
  if (act && !aligned16(act)) return MOE_EINVAL;
  for (int l = 0; l < n_layers; ++l)
    if (layers[l].tid2eid && !token_ids) return MOE_EINVAL;
  const size_t plane = (size_t)T * cfg->hidden_size;
  if (schedule(*cfg, T, false) == MOE_SCHED_SINGLE &&
      layer_stack_supported(cfg->hidden_size, cfg->moe_intermediate, cfg->n_routed_experts, T, cfg->top_k)) {
    // Every layer is one single-launch layer: up to kStackChunk of them per
    // launch, each layer's output rows handed to the next inside the launch.
    // Every layer's arguments are checked before anything is launched.
    if (!aligned16(x) || !aligned16(out)) return MOE_EINVAL;
    for (int l = 0; l < n_layers; ++l) {
      const moe_layer_weights& W = layers[l];
      const bool hash = W.tid2eid != nullptr;
      if (!W.gate_w || !W.w13_codes || !W.w13_scales || !W.w2_codes || !W.w2_scales || !W.sh_w13 ||
          !W.sh_w13_scale || !W.sh_w2 || !W.sh_w2_scale || (hash && W.V <= 0) || (!hash && !W.bias))
        return MOE_EINVAL;
      if (!aligned16(W.gate_w) || !aligned16(W.w13_codes) || !aligned16(W.w13_scales) || !aligned16(W.w2_codes) ||
          !aligned16(W.w2_scales) || !aligned16(W.sh_w13) || !aligned16(W.sh_w2))
        return MOE_EINVAL;
    }
    int rc = check_ws(*cfg, T, workspace, workspace_bytes);
    if (rc) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const Layout L = layout(*cfg, T);
    uint32_t* xfer = at<uint32_t>(workspace, L.xfer);
    int32_t* ids = at<int32_t>(workspace, L.ids);
    float* w = at<float>(workspace, L.w);
    for (int c0 = 0; c0 < n_layers; c0 += kStackChunk) {
      StackArgs sa;
      memset(&sa, 0, sizeof(sa));
      sa.n = std::min(kStackChunk, n_layers - c0);
      for (int j = 0; j < sa.n; ++j) {
        const int l = c0 + j;
        const moe_layer_weights& W = layers[l];
        const bool last = l == n_layers - 1;
        const uint16_t* in = l == 0 ? x : act + (size_t)((l - 1) & 1) * plane;  // read by the launch's first layer
        void* dst = last ? out : static_cast<void*>(act + (size_t)(l & 1) * plane);
        sa.layer[j] = single_layer_args(*cfg, T, in, W.gate_w, W.bias, W.logit_offset, token_ids, W.tid2eid, W.V,
                                        W.w13_codes, W.w13_scales, W.w2_codes, W.w2_scales, W.sh_w13,
                                        W.sh_w13_scale, W.sh_w2, W.sh_w2_scale, dst, last ? out_is_fp32 : 0, ids, w,
                                        xfer);
      }
      rc = status(timed(MOE_KERNEL_ROUTED_W13, st, [&] { return launch_layer_stack(sa, st); }));
      if (rc) return rc;
    }
    return MOE_OK;
  }
  for (int l = 0; l < n_layers; ++l) {
    const moe_layer_weights& W = layers[l];
    const bool hash = W.tid2eid != nullptr;
    const bool last = l == n_layers - 1;
    const uint16_t* in = l == 0 ? x : act + (size_t)((l - 1) & 1) * plane;
    void* dst = last ? out : static_cast<void*>(act + (size_t)(l & 1) * plane);
    const int rc = moe_forward(cfg, T, in, W.gate_w, W.bias, W.logit_offset, hash ? token_ids : nullptr,
                               W.tid2eid, W.V, W.w13_codes, W.w13_scales, W.w2_codes, W.w2_scales, W.sh_w13,
                               W.sh_w13_scale, W.sh_w2, W.sh_w2_scale, dst, last ? out_is_fp32 : 0, nullptr,
                               nullptr, workspace, workspace_bytes, stream);
    if (rc) return rc;
  }
  return MOE_OK;
}

// the split-K linear's arrival words: one per 64 rows of the largest
// projection (64 groups x 65536 rows), from byte 256
constexpr size_t kLinearPartOffset = 256 + (size_t)64 * 65536 / 64 * 4;

size_t moe_linear_workspace_size(int32_t T, int32_t K, int32_t N, int32_t groups) {
  if (T < 0 || T > kMaxT || K <= 0 || N <= 0 || groups <= 0 || K % 128 || N % 256 || K > 65536 || N > 65536 ||
      groups > 64)
    return 0;
  // counters (the GEMM's tile queue), then at decode sizes the split-K pass's
  // arrival words and its fp32 partial sums [split][T][groups*N]. The
  // arrival words sit at a fixed place, sized for the largest projection,
  // so that no call's partial sums land where another shape's words are
  // (the words must be zero before a launch; each call leaves its own zero).
  if (T == 0 || T > kSmallT) return 256;
  const int ks = linear_dec_ks(T, K, N, groups);
  if (ks == 0) return 0;
  const size_t rows = (size_t)groups * N;
  return kLinearPartOffset + align256((size_t)(K / ks) * T * rows * 4);
}

int moe_linear_w8a16(int32_t T, int32_t K, int32_t N, int32_t groups, const uint16_t* x, const int8_t* q,
                     const float* scale, void* out, int32_t out_is_fp32, void* workspace, size_t workspace_bytes,
                     void* stream) {
  if (T < 0 || K <= 0 || N <= 0 || groups <= 0) return MOE_EINVAL;
  const size_t need = moe_linear_workspace_size(T, K, N, groups);
  if (need == 0) return MOE_EUNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !q || !scale || !out || !workspace) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(q) || !aligned16(scale) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255))
    return MOE_EINVAL;
  if (workspace_bytes < need) return MOE_EWORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int32_t* counters = static_cast<int32_t*>(workspace);
  const int ldx = groups * K, ldo = groups * N;
  if (T > kSmallT) {  // grouped-GEMM kernel of the shared expert's w2, with no routed slots to add
    for (int g = 0; g < groups; ++g) {
      GemmArgs a;
      memset(&a, 0, sizeof(a));
      a.T = T;
      a.fmt = 1;
      a.mode = kGemmW2Combine;
      a.wq = reinterpret_cast<const uint8_t*>(q + (size_t)g * N * K);
      a.row_scale = scale + (size_t)g * N;
      a.K = K;
      a.routed = 0;
      a.n_ntiles = N / 256;
      a.act = x + (size_t)g * K;
      a.act_ld = ldx;
      a.topk = 0;
      a.out = out_is_fp32 ? static_cast<void*>(static_cast<float*>(out) + (size_t)g * N)
                          : static_cast<void*>(static_cast<uint16_t*>(out) + (size_t)g * N);
      a.out_ld = ldo;
      a.out_is_fp32 = out_is_fp32 ? 1 : 0;
      a.queue = counters;
      const int rc = status(launch_gemm(a, (T + kGemmTokens - 1) / kGemmTokens, st));
      if (rc) return rc;
    }
    return MOE_OK;
  }
  // decode sizes: every group in one split-K launch
  LinearDecArgs a;
  a.T = T;
  a.K = K;
  a.N = N;
  a.G = groups;
  a.ks = linear_dec_ks(T, K, N, groups);
  a.split = K / a.ks;
  a.x = x;
  a.q = q;
  a.scale = scale;
  a.out = out;
  a.out_is_fp32 = out_is_fp32 ? 1 : 0;
  a.count = at<int32_t>(workspace, 256);
  a.part = at<float>(workspace, kLinearPartOffset);
  return status(launch_linear_dec(a, st));
}

int moe_forward_schedule(const moe_config* cfg, int32_t T, int32_t hash) {
  if (!cfg) return MOE_EINVAL;
  if (!cfg_ok(cfg) || T > kMaxT) return MOE_EUNSUPPORTED;
  if (T < 0) return MOE_EINVAL;
  return schedule(*cfg, T, hash != 0);
}

static int forward_impl(const moe_config* cfg, int32_t T, const uint16_t* x, const float* gate_w,
                        const float* bias, const float* logit_offset, const int32_t* token_ids,
                        const int32_t* tid2eid, int32_t V, const uint8_t* w13_codes, const uint8_t* w13_scales,
                        const W2Weights& W2, const int8_t* sh_w13, const float* sh_w13_scale, const int8_t* sh_w2,
                        const float* sh_w2_scale, void* out, int32_t out_is_fp32, int32_t* topk_ids_out,
                        float* topk_w_out, void* workspace, size_t workspace_bytes, void* stream) {
  const uint8_t* w2_codes = W2.codes;
  const uint8_t* w2_scales = W2.scales;
  const bool q3 = W2.fmt == kFmtQ3;
  if (!cfg) return MOE_EINVAL;
  if (!cfg_ok(cfg) || T > kMaxT) return MOE_EUNSUPPORTED;
  if (T < 0) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (q3 && !w2q3_supported(*cfg, T)) return MOE_EUNSUPPORTED;
  const bool hash = token_ids != nullptr;
  if (!x || !gate_w || !w13_codes || !w13_scales || !w2_codes || !w2_scales || !sh_w13 || !sh_w13_scale ||
      !sh_w2 || !sh_w2_scale || !out)
    return MOE_EINVAL;
  if (hash && (!tid2eid || V <= 0)) return MOE_EINVAL;
  if (!hash && !bias) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(gate_w) || !aligned16(w13_codes) || !aligned16(w2_codes) ||
      !aligned16(w13_scales) || !aligned16(w2_scales) || !aligned16(sh_w13) || !aligned16(sh_w2) || !aligned16(out))
    return MOE_EINVAL;
  int rc = check_ws(*cfg, T, workspace, workspace_bytes);
  if (rc) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const Layout L = layout(*cfg, T);
  int32_t* ids = topk_ids_out ? topk_ids_out : at<int32_t>(workspace, L.ids);
  float* w = topk_w_out ? topk_w_out : at<float>(workspace, L.w);
  Perm p = perm_of(workspace, L, at<int32_t>(workspace, L.offsets), at<int32_t>(workspace, L.sorted),
                   at<int32_t>(workspace, L.slot_pos));
  uint16_t* hbuf = at<uint16_t>(workspace, L.hbuf);
  uint16_t* hs = at<uint16_t>(workspace, L.hs);
  float* ybuf = at<float>(workspace, L.ybuf);
  float* zbuf = at<float>(workspace, L.zbuf);
  int sh13_blocks = 0, sh13w_blocks = 0, sh2_blocks = 0;
  const SkinnyArgs s13 = shared_w13_args(*cfg, T, x, sh_w13, sh_w13_scale, hs, &sh13_blocks, true);
  const SkinnyArgs s13w = shared_w13_args(*cfg, T, x, sh_w13, sh_w13_scale, hs, &sh13w_blocks, false);
  const SkinnyArgs s2 = shared_w2_args(*cfg, T, sh_w2, sh_w2_scale, hs, zbuf, &sh2_blocks);
  const SkinnyArgs r13 = routed_w13_args(*cfg, T, x, p, w13_codes, w13_scales, hbuf);
  SkinnyArgs r2 = routed_w2_args(*cfg, T, p, w, w2_codes, w2_scales, hbuf, ybuf);
  if (q3) set_w2q3(*cfg, W2, r2);
  const int r13_blocks = p.max_tiles * r13.n_rowblocks, r2_blocks = p.max_tiles * r2.n_rowblocks;
  int sched = schedule(*cfg, T, hash);
  if (q3) {  // the 3-bit w2 runs in the single launch, the fused streaming launch or the GEMM
    if (sched == MOE_SCHED_SINGLE &&
        !layer_small_supported(cfg->hidden_size, cfg->moe_intermediate, cfg->n_routed_experts, T, cfg->top_k, true))
      sched = MOE_SCHED_DECODE;
    if (sched == MOE_SCHED_TINY) sched = MOE_SCHED_DECODE;
  }
  const bool tiny = sched == MOE_SCHED_TINY;
  const bool decode = sched == MOE_SCHED_DECODE;

  if (sched == MOE_SCHED_SINGLE) {
    // the whole layer in one launch, one block per CU
    LayerArgs la = single_layer_args(*cfg, T, x, gate_w, bias, logit_offset, token_ids, hash ? tid2eid : nullptr,
                                     V, w13_codes, w13_scales, w2_codes, w2_scales, sh_w13, sh_w13_scale, sh_w2,
                                     sh_w2_scale, out, out_is_fp32, ids, w, at<uint32_t>(workspace, L.xfer));
    la.w2tab = W2.table;
    la.w2q3 = q3 ? 1 : 0;
    return status(timed(MOE_KERNEL_ROUTED_W13, st, [&] { return launch_layer_small(la, st); }));
  }
  if (tiny) {
    // router logits + shared w13 | routed w13 (top-k in each block, one tile
    // per slot) | routed w2 + shared w2 + combine
    RouterArgs a = router_args(*cfg, T, x, gate_w, bias, logit_offset, at<float>(workspace, L.scores), ids, w);
    rc = status(timed(MOE_KERNEL_ROUTER, st, [&] { return launch_router_small(a, &s13, sh13_blocks, st); }));
    if (rc) return rc;
    SkinnyArgs t13 = r13;
    t13.routed = 2;
    t13.tile_n = 1;
    t13.n_tiles_grid = T * cfg->top_k;
    t13.act_row = nullptr;
    t13.scores = a.scores;
    t13.keys = a.keys;
    t13.scale = cfg->routed_scaling_factor;
    t13.E = cfg->n_routed_experts;
    t13.topk = cfg->top_k;
    t13.ids_out = ids;
    t13.w_out = w;
    const int t13_blocks = t13.n_tiles_grid * t13.n_rowblocks;
    rc = status(timed(MOE_KERNEL_ROUTED_W13, st, [&] { return launch_w13_deep(t13, t13_blocks, st); }));
    if (rc) return rc;
    W2CombineArgs c2{T, cfg->hidden_size, cfg->moe_intermediate, cfg->top_k, w2_codes, w2_scales, ids, w, hbuf,
                     sh_w2, sh_w2_scale, hs, out, out_is_fp32 ? 1 : 0};
    return status(timed(MOE_KERNEL_ROUTED_W2, st, [&] { return launch_w2_combine_small(c2, st); }));
  }
  if (decode) {
    // router | top-k (or the hash table) + permutation | routed w13 + shared w13 | routed w2 +
    // shared w2 | combine, the expert passes as streaming blocks
    RouterArgs a = router_args(*cfg, T, x, gate_w, hash ? nullptr : bias, hash ? nullptr : logit_offset,
                               at<float>(workspace, L.scores), ids, w);
    if (hash) {
      a.token_ids = token_ids;
      a.tid2eid = tid2eid;
      a.V = V;
    }
    rc = status(timed(MOE_KERNEL_ROUTER, st, [&] { return launch_router_dec(a, st); }));
    if (rc) return rc;
    rc = status(timed(MOE_KERNEL_PERMUTE, st, [&] {
      return launch_topk_permute_small(a, p, at<int32_t>(workspace, L.counters) + kArrivalsInt, st);
    }));
    if (rc) return rc;
    const int H = cfg->hidden_size, I = cfg->moe_intermediate;
    SkinnyArgs g13 = r13, g2 = r2, h13 = s13w, h2 = s2;
    g13.n_rowblocks = h13.n_rowblocks = I / 128;
    g2.n_rowblocks = h2.n_rowblocks = (H + 255) / 256;
    // the same shared tiles for both stages (one launch needs them alike)
    h13.tile_n = h2.tile_n = std::min(shared_stream_tile(T, H), shared_stream_tile(T, I));
    h13.n_tiles_grid = h2.n_tiles_grid = (T + h13.tile_n - 1) / h13.tile_n;
    if (H % 1024 == 0 && I % 1024 == 0) {  // both stages in one launch
      rc = status(timed(MOE_KERNEL_ROUTED_W13, st, [&] {
        return launch_stream_fused(g13, h13, g2, h2, p.max_tiles * g13.n_rowblocks,
                                   h13.n_tiles_grid * h13.n_rowblocks, p.max_tiles * g2.n_rowblocks,
                                   h2.n_tiles_grid * h2.n_rowblocks, p.queues, p.done, p.done + p.max_tiles, st);
      }));
      if (rc) return rc;
    } else {
      rc = status(timed(MOE_KERNEL_ROUTED_W13, st, [&] {
        return launch_stream(kW13, g13, p.max_tiles * g13.n_rowblocks, &h13, h13.n_tiles_grid * h13.n_rowblocks,
                             p.queues, st);
      }));
      if (rc) return rc;
      rc = status(timed(MOE_KERNEL_ROUTED_W2, st, [&] {
        return launch_stream(kW2, g2, p.max_tiles * g2.n_rowblocks, &h2, h2.n_tiles_grid * h2.n_rowblocks,
                             p.queues + 1, st);
      }));
      if (rc) return rc;
    }
  } else {
    // route | permutation | routed w13 + shared w13 | routed w2 + shared w2 | combine
    if (hash) {
      HashArgs h;
      h.T = T;
      h.H = cfg->hidden_size;
      h.E = cfg->n_routed_experts;
      h.k = cfg->top_k;
      h.V = V;
      h.scale = cfg->routed_scaling_factor;
      h.x = x;
      h.token_ids = token_ids;
      h.tid2eid = tid2eid;
      h.gate_w = gate_w;
      h.ids = ids;
      h.w = w;
      h.flags = p.flags;
      rc = status(timed(MOE_KERNEL_ROUTER, st, [&] { return launch_hash_route(h, st); }));
    } else {
      RouterArgs a = router_args(*cfg, T, x, gate_w, bias, logit_offset, at<float>(workspace, L.scores), ids, w);
      rc = status(timed(MOE_KERNEL_ROUTER, st, [&] {
        return launch_router_mfma(a, at<uint16_t>(workspace, L.wsplit), at<float>(workspace, L.plog), st);
      }));
    }
    if (rc) return rc;
    rc = status(timed(MOE_KERNEL_PERMUTE, st, [&] {
      return launch_permute(T, cfg->n_routed_experts, cfg->top_k, ids, p, at<int32_t>(workspace, L.blk_counts),
                            st);
    }));
    if (rc) return rc;
    if (use_gemm(*cfg, T)) {
      // grouped GEMMs; the shared expert's w2 finishes with the combine
      GemmArgs g13 = gemm_routed_w13(*cfg, T, x, p, w13_codes, w13_scales, hbuf);
      GemmArgs h13 = gemm_shared_w13(*cfg, T, x, sh_w13, sh_w13_scale, hs);
      uint16_t* ybf = reinterpret_cast<uint16_t*>(ybuf);  // the slot outputs in bf16 here
      GemmArgs g2 = gemm_routed_w2(*cfg, T, p, w, w2_codes, w2_scales, hbuf, ybf);
      if (q3) set_w2q3(*cfg, W2, g2);
      GemmArgs h2 = gemm_shared_w2_combine(*cfg, T, sh_w2, sh_w2_scale, hs, ybf, out, out_is_fp32 ? 1 : 0);
      g13.queue = gemm_queue(workspace, L, kQRoutedW13);
      h13.queue = gemm_queue(workspace, L, kQSharedW13);
      g2.queue = gemm_queue(workspace, L, kQRoutedW2);
      h2.queue = gemm_queue(workspace, L, kQSharedW2);
      const int sh_tiles = (T + kGemmTokens - 1) / kGemmTokens;
      if (L.mx && !q3) {
        rc = status(routed_gemms_mx(*cfg, T, x, p, w, w13_codes, w13_scales, w2_codes, w2_scales, workspace, L, ybf,
                                    st));
        if (rc) return rc;
        rc = status(timed(MOE_KERNEL_SHARED_W13, st, [&] { return launch_gemm(h13, sh_tiles, st); }));
        if (rc) return rc;
        return status(timed(MOE_KERNEL_SHARED_W2, st, [&] { return launch_gemm(h2, sh_tiles, st); }));
      }
      rc = status(timed(MOE_KERNEL_ROUTED_W13, st, [&] { return launch_gemm(g13, p.max_tiles, st); }));
      if (rc) return rc;
      rc = status(timed(MOE_KERNEL_SHARED_W13, st, [&] { return launch_gemm(h13, sh_tiles, st); }));
      if (rc) return rc;
      rc = status(timed(MOE_KERNEL_ROUTED_W2, st, [&] { return launch_gemm(g2, p.max_tiles, st); }));
      if (rc) return rc;
      return status(timed(MOE_KERNEL_SHARED_W2, st, [&] { return launch_gemm(h2, sh_tiles, st); }));
    }
    rc = status(timed(MOE_KERNEL_ROUTED_W13, st,
                      [&] { return launch_w13(r13, r13_blocks, &s13w, sh13w_blocks, false, st); }));
    if (rc) return rc;
    rc = status(timed(MOE_KERNEL_ROUTED_W2, st, [&] { return launch_w2(r2, r2_blocks, &s2, sh2_blocks, st); }));
    if (rc) return rc;
  }
  CombineArgs cb{T, cfg->hidden_size, cfg->top_k, ybuf, zbuf, out, out_is_fp32 ? 1 : 0, 0};
  return status(timed(MOE_KERNEL_COMBINE, st, [&] { return launch_combine(cb, st); }));
}

int moe_forward(const moe_config* cfg, int32_t T, const uint16_t* x, const float* gate_w, const float* bias,
                const float* logit_offset, const int32_t* token_ids, const int32_t* tid2eid, int32_t V,
                const uint8_t* w13_codes, const uint8_t* w13_scales, const uint8_t* w2_codes,
                const uint8_t* w2_scales, const int8_t* sh_w13, const float* sh_w13_scale,
                const int8_t* sh_w2, const float* sh_w2_scale, void* out, int32_t out_is_fp32,
                int32_t* topk_ids_out, float* topk_w_out, void* workspace, size_t workspace_bytes,
                void* stream) {
  const W2Weights W2{kFmtMx, w2_codes, w2_scales, nullptr};
  return forward_impl(cfg, T, x, gate_w, bias, logit_offset, token_ids, tid2eid, V, w13_codes, w13_scales, W2,
                      sh_w13, sh_w13_scale, sh_w2, sh_w2_scale, out, out_is_fp32, topk_ids_out, topk_w_out,
                      workspace, workspace_bytes, stream);
}

int moe_forward_w2q3(const moe_config* cfg, int32_t T, const uint16_t* x, const float* gate_w, const float* bias,
                     const float* logit_offset, const int32_t* token_ids, const int32_t* tid2eid, int32_t V,
                     const uint8_t* w13_codes, const uint8_t* w13_scales, const uint8_t* w2_codes,
                     const uint16_t* w2_scales, const float* w2_levels, const int8_t* sh_w13,
                     const float* sh_w13_scale, const int8_t* sh_w2, const float* sh_w2_scale, void* out,
                     int32_t out_is_fp32, int32_t* topk_ids_out, float* topk_w_out, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (w2_levels && !aligned16(w2_levels)) return MOE_EINVAL;
  const W2Weights W2{kFmtQ3, w2_codes, reinterpret_cast<const uint8_t*>(w2_scales), w2_levels};
  return forward_impl(cfg, T, x, gate_w, bias, logit_offset, token_ids, tid2eid, V, w13_codes, w13_scales, W2,
                      sh_w13, sh_w13_scale, sh_w2, sh_w2_scale, out, out_is_fp32, topk_ids_out, topk_w_out,
                      workspace, workspace_bytes, stream);
}

}  // extern "C"
