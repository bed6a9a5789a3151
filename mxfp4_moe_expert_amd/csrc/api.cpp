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
constexpr size_t kLdsBudget = 136 * 1024;  // activation tile bytes per block

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct Layout {
  size_t counters, logits, ids, w, offsets, sorted, slot_pos, tile_off, blk_counts, hbuf, hs, ybuf,
      zbuf, total;
};

bool cfg_ok(const moe_config* c) {
  if (!c) return false;
  const int H = c->hidden_size, E = c->n_routed_experts, k = c->top_k, I = c->moe_intermediate;
  if (H < 128 || H % 128 || H > 32768) return false;
  if (I < 128 || I % 128 || I > 32768) return false;
  if (k < 1 || k > kMaxTopK || E < k || E > kMaxExperts) return false;
  if (!(c->routed_scaling_factor == c->routed_scaling_factor)) return false;
  if (!(c->swiglu_limit == c->swiglu_limit)) return false;
  return true;
}

Layout layout(const moe_config& c, int T) {
  const size_t H = c.hidden_size, E = c.n_routed_experts, k = c.top_k, I = c.moe_intermediate;
  const size_t slots = (size_t)T * k;
  const size_t nblk = (slots + kPermBlock - 1) / kPermBlock;
  Layout L;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  L.counters = take(kNumCounters * sizeof(unsigned));
  L.logits = take((size_t)T * E * 4);
  L.ids = take(slots * 4);
  L.w = take(slots * 4);
  L.offsets = take((E + 1) * 4);
  L.sorted = take(slots * 4);
  L.slot_pos = take(slots * 4);
  L.tile_off = take((E + 1) * 4);
  L.blk_counts = take(nblk * E * 4);
  L.hbuf = take(slots * I * 2);
  L.hs = take((size_t)T * I * 2);
  L.ybuf = take(slots * H * 4);
  L.zbuf = take((size_t)T * H * 4);
  L.total = o;
  return L;
}

template <class P>
inline P* at(void* ws, size_t off) {
  return reinterpret_cast<P*>(static_cast<char*>(ws) + off);
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

// Columns per expert tile: as few as the expected tokens per expert need, so
// the LDS activation tile stays small at decode sizes.
int routed_tile_n(const moe_config& c, int T) {
  int tn = T <= 1 ? 1 : (T <= kSmallT ? 4 : 16);
  const int maxk = c.hidden_size > c.moe_intermediate ? c.hidden_size : c.moe_intermediate;
  while (tn > 1 && (size_t)tn * (2 * (size_t)maxk + 16) > kLdsBudget) tn >>= 1;
  return tn;
}

int shared_tile_n(const moe_config& c, int T) {
  int tn = T < 16 ? T : 16;
  const int maxk = c.hidden_size > c.moe_intermediate ? c.hidden_size : c.moe_intermediate;
  while (tn > 1 && (size_t)tn * (2 * (size_t)maxk + 16) > kLdsBudget) tn >>= 1;
  return tn < 1 ? 1 : tn;
}

int routed_max_tiles(const moe_config& c, int T, int tile_n) {
  const long long slots = (long long)T * c.top_k;
  long long by_width = (slots + tile_n - 1) / tile_n + (slots < c.n_routed_experts ? slots : c.n_routed_experts);
  return (int)(by_width < slots ? by_width : slots);
}

SkinnyArgs skinny_common(const moe_config& c, int T) {
  SkinnyArgs a;
  memset(&a, 0, sizeof(a));
  a.T = T;
  a.topk = c.top_k;
  a.E = c.n_routed_experts;
  a.limit = c.swiglu_limit;
  return a;
}

// Routed experts: w13 + SwiGLU -> hbuf (sorted order), w2 x weight -> ybuf (slot order).
int run_routed(const moe_config& c, int T, const uint16_t* x, const int32_t* offsets,
               const int32_t* sorted, const int32_t* tile_off, int tile_n, const float* slot_w,
               const uint8_t* w13c, const uint8_t* w13s, const uint8_t* w2c, const uint8_t* w2s,
               uint16_t* hbuf, float* ybuf, hipStream_t st) {
  const int H = c.hidden_size, I = c.moe_intermediate;
  const int max_tiles = routed_max_tiles(c, T, tile_n);
  SkinnyArgs a = skinny_common(c, T);
  a.routed = 1;
  a.offsets = offsets;
  a.sorted_slots = sorted;
  a.tile_off = tile_off;
  a.tile_n = tile_n;
  a.n_tiles_grid = max_tiles;
  // w13: K = H, rows [0, I) gate and [I, 2I) up, output h [slots][I]
  a.wq = w13c;
  a.wsc = w13s;
  a.q_expert_stride = (long long)2 * I * (H / 2);
  a.s_expert_stride = (long long)2 * I * (H / 32);
  a.K = H;
  a.half = I;
  a.act = x;
  a.act_ld = H;
  a.act_is_x = 1;
  a.n_rowblocks = I / 16;
  a.hout = hbuf;
  a.hout_ld = I;
  int rc = status(launch_skinny_w13_mxfp4(a, max_tiles, st));
  if (rc) return rc;
  // w2: K = I, output rows H, y * w -> ybuf[slot]
  a.wq = w2c;
  a.wsc = w2s;
  a.q_expert_stride = (long long)H * (I / 2);
  a.s_expert_stride = (long long)H * (I / 32);
  a.K = I;
  a.half = 0;
  a.act = hbuf;
  a.act_ld = I;
  a.act_is_x = 0;
  a.n_rowblocks = H / 16;
  a.yout = ybuf;
  a.yout_ld = H;
  a.slot_w = slot_w;
  return status(launch_skinny_w2_mxfp4(a, max_tiles, st));
}

// Shared expert: int8 w13 + SwiGLU -> hs [T][I], int8 w2 -> zbuf [T][H].
int run_shared(const moe_config& c, int T, const uint16_t* x, const int8_t* q13, const float* s13,
               const int8_t* q2, const float* s2, uint16_t* hs, float* zbuf, hipStream_t st) {
  const int H = c.hidden_size, I = c.moe_intermediate;
  const int tn = shared_tile_n(c, T);
  const int ntiles = (T + tn - 1) / tn;
  SkinnyArgs a = skinny_common(c, T);
  a.routed = 0;
  a.tile_n = tn;
  a.n_tiles_grid = ntiles;
  a.wq = reinterpret_cast<const uint8_t*>(q13);
  a.row_scale = s13;
  a.K = H;
  a.half = I;
  a.act = x;
  a.act_ld = H;
  a.n_rowblocks = I / 16;
  a.hout = hs;
  a.hout_ld = I;
  int rc = status(launch_skinny_w13_int8(a, ntiles, st));
  if (rc) return rc;
  a.wq = reinterpret_cast<const uint8_t*>(q2);
  a.row_scale = s2;
  a.K = I;
  a.half = 0;
  a.act = hs;
  a.act_ld = I;
  a.n_rowblocks = H / 16;
  a.yout = zbuf;
  a.yout_ld = H;
  return status(launch_skinny_w2_int8(a, ntiles, st));
}

int check_ws(const moe_config& c, int T, const void* ws, size_t bytes) {
  if (!ws) return MOE_EINVAL;
  if (reinterpret_cast<uintptr_t>(ws) & 255) return MOE_EINVAL;
  if (bytes < layout(c, T).total) return MOE_EWORKSPACE;
  return MOE_OK;
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

const char* moe_version(void) { return "0.1.0"; }

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
  const Layout L = layout(*cfg, T);
  RouterArgs a;
  memset(&a, 0, sizeof(a));
  a.T = T;
  a.H = cfg->hidden_size;
  a.E = cfg->n_routed_experts;
  a.k = cfg->top_k;
  a.scale = cfg->routed_scaling_factor;
  a.x = x;
  a.gate_w = gate_w;
  a.bias = bias;
  a.logit_offset = logit_offset;
  a.logits = at<float>(workspace, L.logits);
  a.ids = topk_ids;
  a.w = topk_w;
  a.counter = at<unsigned>(workspace, L.counters);
  a.perm = 0;
  return status(launch_router(a, static_cast<hipStream_t>(stream)));
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
  PermuteArgs a;
  a.T = T;
  a.E = cfg->n_routed_experts;
  a.k = cfg->top_k;
  a.tile_n = routed_tile_n(*cfg, T);
  a.ids = topk_ids;
  a.offsets = expert_offsets;
  a.sorted_slots = sorted_slots;
  a.slot_pos = slot_pos;
  a.tile_off = at<int32_t>(workspace, L.tile_off);
  a.blk_counts = at<int32_t>(workspace, L.blk_counts);
  return status(launch_permute(a, static_cast<hipStream_t>(stream)));
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
  if (!aligned16(x) || !aligned16(w13_codes) || !aligned16(w2_codes) || !aligned16(routed_out))
    return MOE_EINVAL;
  int rc = check_ws(*cfg, T, workspace, workspace_bytes);
  if (rc) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const Layout L = layout(*cfg, T);
  const int tile_n = routed_tile_n(*cfg, T);
  int32_t* tile_off = at<int32_t>(workspace, L.tile_off);
  rc = status(launch_tile_offsets(cfg->n_routed_experts, tile_n, expert_offsets, tile_off, st));
  if (rc) return rc;
  rc = run_routed(*cfg, T, x, expert_offsets, sorted_slots, tile_off, tile_n, topk_w, w13_codes, w13_scales,
                  w2_codes, w2_scales, at<uint16_t>(workspace, L.hbuf), at<float>(workspace, L.ybuf), st);
  if (rc) return rc;
  CombineArgs cb;
  cb.T = T;
  cb.H = cfg->hidden_size;
  cb.k = cfg->top_k;
  cb.ybuf = at<float>(workspace, L.ybuf);
  cb.zbuf = nullptr;
  cb.out = routed_out;
  cb.out_is_fp32 = 1;
  return status(launch_combine(cb, st));
}

int moe_forward(const moe_config* cfg, int32_t T, const uint16_t* x, const float* gate_w, const float* bias,
                const float* logit_offset, const int32_t* token_ids, const int32_t* tid2eid, int32_t V,
                const uint8_t* w13_codes, const uint8_t* w13_scales, const uint8_t* w2_codes,
                const uint8_t* w2_scales, const int8_t* sh_w13, const float* sh_w13_scale,
                const int8_t* sh_w2, const float* sh_w2_scale, void* out, int32_t out_is_fp32,
                int32_t* topk_ids_out, float* topk_w_out, void* workspace, size_t workspace_bytes,
                void* stream) {
  if (!cfg) return MOE_EINVAL;
  if (!cfg_ok(cfg) || T > kMaxT) return MOE_EUNSUPPORTED;
  if (T < 0) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  const bool hash = token_ids != nullptr;
  if (!x || !gate_w || !w13_codes || !w13_scales || !w2_codes || !w2_scales || !sh_w13 || !sh_w13_scale ||
      !sh_w2 || !sh_w2_scale || !out)
    return MOE_EINVAL;
  if (hash && (!tid2eid || V <= 0)) return MOE_EINVAL;
  if (!hash && !bias) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(gate_w) || !aligned16(w13_codes) || !aligned16(w2_codes) ||
      !aligned16(sh_w13) || !aligned16(sh_w2) || !aligned16(out))
    return MOE_EINVAL;
  int rc = check_ws(*cfg, T, workspace, workspace_bytes);
  if (rc) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const Layout L = layout(*cfg, T);
  const int tile_n = routed_tile_n(*cfg, T);
  int32_t* ids = topk_ids_out ? topk_ids_out : at<int32_t>(workspace, L.ids);
  float* w = topk_w_out ? topk_w_out : at<float>(workspace, L.w);
  int32_t* offsets = at<int32_t>(workspace, L.offsets);
  int32_t* sorted = at<int32_t>(workspace, L.sorted);
  int32_t* slot_pos = at<int32_t>(workspace, L.slot_pos);
  int32_t* tile_off = at<int32_t>(workspace, L.tile_off);

  bool permuted = false;
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
    rc = status(launch_hash_route(h, st));
  } else {
    RouterArgs a;
    memset(&a, 0, sizeof(a));
    a.T = T;
    a.H = cfg->hidden_size;
    a.E = cfg->n_routed_experts;
    a.k = cfg->top_k;
    a.scale = cfg->routed_scaling_factor;
    a.x = x;
    a.gate_w = gate_w;
    a.bias = bias;
    a.logit_offset = logit_offset;
    a.logits = at<float>(workspace, L.logits);
    a.ids = ids;
    a.w = w;
    a.counter = at<unsigned>(workspace, L.counters);
    a.perm = T <= kSmallT ? 1 : 0;
    a.tile_n = tile_n;
    a.offsets = offsets;
    a.sorted_slots = sorted;
    a.slot_pos = slot_pos;
    a.tile_off = tile_off;
    permuted = a.perm != 0;
    rc = status(launch_router(a, st));
  }
  if (rc) return rc;
  if (!permuted) {
    PermuteArgs p;
    p.T = T;
    p.E = cfg->n_routed_experts;
    p.k = cfg->top_k;
    p.tile_n = tile_n;
    p.ids = ids;
    p.offsets = offsets;
    p.sorted_slots = sorted;
    p.slot_pos = slot_pos;
    p.tile_off = tile_off;
    p.blk_counts = at<int32_t>(workspace, L.blk_counts);
    rc = status(launch_permute(p, st));
    if (rc) return rc;
  }
  rc = run_shared(*cfg, T, x, sh_w13, sh_w13_scale, sh_w2, sh_w2_scale, at<uint16_t>(workspace, L.hs),
                  at<float>(workspace, L.zbuf), st);
  if (rc) return rc;
  rc = run_routed(*cfg, T, x, offsets, sorted, tile_off, tile_n, w, w13_codes, w13_scales, w2_codes, w2_scales,
                  at<uint16_t>(workspace, L.hbuf), at<float>(workspace, L.ybuf), st);
  if (rc) return rc;
  CombineArgs cb;
  cb.T = T;
  cb.H = cfg->hidden_size;
  cb.k = cfg->top_k;
  cb.ybuf = at<float>(workspace, L.ybuf);
  cb.zbuf = at<float>(workspace, L.zbuf);
  cb.out = out;
  cb.out_is_fp32 = out_is_fp32 ? 1 : 0;
  return status(launch_combine(cb, st));
}

}  // extern "C"
