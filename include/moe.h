/*
 * moe.h — C ABI of a DeepSeek-V4-Flash MoE feed-forward layer for AMD
 * Instinct MI355X (gfx950).
 *
 * The layer (page "DeepSeek-V4-Flash export design", section "Source
 * configuration"; page "deepseek-v4-mxfp4-int8 config.json"):
 *   scores  s[t,e] = sqrt(softplus(x_t . Wg_e (+ logit_offset_e)))
 *   select  the top_k experts of s[t,e] + e_score_correction_bias[e]
 *           (bias selects only; page "DeepSeek-V4-Flash-0731", section
 *           "Checked in its code", rows "Mixture of experts" and
 *           "Auxiliary-loss-free load balancing (selection bias)")
 *   weights w[t,j] = routed_scaling_factor * s[t,e_j] / sum_j s[t,e_j]
 *           (norm_topk_prob, routed_scaling_factor 1.5)
 *   or, on hash layers, e_j = tid2eid[token_id[t], j] (num_hash_layers 3)
 *   expert  y = W2 * (silu(min(W1 x, L)) * clamp(W3 x, -L, L)), L = swiglu_limit
 *           (same section, row "SwiGLU feed-forward")
 *   out[t]  = sum_j w[t,j] * y_{e_j}(x_t) + shared(x_t)
 *           (same section, row "Shared expert")
 *
 * Data formats (page "deepseek-v4-mxfp4-int8 config.json",
 * quantization_config):
 *   routed experts, "w4a16": MXFP4 — E2M1 codes, two per byte, element 2i in
 *     the low nibble of byte i; one E8M0 exponent byte per 32 consecutive
 *     weights along the input dimension (value 2^(b-127)). Layouts:
 *       w13_codes  [E][2I][H/2]  u8   rows [0,I) gate (w1), rows [I,2I) up (w3)
 *       w13_scales [E][2I][H/32] u8
 *       w2_codes   [E][H][I/2]   u8
 *       w2_scales  [E][H][I/32]  u8
 *   shared expert, "w8a16": int8, symmetric, one fp32 scale per output row:
 *       sh_w13 [2I][H] i8 + sh_w13_scale [2I] f32; sh_w2 [H][I] i8 + sh_w2_scale [H] f32
 *   router ("*.gate.*" is not quantised): gate_w [E][H] f32, bias [E] f32
 *   activations: x [T][H] bf16 (raw 16-bit patterns); the intermediate
 *     activation entering w2 is rounded to bf16.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers (HIP), row-major, contiguous.
 *     The caller owns every buffer. Inputs are read only; outputs are
 *     overwritten (never accumulated into).
 *   - `stream` is a hipStream_t (NULL = the default stream). Work is queued
 *     on it asynchronously; the library never synchronises the host with the
 *     device and never allocates or frees device memory.
 *   - The return value reports host-side argument checks and launch errors
 *     only: MOE_OK, or a negative MOE_E* code, in which case nothing was
 *     launched (argument errors) or a launch failed (MOE_EHIP).
 *   - Device-side values are trusted: expert ids must lie in [0, E), token
 *     ids in [0, V); E8M0 scale bytes should not be 0xFF (NaN).
 *   - `workspace` is device scratch of at least moe_workspace_size() bytes,
 *     256-byte aligned. Zero-fill it once before its first use
 *     (moe_workspace_init, or any zero fill): bytes 64 .. 67 count the
 *     blocks of the decode-size top-k, bytes 96 .. 239 hold the tile
 *     queues of the grouped GEMMs (MOE_SCHED_LARGE), and bytes 256 ..
 *     136447 hold the hand-off state of the single-launch layer
 *     (MOE_SCHED_SINGLE); every call leaves all three ready for the next,
 *     and every other workspace value is written before it is read. Calls that share one workspace must be
 *     ordered on one stream. If a single-launch call's bounded wait for
 *     another block of its grid expires (about a second), its output is
 *     NaN; the hand-off state stays consistent.
 *   - Supported shapes: H and I multiples of 128, 1 <= top_k <= 8,
 *     top_k <= E <= 256, 0 <= T <= 65536. Device pointers must be 16-byte
 *     aligned.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Layer hyper-parameters; the names are those of the checkpoint's config.json. */
typedef struct moe_config {
  int32_t hidden_size;          /* H: 4096 */
  int32_t n_routed_experts;     /* E: 256 */
  int32_t top_k;                /* num_experts_per_tok: 6 */
  int32_t moe_intermediate;     /* I: moe_intermediate_size, 2048 */
  float routed_scaling_factor;  /* 1.5 */
  float swiglu_limit;           /* 10.0 */
} moe_config;

enum {
  MOE_OK = 0,
  MOE_EINVAL = -1,       /* null pointer, negative size, misaligned pointer */
  MOE_EUNSUPPORTED = -2, /* shape outside the supported limits */
  MOE_EWORKSPACE = -3,   /* workspace too small */
  MOE_EHIP = -4          /* a HIP launch or runtime call failed */
};

/* Human-readable name of a status code (static string). */
const char* moe_status_string(int status);

/* Library version, "major.minor.patch". */
const char* moe_version(void);

/* Bytes of workspace every entry point needs for T tokens with this
 * configuration (one size serves all entry points). Returns 0 if cfg is
 * invalid or unsupported. */
size_t moe_workspace_size(const moe_config* cfg, int32_t T);

/* Zero-fill a workspace on `stream` (with a fill kernel, so it may be
 * captured in a HIP graph). Needed once before a workspace's first use,
 * unless it was allocated zeroed. */
int moe_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/* Learned router: scores, bias-assisted top-k, renormalised weights.
 *   x            [T][H] bf16
 *   gate_w       [E][H] f32   router weight
 *   bias         [E]    f32   e_score_correction_bias (selection only)
 *   logit_offset [E]    f32 or NULL: added to every logit of expert e before
 *                the score (a synthetic load-skew knob; NULL = the model)
 *   topk_ids     [T][k] i32 out: chosen experts, by biased score descending,
 *                ties to the lower expert id
 *   topk_w       [T][k] f32 out: routed_scaling_factor * s / sum(s)
 * Logits are fp32 sums of bf16 x times fp32 Wg; the selection is decided on
 * the fp32 values s + bias. */
int moe_route(const moe_config* cfg, int32_t T, const uint16_t* x, const float* gate_w,
              const float* bias, const float* logit_offset, int32_t* topk_ids, float* topk_w,
              void* workspace, size_t workspace_bytes, void* stream);

/* Hash router of the first num_hash_layers layers (page "Tidalluna/
 * DeepSeek-V4-Flash-0731-Tina-CQ4KM", section "Compatibility", item 2):
 *   topk_ids[t][j] = tid2eid[token_ids[t]][j], in table order;
 *   topk_w[t][j]   = routed_scaling_factor * s[t,e_j] / sum_j s[t,e_j] with the
 *                    sqrt-softplus scores of those experts (no bias).
 *   token_ids [T] i32 in [0, V);  tid2eid [V][k] i32 in [0, E). */
int moe_hash_route(const moe_config* cfg, int32_t T, const uint16_t* x, const int32_t* token_ids,
                   const int32_t* tid2eid, int32_t V, const float* gate_w, int32_t* topk_ids,
                   float* topk_w, void* stream);

/* Stable counting sort of the T*k slots (slot = t*k + j) by expert:
 *   expert_offsets [E+1] i32 out: first sorted position of each expert,
 *                  expert_offsets[E] = T*k
 *   sorted_slots   [T*k] i32 out: slot at each sorted position; slots of one
 *                  expert appear in ascending slot order
 *   slot_pos       [T*k] i32 out: sorted position of each slot (inverse). */
int moe_permute(const moe_config* cfg, int32_t T, const int32_t* topk_ids,
                int32_t* expert_offsets, int32_t* sorted_slots, int32_t* slot_pos, void* workspace,
                size_t workspace_bytes, void* stream);

/* Routed experts only, given a permutation from moe_permute:
 *   routed_out[t] = sum_j topk_w[t][j] * y_{e_j}(x_t), fp32 [T][H], written in
 *   slot order j = 0..k-1 for each token (deterministic).
 * expert_offsets, sorted_slots: as written by moe_permute for the same
 * topk ids; topk_w [T][k] f32. */
int moe_expert_ffn(const moe_config* cfg, int32_t T, const uint16_t* x,
                   const int32_t* expert_offsets, const int32_t* sorted_slots, const float* topk_w,
                   const uint8_t* w13_codes, const uint8_t* w13_scales, const uint8_t* w2_codes,
                   const uint8_t* w2_scales, float* routed_out, void* workspace,
                   size_t workspace_bytes, void* stream);

/* The whole layer: route (learned, or hash when token_ids != NULL), permute,
 * routed experts, shared expert, combine.
 *   out         [T][H]: bf16 if out_is_fp32 == 0, else fp32. The bf16 output
 *               is the round-to-nearest-even of the fp32 output.
 *   topk_ids_out, topk_w_out: optional [T][k] copies of the routing (NULL to skip).
 * On a hash layer bias and logit_offset are ignored and tid2eid/V are used. */
int moe_forward(const moe_config* cfg, int32_t T, const uint16_t* x, const float* gate_w,
                const float* bias, const float* logit_offset, const int32_t* token_ids,
                const int32_t* tid2eid, int32_t V, const uint8_t* w13_codes,
                const uint8_t* w13_scales, const uint8_t* w2_codes, const uint8_t* w2_scales,
                const int8_t* sh_w13, const float* sh_w13_scale, const int8_t* sh_w2,
                const float* sh_w2_scale, void* out, int32_t out_is_fp32, int32_t* topk_ids_out,
                float* topk_w_out, void* workspace, size_t workspace_bytes, void* stream);

/* The launch sequence moe_forward takes. */
enum {
  MOE_SCHED_SINGLE = 1,  /* T <= 2, learned router, shapes with a single-launch kernel whose whole
                          * grid the device holds at once: the layer in one launch */
  MOE_SCHED_TINY = 2,    /* T * (top_k + 1) <= 16 otherwise: three launches */
  MOE_SCHED_DECODE = 3,  /* T <= 64: router, top-k + permutation, streaming w13, streaming w2, combine */
  MOE_SCHED_LARGE = 4    /* larger T or a hash layer: route, permutation, grouped GEMMs, combine */
};

/* Which of the MOE_SCHED_* sequences moe_forward takes for T tokens on the
 * current device (hash != 0: a hash layer). Returns a negative MOE_E* code
 * if cfg or T is invalid or unsupported. May query the device (occupancy),
 * never launches anything. */
int moe_forward_schedule(const moe_config* cfg, int32_t T, int32_t hash);

/* Kernels that moe_set_kernel_events can bracket. */
enum {
  MOE_KERNEL_NONE = 0,
  MOE_KERNEL_ROUTER = 1,       /* router logits (+ top-k, + small-T permutation) */
  MOE_KERNEL_PERMUTE = 2,      /* multi-block permutation (large T only) */
  MOE_KERNEL_ROUTED_W13 = 3,   /* routed experts: MXFP4 w13 + clamped SwiGLU (MOE_SCHED_SINGLE: the
                                * whole layer's one launch) */
  MOE_KERNEL_ROUTED_W2 = 4,    /* routed experts: MXFP4 w2 x routing weight */
  MOE_KERNEL_SHARED_W13 = 5,   /* shared expert: int8 w13 + clamped SwiGLU */
  MOE_KERNEL_SHARED_W2 = 6,    /* shared expert: int8 w2 */
  MOE_KERNEL_COMBINE = 7       /* weighted sum of the slots + shared expert */
};

/* Diagnostics for measurement (not part of the layer): from now on, every
 * launch of `kernel_id` made by moe_forward / moe_expert_ffn is bracketed by
 * hipEventRecord(start_event) and hipEventRecord(stop_event) on the call's
 * stream, so hipEventElapsedTime(start, stop) is that kernel's duration.
 * start_event/stop_event are hipEvent_t created by the caller; pass
 * MOE_KERNEL_NONE (or NULL events) to stop. Process-wide setting, not
 * thread-safe: meant for a benchmark driving one stream. */
int moe_set_kernel_events(int32_t kernel_id, void* start_event, void* stop_event);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
