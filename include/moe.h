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
 *   - Device-side values are checked where an index comes from the caller:
 *     a token id outside [0, V), a tid2eid entry outside [0, E), an expert
 *     id outside [0, E) given to moe_permute, or an inconsistent permutation
 *     given to moe_expert_ffn is never used to index memory. The kernels
 *     substitute an in-range value (token row 0, expert 0, slot 0), write NaN
 *     routing weights for such a hash-layer token, and set a bit of the
 *     device error flags (MOE_FLAG_*, read with moe_device_flags); the
 *     return code cannot report them, since it is produced before the
 *     kernels run. E8M0 scale bytes should not be 0xFF (NaN).
 *   - `workspace` is device scratch of at least moe_workspace_size() bytes,
 *     256-byte aligned. Zero-fill it once before its first use
 *     (moe_workspace_init, or any zero fill): bytes 64 .. 67 count the
 *     blocks of the decode-size top-k, bytes 96 .. 239 hold the tile
 *     queues of the grouped GEMMs (MOE_SCHED_LARGE), and bytes 256 ..
 *     169215 hold the hand-off state of the single-launch layer
 *     (MOE_SCHED_SINGLE); every call leaves all three ready for the next,
 *     and every other workspace value is written before it is read. Calls
 *     that share one workspace must be ordered on one stream. If a bounded
 *     wait of one block for another block of the same launch expires (about
 *     a second; it does not happen when the whole grid is resident, which
 *     the launchers check), the outputs that depend on it are NaN, the
 *     device flag MOE_FLAG_WAIT_EXPIRED is set, and the hand-off state stays
 *     consistent for the next call.
 *   - Supported shapes: H and I multiples of 128 up to 8192, 1 <= top_k <=
 *     8, top_k <= E <= 256, 0 <= T <= 65536 (other shapes: MOE_EUNSUPPORTED,
 *     and moe_workspace_size returns 0). Device pointers must be 16-byte
 *     aligned.
 *   - Buffers a call writes (outputs, act, workspace) must not overlap each
 *     other or any buffer the call reads.
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
  int32_t norm_topk_prob;       /* 1: the top-k scores are renormalised (the model's true);
                                   0 is not supported (MOE_EUNSUPPORTED) */
} moe_config;

enum {
  MOE_OK = 0,
  MOE_EINVAL = -1,       /* null pointer, negative size, misaligned pointer */
  MOE_EUNSUPPORTED = -2, /* shape outside the supported limits */
  MOE_EWORKSPACE = -3,   /* workspace too small */
  MOE_EHIP = -4          /* a HIP launch or runtime call failed */
};

/* Device error flags: bits of a word kept by the library in device memory,
 * one per GPU, set by kernels (atomic OR) and cleared only by
 * moe_device_flags(..., clear = 1, ...). */
enum {
  MOE_FLAG_TOKEN_ID = 1,      /* a hash-layer token id outside [0, V) */
  MOE_FLAG_TABLE_ENTRY = 2,   /* a tid2eid entry outside [0, E) */
  MOE_FLAG_EXPERT_ID = 4,     /* an expert id outside [0, E) given to moe_permute */
  MOE_FLAG_WAIT_EXPIRED = 8,  /* a bounded wait between blocks of one launch expired */
  MOE_FLAG_PERMUTATION = 16   /* offsets or sorted slots given to moe_expert_ffn are inconsistent */
};

/* Reads the current device's error flags into *flags (if not NULL) after the
 * work queued on `stream` so far, and clears them if clear != 0. Waits for
 * the stream (host synchronisation): a diagnostic, not for the hot path. */
int moe_device_flags(uint32_t* flags, int32_t clear, void* stream);

/* Measurement aid, not part of the layer: reads `bytes` of device memory at
 * `buf` once with a plain streaming kernel of `blocks` blocks of 256
 * threads (32 KB chunks per block; 16-byte loads, 1 KB per wave-wide load,
 * eight in flight per lane) on `stream`, so that timing it gives the HBM
 * read rate this GPU reaches, the denominator beside the published 8 TB/s
 * for paths that only read. sink: [blocks] u32 device words; a word is
 * written only if the folded data of its block takes one particular value
 * (never for a buffer of zeros or ones). buf 16-byte aligned, bytes a
 * multiple of 16, blocks > 0, else MOE_EINVAL. */
int moe_read_probe(const void* buf, size_t bytes, int32_t blocks, uint32_t* sink, void* stream);

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

/* moe_forward with the routed experts' down projection (w2) in 3-bit
 * blocks: 14 bytes per 32 weights, one code book for every block (uniform)
 * or a small table per expert (adaptive); page
 * "Geometric-AI/DeepSeek-V4-Flash-0731-ROCmFP3-MIX", introduction and
 * section "What 'adaptive' means here". The pages fix the byte count only;
 * the field layout is this library's own:
 *   w2_codes  [E][H][I/32][12] u8: per 32 consecutive weights along I, 12
 *             bytes b[0..11] of 3-bit codes. Byte j + 4q (j < 4, q < 3)
 *             holds the code of weight 8q + j in bits 0..2 and of weight
 *             8q + 4 + j in bits 3..5; weight 24 + j has its code bits 0..1
 *             in bits 6..7 of byte j and bit 2 in bit 6 of byte 8 + j;
 *             weight 28 + j has bits 0..1 in bits 6..7 of byte 4 + j and bit
 *             2 in bit 7 of byte 8 + j.
 *   w2_scales [E][H][I/32] u16: IEEE binary16 scale d of each block.
 *   w2_levels [E][8] f32: expert e's levels, or NULL for the uniform code
 *             book level[c] = c - 4.
 *   weight = d * level[code]. The kernels round each decoded weight to bf16
 *   (nearest even) before the bf16 MFMA; every other argument is as in
 *   moe_forward. Supported: T <= 64 with H and I multiples of 1024 (the
 *   single-launch layer where moe_forward takes it, else one streaming
 *   launch for both stages), T > 64 with H a multiple of 256 (the grouped
 *   GEMMs); else MOE_EUNSUPPORTED. w2_codes need 4-byte alignment
 *   of each block (its 16-byte pointer alignment suffices), w2_levels
 *   16-byte alignment. */
int moe_forward_w2q3(const moe_config* cfg, int32_t T, const uint16_t* x, const float* gate_w,
                     const float* bias, const float* logit_offset, const int32_t* token_ids,
                     const int32_t* tid2eid, int32_t V, const uint8_t* w13_codes,
                     const uint8_t* w13_scales, const uint8_t* w2_codes, const uint16_t* w2_scales,
                     const float* w2_levels, const int8_t* sh_w13, const float* sh_w13_scale,
                     const int8_t* sh_w2, const float* sh_w2_scale, void* out, int32_t out_is_fp32,
                     int32_t* topk_ids_out, float* topk_w_out, void* workspace, size_t workspace_bytes,
                     void* stream);

/* The model's other int8 linear layers ("w8a16": int8, symmetric, one fp32
 * scale per output channel, 16-bit activations; page "deepseek-v4-mxfp4-int8
 * config.json", quantization_config, config group linears_w8a16, targets
 * attn.fused_wqa_wkv, attn.wq_b, attn.wo_a, attn.wo_b, attn.indexer.wq_b,
 * attn.indexer.compressor.wkv): y = x W^T with W[n][k] = scale[n] * q[n][k].
 *   groups > 1: a grouped (block-diagonal) projection such as wo_a
 *   (o_groups): group g maps input features [g K, (g+1) K) to output
 *   features [g N, (g+1) N) with its own rows q[g N .. g N + N) and scales.
 *   x     [T][groups K] bf16
 *   q     [groups N][K] int8;  scale [groups N] f32
 *   out   [T][groups N] bf16 (out_is_fp32 = 0) or f32
 *   workspace: moe_linear_workspace_size(T, K, N, groups) bytes, 256-byte
 *   aligned, zero-filled before its first use (its counters, bytes 0 .. 36
 *   and 256 .. 262399, are left at zero by every call; at T <= 64 the rest
 *   holds partial sums, written before they are read); calls sharing one
 *   must be ordered on one stream.
 *   T <= 64: one launch that splits K over blocks of 64 rows (the last block
 *   of each row block adds the slices in order: deterministic); T > 64: the
 *   shared expert's grouped GEMM, one launch per group.
 * Supported: K a multiple of 128, N of 256 (each at most 65536), groups at
 * most 64, 0 <= T <= 65536. Errors as for moe_forward. */
size_t moe_linear_workspace_size(int32_t T, int32_t K, int32_t N, int32_t groups);
int moe_linear_w8a16(int32_t T, int32_t K, int32_t N, int32_t groups, const uint16_t* x, const int8_t* q,
                     const float* scale, void* out, int32_t out_is_fp32, void* workspace, size_t workspace_bytes,
                     void* stream);

/* One MoE layer's parameters for moe_forward_stack (device pointers, layouts
 * as for moe_forward). tid2eid != NULL makes it a hash layer (V rows); then
 * bias and logit_offset are ignored. */
typedef struct moe_layer_weights {
  const float* gate_w;         /* [E][H] */
  const float* bias;           /* [E] (learned router) */
  const float* logit_offset;   /* [E] or NULL */
  const int32_t* tid2eid;      /* [V][k] or NULL */
  int32_t V;
  const uint8_t* w13_codes;    /* [E][2I][H/2] */
  const uint8_t* w13_scales;   /* [E][2I][H/32] */
  const uint8_t* w2_codes;     /* [E][H][I/2] */
  const uint8_t* w2_scales;    /* [E][H][I/32] */
  const int8_t* sh_w13;        /* [2I][H] */
  const float* sh_w13_scale;   /* [2I] */
  const int8_t* sh_w2;         /* [H][I] */
  const float* sh_w2_scale;    /* [H] */
} moe_layer_weights;

/* A stack of MoE layers run back to back on `stream`, as the model's 43 MoE
 * layers are, the first num_hash_layers routed by the token-id table (page
 * "DeepSeek-V4-Flash export design", section "Source configuration"; page
 * "deepseek-v4-mxfp4-int8 config.json", num_hidden_layers,
 * num_hash_layers): layer 0 reads x, layer l + 1 reads the bf16 output of
 * layer l (the attention and residual steps the model has between its MoE
 * layers are not part of this library), and the last layer writes out (bf16,
 * or fp32 if out_is_fp32).
 *   layers     host array of n_layers parameter sets (read during the call)
 *   token_ids  [T] i32, used by the hash layers (may be NULL if none is)
 *   act        [2][T][H] bf16 device scratch for the layers' outputs (the
 *              output of layer l, l < n_layers - 1, is left in act[l % 2])
 *   workspace  as for moe_forward (moe_workspace_size(cfg, T) bytes), shared
 *              by the layers in turn
 * Where moe_forward would run the layers as single launches (T <= 2 at
 * shapes that have one), up to 8 layers run in one launch, each layer's
 * output rows handed to the next inside it (also written to act as above);
 * the results are those of the layers called one by one, bit for bit, and
 * every layer's arguments are checked before anything is launched.
 * Otherwise each layer takes the schedule moe_forward takes for it and a
 * failed layer stops the stack. Errors as for moe_forward. */
int moe_forward_stack(const moe_config* cfg, int32_t n_layers, const moe_layer_weights* layers, int32_t T,
                      const uint16_t* x, const int32_t* token_ids, uint16_t* act, void* out,
                      int32_t out_is_fp32, void* workspace, size_t workspace_bytes, void* stream);

/* moe_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). Its workspace is a fixed scratch array
 * in the library's device memory, one per GPU, held until the process ends
 * (moe_noalloc_max_bytes() bytes, 16 MiB: enough for T <= 64 at the full
 * shape). The first call on a device zero-fills it on `stream` (and waits,
 * unless the stream is being captured), and so does the first call after one
 * that returned MOE_EHIP (a failed launch can leave its counters non-zero).
 * It allocates nothing and calls no
 * allocating routine. Every call on one GPU shares that GPU's scratch: calls
 * that overlap in time on one GPU (different streams, no ordering) race;
 * order them on one stream. Returns MOE_EWORKSPACE, launching nothing, when
 * moe_workspace_size(cfg, T) exceeds the scratch; otherwise as moe_forward,
 * with the same kernels and outputs. */
int moe_forward_noalloc(const moe_config* cfg, int32_t T, const uint16_t* x, const float* gate_w,
                        const float* bias, const float* logit_offset, const int32_t* token_ids,
                        const int32_t* tid2eid, int32_t V, const uint8_t* w13_codes,
                        const uint8_t* w13_scales, const uint8_t* w2_codes, const uint8_t* w2_scales,
                        const int8_t* sh_w13, const float* sh_w13_scale, const int8_t* sh_w2,
                        const float* sh_w2_scale, void* out, int32_t out_is_fp32, int32_t* topk_ids_out,
                        float* topk_w_out, void* stream);

/* Size in bytes of moe_forward_noalloc's scratch (its largest workspace). */
size_t moe_noalloc_max_bytes(void);

/* The launch sequence moe_forward takes. */
enum {
  MOE_SCHED_SINGLE = 1,  /* T * (top_k + 1) <= 16, shapes with a single-launch kernel whose whole
                          * grid the device holds at once: the layer in one launch (learned
                          * router or hash layer) */
  MOE_SCHED_TINY = 2,    /* T * (top_k + 1) <= 16 otherwise, learned router: three launches */
  MOE_SCHED_DECODE = 3,  /* T <= 64 otherwise: router, top-k (or the hash table) + permutation,
                          * streaming w13, streaming w2, combine */
  MOE_SCHED_LARGE = 4    /* T > 64: route, permutation, grouped GEMMs, combine */
};

/* Which of the MOE_SCHED_* sequences moe_forward takes for T tokens on the
 * current device (hash != 0: a hash layer). Returns a negative MOE_E* code
 * if cfg or T is invalid or unsupported. May query the device (occupancy),
 * never launches anything. */
int moe_forward_schedule(const moe_config* cfg, int32_t T, int32_t hash);

/* Process-wide options (not thread-safe; set them before the calls they
 * should affect, and query moe_workspace_size after setting them: the
 * workspace size depends on them). */
enum {
  /* 1: the routed grouped GEMMs of batches above 64 tokens run on gfx950's
   * block-scaled MFMA (v_mfma_scale_f32_32x32x64_f8f6f4): MXFP4 weights as
   * stored, E8M0 exponents as the hardware scales, and each bf16 activation
   * split exactly into two fp8 (E4M3) values with their own E8M0 exponents
   * per 32, so the sums equal the bf16 path's up to summation order
   * (page "deepseek-v4-mxfp4-int8 config.json", quantization_config,
   * experts_w4a16: scale_mode native_e8m0). Needs H % 256 == 0 and
   * I % 128 == 0; other shapes keep the default. 0 (default): bf16 MFMA on
   * weights converted to bf16 in registers. */
  MOE_OPTION_PREFILL_BLOCK_SCALED = 1
};

/* Sets an option; MOE_EINVAL for an unknown option or value. */
int moe_set_option(int32_t option, int32_t value);

/* The current value of an option, or MOE_EINVAL for an unknown option. */
int moe_get_option(int32_t option);

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
