// Internal interfaces between the host entry points and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kSmallT = 64;        // T at or below: decode schedule (one-block top-k + permutation)
constexpr int kMaxTopK = 8;
constexpr int kMaxExperts = 256;
constexpr int kPermBlock = 1024;   // slots per block of the multi-block permutation
constexpr int kThreads = 512;      // threads of every expert / router block (8 waves)
constexpr int kWaves = kThreads / 64;

// Permutation of the T*k slots by expert, plus the table of expert tiles
// (groups of at most tile_n consecutive sorted positions of one expert) that
// the expert kernels take one block column each.
struct Perm {
  int32_t* offsets;       // [E+1] first sorted position of each expert
  int32_t* sorted_slots;  // [T*k] slot (t*k+j) at each sorted position
  int32_t* slot_pos;      // [T*k] sorted position of each slot
  int32_t* sorted_tok;    // [T*k] token of each sorted position
  int4* tile_info;        // [max_tiles] {expert, first position, columns, 0}
  int32_t* n_tiles;       // [1] tiles in use
  int32_t* tile_rec;      // [max_tiles][kRecInts] tile records (decode sizes)
  int32_t* queues;        // [2] unit counters of the streaming w13 and w2 passes
  int32_t* done;          // [max_tiles + kSmallT] finished w13 units per routed, then shared, tile
  int tile_n;
  int max_tiles;
  uint32_t* flags;        // device error-flag word (MOE_FLAG_* bits)
};

// Tile record, one per routed tile, written with the tile table at decode
// sizes (write_tile_records, or the decode top-k) and read by the streaming
// passes, kRecInts ints: expert, first position, columns, 0, then for
// columns c < 16 the token of the position, the slot, and the slot's routing
// weight (float bits). Only columns below the tile's count are defined (the
// passes clamp or mask the others).
constexpr int kRecInts = 52;

// routed MXFP4 / shared int8 / routed w2 in 3-bit blocks (12 code bytes +
// a binary16 scale per 32 weights, 8 levels per expert table)
enum { kFmtMx = 0, kFmtI8 = 1, kFmtQ3 = 2 };
enum { kW13 = 0, kW2 = 1 };        // expert stage

struct RouterArgs {
  int T, H, E, k;
  float scale;
  const uint16_t* x;
  const float* gate_w;
  const float* bias;
  const float* logit_offset;
  float* scores;  // [T][E] s = sqrt(softplus(logit)), fp32
  float* keys;    // [T][E] selection values fp32(s + bias)
  int32_t* ids;   // [T][k]
  float* w;       // [T][k]
  // hash layers (tid2eid != null): the experts come from the token-id table
  // (the decode-size top-k kernel); bias may then be null
  const int32_t* token_ids;  // [T]
  const int32_t* tid2eid;    // [V][k]
  int V;
  uint32_t* flags;           // device error-flag word
};

struct HashArgs {
  int T, H, E, k, V;
  float scale;
  const uint16_t* x;
  const int32_t* token_ids;
  const int32_t* tid2eid;
  const float* gate_w;
  int32_t* ids;
  float* w;
  uint32_t* flags;  // device error-flag word: out-of-range token ids / table entries
};

// One expert GEMM pass on the "skinny" kernel: 16 weight rows per block (for
// w13, 16 gate rows and the 16 matching up rows) against one tile of at most
// 16 activation columns; K split over the 8 waves of the block.
struct SkinnyArgs {
  const uint8_t* wq;          // MXFP4 codes [E][N][K/2], 3-bit codes [E][N][K/32][12] or int8 [N][K]
  const uint8_t* wsc;         // MXFP4 E8M0 [E][N][K/32], 3-bit binary16 [E][N][K/32] (null for int8)
  const float* table;         // 3-bit: levels [E][8], null for the uniform book
  int fmt;                    // kFmtQ3 for a routed w2 pass in 3-bit blocks (else unused)
  const float* row_scale;     // int8 per-row scales [N] (null for MXFP4)
  long long q_expert_stride;  // bytes between experts of wq
  long long s_expert_stride;  // bytes between experts of wsc
  int K;                      // input features
  int half;                   // w13: I (up rows start there); w2: 0
  int rows;                   // weight rows of the pass (w13: 2I, w2: H)
  int n_rowblocks;            // output rows / 16
  int routed;                 // 1: tiles from perm.tile_info; 0: tiles of consecutive tokens;
                              // 2: one tile per slot, expert from the top-k computed in the block
  const int4* tile_info;
  const int32_t* n_tiles;
  int tile_n;                 // columns per tile (shared: tokens per tile)
  int n_tiles_grid;           // tiles per row block in the grid
  int T;
  const uint16_t* act;        // bf16 activation rows
  int act_ld;
  const int32_t* act_row;     // row of act for each sorted position (null: the position itself)
  uint16_t* hout;             // w13: bf16 h rows, by sorted position (routed) or token (shared)
  int hout_ld;
  float* yout;                // w2: fp32 rows, by slot (routed) or token (shared)
  int yout_ld;
  const int32_t* sorted_slots;
  const float* slot_w;        // w2 routed: combine weight of each slot
  const int32_t* tile_rec;    // routed tile records (streaming passes)
  float limit;
  // routed == 2 only: router scores and selection values, and the routing
  // outputs this pass writes
  const float* scores;        // [T][E]
  const float* keys;          // [T][E]
  float scale;
  int E, topk;
  int32_t* ids_out;           // [T][k]
  float* w_out;               // [T][k]
  uint32_t* flags;            // device error-flag word (expired waits of the fused passes)
};

// Routed w2 + shared w2 + combine for T*(k+1) <= 16 ("output-stationary"):
// each block owns 16 output rows of every token; slot j is MFMA column j and
// token t's shared-expert input is column T*k + t.
struct W2CombineArgs {
  int T, H, I, k;
  const uint8_t* w2c;
  const uint8_t* w2s;
  const int32_t* ids;    // [T*k] experts of the slots
  const float* w;        // [T*k] routing weights
  const uint16_t* hbuf;  // [T*k][I] bf16 h of each slot
  const int8_t* sh_w2;   // [H][I] shared expert w2 (int8)
  const float* sh_w2_scale;  // [H]
  const uint16_t* hs;    // [T][I] bf16 h of the shared expert
  void* out;             // [T][H]
  int out_is_fp32;
};

// Grouped GEMM (gemm.hip) for large T: tiles of 128 token positions x 256
// weight rows.
enum { kGemmW13 = 0, kGemmW2 = 1, kGemmW2Combine = 2 };
struct GemmArgs {
  int fmt;                    // kFmtMx (routed), kFmtI8 (shared), kFmtQ3 (routed w2 only)
  int mode;                   // kGemmW13: SwiGLU -> hout; kGemmW2: x slot weight -> yout[slot];
                              // kGemmW2Combine: shared w2 + sum of the slots' ybuf -> out
  const uint8_t* wq;
  const uint8_t* wsc;
  const float* table;         // 3-bit: levels [E][8], null for the uniform book
  const float* row_scale;     // int8 per-row scales
  long long q_expert_stride, s_expert_stride;
  int K, half;
  int routed;                 // tiles from tile_info (routed) or consecutive tokens (shared)
  const int4* tile_info;
  const int32_t* n_tiles;
  int n_ntiles;               // tiles along the weight rows
  int T;
  const uint16_t* act;
  int act_ld;
  const int32_t* act_row;     // row of act for each position (null: the position)
  uint16_t* hout;
  int hout_ld;
  uint16_t* yout;             // w2 routed: bf16 rows (x routing weight), by slot
  int yout_ld;
  const int32_t* sorted_slots;
  const float* slot_w;
  const uint16_t* ybuf;       // combine: [T*k][H] bf16
  int* queue;                 // [9] tile counters per XCD and blocks done: zero before the launch, left zero
  int topk;
  void* out;
  int out_ld, out_is_fp32;
  float limit;
};
constexpr int kGemmTokens = 128;  // token positions per GEMM tile

// Routed grouped GEMM on the block-scaled MFMA (gemm_mx.hip): MXFP4 weights x
// activations split exactly into hi and lo fp8 (E4M3) halves with E8M0
// exponents per 32 along K. Tiles of kGemmMxTokens positions x 512 weight
// rows (w13: 256 gate + the matching 256 up rows).
constexpr int kGemmMxTokens = 128;
struct MxGemmArgs {
  int mode;                   // kGemmW13: SwiGLU -> h split (hi/lo + exponents); kGemmW2: x slot weight -> yout
  const uint8_t* wq;          // codes [E][rows][K/2]
  const uint8_t* wsc;         // E8M0 [E][rows][K/32]
  long long q_expert_stride, s_expert_stride;
  int K;                      // input features
  int half;                   // w13: I (the up rows start there)
  int N;                      // output features (w13: I, w2: H)
  const int4* tile_info;
  const int32_t* n_tiles;
  int n_ntiles;               // N tiles (w13: I / 256, w2: H / 512)
  const uint8_t* a_hi;        // activations fp8 [rows][K]
  const uint8_t* a_lo;
  const uint8_t* as_hi;       // E8M0 [rows][K/32]
  const uint8_t* as_lo;
  const int32_t* act_row;     // activation row of each sorted position (null: the position)
  uint8_t* h_hi;              // w13: h by sorted position, fp8 [slots][I] and E8M0 [slots][I/32]
  uint8_t* h_lo;
  uint8_t* hs_hi;
  uint8_t* hs_lo;
  int I;
  uint16_t* yout;             // w2: bf16 rows by slot (x routing weight)
  int yout_ld;
  const int32_t* sorted_slots;
  const float* slot_w;
  int* queue;                 // [9] as GemmArgs::queue
  float limit;
  int order;                  // 0: the N tiles of a token tile adjacent; 1: the token tiles of an N tile adjacent
};
bool gemm_mx_supported(int H, int I);
// x [rows][K] bf16 -> hi, lo fp8 [rows][K] and E8M0 [rows][K/32] each (the exact split)
hipError_t launch_quant_rows(const uint16_t* x, long long rows, int K, uint8_t* hi, uint8_t* lo, uint8_t* sh,
                             uint8_t* sl, hipStream_t st);
hipError_t launch_gemm_mx(const MxGemmArgs& p, int tiles, hipStream_t st);

struct CombineArgs {
  int T, H, k;
  const void* ybuf;   // [T*k][H] weighted expert outputs in slot order: fp32, or bf16 if y_bf16
  const float* zbuf;  // [T][H] shared expert or null
  void* out;          // [T][H]
  int out_is_fp32;
  int y_bf16;
};

// Routers
hipError_t launch_router_small(const RouterArgs& r, const SkinnyArgs* shared_w13, int shared_blocks,
                               hipStream_t st);
// Decode router (H = 1024, 2048 or 4096; other sizes use launch_router_small).
hipError_t launch_router_dec(const RouterArgs& r, hipStream_t st);
// Top-k of every token and the permutation; arrivals: an int of the
// workspace that is zero before the call and is zero again after it.
hipError_t launch_topk_permute_small(const RouterArgs& r, const Perm& p, int* arrivals, hipStream_t st);
// Workspace ints (in the counters region): the top-k blocks' arrival count,
// then the streaming passes' two unit counters.
constexpr int kArrivalsInt = 16;
constexpr int kQueueInts = 17;
// the grouped GEMMs' tile queues, 9 ints per launch: routed w13, shared w13,
// routed w2, shared w2 + combine
constexpr int kGemmQueueInts = 24;
enum { kQRoutedW13 = 0, kQSharedW13 = 1, kQRoutedW2 = 2, kQSharedW2 = 3 };
// Large-T learned router on bf16 MFMA (fp32 router rows split into three
// bf16 planes, wsplit [3][E][H]; partial logits plog [KS][T][E] with KS =
// router_mfma_splits(T, H)).
struct RouterMfmaArgs {
  int T, H, E, KS;
  const uint16_t* x;
  const uint16_t* wsplit;
  float* plog;
};
int router_mfma_splits(int T, int H);
hipError_t launch_router_mfma(const RouterArgs& r, uint16_t* wsplit, float* plog, hipStream_t st);
hipError_t launch_hash_route(const HashArgs& a, hipStream_t st);
// Permutation and tiles
hipError_t launch_permute(int T, int E, int k, const int32_t* ids, const Perm& p, int32_t* blk_counts,
                          hipStream_t st);
// Tile table from a permutation given by the caller: user_offsets and
// user_sorted are checked (offsets from 0 to T*k, non-decreasing; slots in
// [0, T*k)) and copied into p.offsets / p.sorted_slots, so the expert
// kernels never index with a caller's value; a violation sets
// kFlagPermutation and leaves no tiles (or the slot clamped).
hipError_t launch_tiles_from_offsets(int T, int E, int k, const int32_t* user_offsets, const int32_t* user_sorted,
                                     const Perm& p, hipStream_t st);
// Expert passes; `b` (optional) runs in the same launch as `a`
hipError_t launch_w13(const SkinnyArgs& a, int a_blocks, const SkinnyArgs* b, int b_blocks, bool b_is_shared_w2,
                      hipStream_t st);
hipError_t launch_w2(const SkinnyArgs& a, int a_blocks, const SkinnyArgs* b, int b_blocks, hipStream_t st);
hipError_t launch_shared_w13(const SkinnyArgs& a, int blocks, hipStream_t st);
hipError_t launch_w13_deep(const SkinnyArgs& a, int blocks, hipStream_t st);
hipError_t launch_combine(const CombineArgs& a, hipStream_t st);
hipError_t launch_gemm(const GemmArgs& p, int tiles, hipStream_t st);
// Streaming expert pass (batched decode): routed MXFP4 pass a and int8 shared
// pass b of stage `mode` (kW13 / kW2) in one grid; n_rowblocks of each holds
// its row groups (w13: I/64, w2: H/128).
// queue: the pass's unit counter, zero before the launch (the tile-record
// writers reset it).
hipError_t launch_stream(int mode, const SkinnyArgs& a, int a_blocks, const SkinnyArgs* b, int b_blocks,
                         int* queue, hipStream_t st);
// Both decode stages in one launch (H and I multiples of 1024, the shared
// tiles of w13 and w2 alike): done_r / done_s count the finished w13 units of
// each routed / shared tile and must be zero before the launch.
hipError_t launch_stream_fused(const SkinnyArgs& a13, const SkinnyArgs& b13, const SkinnyArgs& a2,
                               const SkinnyArgs& b2, int a_blocks13, int b_blocks13, int a_blocks2, int b_blocks2,
                               int* queue, int* done_r, int* done_s, hipStream_t st);
// Tile records and queue reset for tiles built by launch_tiles_from_offsets.
hipError_t launch_tile_records(const Perm& p, const float* slot_w, hipStream_t st);
hipError_t launch_w2_combine_small(const W2CombineArgs& a, hipStream_t st);
// LDS bytes of k_w2_combine_small for T tokens of k slots at intermediate I
// (at most 160 KB fit a block).
size_t w2_combine_small_lds(int T, int k, int I);
// LDS bytes of one streaming unit over K input features with tile_n
// activation rows (the routed tile, plus the unit's 256 rows of scales).
size_t stream_unit_lds(int tile_n, int K, bool q3);
constexpr size_t kLdsBlockMax = 160 * 1024;  // LDS one block can have on gfx950
// Hand-off region of the single-launch layer, at a fixed offset at the start
// of every workspace (zero on first use): per-block layer counters, then two
// buffers, used by alternate layers, of router scores, h columns and (for
// layers run back to back in one launch) the layer's input rows.
constexpr int kXferBlocks = 256;  // blocks tracked: the largest single-launch grid
constexpr int kXferTokens = 2, kXferCols = 16, kXferMaxI = 2048, kXferMaxH = 4096;
constexpr size_t kXferScoreWords = (size_t)kXferTokens * kXferBlocks;  // [2 tokens][256 experts]
constexpr size_t kXferHWords = (size_t)kXferCols * (kXferMaxI / 2);     // [16 columns][1024 bf16 pairs]
constexpr size_t kXferXWords = (size_t)kXferTokens * (kXferMaxH / 2);   // [2 tokens][2048 bf16 pairs]
constexpr size_t kXferBytes = ((size_t)kXferBlocks + 2 * (kXferScoreWords + kXferHWords + kXferXWords)) * 4;

// The whole layer for T <= 2 tokens (T*(k+1) <= 16) in one launch of one
// block per CU.
struct LayerArgs {
  int T, H, I, E, k;
  float scale, limit;
  const uint16_t* x;           // [T][H] bf16
  const float* gate_w;         // [E][H] fp32 router
  const float* bias;           // [E]
  const float* logit_offset;   // [E] or null
  const uint8_t* w13c;         // [E][2I][H/2]
  const uint8_t* w13s;         // [E][2I][H/32]
  const uint8_t* w2c;          // [E][H][I/2] (3-bit: [E][H][I/32][12])
  const uint8_t* w2s;          // [E][H][I/32] (3-bit: binary16 [E][H][I/32])
  const float* w2tab;          // 3-bit: levels [E][8], null for the uniform book
  int w2q3;                    // routed w2 in 3-bit blocks
  const int8_t* sh13;          // [2I][H]
  const float* sh13s;          // [2I]
  const int8_t* sh2;           // [H][I]
  const float* sh2s;           // [H]
  void* out;                   // [T][H]
  int out_is_fp32;
  int32_t* ids_out;            // [T][k]
  float* w_out;                // [T][k]
  uint32_t* xfer;              // hand-off region (kXferBytes, workspace)
  uint32_t* flags;             // device error-flag word (expired hand-off waits)
  const int32_t* token_ids;    // hash layer (tid2eid != null): [T] token ids
  const int32_t* tid2eid;      // [V][k] token-id table, or null (learned router)
  int V;
};
// Whether the single-launch layer has a kernel for this shape whose whole
// grid the current device holds at once.
bool layer_small_supported(int H, int I, int E, int T, int k, bool w2q3 = false);

// int8 per-channel linear at decode sizes (linear.hip): x [T][G*K] bf16,
// q [G*N][K] int8, scale [G*N] -> out [T][G*N]; blocks of 64 rows x a K slice
// of ks (linear_dec_ks), split = K / ks slices added by the last block of
// each row block.
struct LinearDecArgs {
  int T, K, N, G;
  int ks, split;
  const uint16_t* x;
  const int8_t* q;
  const float* scale;
  void* out;
  int out_is_fp32;
  float* part;  // [split][T][G*N] fp32 partial sums (split > 1)
  int* count;   // [G*N/64] arrivals per row block: zero before the launch, left zero
};
int linear_dec_ks(int T, int K, int N, int G);  // 0: not supported
hipError_t launch_linear_dec(const LinearDecArgs& a, hipStream_t st);
hipError_t launch_layer_small(const LayerArgs& a, hipStream_t st);

// Layers run back to back in one launch of the single-launch layer (a stack
// of MoE layers at T <= 2): each layer's output rows go to the next through
// the hand-off region instead of a kernel boundary. Up to kStackChunk layers
// per launch, their arguments passed as kernel arguments: layer j > 0 of a
// launch takes its input from layer j - 1 (its x is not read), and writes
// out too (bf16) unless it is the launch's last layer.
constexpr int kStackChunk = 8;
struct StackArgs {
  int n;  // layers in this launch, 1 .. kStackChunk
  LayerArgs layer[kStackChunk];
};
// Whether launch_layer_stack has a kernel for this shape whose whole grid the
// current device holds at once.
bool layer_stack_supported(int H, int I, int E, int T, int k);
hipError_t launch_layer_stack(const StackArgs& a, hipStream_t st);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st);

// Device error flags (values of MOE_FLAG_* in moe.h), one word per GPU in
// library-owned device memory; the address for the current device, or null
// if it cannot be obtained.
constexpr uint32_t kFlagTokenId = 1u, kFlagTableEntry = 2u, kFlagExpertId = 4u, kFlagWaitExpired = 8u,
                   kFlagPermutation = 16u;
uint32_t* device_flags();

}  // namespace moe
