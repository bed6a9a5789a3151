// Internal interfaces between the host entry points and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kSmallT = 64;         // T at or below this uses the one-launch router
constexpr int kMaxTopK = 8;
constexpr int kMaxExperts = 256;
constexpr int kPermBlock = 1024;    // slots per block in the multi-block permutation
constexpr int kNumCounters = 64;

struct RouterArgs {
  int T, H, E, k;
  float scale;
  const uint16_t* x;
  const float* gate_w;
  const float* bias;
  const float* logit_offset;
  float* logits;       // [T][E] workspace
  int32_t* ids;        // [T][k]
  float* w;            // [T][k]
  unsigned* counter;   // last-block counter (zero between calls)
  // small-T path only: build the permutation in the same launch
  int perm;
  int tile_n;
  int32_t* offsets;
  int32_t* sorted_slots;
  int32_t* slot_pos;
  int32_t* tile_off;
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
};

struct PermuteArgs {
  int T, E, k, tile_n;
  const int32_t* ids;
  int32_t* offsets;
  int32_t* sorted_slots;
  int32_t* slot_pos;
  int32_t* tile_off;
  int32_t* blk_counts;  // [nblk][E] workspace
};

// One pass of the small-column ("skinny") expert GEMM: up to 16 activation
// columns per tile against 16 weight rows per block, MFMA 16x16x32 bf16.
struct SkinnyArgs {
  const uint8_t* wq;          // MXFP4 codes [E][N][K/2] or int8 [N][K]
  const uint8_t* wsc;         // MXFP4 scales [E][N][K/32] (null for int8)
  const float* row_scale;     // int8 per-row scales [N] (null for MXFP4)
  long long q_expert_stride;  // bytes between experts of wq
  long long s_expert_stride;  // bytes between experts of wsc
  int K;                      // input features
  int half;                   // w13: I (up rows start there); w2: 0
  const uint16_t* act;        // bf16 activation rows
  int act_ld;
  int act_is_x;               // routed w13: activation row = token of the slot
  int T, topk, E;
  int routed;                 // tiles from tile_off (routed) or 16-token tiles (shared)
  const int32_t* offsets;
  const int32_t* sorted_slots;
  const int32_t* tile_off;
  int tile_n;                 // columns per tile, 1..16
  int n_tiles_grid;           // tiles in the grid (block = tile + n_tiles_grid * rowblock)
  int n_rowblocks;            // output rows / 16
  uint16_t* hout;             // w13: bf16 h rows
  int hout_ld;
  float* yout;                // w2: fp32 rows
  int yout_ld;
  const float* slot_w;        // w2 routed: combine weight of each slot
  float limit;
};

struct CombineArgs {
  int T, H, k;
  const float* ybuf;    // [T*k][H] weighted expert outputs in slot order
  const float* zbuf;    // [T][H] shared expert or null
  void* out;            // [T][H]
  int out_is_fp32;
};

hipError_t launch_router(const RouterArgs& a, hipStream_t st);
hipError_t launch_hash_route(const HashArgs& a, hipStream_t st);
hipError_t launch_permute(const PermuteArgs& a, hipStream_t st);
hipError_t launch_tile_offsets(int E, int tile_n, const int32_t* offsets, int32_t* tile_off,
                               hipStream_t st);
hipError_t launch_skinny_w13_mxfp4(const SkinnyArgs& a, int max_tiles, hipStream_t st);
hipError_t launch_skinny_w2_mxfp4(const SkinnyArgs& a, int max_tiles, hipStream_t st);
hipError_t launch_skinny_w13_int8(const SkinnyArgs& a, int max_tiles, hipStream_t st);
hipError_t launch_skinny_w2_int8(const SkinnyArgs& a, int max_tiles, hipStream_t st);
hipError_t launch_combine(const CombineArgs& a, hipStream_t st);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st);

}  // namespace moe
