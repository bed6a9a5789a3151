// Token permutation by expert on gfx950: a stable counting sort of the T*k
// (token, slot) pairs by expert id, so each expert's activation rows can be
// gathered into one contiguous group (the dispatch step of the MoE block:
// page "DeepSeek-V4-Flash-0731", section "Checked in its code", row "Shared
// expert", where the routed experts are called with the flat tokens, the
// chosen indices and their weights).
//
// Three launches for any T (the small-T router builds the same outputs in its
// own last block):
//   k_perm_count   per block of kPermBlock slots, a histogram over experts
//   k_perm_scan    one block: per-expert exclusive prefix over blocks, expert
//                  offsets, and the tile prefix used by the expert GEMMs
//   k_perm_scatter per block, the stable rank of each slot among the block's
//                  earlier slots of the same expert -> its sorted position
#include "device.h"
#include "internal.h"

namespace moe {

__global__ __launch_bounds__(256) void k_perm_count(PermuteArgs a) {
  __shared__ int hist[kMaxExperts];
  const int tid = threadIdx.x, b = blockIdx.x;
  const int n = a.T * a.k;
  hist[tid] = 0;
  __syncthreads();
  const int beg = b * kPermBlock, end = min(n, beg + kPermBlock);
  for (int i = beg + tid; i < end; i += 256) atomicAdd(&hist[a.ids[i]], 1);
  __syncthreads();
  if (tid < a.E) a.blk_counts[(size_t)b * a.E + tid] = hist[tid];
}

__global__ __launch_bounds__(256) void k_perm_scan(PermuteArgs a, int nblk) {
  __shared__ int tmp[256];
  const int tid = threadIdx.x;
  int running = 0;
  if (tid < a.E) {
    for (int b = 0; b < nblk; ++b) {
      int c = a.blk_counts[(size_t)b * a.E + tid];
      a.blk_counts[(size_t)b * a.E + tid] = running;
      running += c;
    }
  }
  int total;
  int off = block_exclusive_scan_256(tid < a.E ? running : 0, tmp, &total);
  int nt = tid < a.E ? (running + a.tile_n - 1) / a.tile_n : 0;
  int ttotal;
  int toff = block_exclusive_scan_256(nt, tmp, &ttotal);
  if (tid < a.E) {
    a.offsets[tid] = off;
    a.tile_off[tid] = toff;
    for (int b = 0; b < nblk; ++b) a.blk_counts[(size_t)b * a.E + tid] += off;
  }
  if (tid == 0) {
    a.offsets[a.E] = total;
    a.tile_off[a.E] = ttotal;
  }
}

__global__ __launch_bounds__(256) void k_perm_scatter(PermuteArgs a) {
  __shared__ int chunk[256];
  __shared__ int seen[kMaxExperts];
  const int tid = threadIdx.x, b = blockIdx.x;
  const int n = a.T * a.k;
  seen[tid] = 0;
  const int beg = b * kPermBlock, end = min(n, beg + kPermBlock);
  for (int c0 = beg; c0 < end; c0 += 256) {
    const int i = c0 + tid;
    const int e = i < end ? a.ids[i] : -1;
    chunk[tid] = e;
    __syncthreads();
    if (e >= 0) {
      int rank = 0;
      for (int j = 0; j < tid; ++j) rank += (chunk[j] == e);
      const int pos = a.blk_counts[(size_t)b * a.E + e] + seen[e] + rank;
      a.sorted_slots[pos] = i;
      a.slot_pos[i] = pos;
    }
    __syncthreads();
    if (e >= 0) atomicAdd(&seen[e], 1);
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void k_tile_offsets(int E, int tile_n, const int32_t* offsets,
                                                       int32_t* tile_off) {
  __shared__ int tmp[256];
  const int tid = threadIdx.x;
  int c = tid < E ? offsets[tid + 1] - offsets[tid] : 0;
  int total;
  int toff = block_exclusive_scan_256((c + tile_n - 1) / tile_n, tmp, &total);
  if (tid < E) tile_off[tid] = toff;
  if (tid == 0) tile_off[E] = total;
}

hipError_t launch_permute(const PermuteArgs& a, hipStream_t st) {
  const int n = a.T * a.k;
  if (n <= 0) {  // every expert empty: zero offsets and tiles
    k_perm_scan<<<1, 256, 0, st>>>(a, 0);
    return hipGetLastError();
  }
  const int nblk = (n + kPermBlock - 1) / kPermBlock;
  k_perm_count<<<nblk, 256, 0, st>>>(a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  k_perm_scan<<<1, 256, 0, st>>>(a, nblk);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  k_perm_scatter<<<nblk, 256, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_tile_offsets(int E, int tile_n, const int32_t* offsets, int32_t* tile_off,
                               hipStream_t st) {
  k_tile_offsets<<<1, 256, 0, st>>>(E, tile_n, offsets, tile_off);
  return hipGetLastError();
}

}  // namespace moe
