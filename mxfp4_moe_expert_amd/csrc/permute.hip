// Token permutation by expert on gfx950: a stable counting sort of the T*k
// (token, slot) pairs by expert id, so each expert's activation rows form one
// contiguous group (the dispatch step of the MoE block: page
// "DeepSeek-V4-Flash-0731", section "Checked in its code", row "Shared
// expert", where the routed experts are called with the flat tokens, the
// chosen indices and their weights). It also writes the expert tile table
// the expert kernels read with one load per block.
//
// Three launches for any T (decode sizes use the one-block version in
// route.hip):
//   k_perm_count   per block of kPermBlock slots, a histogram over experts
//   k_perm_scan    one block: per-expert prefix over blocks, expert offsets,
//                  the tile table
//   k_perm_scatter per block, the stable rank of each slot among the block's
//                  earlier slots of the same expert (wave ballots) -> its
//                  sorted position
#include "device.h"
#include "internal.h"
#include "tilerec.h"

namespace moe {

struct PermArgs {
  int T, E, k;
  const int32_t* ids;
  Perm p;
  int32_t* blk_counts;  // [nblk][E]
};

__device__ void write_tiles(int c, int off, int E, const Perm& p, int* scan_tmp) {
  const int tid = threadIdx.x;
  const int nt = tid < E ? (c + p.tile_n - 1) / p.tile_n : 0;
  int total;
  const int toff = block_exclusive_scan(nt, scan_tmp, &total);
  if (tid < E) {
    for (int i = 0; i < nt; ++i) {
      const int first = i * p.tile_n;
      p.tile_info[toff + i] = make_int4(tid, off + first, min(p.tile_n, c - first), 0);
    }
  }
  if (tid == 0) *p.n_tiles = total;
}

__global__ __launch_bounds__(256) void k_perm_count(PermArgs a) {
  __shared__ int hist[kMaxExperts];
  const int tid = threadIdx.x, b = blockIdx.x;
  const int n = a.T * a.k;
  hist[tid] = 0;
  __syncthreads();
  const int beg = b * kPermBlock, end = min(n, beg + kPermBlock);
  bool bad = false;
  for (int i = beg + tid; i < end; i += 256) {
    const int e = a.ids[i];
    const bool ok = (unsigned)e < (unsigned)a.E;  // an id outside [0, E) counts as expert 0, flagged
    bad = bad || !ok;
    atomicAdd(&hist[ok ? e : 0], 1);
  }
  if (bad && a.p.flags) atomicOr(a.p.flags, kFlagExpertId);
  __syncthreads();
  if (tid < a.E) a.blk_counts[(size_t)b * a.E + tid] = hist[tid];
}

// Thread e: the exclusive prefix of expert e's counts over the blocks (its
// count in blocks before b), loaded in batches of independent loads; the
// expert offsets and the tile table. The scatter adds the offsets.
__global__ __launch_bounds__(256) void k_perm_scan(PermArgs a, int nblk) {
  __shared__ int tmp[256];
  const int tid = threadIdx.x;
  constexpr int kBatch = 16;
  int running = 0;
  if (tid < a.E) {
    for (int b0 = 0; b0 < nblk; b0 += kBatch) {
      int c[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) c[j] = a.blk_counts[(size_t)min(b0 + j, nblk - 1) * a.E + tid];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if (b0 + j < nblk) {
          a.blk_counts[(size_t)(b0 + j) * a.E + tid] = running;
          running += c[j];
        }
      }
    }
  }
  int total;
  const int off = block_exclusive_scan(tid < a.E ? running : 0, tmp, &total);
  if (tid < a.E) a.p.offsets[tid] = off;
  if (tid == 0) a.p.offsets[a.E] = total;
  write_tiles(running, off, a.E, a.p, tmp);
}

// Per block of kPermBlock slots, in chunks of 256 (4 waves): each slot's
// rank among the earlier slots of its expert. Within a wave, the lanes with
// the same expert come from 8 ballots (one per bit of the id) and the rank
// is the number of such lanes below; the waves then take their turns, in
// order, adding their group sizes to the block's running count per expert.
// Sorted position = expert offset + the expert's count in earlier blocks +
// the running count + the rank.
__global__ __launch_bounds__(256) void k_perm_scatter(PermArgs a) {
  __shared__ int seen[kMaxExperts];
  const int tid = threadIdx.x, b = blockIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = a.T * a.k;
  seen[tid] = 0;  // 256 threads, kMaxExperts = 256
  const int beg = b * kPermBlock, end = min(n, beg + kPermBlock);
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int c0 = beg; c0 < end; c0 += 256) {
    const int i = c0 + tid;
    int e = i < end ? a.ids[i] : -1;
    if (i < end && (unsigned)e >= (unsigned)a.E) e = 0;  // as in k_perm_count
    unsigned long long m = __ballot(e >= 0);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const bool set = ((e >> bit) & 1) != 0;
      const unsigned long long bs = __ballot(set);
      m &= set ? bs : ~bs;
    }
    const int rank = __popcll(m & below);
    const int group = __popcll(m);
    int base = 0;
    for (int w = 0; w < 4; ++w) {
      __syncthreads();
      if (wave == w && e >= 0) {
        base = seen[e];  // every lane of the group reads before its first lane adds
        if (rank == 0) seen[e] = base + group;
      }
    }
    __syncthreads();
    if (e >= 0) {
      const int pos = a.p.offsets[e] + a.blk_counts[(size_t)b * a.E + e] + base + rank;
      a.p.sorted_slots[pos] = i;
      a.p.slot_pos[i] = pos;
      a.p.sorted_tok[pos] = i / a.k;
    }
  }
}

// Tile table and token-of-position from expert offsets and sorted slots given
// by the caller (moe_expert_ffn), copied into the workspace's permutation
// after checking them: block 0 checks the offsets (0 first, T*k last,
// non-decreasing) and writes the tiles (none if the check fails), every
// block a slice of the sorted slots (each in [0, T*k), else clamped to 0)
// and of sorted_tok. Any violation sets kFlagPermutation.
__global__ __launch_bounds__(256) void k_tiles_from_offsets(int T, int E, int k, const int32_t* user_offsets,
                                                            const int32_t* user_sorted, Perm p) {
  __shared__ int tmp[256];
  __shared__ int bad;
  const int tid = threadIdx.x;
  const int n = T * k;
  if (blockIdx.x == 0) {
    if (tid == 0) bad = 0;
    __syncthreads();
    const int lo = tid < E ? user_offsets[tid] : 0, hi = tid < E ? user_offsets[tid + 1] : 0;
    if (tid < E && (hi < lo || lo < 0 || hi > n || (tid == 0 && lo != 0) || (tid == E - 1 && hi != n))) bad = 1;
    __syncthreads();
    const bool ok = bad == 0;
    if (tid < E) p.offsets[tid] = ok ? lo : 0;
    if (tid == 0) p.offsets[E] = ok ? n : 0;
    if (!ok && tid == 0 && p.flags) atomicOr(p.flags, kFlagPermutation);
    write_tiles(ok && tid < E ? hi - lo : 0, ok && tid < E ? lo : 0, E, p, tmp);
  }
  bool clamped = false;
  for (int i = blockIdx.x * 256 + tid; i < n; i += gridDim.x * 256) {
    int s = user_sorted[i];
    if ((unsigned)s >= (unsigned)n) {
      s = 0;
      clamped = true;
    }
    p.sorted_slots[i] = s;
    p.sorted_tok[i] = s / k;
  }
  if (clamped && p.flags) atomicOr(p.flags, kFlagPermutation);
}

hipError_t launch_permute(int T, int E, int k, const int32_t* ids, const Perm& p, int32_t* blk_counts,
                          hipStream_t st) {
  PermArgs a{T, E, k, ids, p, blk_counts};
  const int n = T * k;
  const int nblk = (n + kPermBlock - 1) / kPermBlock;
  if (nblk > 0) {
    k_perm_count<<<nblk, 256, 0, st>>>(a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  k_perm_scan<<<1, 256, 0, st>>>(a, nblk);  // nblk == 0: all experts empty
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || nblk == 0) return err;
  k_perm_scatter<<<nblk, 256, 0, st>>>(a);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_tile_records(Perm p, const float* slot_w) {
  write_tile_records(p, slot_w, blockIdx.x * 256 + threadIdx.x, gridDim.x * 256);
}

hipError_t launch_tile_records(const Perm& p, const float* slot_w, hipStream_t st) {
  const int blocks = (p.max_tiles * kRecInts + 255) / 256;
  k_tile_records<<<blocks < 1 ? 1 : blocks, 256, 0, st>>>(p, slot_w);
  return hipGetLastError();
}

hipError_t launch_tiles_from_offsets(int T, int E, int k, const int32_t* user_offsets, const int32_t* user_sorted,
                                     const Perm& p, hipStream_t st) {
  if (E > 256 || !user_offsets || !user_sorted) return hipErrorInvalidValue;  // one thread per expert
  const int n = T * k;
  int blocks = (n + 255) / 256;
  blocks = blocks < 1 ? 1 : (blocks > 1024 ? 1024 : blocks);
  k_tiles_from_offsets<<<blocks, 256, 0, st>>>(T, E, k, user_offsets, user_sorted, p);
  return hipGetLastError();
}

}  // namespace moe
