// Streaming expert pass for batched decode (2 < T <= 64) on gfx950: each
// wave owns its weight rows over the whole of K, so a block needs no
// cross-wave reduction, and every wave keeps D stages of its rows in flight
// through a branch-free register pipeline. MXFP4 routed experts ("w4a16")
// and the int8 per-channel shared expert ("w8a16"): page
// "deepseek-v4-mxfp4-int8 config.json", quantization_config. The w13 pass
// applies the clamped SwiGLU (page "DeepSeek-V4-Flash-0731", section
// "Checked in its code", row "SwiGLU feed-forward"); the routed w2 pass
// scales each slot by its routing weight, the shared w2 pass by the output
// channel's int8 scale.
//
// Unit (8 waves, one block per CU) = one tile of at most 16 activation
// columns (an expert's sorted positions, or consecutive tokens for the
// shared expert) x one row group: w13 = 128 h columns (wave w: gate rows and
// up rows of columns 16w .. 16w+15), w2 = 256 output rows (wave w: rows
// 32w .. 32w+31; rows past H in the last group are clamped on load and not
// stored).
//   - K runs in stages of 128. Lane (r = l%16, g = l/16) reads, per stage and
//     row block, 32 K-values of row r: MXFP4, the range 128 st + 32g .. +32
//     (16 bytes of E2M1 pairs, exactly one E8M0 group, whose byte the block
//     staged in LDS with all its rows' scales); int8, the two 16-value ranges
//     128 st + 16g and 128 st + 64 + 16g, so that each of the stage's two
//     loads covers 64 contiguous bytes of every row. Converted to bf16 in
//     registers, they feed four MFMA 16x16x32 bf16 per row block; the
//     activation fragments for the same K-values come from the tile's
//     columns in LDS. Any permutation of K shared by both operands leaves
//     the sums unchanged.
//
// Persistent grid with a work queue: only as many blocks as the chip holds
// at once; block b starts with unit b and then takes units from the pass's
// counter (one atomic per unit), so blocks that run faster take more units. (Two blocks sharing a CU do not
// stream at the same rate, so any fixed split leaves a tail.) Queue order:
// the shared units first, then the routed units, row group fastest; the
// live routed tile count is read on the device. A block grabs its units two
// ahead and loads their tile records (expert, first position, columns, the
// columns' activation rows, slots and routing weights: one 208-byte row
// written with the tile table) one ahead, so every look-up is ready before
// it is needed. Per unit:
//   - loads for stage st + D are issued right after stage st is consumed;
//   - in the last D stages the loads are the next unit's scales, activation
//     columns and epilogue scales, its tile record's successor and the next
//     grab, then its first D stages: the weight stream never drains between
//     units (after the block's last unit the same loads re-read that unit's
//     last stages, a cache hit, so that no load is conditional and the
//     compiler's waits count exactly);
//   - epilogue, barrier, the next unit's scales and columns to LDS, barrier.
#include "device.h"
#include "internal.h"
#include "skinny.h"

namespace moe {

constexpr int kStreamThreads = 512;
constexpr int kUnitRows = 256;  // weight rows per unit

// LDS row of a unit's scales: the row's E8M0 bytes (K/32) or binary16 scales
// (K/16), padded by 16 bytes so that the 16 rows a wave's lanes read in one
// instruction fall in different banks (unpadded, rows 64 or 128 bytes apart
// shared two banks).
__host__ __device__ inline int stream_scale_row(int K, bool q3) { return (q3 ? K / 16 : K / 32) + 16; }

template <int FMT>
struct StreamStage {
  uint4 q[FMT == kFmtI8 ? 2 : 1];
};

template <int FMT>
__device__ __forceinline__ void stream_load(const uint8_t* q, int st, StreamStage<FMT>& d) {
  if constexpr (FMT == kFmtMx) {
    d.q[0] = *reinterpret_cast<const uint4*>(q + (size_t)st * 64);
  } else if constexpr (FMT == kFmtQ3) {  // one 32-weight block: 12 bytes
    const uint32_t* s = reinterpret_cast<const uint32_t*>(q + (size_t)st * 48);
    d.q[0] = make_uint4(s[0], s[1], s[2], 0u);
  } else {
    d.q[0] = *reinterpret_cast<const uint4*>(q + (size_t)st * 128);
    d.q[1] = *reinterpret_cast<const uint4*>(q + (size_t)st * 128 + 64);
  }
}

// Per row block and stage, what turns the lane's codes into bf16: the E8M0
// scale operand (MXFP4), the scaled code book (3-bit), nothing (int8).
template <int FMT>
struct StreamDec {
  float sc;
};
template <>
struct StreamDec<kFmtQ3> {
  Q3Book book;
};

template <int FMT>
__device__ __forceinline__ bf16x8_t stream_frag(const StreamStage<FMT>& d, int kk, const StreamDec<FMT>& dec) {
  if constexpr (FMT == kFmtMx) {
    const uint32_t w = kk == 0 ? d.q[0].x : kk == 1 ? d.q[0].y : kk == 2 ? d.q[0].z : d.q[0].w;
    return fp4x8_to_bf16x8(w, dec.sc);
  } else if constexpr (FMT == kFmtQ3) {
    return q3_frag(d.q[0].x, d.q[0].y, d.q[0].z, kk, dec.book);
  } else {
    const uint4 u = d.q[kk >> 1];
    return i8x8_to_bf16x8((kk & 1) ? u.z : u.x, (kk & 1) ? u.w : u.y);
  }
}

// A unit of the queue: its index, this lane's int of its tile record, and
// the record's uniform fields.
struct SUnit {
  int idx, rec, e, pos0, ncols, rg;
};

// Units of one format while the queue hands them out: queue indices
// [lo, hi). idx holds the current unit and the two grabbed after it
// (uniform; idx[0] in range on entry). Returns with idx[0] the first unit
// handed out that is not of this format (or past the end), followed by the
// two grabbed after it. NS scale pieces and NA activation pieces per thread
// travel in registers; any beyond are loaded at the unit boundary.
//
// FUSED (w13 and w2 in one launch): a w13 unit writes its h with coherent
// (write-through) stores and counts itself in done[its tile] once they are
// complete (the count is issued at the block's next unit boundary, after
// every wave has waited for its stores); a w2 unit reads its h with
// coherent loads, after done[its tile] has reached done_target (the tile's
// w13 units). The count of the unit after next is polled one unit ahead.
template <int FMT, int MODE, int D, int NS, int NA, bool FUSED = false>
__device__ __forceinline__ void stream_loop(const SkinnyArgs& p, int lo, int hi, int* queue, int (&idx)[3],
                                            unsigned char* lds, int* sh, int* done = nullptr,
                                            int done_target = 0) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, g = lane >> 4;
  const int K = p.K, S = K >> 7, n16 = K >> 3, row_bytes = 2 * K + 16;
  const int nrb = p.n_rowblocks;
  // scale bytes per row (a multiple of 4): one E8M0 byte or one binary16 per 32 weights
  const int srow = FMT == kFmtQ3 ? K / 16 : K / 32;          // scale bytes per weight row
  const int srow_l = stream_scale_row(K, FMT == kFmtQ3);      // its padded LDS row
  unsigned char* lds_sc = lds + (size_t)p.tile_n * row_bytes;  // [256 rows][srow_l]
  // LDS place of piece i (of `piece` bytes) of the unit's scales
  auto sc_dst = [&](int i, int piece) {
    const int row = (i * piece) / srow;
    return lds_sc + (size_t)row * srow_l + (i * piece - row * srow);
  };
  const bool sc16 = srow % 16 == 0;                            // rows of whole 16-byte pieces
  const int nsc = FMT != kFmtI8 ? kUnitRows * srow / (sc16 ? 16 : 4) : 0;
  // this lane's two block rows (of the unit's 256)
  const int brA = MODE == kW13 ? wave * 16 + r : wave * 32 + r;
  const int brB = MODE == kW13 ? 128 + wave * 16 + r : wave * 32 + 16 + r;

  auto in_range = [&](int i) { return i >= lo && i < hi; };
  auto local = [&](int i) { return min(max(i, lo), hi - 1) - lo; };  // clamped into the range
  // the lane's int of unit i's tile record: routed tiles from the table,
  // shared tiles (consecutive tokens) computed
  auto rec_of = [&](int i) -> int {
    const int tile = local(i) / nrb;
    if constexpr (FMT != kFmtI8) {
      return p.tile_rec[(size_t)tile * kRecInts + min(lane, kRecInts - 1)];
    } else {
      const int pos0 = tile * p.tile_n, ncols = min(p.tile_n, p.T - pos0);
      return lane == 1 ? pos0 : lane == 2 ? ncols : (lane >= 4 && lane < 20) ? pos0 + min(lane - 4, ncols - 1) : 0;
    }
  };
  auto unit_of = [&](int i, int rec) {
    SUnit x;
    x.idx = i;
    x.rec = rec;
    x.e = __builtin_amdgcn_readlane(rec, 0);
    x.pos0 = __builtin_amdgcn_readlane(rec, 1);
    x.ncols = __builtin_amdgcn_readlane(rec, 2);
    x.rg = local(i) % nrb;
    return x;
  };
  auto grow = [&](const SUnit& x, int br) {  // weight row of block row br (clamped to the last)
    return MODE == kW13 ? (br < 128 ? x.rg * 128 + br : p.half + x.rg * 128 + (br - 128))
                        : min(x.rg * kUnitRows + br, p.rows - 1);
  };
  auto wptr = [&](const SUnit& x, int br) -> const uint8_t* {
    if (FMT == kFmtMx) return p.wq + (long long)x.e * p.q_expert_stride + (size_t)grow(x, br) * (K / 2) + g * 16;
    if (FMT == kFmtQ3)
      return p.wq + (long long)x.e * p.q_expert_stride + (size_t)grow(x, br) * (K / 32 * 12) + g * 12;
    return p.wq + (size_t)grow(x, br) * K + g * 16;
  };
  auto sc_src = [&](const SUnit& x, int i, int piece) {  // piece i of the unit's scales
    const int row = (i * piece) / srow;
    return p.wsc + (long long)x.e * p.s_expert_stride + (size_t)grow(x, row) * srow + (i * piece - row * srow);
  };
  // piece i (16 bytes) of the unit's columns; the row of its column from the
  // tile record (a shuffle: every lane must take part) or, in divergent
  // code, from memory
  auto act_src = [&](const SUnit& x, int i) {
    const int c = min(i / n16, x.ncols - 1), o = i - (i / n16) * n16;
    const int row = p.act_row ? __shfl(x.rec, 4 + c) : x.pos0 + c;
    return reinterpret_cast<const u32x4_t*>(p.act + (size_t)row * p.act_ld) + o;
  };
  auto act_src_mem = [&](const SUnit& x, int i) {
    const int c = i / n16, o = i - c * n16;
    const int row = p.act_row ? p.act_row[x.pos0 + c] : x.pos0 + c;
    return reinterpret_cast<const u32x4_t*>(p.act + (size_t)row * p.act_ld) + o;
  };
  auto act_dst = [&](int i) { return reinterpret_cast<u32x4_t*>(lds + (i / n16) * row_bytes + (i % n16) * 16); };
  auto act_load = [&](const u32x4_t* src) -> u32x4_t {
    if constexpr (FUSED && MODE == kW2) return load_agent_u32x4(src);
    else return *src;
  };
  // FUSED: tiles of units, their published counts, and the wait for a w2
  // unit's tile (bounded; every w13 unit is grabbed before any w2 unit and
  // its block finishes it without waiting, so the count always arrives)
  auto tile_of = [&](int i) { return local(i) / nrb; };
  auto poll = [&](int i) -> int {
    if constexpr (FUSED && MODE == kW2) return (int)load_agent(reinterpret_cast<const uint32_t*>(done + tile_of(i)));
    else return 0;
  };
  // returns false if the wait expired: the unit's outputs are then NaN and
  // the device error flag is set (never a silent value from a stale h)
  auto wait_tile = [&](int i, int seen) __attribute__((always_inline)) -> bool {
    if constexpr (FUSED && MODE == kW2) {
      int v = __builtin_amdgcn_readfirstlane(seen);
      for (int it = 0; v < done_target && it < (1 << 22); ++it) {
        __builtin_amdgcn_s_sleep(2);
        v = __builtin_amdgcn_readfirstlane(poll(i));
      }
      if (v < done_target) {
        if (threadIdx.x == 0 && p.flags) atomicOr(p.flags, kFlagWaitExpired);
        return false;
      }
    }
    return true;
  };
  int pub = -1;  // FUSED w13: tile of the unit whose completion is counted at the next boundary

  // register-staged operands of a unit: scales, activation pieces and the
  // int8 epilogue's row scales (every load unconditional: clamped indices)
  u32x4_t sv[NS], av[NA];
  float es[8] = {};
  auto load_ops = [&](const SUnit& x) __attribute__((always_inline)) {
    if constexpr (FMT != kFmtI8) {
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        // rows of dword pieces are loaded at the boundary; meanwhile a
        // harmless 16-byte read at the start of the expert's scales
        const uint8_t* src = sc16 ? sc_src(x, min(tid + j * kStreamThreads, nsc - 1), 16)
                                  : p.wsc + (long long)x.e * p.s_expert_stride;
        sv[j] = *reinterpret_cast<const u32x4_t*>(src);
      }
    }
    const int nact = x.ncols * n16;
#pragma unroll
    for (int j = 0; j < NA; ++j) av[j] = act_load(act_src(x, min(tid + j * kStreamThreads, nact - 1)));
    if constexpr (FMT == kFmtI8) {
      const int base = MODE == kW13 ? x.rg * 128 + wave * 16 + 4 * g : x.rg * kUnitRows + wave * 32 + 4 * g;
      const int off = MODE == kW13 ? p.half : 16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        es[i] = p.row_scale[min(base + i, p.rows - 1)];
        es[4 + i] = p.row_scale[min(base + off + i, p.rows - 1)];
      }
    }
    asm volatile("" ::: "memory");
  };
  auto store_ops = [&](const SUnit& x) __attribute__((always_inline)) {
    if constexpr (FMT != kFmtI8) {
      if (sc16) {
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          const int i = tid + j * kStreamThreads;
          if (i < nsc) *reinterpret_cast<u32x4_t*>(sc_dst(i, 16)) = sv[j];
        }
        for (int i = tid + NS * kStreamThreads; i < nsc; i += kStreamThreads)
          *reinterpret_cast<u32x4_t*>(sc_dst(i, 16)) = *reinterpret_cast<const u32x4_t*>(sc_src(x, i, 16));
      } else {
        for (int i = tid; i < nsc; i += kStreamThreads)
          *reinterpret_cast<uint32_t*>(sc_dst(i, 4)) = *reinterpret_cast<const uint32_t*>(sc_src(x, i, 4));
      }
    }
    const int nact = x.ncols * n16;
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      const int i = tid + j * kStreamThreads;
      if (i < nact) *act_dst(i) = av[j];
    }
    for (int i = tid + NA * kStreamThreads; i < nact; i += kStreamThreads) *act_dst(i) = act_load(act_src_mem(x, i));
  };

  // MXFP4 stages come in pairs whose loads are issued back to back: the two
  // 64-byte halves of each 128-byte line of a row (one int8 stage reads a
  // whole line in two adjacent loads already)
  constexpr int P = (FMT != kFmtI8 && D % 2 == 0) ? 2 : 1;

  // first unit: its record, its first D stages, its operands; the next
  // unit's record
  SUnit cur = unit_of(idx[0], rec_of(idx[0]));
  int rec_nxt = rec_of(idx[1]);
  float lv[8] = {};  // 3-bit: the current unit's expert's levels
  if constexpr (FMT == kFmtQ3) q3_levels(p.table, cur.e, lv);
  const uint8_t* qA = wptr(cur, brA);
  const uint8_t* qB = wptr(cur, brB);
  StreamStage<FMT> wA[D], wB[D];
#pragma unroll
  for (int i = 0; i < D; ++i) {
    stream_load<FMT>(qA, i, wA[i]);
    stream_load<FMT>(qB, i, wB[i]);
  }
  bool cur_ok = wait_tile(idx[0], poll(idx[0]));
  int poll_nxt = poll(idx[1]);
  load_ops(cur);
  store_ops(cur);
  __syncthreads();
  // FUSED w13: at a unit's last stages a wave's h stores of the unit before
  // are complete once at most the last main-loop iteration's loads are
  // outstanding (vmcnt(16): 8 MXFP4 stages x 2 loads, or 4 int8 stages x 4),
  // if the main loop ran at all; else once nothing is outstanding
  static_assert(!FUSED || MODE != kW13 || (FMT == kFmtMx ? 2 * D : 4 * D) == 16, "vmcnt of the h-store wait");
  const bool deep = S >= 2 * D;

  const bf16x8_t zero8 = {};
  for (;;) {
    f32x4_t accA = {0.f, 0.f, 0.f, 0.f}, accB = {0.f, 0.f, 0.f, 0.f};
    const bool live = r < cur.ncols;
    const unsigned char* bcol = lds + (live ? r : 0) * row_bytes + g * (FMT != kFmtI8 ? 64 : 32);
    // the scale of block 4 st + g of each row (MXFP4: a byte, 3-bit: a binary16)
    const unsigned char* scA = lds_sc + (size_t)brA * srow_l + g * (FMT == kFmtQ3 ? 2 : 1);
    const unsigned char* scB = lds_sc + (size_t)brB * srow_l + g * (FMT == kFmtQ3 ? 2 : 1);
    // byte offset in the column of fragment kk (the lane's K-values of it)
    auto kbyte = [](int kk) { return FMT != kFmtI8 ? kk * 16 : (kk >> 1) * 128 + (kk & 1) * 16; };
    auto dec_of = [&](const unsigned char* sc, int st) __attribute__((always_inline)) {
      StreamDec<FMT> d{};
      if constexpr (FMT == kFmtMx) d.sc = e8m0_scale_operand(sc[st * 4]);
      if constexpr (FMT == kFmtQ3)
        d.book = q3_book(lv, f16_bits_to_f32(*reinterpret_cast<const uint16_t*>(sc + st * 8)));
      return d;
    };
    auto stage = [&](int i, int st) __attribute__((always_inline)) {
      bf16x8_t b[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        b[kk] = live ? *reinterpret_cast<const bf16x8_t*>(bcol + st * 256 + kbyte(kk)) : zero8;
      const StreamDec<FMT> decA = dec_of(scA, st), decB = dec_of(scB, st);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        accA = mfma_16x16x32(stream_frag<FMT>(wA[i], kk, decA), b[kk], accA);
        accB = mfma_16x16x32(stream_frag<FMT>(wB[i], kk, decB), b[kk], accB);
      }
    };
    // Main loop: consume stages st0 .. st0+D-1, request st0+D .. st0+2D-1.
    // Every requested stage is below S by the loop condition; the launchers
    // require S to be a multiple of D (and S >= D), so the loop ends with
    // st0 = S - D and the last D stages below cover the rest exactly.
    int st0 = 0;
    for (; st0 + 2 * D <= S; st0 += D) {
#pragma unroll
      for (int i = 0; i < D; i += P) {
#pragma unroll
        for (int j = 0; j < P; ++j) stage(i + j, st0 + i + j);
#pragma unroll
        for (int j = 0; j < P; ++j) stream_load<FMT>(qA, st0 + i + j + D, wA[i + j]);
#pragma unroll
        for (int j = 0; j < P; ++j) stream_load<FMT>(qB, st0 + i + j + D, wB[i + j]);
      }
    }
    // the last D stages request the next unit: operands, the record after
    // it, the next grab, then its first stages
    const bool more = in_range(idx[1]);
    const SUnit nxt = unit_of(more ? idx[1] : idx[0], more ? rec_nxt : cur.rec);
    float lv_nxt[8] = {};
    if constexpr (FMT == kFmtQ3) q3_levels(p.table, nxt.e, lv_nxt);
    const uint8_t* nA = more ? wptr(nxt, brA) : qA;
    const uint8_t* nB = more ? wptr(nxt, brB) : qB;
    const int nst = more ? 0 : S - D;
    float ec[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) ec[i] = es[i];
    if constexpr (FUSED && MODE == kW13) {
      // vmcnt(16) / vmcnt(0), expcnt and lgkmcnt not waited for
      if (deep) __builtin_amdgcn_s_waitcnt((1 << 14) | (15 << 8) | (7 << 4));
      else __builtin_amdgcn_s_waitcnt((15 << 8) | (7 << 4));
    }
    const bool nxt_ok = more ? wait_tile(idx[1], poll_nxt) : true;
    load_ops(nxt);
    const int rec_after = rec_of(idx[2]);
    const int poll_after = poll(idx[2]);
    int grabbed = 0;
    if (tid == 0) grabbed = (int)gridDim.x + atomicAdd(queue, 1);
#pragma unroll
    for (int i = 0; i < D; i += P) {
#pragma unroll
      for (int j = 0; j < P; ++j) stage(i + j, st0 + i + j);
#pragma unroll
      for (int j = 0; j < P; ++j) stream_load<FMT>(nA, nst + i + j, wA[i + j]);
#pragma unroll
      for (int j = 0; j < P; ++j) stream_load<FMT>(nB, nst + i + j, wB[i + j]);
    }

    // epilogue: lane (r, g) holds rows 4g .. 4g+3 of each row block, column r
    int slot = 0;
    float wv = 0.0f;
    if (FMT != kFmtI8 && MODE == kW2) {  // every lane takes part in the shuffles
      slot = __shfl(cur.rec, 20 + r);
      wv = __int_as_float(__shfl(cur.rec, 36 + r));
    }
    if (live) {
      if (MODE == kW13) {
        const int hc = cur.rg * 128 + wave * 16 + 4 * g;
        uint16_t h[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float gv = accA[i], uv = accB[i];
          if (FMT == kFmtI8) {
            gv *= ec[i];
            uv *= ec[4 + i];
          }
          h[i] = f32_to_bf16(swiglu_clamped(gv, uv, p.limit));
        }
        uint2 packed;
        packed.x = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
        packed.y = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
        uint16_t* hdst = p.hout + (size_t)(cur.pos0 + r) * p.hout_ld + hc;
        if constexpr (FUSED) {
          __hip_atomic_store(reinterpret_cast<uint64_t*>(hdst), (uint64_t)packed.x | ((uint64_t)packed.y << 32),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
          *reinterpret_cast<uint2*>(hdst) = packed;
        }
      } else {
        const int n0 = cur.rg * kUnitRows + wave * 32 + 4 * g;
        float* dst;
        float4 ya, yb;
        if (!cur_ok) wv = __builtin_nanf("");  // the wait for this unit's h expired
        if (FMT != kFmtI8) {
          ya = make_float4(accA[0] * wv, accA[1] * wv, accA[2] * wv, accA[3] * wv);
          yb = make_float4(accB[0] * wv, accB[1] * wv, accB[2] * wv, accB[3] * wv);
          dst = p.yout + (size_t)slot * p.yout_ld;
        } else {
          if (!cur_ok) {
#pragma unroll
            for (int i = 0; i < 8; ++i) ec[i] = __builtin_nanf("");
          }
          ya = make_float4(accA[0] * ec[0], accA[1] * ec[1], accA[2] * ec[2], accA[3] * ec[3]);
          yb = make_float4(accB[0] * ec[4], accB[1] * ec[5], accB[2] * ec[6], accB[3] * ec[7]);
          dst = p.yout + (size_t)(cur.pos0 + r) * p.yout_ld;
        }
        if (n0 < p.rows) *reinterpret_cast<float4*>(dst + n0) = ya;  // rows come in whole blocks of 16
        if (n0 + 16 < p.rows) *reinterpret_cast<float4*>(dst + n0 + 16) = yb;
      }
    }
    // every wave is done with this unit's LDS; hand the grab to every thread
    __syncthreads();
    if constexpr (FUSED && MODE == kW13) {  // every wave has waited for the unit before's h stores
      if (tid == 0 && pub >= 0) atomicAdd(done + pub, 1);
      pub = tile_of(cur.idx);
    }
    if (tid == 0) sh[0] = grabbed;
    if (more) store_ops(nxt);
    __syncthreads();
    idx[0] = idx[1];
    idx[1] = idx[2];
    idx[2] = __builtin_amdgcn_readfirstlane(sh[0]);
    if (!more) break;
    cur = nxt;
    cur_ok = nxt_ok;
    if constexpr (FMT == kFmtQ3) {
#pragma unroll
      for (int c = 0; c < 8; ++c) lv[c] = lv_nxt[c];
    }
    rec_nxt = rec_after;
    poll_nxt = poll_after;
    qA = nA;
    qB = nB;
  }
  __builtin_amdgcn_s_waitcnt(0);  // the last unit's re-reads have landed before the registers are reused
  if constexpr (FUSED && MODE == kW13) {  // and its h stores are complete in every wave
    __syncthreads();
    if (tid == 0) atomicAdd(done + pub, 1);
  }
}

// Pass b (int8 shared) and pass a (MXFP4 routed) of the same stage in one
// persistent grid fed by one queue: indices [0, nb) are the shared units,
// [nb, nb + na) the routed ones (row group fastest in both).
template <int MODE, int DA, int DB>
__global__ __launch_bounds__(kStreamThreads) void k_stream(SkinnyArgs a, int has_a, SkinnyArgs b, int has_b,
                                                           int* queue) {
  extern __shared__ __align__(16) unsigned char lds[];
  __shared__ int sh[4];
  const int na = has_a ? (a.routed ? min(*a.n_tiles, a.n_tiles_grid) : a.n_tiles_grid) * a.n_rowblocks : 0;
  const int nb = has_b ? b.n_tiles_grid * b.n_rowblocks : 0;
  // the block's first unit is its own index; the queue hands out the rest,
  // from gridDim.x on
  const int G = gridDim.x;
  if (threadIdx.x == 0) sh[0] = G + atomicAdd(queue, 2);
  __syncthreads();
  const int next = __builtin_amdgcn_readfirstlane(sh[0]);
  int idx[3] = {(int)blockIdx.x, next, next + 1};
  constexpr int NSA = MODE == kW13 ? 4 : 2;  // all scale pieces of K = 4096 / 2048
  constexpr int NAA = MODE == kW13 ? 6 : 3;  // 6 columns of K = 4096 / 2048
  constexpr int NAB = MODE == kW13 ? 8 : 4;  // 8 columns
  if (idx[0] < nb) stream_loop<kFmtI8, MODE, DB, 1, NAB>(b, 0, nb, queue, idx, lds, sh);
  if (idx[0] >= nb && idx[0] < nb + na) stream_loop<kFmtMx, MODE, DA, NSA, NAA>(a, nb, nb + na, queue, idx, lds, sh);
}

// Both stages of the decode layer in one persistent grid fed by one queue:
// [0, e0) shared w13 units, [e0, e1) routed w13, [e1, e2) shared w2,
// [e2, e3) routed w2 (row group fastest in each). Every w13 unit is handed
// out before any w2 unit, so a block's w2 phase overlaps the other blocks'
// last w13 units and the w2 units start without a launch in between; a w2
// unit waits (rarely) for its tile's w13 units through done_r (routed tiles)
// and done_s (shared tiles), which the tile builders zero.
// Q3: the routed w2 pass reads 3-bit blocks; a unit's binary16 scales (256
// rows x K/16 bytes) are 4 pieces per thread at K = 2048.
template <int DA, int DB, bool Q3>
__global__ __launch_bounds__(kStreamThreads) void k_stream_fused(SkinnyArgs a13, SkinnyArgs b13, SkinnyArgs a2,
                                                                 SkinnyArgs b2, int* queue, int* done_r,
                                                                 int* done_s) {
  extern __shared__ __align__(16) unsigned char lds[];
  __shared__ int sh[4];
  const int tiles = min(*a13.n_tiles, a13.n_tiles_grid);
  const int e0 = b13.n_tiles_grid * b13.n_rowblocks;
  const int e1 = e0 + tiles * a13.n_rowblocks;
  const int e2 = e1 + b2.n_tiles_grid * b2.n_rowblocks;
  const int e3 = e2 + tiles * a2.n_rowblocks;
  const int G = gridDim.x;
  if (threadIdx.x == 0) sh[0] = G + atomicAdd(queue, 2);
  __syncthreads();
  const int next = __builtin_amdgcn_readfirstlane(sh[0]);
  int idx[3] = {(int)blockIdx.x, next, next + 1};
  if (idx[0] < e0) stream_loop<kFmtI8, kW13, DB, 1, 8, true>(b13, 0, e0, queue, idx, lds, sh, done_s, 0);
  if (idx[0] >= e0 && idx[0] < e1)
    stream_loop<kFmtMx, kW13, DA, 4, 6, true>(a13, e0, e1, queue, idx, lds, sh, done_r, 0);
  if (idx[0] >= e1 && idx[0] < e2)
    stream_loop<kFmtI8, kW2, DB, 1, 4, true>(b2, e1, e2, queue, idx, lds, sh, done_s, b13.n_rowblocks);
  if (idx[0] >= e2 && idx[0] < e3)
    stream_loop<Q3 ? kFmtQ3 : kFmtMx, kW2, DA, Q3 ? 4 : 2, 3, true>(a2, e2, e3, queue, idx, lds, sh, done_r,
                                                                   a13.n_rowblocks);
}

// Blocks of kernel k with lds bytes that the current device holds at once
// (0 if unknown), cached per device, kernel and size.
static int stream_resident(const void* k, size_t lds) {
  constexpr int kDev = 16, kSlots = 16;
  struct Entry {
    const void* k;
    size_t lds;
    int n;
  };
  static Entry seen[kDev][kSlots];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDev) return 0;
  for (int i = 0; i < kSlots; ++i)
    if (seen[dev][i].k == k && seen[dev][i].lds == lds) return seen[dev][i].n;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, kStreamThreads, lds) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  for (int i = 0; i < kSlots; ++i)
    if (!seen[dev][i].k) {
      seen[dev][i] = Entry{k, lds, per_cu * cus};
      break;
    }
  return per_cu * cus;
}

// The stage loop of stream_loop needs the stage count S = K / 128 to be a
// multiple of the stage depth D and at least D: the main loop steps D stages
// at a time and the last D stages (and the next unit's first D, or the
// re-read of the last D) are handled after it.
inline bool stream_depth_ok(int K, int D) {
  const int S = K >> 7;
  return K % 128 == 0 && S >= D && S % D == 0;
}

template <int MODE, int DA, int DB>
static hipError_t launch_stream_t(const SkinnyArgs& a, int a_blocks, const SkinnyArgs& b, int b_blocks, int* queue,
                                  hipStream_t st) {
  const long long nblk = (long long)a_blocks + b_blocks;
  if (nblk <= 0) return hipSuccess;
  if (nblk > 0x3fffffffLL || !queue) return hipErrorInvalidValue;
  if ((a_blocks > 0 && !stream_depth_ok(a.K, DA)) || (b_blocks > 0 && !stream_depth_ok(b.K, DB)))
    return hipErrorInvalidValue;
  if ((a_blocks > 0 && (a.tile_n > 16 || a.tile_n < 1 || !a.tile_rec)) ||
      (b_blocks > 0 && (b.tile_n > 16 || b.tile_n < 1)))
    return hipErrorInvalidValue;
  size_t lds = 0;
  if (a_blocks > 0) lds = (size_t)a.tile_n * (2 * (size_t)a.K + 16) + kUnitRows * (size_t)stream_scale_row(a.K, false);
  if (b_blocks > 0) {
    const size_t lb = (size_t)b.tile_n * (2 * (size_t)b.K + 16);
    lds = lb > lds ? lb : lds;
  }
  auto kern = &k_stream<MODE, DA, DB>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  // one block per resident slot, never more than there are units
  const int res = stream_resident(reinterpret_cast<const void*>(kern), lds);
  if (res <= 0) return hipErrorInvalidValue;
  const long long grid = nblk < res ? nblk : res;
  kern<<<(unsigned)grid, kStreamThreads, lds, st>>>(a, a_blocks > 0 ? 1 : 0, b, b_blocks > 0 ? 1 : 0, queue);
  return hipGetLastError();
}

size_t stream_unit_lds(int tile_n, int K, bool q3) {
  return (size_t)tile_n * (2 * (size_t)K + 16) + kUnitRows * (size_t)stream_scale_row(K, q3);
}

static size_t stream_lds(const SkinnyArgs& a, int a_blocks, const SkinnyArgs& b, int b_blocks) {
  size_t lds = 0;
  if (a_blocks > 0)
    lds = (size_t)a.tile_n * (2 * (size_t)a.K + 16) + kUnitRows * (size_t)stream_scale_row(a.K, a.fmt == kFmtQ3);
  if (b_blocks > 0) {
    const size_t lb = (size_t)b.tile_n * (2 * (size_t)b.K + 16);
    lds = lb > lds ? lb : lds;
  }
  return lds;
}

hipError_t launch_stream_fused(const SkinnyArgs& a13, const SkinnyArgs& b13, const SkinnyArgs& a2,
                               const SkinnyArgs& b2, int a_blocks13, int b_blocks13, int a_blocks2, int b_blocks2,
                               int* queue, int* done_r, int* done_s, hipStream_t st) {
  if (a13.K % 1024 || a2.K % 1024 || !queue || !done_r || !done_s || !a13.tile_rec || !a2.tile_rec ||
      b13.tile_n != b2.tile_n || b13.n_tiles_grid != b2.n_tiles_grid || a13.tile_n > 16 || b13.tile_n > 16 ||
      a13.tile_n < 1 || b13.tile_n < 1 || a_blocks13 <= 0 || b_blocks13 <= 0)
    return hipErrorInvalidValue;
  constexpr int kDA = 8, kDB = 4;  // stage depths of k_stream_fused<kDA, kDB>
  if (!stream_depth_ok(a13.K, kDA) || !stream_depth_ok(a2.K, kDA) || !stream_depth_ok(b13.K, kDB) ||
      !stream_depth_ok(b2.K, kDB))
    return hipErrorInvalidValue;
  const long long nblk = (long long)a_blocks13 + b_blocks13 + a_blocks2 + b_blocks2;
  if (nblk > 0x3fffffffLL) return hipErrorInvalidValue;
  const bool q3 = a2.fmt == kFmtQ3;
  if (a13.fmt == kFmtQ3) return hipErrorInvalidValue;  // 3-bit blocks are a w2 format
  size_t lds = stream_lds(a13, a_blocks13, b13, b_blocks13);
  const size_t l2 = stream_lds(a2, a_blocks2, b2, b_blocks2);
  lds = l2 > lds ? l2 : lds;
  auto kern = q3 ? &k_stream_fused<kDA, kDB, true> : &k_stream_fused<kDA, kDB, false>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const int res = stream_resident(reinterpret_cast<const void*>(kern), lds);
  if (res <= 0) return hipErrorInvalidValue;
  const long long grid = nblk < res ? nblk : res;
  kern<<<(unsigned)grid, kStreamThreads, lds, st>>>(a13, b13, a2, b2, queue, done_r, done_s);
  return hipGetLastError();
}

// Row groups: w13 I/128 (128 h columns each), w2 ceil(H/256) (256 rows
// each); the caller sets n_rowblocks to that count, rows to the pass's
// weight rows, and a_blocks / b_blocks to the most units each pass can have
// (tiles x row groups). Stage depth D: 8
// (MXFP4) and 4 (int8) when the stage count is a multiple of 8, else the
// largest that divides it of 4 and 1.
hipError_t launch_stream(int mode, const SkinnyArgs& a, int a_blocks, const SkinnyArgs* b, int b_blocks, int* queue,
                         hipStream_t st) {
  if (a_blocks > 0 && a.fmt == kFmtQ3) return hipErrorInvalidValue;  // 3-bit w2 runs in the fused launch only
  SkinnyArgs bb{};
  if (b) bb = *b; else b_blocks = 0;
  const int K = a_blocks > 0 ? a.K : bb.K;
  if (K % 128 || (a_blocks > 0 && b_blocks > 0 && a.K != bb.K)) return hipErrorInvalidValue;
  const int S = K / 128;
  if (mode == kW13) {
    if (S % 8 == 0) return launch_stream_t<kW13, 8, 4>(a, a_blocks, bb, b_blocks, queue, st);
    if (S % 4 == 0) return launch_stream_t<kW13, 4, 4>(a, a_blocks, bb, b_blocks, queue, st);
    return launch_stream_t<kW13, 1, 1>(a, a_blocks, bb, b_blocks, queue, st);
  }
  if (S % 8 == 0) return launch_stream_t<kW2, 8, 4>(a, a_blocks, bb, b_blocks, queue, st);
  if (S % 4 == 0) return launch_stream_t<kW2, 4, 4>(a, a_blocks, bb, b_blocks, queue, st);
  return launch_stream_t<kW2, 1, 1>(a, a_blocks, bb, b_blocks, queue, st);
}

}  // namespace moe
