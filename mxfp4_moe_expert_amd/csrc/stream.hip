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
// Unit (4 waves) = one tile of at most 16 activation columns (an expert's
// sorted positions, or consecutive tokens for the shared expert) x one row
// group: w13 = 64 h columns (wave w: gate rows and up rows of columns
// 16w .. 16w+15), w2 = 128 output rows (wave w: rows 32w .. 32w+31).
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
// Persistent grid: only as many blocks as the chip holds at once, so no
// block waits for the dispatcher and no block is spent on a tile that
// routing left empty (the live tile count is read on the device). The
// shared units go to the first blocks, the routed units to the rest, in
// proportion to their weight bytes; each block takes a contiguous run of
// units, row group fastest, so consecutive units mostly share a tile. Per
// run of at most kMetaTiles tiles the block stages their metadata in LDS
// (expert, first position, columns, each column's activation row and, for
// the routed w2 pass, slot and routing weight); every later look-up is an
// LDS read. Per unit:
//   - loads for stage st + D are issued right after stage st is consumed;
//   - in the last D stages the loads are the next unit's first D stages,
//     after its scales and epilogue scales: the weight stream never drains
//     between units (after the block's last unit the same loads re-read
//     that unit's last stages, a cache hit, so that no load is conditional
//     and the compiler's waits count exactly);
//   - epilogue, barrier, the next unit's scales to LDS (and its activation
//     columns, if its tile differs), barrier.
#include "device.h"
#include "internal.h"
#include "skinny.h"

namespace moe {

constexpr int kStreamThreads = 256;
constexpr int kMetaTiles = 16;  // tiles whose metadata is staged at once
// per tile: expert, first position, columns, unused, then per column its
// activation row, its slot and its routing weight (bits)
constexpr int kMetaInts = 4 + 3 * 16;
constexpr int kMetaBytes = kMetaTiles * kMetaInts * 4;

template <int FMT>
struct StreamStage {
  uint4 q[FMT == kFmtMx ? 1 : 2];
};

template <int FMT>
__device__ __forceinline__ void stream_load(const uint8_t* q, int st, StreamStage<FMT>& d) {
  if constexpr (FMT == kFmtMx) {
    d.q[0] = *reinterpret_cast<const uint4*>(q + (size_t)st * 64);
  } else {
    d.q[0] = *reinterpret_cast<const uint4*>(q + (size_t)st * 128);
    d.q[1] = *reinterpret_cast<const uint4*>(q + (size_t)st * 128 + 64);
  }
}

// scale: the E8M0 byte of the lane's group (MXFP4), unused for int8
template <int FMT>
__device__ __forceinline__ bf16x8_t stream_frag(const StreamStage<FMT>& d, int kk, uint32_t scale) {
  if constexpr (FMT == kFmtMx) {
    const uint32_t w = kk == 0 ? d.q[0].x : kk == 1 ? d.q[0].y : kk == 2 ? d.q[0].z : d.q[0].w;
    return fp4x8_to_bf16x8(w, e8m0_scale_operand(scale));
  } else {
    const uint4 u = d.q[kk >> 1];
    return i8x8_to_bf16x8((kk & 1) ? u.z : u.x, (kk & 1) ? u.w : u.y);
  }
}

// Metadata of tiles t0 .. t0+nt-1 -> LDS (two rounds: tile entries, then the
// per-column values that depend on them). Starts with a barrier: the
// previous run's units may still be reading the region.
template <int FMT, int MODE>
__device__ __forceinline__ void stage_meta(const SkinnyArgs& p, int t0, int nt, int* meta) {
  const int tid = threadIdx.x;
  __syncthreads();
  if (tid < nt) {
    const int t = t0 + tid;
    int e = 0, pos0, ncols;
    if (p.routed) {
      const int4 ti = p.tile_info[t];
      e = ti.x;
      pos0 = ti.y;
      ncols = ti.z;
    } else {
      pos0 = t * p.tile_n;
      ncols = min(p.tile_n, p.T - pos0);
    }
    meta[tid * kMetaInts + 0] = e;
    meta[tid * kMetaInts + 1] = pos0;
    meta[tid * kMetaInts + 2] = ncols;
  }
  __syncthreads();
  if (tid < nt * 16) {  // nt * 16 <= kStreamThreads
    int* m = meta + (tid >> 4) * kMetaInts;
    const int c = tid & 15;
    const int pos = m[1] + min(c, m[2] - 1);  // columns past the tile repeat its last one
    m[4 + c] = p.act_row ? p.act_row[pos] : pos;
    if (FMT == kFmtMx && MODE == kW2) {
      const int slot = p.sorted_slots[pos];
      m[20 + c] = slot;
      m[36 + c] = __float_as_int(p.slot_w[slot]);
    }
  }
  __syncthreads();
}

// Units [u0, u1) of one run (their tiles' metadata at meta, tile t0 first).
// NS scale pieces per thread travel in registers from the previous unit's
// last stages (any beyond are loaded at the unit boundary); the activation
// columns are loaded at the boundary when the tile changes, which a run of
// consecutive units seldom does.
template <int FMT, int MODE, int D, int NS>
__device__ __forceinline__ void stream_run(const SkinnyArgs& p, int u0, int u1, int t0, unsigned char* lds,
                                           const int* meta) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, g = lane >> 4;
  const int K = p.K, S = K >> 7, n16 = K >> 3, row_bytes = 2 * K + 16;
  const int nrb = p.n_rowblocks;
  const int srow = K / 32;  // scale bytes per row (a multiple of 4)
  unsigned char* lds_sc = lds + (size_t)p.tile_n * row_bytes;  // [128 rows][srow]
  const bool sc16 = srow % 16 == 0;                            // rows of whole 16-byte pieces
  const int nsc = FMT == kFmtMx ? 128 * srow / (sc16 ? 16 : 4) : 0;
  // this lane's two block rows (of the unit's 128)
  const int brA = MODE == kW13 ? wave * 16 + r : wave * 32 + r;
  const int brB = MODE == kW13 ? 64 + wave * 16 + r : wave * 32 + 16 + r;

  struct Unit {
    int e, pos0, ncols, rg, tl;
  };
  auto unit_at = [&](int u) {
    Unit x;
    const int tg = u / nrb;
    x.rg = u - tg * nrb;
    x.tl = tg - t0;
    const int* m = meta + x.tl * kMetaInts;
    x.e = __builtin_amdgcn_readfirstlane(m[0]);
    x.pos0 = __builtin_amdgcn_readfirstlane(m[1]);
    x.ncols = __builtin_amdgcn_readfirstlane(m[2]);
    return x;
  };
  auto grow = [&](const Unit& x, int br) {  // weight row of block row br
    return MODE == kW13 ? (br < 64 ? x.rg * 64 + br : p.half + x.rg * 64 + (br - 64)) : x.rg * 128 + br;
  };
  auto wptr = [&](const Unit& x, int br) -> const uint8_t* {
    if (FMT == kFmtMx) return p.wq + (long long)x.e * p.q_expert_stride + (size_t)grow(x, br) * (K / 2) + g * 16;
    return p.wq + (size_t)grow(x, br) * K + g * 16;
  };
  auto sc_src = [&](const Unit& x, int i, int piece) {  // piece i of the unit's scales
    const int row = (i * piece) / srow;
    return p.wsc + (long long)x.e * p.s_expert_stride + (size_t)grow(x, row) * srow + (i * piece - row * srow);
  };
  auto act_src = [&](const Unit& x, int i) {  // piece i (16 bytes) of the unit's columns
    const int c = min(i / n16, x.ncols - 1), o = i - (i / n16) * n16;
    const int row = meta[x.tl * kMetaInts + 4 + c];
    return reinterpret_cast<const u32x4_t*>(p.act + (size_t)row * p.act_ld) + o;
  };
  auto act_dst = [&](int i) { return reinterpret_cast<u32x4_t*>(lds + (i / n16) * row_bytes + (i % n16) * 16); };

  // register-staged operands of a unit: scales and the int8 epilogue's row
  // scales (every load unconditional: clamped indices)
  u32x4_t sv[NS];
  float es[8] = {};
  auto load_ops = [&](const Unit& x) __attribute__((always_inline)) {
    if constexpr (FMT == kFmtMx) {
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        // rows of dword pieces are loaded at the boundary; meanwhile a
        // harmless 16-byte read at the start of the expert's scales
        const uint8_t* src = sc16 ? sc_src(x, min(tid + j * kStreamThreads, nsc - 1), 16)
                                  : p.wsc + (long long)x.e * p.s_expert_stride;
        sv[j] = *reinterpret_cast<const u32x4_t*>(src);
      }
    }
    if constexpr (FMT == kFmtI8) {
      const int base = MODE == kW13 ? x.rg * 64 + wave * 16 + 4 * g : x.rg * 128 + wave * 32 + 4 * g;
      const int off = MODE == kW13 ? p.half : 16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        es[i] = p.row_scale[base + i];
        es[4 + i] = p.row_scale[base + off + i];
      }
    }
    asm volatile("" ::: "memory");
  };
  auto store_ops = [&](const Unit& x, bool new_tile) __attribute__((always_inline)) {
    if constexpr (FMT == kFmtMx) {
      if (sc16) {
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          const int i = tid + j * kStreamThreads;
          if (i < nsc) *reinterpret_cast<u32x4_t*>(lds_sc + i * 16) = sv[j];
        }
        for (int i = tid + NS * kStreamThreads; i < nsc; i += kStreamThreads)
          *reinterpret_cast<u32x4_t*>(lds_sc + i * 16) = *reinterpret_cast<const u32x4_t*>(sc_src(x, i, 16));
      } else {
        for (int i = tid; i < nsc; i += kStreamThreads)
          *reinterpret_cast<uint32_t*>(lds_sc + i * 4) = *reinterpret_cast<const uint32_t*>(sc_src(x, i, 4));
      }
    }
    if (new_tile) {
      const int nact = x.ncols * n16;
      for (int i0 = 0; i0 < nact; i0 += 4 * kStreamThreads) {  // 4 pieces per thread in flight
        u32x4_t v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = *act_src(x, min(i0 + tid + j * kStreamThreads, nact - 1));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = i0 + tid + j * kStreamThreads;
          if (i < nact) *act_dst(i) = v[j];
        }
      }
    }
  };

  // MXFP4 stages come in pairs whose loads are issued back to back: the two
  // 64-byte halves of each 128-byte line of a row (one int8 stage reads a
  // whole line in two adjacent loads already)
  constexpr int P = (FMT == kFmtMx && D % 2 == 0) ? 2 : 1;

  // first unit: its first D stages, then its operands
  Unit cur = unit_at(u0);
  const uint8_t* qA = wptr(cur, brA);
  const uint8_t* qB = wptr(cur, brB);
  StreamStage<FMT> wA[D], wB[D];
#pragma unroll
  for (int i = 0; i < D; ++i) {
    stream_load<FMT>(qA, i, wA[i]);
    stream_load<FMT>(qB, i, wB[i]);
  }
  load_ops(cur);
  store_ops(cur, true);
  __syncthreads();

  const bf16x8_t zero8 = {};
  for (int u = u0;; ++u) {
    f32x4_t accA = {0.f, 0.f, 0.f, 0.f}, accB = {0.f, 0.f, 0.f, 0.f};
    const bool live = r < cur.ncols;
    const unsigned char* bcol = lds + (live ? r : 0) * row_bytes + g * (FMT == kFmtMx ? 64 : 32);
    const unsigned char* scA = lds_sc + (size_t)brA * srow + g;  // group 4 st + g of each row
    const unsigned char* scB = lds_sc + (size_t)brB * srow + g;
    // byte offset in the column of fragment kk (the lane's K-values of it)
    auto kbyte = [](int kk) { return FMT == kFmtMx ? kk * 16 : (kk >> 1) * 128 + (kk & 1) * 16; };
    auto stage = [&](int i, int st) __attribute__((always_inline)) {
      bf16x8_t b[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        b[kk] = live ? *reinterpret_cast<const bf16x8_t*>(bcol + st * 256 + kbyte(kk)) : zero8;
      const uint32_t scaleA = FMT == kFmtMx ? scA[st * 4] : 0u;
      const uint32_t scaleB = FMT == kFmtMx ? scB[st * 4] : 0u;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        accA = mfma_16x16x32(stream_frag<FMT>(wA[i], kk, scaleA), b[kk], accA);
        accB = mfma_16x16x32(stream_frag<FMT>(wB[i], kk, scaleB), b[kk], accB);
      }
    };
    int st0 = 0;
    for (; st0 + D < S; st0 += D) {  // S is a multiple of D
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
    // the last D stages request the next unit: operands, then first stages
    const bool more = u + 1 < u1;
    const Unit nxt = unit_at(more ? u + 1 : u);
    const uint8_t* nA = more ? wptr(nxt, brA) : qA;
    const uint8_t* nB = more ? wptr(nxt, brB) : qB;
    const int nst = more ? 0 : S - D;
    float ec[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) ec[i] = es[i];
    load_ops(nxt);
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
    if (live) {
      if (MODE == kW13) {
        const int hc = cur.rg * 64 + wave * 16 + 4 * g;
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
        *reinterpret_cast<uint2*>(p.hout + (size_t)(cur.pos0 + r) * p.hout_ld + hc) = packed;
      } else {
        const int n0 = cur.rg * 128 + wave * 32 + 4 * g;
        float* dst;
        float4 ya, yb;
        if (FMT == kFmtMx) {
          const int* m = meta + cur.tl * kMetaInts;
          const float wv = __int_as_float(m[36 + r]);
          ya = make_float4(accA[0] * wv, accA[1] * wv, accA[2] * wv, accA[3] * wv);
          yb = make_float4(accB[0] * wv, accB[1] * wv, accB[2] * wv, accB[3] * wv);
          dst = p.yout + (size_t)m[20 + r] * p.yout_ld;
        } else {
          ya = make_float4(accA[0] * ec[0], accA[1] * ec[1], accA[2] * ec[2], accA[3] * ec[3]);
          yb = make_float4(accB[0] * ec[4], accB[1] * ec[5], accB[2] * ec[6], accB[3] * ec[7]);
          dst = p.yout + (size_t)(cur.pos0 + r) * p.yout_ld;
        }
        *reinterpret_cast<float4*>(dst + n0) = ya;
        *reinterpret_cast<float4*>(dst + n0 + 16) = yb;
      }
    }
    if (!more) break;
    __syncthreads();  // every wave is done with this unit's LDS
    store_ops(nxt, nxt.tl != cur.tl);
    __syncthreads();
    cur = nxt;
    qA = nA;
    qB = nB;
  }
  __builtin_amdgcn_s_waitcnt(0);  // the last unit's re-reads have landed before the registers are reused
}

// Units [u0, u1) of one pass, in runs of at most kMetaTiles tiles.
template <int FMT, int MODE, int D, int NS>
__device__ __forceinline__ void stream_units(const SkinnyArgs& p, long long u0, long long u1, unsigned char* lds) {
  const int nrb = p.n_rowblocks;
  int* meta = reinterpret_cast<int*>(lds + (size_t)p.tile_n * (2 * (size_t)p.K + 16) +
                                     (FMT == kFmtMx ? 128 * (size_t)(p.K / 32) : 0));
  for (long long s0 = u0; s0 < u1;) {
    const int t0 = (int)(s0 / nrb);
    const long long s1 = min(u1, (long long)(t0 + kMetaTiles) * nrb);
    const int nt = (int)((s1 - 1) / nrb) - t0 + 1;
    stage_meta<FMT, MODE>(p, t0, nt, meta);
    stream_run<FMT, MODE, D, NS>(p, (int)s0, (int)s1, t0, lds, meta);
    s0 = s1;
  }
}

// Pass b (int8 shared) and pass a (MXFP4 routed) of the same stage in one
// persistent grid: blocks [0, gb) take the shared units, the rest the routed
// ones; gb splits the grid in proportion to the weight bytes of the two
// (per row: K int8 bytes; K/2 code bytes + K/32 scale bytes).
template <int MODE, int DA, int DB>
__global__ __launch_bounds__(kStreamThreads) void k_stream(SkinnyArgs a, int has_a, SkinnyArgs b, int has_b) {
  extern __shared__ __align__(16) unsigned char lds[];
  const long long a_tiles = has_a ? (a.routed ? min(*a.n_tiles, a.n_tiles_grid) : a.n_tiles_grid) : 0;
  const long long na = a_tiles * a.n_rowblocks;
  const long long nb = has_b ? (long long)b.n_tiles_grid * b.n_rowblocks : 0;
  const long long G = gridDim.x, x = blockIdx.x;
  long long gb = 0;
  if (nb > 0 && na == 0) {
    gb = G;
  } else if (nb > 0) {
    const long long cb = nb * 32, tot = cb + na * 17;
    gb = max(1LL, min(G - 1, (G * cb + tot / 2) / tot));
  }
  constexpr int NSA = MODE == kW13 ? 4 : 2;  // all scale pieces of K = 4096 / 2048
  if (x < gb) {
    stream_units<kFmtI8, MODE, DB, 1>(b, nb * x / gb, nb * (x + 1) / gb, lds);
  } else {
    const long long m = G - gb, i = x - gb;
    stream_units<kFmtMx, MODE, DA, NSA>(a, na * i / m, na * (i + 1) / m, lds);
  }
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

template <int MODE, int DA, int DB>
static hipError_t launch_stream_t(const SkinnyArgs& a, int a_blocks, const SkinnyArgs& b, int b_blocks,
                                  hipStream_t st) {
  const long long nblk = (long long)a_blocks + b_blocks;
  if (nblk <= 0) return hipSuccess;
  if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
  if ((a_blocks > 0 && (a.tile_n > 16 || a.tile_n < 1)) || (b_blocks > 0 && (b.tile_n > 16 || b.tile_n < 1)))
    return hipErrorInvalidValue;
  size_t lds = 0;
  if (a_blocks > 0) lds = (size_t)a.tile_n * (2 * (size_t)a.K + 16) + 128 * (size_t)(a.K / 32);
  if (b_blocks > 0) {
    const size_t lb = (size_t)b.tile_n * (2 * (size_t)b.K + 16);
    lds = lb > lds ? lb : lds;
  }
  lds += kMetaBytes;
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
  kern<<<(unsigned)grid, kStreamThreads, lds, st>>>(a, a_blocks > 0 ? 1 : 0, b, b_blocks > 0 ? 1 : 0);
  return hipGetLastError();
}

// Row groups: w13 I/64 (64 h columns each), w2 H/128 (128 rows each); the
// caller sets n_rowblocks to that count, and a_blocks / b_blocks to the
// most units each pass can have (tiles x row groups). Stage depth D: 8
// (MXFP4) and 4 (int8) when the stage count is a multiple of 8, else the
// largest that divides it of 4 and 1.
hipError_t launch_stream(int mode, const SkinnyArgs& a, int a_blocks, const SkinnyArgs* b, int b_blocks,
                         hipStream_t st) {
  SkinnyArgs bb{};
  if (b) bb = *b; else b_blocks = 0;
  const int K = a_blocks > 0 ? a.K : bb.K;
  if (K % 128 || (a_blocks > 0 && b_blocks > 0 && a.K != bb.K)) return hipErrorInvalidValue;
  const int S = K / 128;
  if (mode == kW13) {
    if (S % 8 == 0) return launch_stream_t<kW13, 8, 4>(a, a_blocks, bb, b_blocks, st);
    if (S % 4 == 0) return launch_stream_t<kW13, 4, 4>(a, a_blocks, bb, b_blocks, st);
    return launch_stream_t<kW13, 1, 1>(a, a_blocks, bb, b_blocks, st);
  }
  if (S % 8 == 0) return launch_stream_t<kW2, 8, 4>(a, a_blocks, bb, b_blocks, st);
  if (S % 4 == 0) return launch_stream_t<kW2, 4, 4>(a, a_blocks, bb, b_blocks, st);
  return launch_stream_t<kW2, 1, 1>(a, a_blocks, bb, b_blocks, st);
}

}  // namespace moe
