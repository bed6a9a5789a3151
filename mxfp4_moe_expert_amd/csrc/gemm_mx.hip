// Routed-expert grouped GEMM for large token counts on gfx950's block-scaled
// matrix cores: MXFP4 weights go to v_mfma_scale_f32_32x32x64_f8f6f4 as they
// are stored (E2M1 codes, one E8M0 exponent per 32 weights along K; page
// "deepseek-v4-mxfp4-int8 config.json", quantization_config, experts_w4a16),
// and every bf16 activation x is split exactly into two fp8 (E4M3) values with
// their own E8M0 block exponents, x = hi * 2^(sh-127) + lo * 2^(sl-127), so
// that W x = W hi + W lo: two scaled MFMAs per 64-K step replace the bf16
// MFMAs and the FP4 -> bf16 converts. The split is exact: a bf16 value has 8
// significant bits, hi keeps the leading 4 (E4M3), and the remainder has at
// most 4 significant bits, which lo holds exactly for every element within
// 2^13 of its 32-block's largest magnitude (smaller ones, whose remainder
// could round, are below 2^-21 of that maximum). The products are exact and
// the MFMA sums in fp32, so the result matches the bf16 path up to
// summation order.
//
// Operand layout of the instruction (measured on gfx950 with one-hot inputs):
// for a 32 x 32 x 64 step, lane l = 32 g + c holds
//   A: the 16 bytes of E2M1 codes of weight row c, group g of the step
//      (K 32g .. 32g+31), and that group's E8M0 byte as its scale;
//   B: for token c, K 16g .. 16g+15 and 32+16g .. 32+16g+15 (fp8), and the
//      E8M0 byte of token c's group g as its scale;
//   D: token c, weight rows 8 (i/4) + 4 g + i%4, i = 0 .. 15.
//
// Tile: 256 weight rows x 128 token positions, one block of 4 waves (one per
// SIMD, each with up to 512 registers). Wave w owns 64 rows (two 32-row blocks; for w13 32 gate rows and the matching 32
// up rows, so the clamped SwiGLU is computed in registers) x all 128 tokens
// (four 32-token blocks): 8 accumulators of 32 x 32.
//   - K runs in stages of 128. Per stage and row block, a lane loads its 16
//     code bytes for each of the two 64-K steps straight into registers, and
//     one dword of its row's E8M0 bytes (the stage's four groups), two stages
//     ahead.
//   - The tile's gathered activation rows (hi and lo, 128 bytes each per
//     stage) go global -> registers -> LDS, double-buffered, one stage ahead,
//     stored fragment-major: for each (token block, 64-K step, hi/lo, half of
//     the lane's 32 bytes) the 64 lanes' 16-byte pieces lie contiguously in
//     lane order, so each MFMA operand is two conflict-free 1 KB reads. The
//     tokens' E8M0 dwords (four groups per stage, hi and lo) go to LDS too.
//   - w13 epilogue: h = bf16(SwiGLU), then split into hi/lo fp8 per 32 h
//     columns (the 32 rows of a row block: lanes c and c+32 hold 16 each; one
//     lane swap gives the block maximum) and stored by sorted position with
//     its E8M0 bytes: the w2 pass reads them as its activations.
//   - w2 epilogue: y times the slot's routing weight, bf16, by slot.
//   - Persistent and XCD-aware: one block per CU walks the logical tiles, N
//     tile outermost, so consecutive tiles are the token tiles of one expert
//     and N tile, which share its weights; XCD x owns a contiguous run (its
//     L2 serves those weights to all of them), handed out by its counter in
//     the workspace. The activations, re-read once per N tile, are small
//     enough to stay in the last-level cache.
#include "device.h"
#include "internal.h"

namespace moe {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kXBM = 128;                // token positions per tile
constexpr int kXBN = 256;                // weight rows per tile
constexpr int kXThreads = 256;           // 4 waves, one per SIMD (each may use 512 registers)
constexpr int kXBK = 128;                // K per stage
constexpr int kXTB = kXBM / 32;          // 32-token blocks per tile
constexpr int kXStage = kXBM * kXBK * 2; // LDS bytes per stage (hi + lo)

// One 32 x 32 x 64 step: a = the lane's 16 code bytes, b = its 32 fp8 bytes,
// sa / sb = E8M0 bytes (low byte of the register).
__device__ __forceinline__ f32x16_t mfma_mx(const u32x4_t& a, const i32x8_t& b, const f32x16_t& c, uint32_t sa,
                                            uint32_t sb) {
  const i32x8_t a8 = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b, c, 4, 0, 0, (int)sa, 0, (int)sb);
}

// The E8M0 bytes of a 32-block whose largest magnitude is m (a finite bf16
// value): sh puts m in [128, 256) (never above E4M3's 448), sl = sh - 4
// leaves room for the remainder (at most 8 units of hi); both at least 0.
// inv_h = 2^(127 - sh), f_l = 2^(sh - sl) (scales from hi units to lo units).
struct MxSplit {
  uint32_t sh, sl;
  float inv_h, f_l;
};
__device__ __forceinline__ MxSplit mx_split_scales(float m) {
  const int E = (int)((__float_as_uint(m) >> 23) & 0xff);  // biased exponent of m (0 for zero)
  int sh = E == 0 ? 127 : E - 7;
  sh = sh < 0 ? 0 : sh;
  const int sl = sh >= 4 ? sh - 4 : 0;
  MxSplit s;
  s.sh = (uint32_t)sh;
  s.sl = (uint32_t)sl;
  s.inv_h = __uint_as_float((uint32_t)(254 - sh) << 23);
  s.f_l = __uint_as_float((uint32_t)(127 + sh - sl) << 23);
  return s;
}

// Four values (exact bf16 values as float) -> their hi and lo fp8 bytes,
// packed in the byte order of the values.
__device__ __forceinline__ void mx_split4(float v0, float v1, float v2, float v3, const MxSplit& s, uint32_t& hi,
                                          uint32_t& lo) {
  const float a0 = v0 * s.inv_h, a1 = v1 * s.inv_h, a2 = v2 * s.inv_h, a3 = v3 * s.inv_h;
  int h = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false);
  h = __builtin_amdgcn_cvt_pk_fp8_f32(a2, a3, h, true);
  const auto d01 = __builtin_amdgcn_cvt_pk_f32_fp8(h, false);
  const auto d23 = __builtin_amdgcn_cvt_pk_f32_fp8(h, true);
  int l = __builtin_amdgcn_cvt_pk_fp8_f32((a0 - d01[0]) * s.f_l, (a1 - d01[1]) * s.f_l, 0, false);
  l = __builtin_amdgcn_cvt_pk_fp8_f32((a2 - d23[0]) * s.f_l, (a3 - d23[1]) * s.f_l, l, true);
  hi = (uint32_t)h;
  lo = (uint32_t)l;
}

// x [R][K] bf16 -> hi, lo [R][K] fp8 and their E8M0 bytes sh, sl [R][K/32];
// one thread per 32-block.
__global__ __launch_bounds__(256) void k_quant_rows(const uint16_t* x, long long nblocks, uint8_t* hi, uint8_t* lo,
                                                    uint8_t* sh, uint8_t* sl) {
  const long long b = (long long)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblocks) return;
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(x + b * 32);
  u32x4_t v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = src[i];
  float f[32];
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f[8 * i + 2 * j] = bf16_to_f32(v[i][j] & 0xffffu);
      f[8 * i + 2 * j + 1] = bf16_to_f32(v[i][j] >> 16);
      m = fmaxf(m, fmaxf(fabsf(f[8 * i + 2 * j]), fabsf(f[8 * i + 2 * j + 1])));
    }
  const MxSplit s = mx_split_scales(m);
  u32x4_t oh[2], ol[2];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t h, l;
    mx_split4(f[4 * i], f[4 * i + 1], f[4 * i + 2], f[4 * i + 3], s, h, l);
    oh[i >> 2][i & 3] = h;
    ol[i >> 2][i & 3] = l;
  }
  u32x4_t* dh = reinterpret_cast<u32x4_t*>(hi + b * 32);
  u32x4_t* dl = reinterpret_cast<u32x4_t*>(lo + b * 32);
  dh[0] = oh[0];
  dh[1] = oh[1];
  dl[0] = ol[0];
  dl[1] = ol[1];
  sh[b] = (uint8_t)s.sh;
  sl[b] = (uint8_t)s.sl;
}

// A wave's weights of one stage: two row blocks x two 64-K steps of 16 code
// bytes, and the row's E8M0 dword of the stage (groups 4 st .. 4 st + 3).
struct MxW {
  u32x4_t q[2][2];
  uint32_t s[2];
};

__device__ __forceinline__ void mx_load_w(const uint8_t* const (&wrow)[2], const uint8_t* const (&srow)[2], int st,
                                          MxW& w) {
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
    for (int c = 0; c < 2; ++c) w.q[rb][c] = *reinterpret_cast<const u32x4_t*>(wrow[rb] + st * 64 + c * 32);
    w.s[rb] = *reinterpret_cast<const uint32_t*>(srow[rb] + st * 4);
  }
}

// A thread's share of one stage of the tile's activations. The stage's LDS
// image is 32 regions of 1 KB, region ((tb * 2 + c) * 2 + part) * 2 + jj
// holding, in lane order, lane l's 16 bytes jj of the B operand (token
// 32 tb + l % 32, 64-K step c, hi or lo). Wave w fills regions 8w .. 8w+7
// (token block w; both steps, hi and lo, both halves), so every LDS store of
// a wave is one contiguous 1 KB. Every thread also carries one E8M0 dword of
// a token (the stage's four groups; hi for ids 0..127, lo for 128..255).
struct MxA {
  u32x4_t v[8];  // [c][part][jj]
  uint32_t s;
  __device__ __forceinline__ void load(const uint8_t* srch, const uint8_t* srcl, const uint8_t* srcs, int st) {
    const int o = st * kXBK;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      v[c * 4 + 0] = *reinterpret_cast<const u32x4_t*>(srch + o + 64 * c);
      v[c * 4 + 1] = *reinterpret_cast<const u32x4_t*>(srch + o + 64 * c + 32);
      v[c * 4 + 2] = *reinterpret_cast<const u32x4_t*>(srcl + o + 64 * c);
      v[c * 4 + 3] = *reinterpret_cast<const u32x4_t*>(srcl + o + 64 * c + 32);
    }
    s = *reinterpret_cast<const uint32_t*>(srcs + st * 4);
    asm volatile("" ::: "memory");
  }
  __device__ __forceinline__ void store(unsigned char* buf, uint32_t* sbuf, int off, int soff) const {
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4_t*>(buf + off + i * 1024) = v[i];
    sbuf[soff] = s;
  }
};

// One stage of MFMAs. The B operands of the four token blocks (a 64-K step,
// hi or lo) come from LDS one group ahead: the next group is requested
// before the MFMAs of the current one. The MFMAs run hi for every (token
// block, row block), then lo, so an accumulator's next MFMA is eight
// instructions behind its last one.
__device__ __forceinline__ void mx_compute(f32x16_t (&acc)[2][kXTB], const MxW& w, const unsigned char* buf,
                                           const uint32_t* sbuf, int lane) {
  const int g = lane >> 5, tok = lane & 31;
  auto rd = [&](int c, int tb, int part) -> i32x8_t {
    const unsigned char* base = buf + ((((tb * 2 + c) * 2 + part) * 2) * 1024) + lane * 16;
    const u32x4_t a = *reinterpret_cast<const u32x4_t*>(base);
    const u32x4_t b = *reinterpret_cast<const u32x4_t*>(base + 1024);
    return (i32x8_t){(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
  };
  uint32_t bs[2][kXTB];  // the token's E8M0 dwords (hi, lo) of each token block
#pragma unroll
  for (int tb = 0; tb < kXTB; ++tb) {
    bs[0][tb] = sbuf[tb * 32 + tok];
    bs[1][tb] = sbuf[kXBM + tb * 32 + tok];
  }
  i32x8_t b[2][kXTB];  // groups alternate between the two sets
#pragma unroll
  for (int tb = 0; tb < kXTB; ++tb) b[0][tb] = rd(0, tb, 0);
#pragma unroll
  for (int grp = 0; grp < 4; ++grp) {  // (step c, part) = (grp / 2, grp % 2)
    const int c = grp >> 1, part = grp & 1;
    if (grp + 1 < 4) {
#pragma unroll
      for (int tb = 0; tb < kXTB; ++tb) b[(grp + 1) & 1][tb] = rd((grp + 1) >> 1, tb, (grp + 1) & 1);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int tb = 0; tb < kXTB; ++tb) {
      const uint32_t sb = __builtin_amdgcn_ubfe(bs[part][tb], 8 * (2 * c + g), 8);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
        acc[rb][tb] = mfma_mx(w.q[rb][c], b[grp & 1][tb], acc[rb][tb],
                              __builtin_amdgcn_ubfe(w.s[rb], 8 * (2 * c + g), 8), sb);
    }
  }
}

template <int MODE>
__global__ __launch_bounds__(kXThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_gemm_mx(MxGemmArgs p) {
  __shared__ __align__(16) unsigned char lds_b[2][kXStage];
  __shared__ __align__(16) uint32_t lds_s[2][2 * kXBM];  // [buffer][hi tokens 0..127, lo tokens 0..127]
  __shared__ int grabbed;

  const int ntt = *p.n_tiles;  // live token tiles
  const int nblk = ntt * p.n_ntiles;
  if (nblk <= 0) return;  // no tiles: the whole grid leaves, the queue untouched
  const int G = gridDim.x;
  const int xcd = blockIdx.x & 7, inx = blockIdx.x >> 3;
  const int nx = (G - xcd + 7) >> 3;  // blocks on this XCD
  const int per = nblk >> 3, extra = nblk & 7;
  const int lo = xcd * per + min(xcd, extra), hi = lo + per + (xcd < extra ? 1 : 0);
  int* const q = p.queue;  // [8] tiles handed out per XCD, [8] blocks done
  const int K = p.K, nst = K / kXBK, last = nst - 1;

  // logical tile lg -> (token tile, N tile): order 0 keeps the N tiles of one token tile adjacent
  // (its gathered activations are reused from the XCD's L2), order 1 the token tiles of one N tile
  // (the expert's weights of that N tile are shared by its token tiles running at once)
  auto tt_of = [&](int lg) { return p.order ? lg % ntt : lg / p.n_ntiles; };
  auto nt_of = [&](int lg) { return p.order ? lg / ntt : lg % p.n_ntiles; };
  auto record = [&](int lg) -> int4 {
    int4 t = p.tile_info[tt_of(min(lg, nblk - 1))];
    t.x = __builtin_amdgcn_readfirstlane(t.x);
    t.y = __builtin_amdgcn_readfirstlane(t.y);
    t.z = __builtin_amdgcn_readfirstlane(t.z);
    return t;
  };

  int cur = lo + inx, nxt = lo + nx + inx;
  int4 rec = record(cur);
  while (cur < hi) {
    int tid;  // an opaque copy: per-lane values are recomputed per tile instead of living across it
    asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"((int)threadIdx.x));
    const int wave = tid >> 6, lane = tid & 63;
    const int g = lane >> 5, c32 = lane & 31;
    int grab = 0;
    if (tid == 0) grab = atomicAdd(q + xcd, 1);
    const int4 rec_n = record(nxt);
    const int e = rec.x, pos0 = rec.y, ncols = rec.z;
    const int nt = nt_of(cur);

    // the wave's weight rows: w13 gate rows 128 nt + 32 w + c and the matching up rows;
    // w2 rows 256 nt + 64 w + 32 rb + c
    const uint8_t* qe = p.wq + (long long)e * p.q_expert_stride;
    const uint8_t* se = p.wsc + (long long)e * p.s_expert_stride;
    const uint8_t* wrow[2];
    const uint8_t* srow[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int row = MODE == kGemmW13 ? rb * p.half + nt * (kXBN / 2) + wave * 32 + c32
                                       : nt * kXBN + wave * 64 + rb * 32 + c32;
      wrow[rb] = qe + (size_t)row * (K / 2) + 16 * g;
      srow[rb] = se + (size_t)row * (K / 32);
    }
    // this thread's activation pieces: token 32 w + c32 of the tile, bytes 64 c + 16 g (jj = 0) and
    // 64 c + 32 + 16 g (jj = 1) of the stage for both 64-K steps c, hi and lo
    const int atok = 32 * wave + c32;
    const int arow = p.act_row ? p.act_row[pos0 + min(atok, ncols - 1)] : pos0 + min(atok, ncols - 1);
    const uint8_t* srch = p.a_hi + (size_t)arow * K + 16 * g;
    const uint8_t* srcl = p.a_lo + (size_t)arow * K + 16 * g;
    const int off = (8 * wave) * 1024 + lane * 16;  // regions 8w .. 8w + 7
    // E8M0 dwords: thread ids 0..127 the hi bytes of token id, 128..255 the lo bytes of token id - 128
    const int sj = min(tid & (kXBM - 1), ncols - 1);
    const int srow_act = p.act_row ? p.act_row[pos0 + sj] : pos0 + sj;
    const uint8_t* srcs = ((tid & kXBM) ? p.as_lo : p.as_hi) + (size_t)srow_act * (K / 32);
    const int soff = tid;

    // w2: the slot and routing weight of the lane's tokens, in flight during the K loop
    int slot[kXTB];
    float wsl[kXTB];
#pragma unroll
    for (int t2 = 0; t2 < kXTB; ++t2) {
      slot[t2] = 0;
      wsl[t2] = 0.0f;
    }
    if (MODE == kGemmW2) {
#pragma unroll
      for (int t2 = 0; t2 < kXTB; ++t2) slot[t2] = p.sorted_slots[pos0 + min(t2 * 32 + c32, ncols - 1)];
#pragma unroll
      for (int t2 = 0; t2 < kXTB; ++t2) wsl[t2] = p.slot_w[slot[t2]];
    }

    f32x16_t acc[2][kXTB];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int t2 = 0; t2 < kXTB; ++t2)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[rb][t2][i] = 0.0f;

    // pipeline: stage st computes from LDS buffer st % 2 and weight set st % 2. Activations go
    // global -> registers -> LDS: set a1 / a0 is stored as stage st + 1 at the top of stage st and
    // then requested again for stage st + 3, so each has two stages to arrive; weights are
    // requested two stages ahead, after the stage that used their registers
    MxW w0, w1;
    MxA a0, a1;
    mx_load_w(wrow, srow, 0, w0);
    a0.load(srch, srcl, srcs, 0);
    mx_load_w(wrow, srow, min(1, last), w1);
    a1.load(srch, srcl, srcs, min(1, last));
    a0.store(lds_b[0], lds_s[0], off, soff);
    a0.load(srch, srcl, srcs, min(2, last));
    int st = 0;
    for (; st + 1 < nst; st += 2) {
      __syncthreads();  // buffer 0 holds stage st; buffer 1 is free
      a1.store(lds_b[1], lds_s[1], off, soff);  // stage st + 1
      a1.load(srch, srcl, srcs, min(st + 3, last));
      mx_compute(acc, w0, lds_b[0], lds_s[0], lane);
      mx_load_w(wrow, srow, min(st + 2, last), w0);
      __syncthreads();  // buffer 1 holds stage st + 1; buffer 0 is free
      a0.store(lds_b[0], lds_s[0], off, soff);  // stage st + 2
      a0.load(srch, srcl, srcs, min(st + 4, last));
      mx_compute(acc, w1, lds_b[1], lds_s[1], lane);
      mx_load_w(wrow, srow, min(st + 3, last), w1);
    }
    if (nst & 1) {  // the last stage (buffer 0, w0)
      __syncthreads();
      mx_compute(acc, w0, lds_b[0], lds_s[0], lane);
    }

    // epilogue: lane holds acc[rb][tb][i] = D[row 8 (i/4) + 4 g + i%4 of block rb][token 32 tb + c32]
#pragma unroll
    for (int t2 = 0; t2 < kXTB; ++t2) {
      const int tok = t2 * 32 + c32;
      const bool live = tok < ncols;
      const int pos = pos0 + tok;
      if (MODE == kGemmW13) {
        float hv[16];
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          hv[i] = bf16_to_f32(f32_to_bf16(swiglu_clamped(acc[0][t2][i], acc[1][t2][i], p.limit)));
          m = fmaxf(m, fabsf(hv[i]));
        }
        // the block's other 16 values are in lane c32 + 32 (or c32): exchange the maxima
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
        m = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        const MxSplit s = mx_split_scales(m);
        const int col0 = nt * (kXBN / 2) + wave * 32;  // the block's first h column
        if (live) {
          uint8_t* dh = p.h_hi + (size_t)pos * p.I + col0 + 4 * g;
          uint8_t* dl = p.h_lo + (size_t)pos * p.I + col0 + 4 * g;
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            uint32_t h, l;
            mx_split4(hv[4 * qq], hv[4 * qq + 1], hv[4 * qq + 2], hv[4 * qq + 3], s, h, l);
            *reinterpret_cast<uint32_t*>(dh + 8 * qq) = h;
            *reinterpret_cast<uint32_t*>(dl + 8 * qq) = l;
          }
          if (g == 0) {
            p.hs_hi[(size_t)pos * (p.I / 32) + col0 / 32] = (uint8_t)s.sh;
            p.hs_lo[(size_t)pos * (p.I / 32) + col0 / 32] = (uint8_t)s.sl;
          }
        }
      } else if (live) {
        const float wv = wsl[t2];
        uint16_t* dst = p.yout + (size_t)slot[t2] * p.yout_ld;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const int n0 = nt * kXBN + wave * 64 + rb * 32 + 4 * g;
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            uint2 pk;
            pk.x = (uint32_t)f32_to_bf16(acc[rb][t2][4 * qq] * wv) |
                   ((uint32_t)f32_to_bf16(acc[rb][t2][4 * qq + 1] * wv) << 16);
            pk.y = (uint32_t)f32_to_bf16(acc[rb][t2][4 * qq + 2] * wv) |
                   ((uint32_t)f32_to_bf16(acc[rb][t2][4 * qq + 3] * wv) << 16);
            *reinterpret_cast<uint2*>(dst + n0 + 8 * qq) = pk;
          }
        }
      }
    }
    if (tid == 0) grabbed = lo + 2 * nx + grab;
    __syncthreads();  // every wave is done with this tile's LDS; the grab is visible
    cur = nxt;
    nxt = __builtin_amdgcn_readfirstlane(grabbed);
    rec = rec_n;
  }
  // the last block out sets the counters back to zero for the next launch
  if (threadIdx.x == 0 && atomicAdd(q + 8, 1) == G - 1) {
#pragma unroll
    for (int i = 0; i < 9; ++i) q[i] = 0;
  }
}

bool gemm_mx_supported(int H, int I) { return H % kXBN == 0 && I % (kXBN / 2) == 0 && H % kXBK == 0 && I % kXBK == 0; }

hipError_t launch_quant_rows(const uint16_t* x, long long rows, int K, uint8_t* hi, uint8_t* lo, uint8_t* sh,
                             uint8_t* sl, hipStream_t st) {
  if (K % 32) return hipErrorInvalidValue;
  const long long nb = rows * (K / 32);
  if (nb <= 0) return hipSuccess;
  k_quant_rows<<<(unsigned)((nb + 255) / 256), 256, 0, st>>>(x, nb, hi, lo, sh, sl);
  return hipGetLastError();
}

// Blocks of k_gemm_mx<MODE> the current device holds at once (cached per device).
template <int MODE>
static int gemm_mx_resident() {
  constexpr int kDev = 16;
  static int cache[kDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDev) return 0;
  if (cache[dev] > 0) return cache[dev];
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(&k_gemm_mx<MODE>),
                                                   kXThreads, 0) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  cache[dev] = per_cu * cus;
  return cache[dev];
}

hipError_t launch_gemm_mx(const MxGemmArgs& p, int tiles, hipStream_t st) {
  if (tiles <= 0) return hipSuccess;
  if (!p.queue || p.K % kXBK || (p.mode != kGemmW13 && p.mode != kGemmW2)) return hipErrorInvalidValue;
  if (p.n_ntiles * (p.mode == kGemmW13 ? kXBN / 2 : kXBN) != p.N) return hipErrorInvalidValue;
  if (p.mode == kGemmW13 && (p.half != p.N || p.I != p.N)) return hipErrorInvalidValue;
  const long long nblk = (long long)tiles * p.n_ntiles;
  const int resident = p.mode == kGemmW13 ? gemm_mx_resident<kGemmW13>() : gemm_mx_resident<kGemmW2>();
  if (resident <= 0) return hipErrorInvalidValue;
  const long long grid = nblk < resident ? nblk : resident;
  if (p.mode == kGemmW13) k_gemm_mx<kGemmW13><<<(unsigned)grid, kXThreads, 0, st>>>(p);
  else k_gemm_mx<kGemmW2><<<(unsigned)grid, kXThreads, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace moe
