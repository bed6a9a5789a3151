/*
 * CPU ORACLE for the DeepSeek-V4-Flash MoE feed-forward layer.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. The GPU library never
 * calls it and shares no code, header, table or constant generator with it.
 *
 * It is the plain definition of the layer, written out: scalar loops, sums
 * in fp64 in ascending index order, weights decoded exactly from their codes.
 * Where floating point decides an integer (which 6 experts a token goes to),
 * the decision is taken on fp32 values, the precision the GPU kernels use.
 *
 * What it follows:
 *  - Layer constants (256 routed experts, 6 per token, intermediate 2048,
 *    one shared expert, routed scale 1.5, sqrt(softplus(logit)) scores
 *    that are normalised, the first three layers routed by a token-id
 *    table): page "DeepSeek-V4-Flash export design", section "Source
 *    configuration"; page "deepseek-v4-mxfp4-int8 config.json", keys
 *    n_routed_experts, num_experts_per_tok, moe_intermediate_size,
 *    n_shared_experts, norm_topk_prob, routed_scaling_factor,
 *    scoring_func, topk_method, swiglu_limit, num_hash_layers.
 *  - Selection by score + e_score_correction_bias, weights gathered from
 *    the unbiased scores: page "DeepSeek-V4-Flash-0731", section "Checked
 *    in its code", rows "Mixture of experts" and "Auxiliary-loss-free load
 *    balancing (selection bias)".
 *  - routed + shared_experts(x), shared expert added unscaled: same
 *    section, row "Shared expert".
 *  - Gate clamped from above at the limit, up clamped to [-limit, limit],
 *    down(silu(gate) * up): same section, row "SwiGLU feed-forward".
 *  - Routed expert weights: 4-bit float, group 32 along the input dim, one
 *    E8M0 exponent per group; activations 16-bit float ("w4a16"). Shared
 *    expert: int8, symmetric, one scale per output channel ("w8a16"): page
 *    "deepseek-v4-mxfp4-int8 config.json", quantization_config,
 *    config_groups experts_w4a16 and linears_w8a16. The packed FP4/E8M0
 *    tensors decode to a finite floating-point value: page
 *    "Tidalluna/DeepSeek-V4-Flash-0731-Tina-CQ4KM", section "Quantization
 *    Scope". The E2M1 bit layout and the E8M0 bias are those of the OCP
 *    Microscaling Formats (MX) v1.0 specification.
 *  - The router ("*.gate.*") is not quantised: config.json, "ignore" list.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 * nibble 2i is the low half of byte i; rows [0, I) of w13 are the gate and
 * rows [I, 2I) the up projection; ties in the top-k go to the lower expert
 * id; no epsilon in the renormalisation; the 1.5 scale applies to the routed
 * weights only; the intermediate activation h entering w2 is bf16 (the a16
 * format of the expert linears) unless round_h is 0; the hash layers weight
 * the 6 table experts by their renormalised sqrt-softplus scores, no bias.
 *
 * Down experts in 3-bit blocks (or_forward_w2q3): page
 * "Geometric-AI/DeepSeek-V4-Flash-0731-ROCmFP3-MIX", introduction and section
 * "What 'adaptive' means here", gives 14 bytes per 32 weights for both its
 * formats, one code book for every block (uniform) or a small table per
 * expert (adaptive), and nothing finer. Readings: 12 bytes of 3-bit codes and
 * a 2-byte IEEE binary16 scale d per 32 consecutive weights along the input
 * dimension; weight = d * level[code]; the uniform code book is level[c] =
 * c - 4 (a scale-only block, like the "_0" formats the name recalls); an
 * adaptive table is 8 fp32 levels per expert; the code bits sit where
 * or_q3_code reads them (a layout of this library's own).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_OK 0
#define OR_EINVAL (-1)

/* Threads the oracle's parallel loops use (OpenMP). */
int or_num_threads(void) { return omp_get_max_threads(); }

/* ---- exact decoders ------------------------------------------------------ */

/* E2M1: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa.
 * Exponent 0 is subnormal: 0.5 * m. Otherwise 2^(e-1) * (1 + m/2). */
double or_e2m1(int code) {
  int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  double mag = (e == 0) ? 0.5 * m : (1.0 + 0.5 * m) * (double)(1 << (e - 1));
  return s ? -mag : mag;
}

/* E8M0: 2^(b - 127); the byte 0xFF is NaN. */
double or_e8m0(int b) {
  if (b == 255) return NAN;
  return ldexp(1.0, b - 127);
}

/* Weight (n, k) of an MXFP4 matrix with K inputs: codes [N][K/2], scales [N][K/32]. */
double or_mxfp4_weight(const uint8_t* codes, const uint8_t* scales, int64_t K, int64_t n, int64_t k) {
  uint8_t byte = codes[n * (K / 2) + k / 2];
  int c = (k & 1) ? (byte >> 4) : (byte & 15);
  return or_e2m1(c) * or_e8m0(scales[n * (K / 32) + k / 32]);
}

double or_bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Round to the nearest bf16 value (8 significant bits), ties to even. */
double or_round_bf16(double v) {
  if (v == 0.0 || !isfinite(v)) return v;
  int e;
  frexp(v, &e);             /* v = m * 2^e, |m| in [0.5, 1) */
  if (e < -125) e = -125;   /* below 2^-126 the bf16 spacing stays 2^-133 */
  double q = nearbyint(ldexp(v, 8 - e));
  return ldexp(q, e - 8);
}

/* Bytes of one block of `group` weights of `bits` bits plus a scale of
 * `scale_bits` bits. */
int64_t or_block_bytes(int bits, int group, int scale_bits) {
  return ((int64_t)bits * group + scale_bits) / 8;
}

/* IEEE 754 binary16: bit 15 sign, bits 14..10 exponent (bias 15), bits 9..0
 * fraction; exponent 0 is subnormal (fraction * 2^-24), 31 is Inf/NaN. */
double or_fp16_value(uint16_t h) {
  int s = (h >> 15) & 1, e = (h >> 10) & 31, f = h & 1023;
  double mag;
  if (e == 31) mag = f ? NAN : INFINITY;
  else if (e == 0) mag = ldexp((double)f, -24);
  else mag = ldexp(1.0 + f / 1024.0, e - 15);
  return s ? -mag : mag;
}

/* The 3-bit code of weight i (0..31) of a 12-byte block b. Weights
 * 0..23 have all three bits in one byte: weight i in byte 4*(i/8) + i%4,
 * bits 0..2 if i%8 < 4, else bits 3..5. Weights 24..31 use the two top bits
 * of three bytes: weight 24 + j has bits 0..1 in bits 6..7 of byte j and
 * bit 2 in bit 6 of byte 8 + j; weight 28 + j has bits 0..1 in bits 6..7 of
 * byte 4 + j and bit 2 in bit 7 of byte 8 + j. */
int or_q3_code(const uint8_t* b, int i) {
  if (i < 24) {
    int byte = 4 * (i / 8) + i % 4;
    int shift = (i % 8 < 4) ? 0 : 3;
    return (b[byte] >> shift) & 7;
  }
  int j = (i - 24) % 4;
  if (i < 28) return ((b[j] >> 6) & 3) | (((b[8 + j] >> 6) & 1) << 2);
  return ((b[4 + j] >> 6) & 3) | (((b[8 + j] >> 7) & 1) << 2);
}

/* Level of code c: the expert's table, or c - 4 for the uniform code book. */
double or_q3_level(const float* levels, int c) { return levels ? (double)levels[c] : (double)(c - 4); }

/* Weight (n, k) of a 3-bit matrix with K inputs: codes [N][K/32][12],
 * scales [N][K/32] binary16 bits, levels [8] or NULL (uniform). */
double or_q3_weight(const uint8_t* codes, const uint16_t* scales, const float* levels, int64_t K, int64_t n,
                    int64_t k) {
  const uint8_t* blk = codes + (n * (K / 32) + k / 32) * 12;
  return or_fp16_value(scales[n * (K / 32) + k / 32]) * or_q3_level(levels, or_q3_code(blk, (int)(k % 32)));
}

/* ---- elementwise pieces -------------------------------------------------- */

double or_softplus(double z) { return (z > 0 ? z : 0.0) + log1p(exp(-fabs(z))); }

double or_score(double logit) { return sqrt(or_softplus(logit)); }

double or_silu(double z) { return z / (1.0 + exp(-z)); }

double or_swiglu(double g, double u, double limit) {
  double gc = g < limit ? g : limit;
  double uc = u < -limit ? -limit : (u > limit ? limit : u);
  return or_silu(gc) * uc;
}

/* ---- routing ------------------------------------------------------------- */

/* Top-k of b[0..E) by value descending, ties to the lower index. Writes the
 * chosen indices in that order; returns the best unchosen index (-1 if none). */
static int topk_desc(const float* b, int E, int k, int32_t* out) {
  unsigned char taken[4096];
  memset(taken, 0, (size_t)E);
  for (int j = 0; j < k; ++j) {
    int best = -1;
    for (int e = 0; e < E; ++e) {
      if (taken[e]) continue;
      if (best < 0 || b[e] > b[best]) best = e; /* strict: equal keeps the lower id */
    }
    out[j] = best;
    taken[best] = 1;
  }
  int nxt = -1;
  for (int e = 0; e < E; ++e)
    if (!taken[e] && (nxt < 0 || b[e] > b[nxt])) nxt = e;
  return nxt;
}

/* Router logit of expert e for one token: sum_h x_h * Wg[e][h], fp64. */
static double logit_of(const uint16_t* xt, const float* gate_w, int H, int e) {
  double acc = 0.0;
  const float* we = gate_w + (int64_t)e * H;
  for (int h = 0; h < H; ++h) acc += or_bf16_value(xt[h]) * (double)we[h];
  return acc;
}

/* Learned router for one token. Outputs ids/w in slot order, the fp32 gap
 * between the k-th chosen and the best unchosen biased score, and that
 * unchosen expert. If force_ids is given, those experts are used instead of
 * the top-k and only the weights are computed. */
static void route_token(const uint16_t* xt, int H, int E, int k, const float* gate_w,
                        const float* bias, const float* offset, double scale,
                        const int32_t* force_ids, int32_t* ids, double* w, double* gap,
                        int32_t* next) {
  double s[4096];
  float b[4096];
  for (int e = 0; e < E; ++e) {
    double l = logit_of(xt, gate_w, H, e);
    if (offset) l += (double)offset[e];
    s[e] = or_score(l);
    b[e] = (float)(s[e] + (double)bias[e]); /* the selection is decided in fp32 */
  }
  int nxt = -1;
  if (force_ids) {
    for (int j = 0; j < k; ++j) ids[j] = force_ids[j];
  } else {
    nxt = topk_desc(b, E, k, ids);
  }
  if (gap) *gap = (nxt >= 0) ? (double)b[ids[k - 1]] - (double)b[nxt] : INFINITY;
  if (next) *next = nxt;
  double sum = 0.0;
  for (int j = 0; j < k; ++j) sum += s[ids[j]];
  for (int j = 0; j < k; ++j) w[j] = scale * s[ids[j]] / sum;
}

/* Hash router for one token: the table row gives the experts, in table
 * order; weights are their renormalised scores times `scale`. */
static void hash_route_token(const uint16_t* xt, int H, int k, const float* gate_w,
                             const int32_t* row, double scale, int32_t* ids, double* w) {
  double s[64];
  double sum = 0.0;
  for (int j = 0; j < k; ++j) {
    ids[j] = row[j];
    s[j] = or_score(logit_of(xt, gate_w, H, row[j]));
    sum += s[j];
  }
  for (int j = 0; j < k; ++j) w[j] = scale * s[j] / sum;
}

int or_route(int T, int H, int E, int k, const uint16_t* x, const float* gate_w, const float* bias,
             const float* offset, double scale, int32_t* ids, double* w, double* gap, int32_t* next) {
  if (T < 0 || H <= 0 || E <= 0 || E > 4096 || k <= 0 || k > E || k > 64) return OR_EINVAL;
#pragma omp parallel for schedule(dynamic, 1)
  for (int t = 0; t < T; ++t)
    route_token(x + (int64_t)t * H, H, E, k, gate_w, bias, offset, scale, NULL, ids + (int64_t)t * k,
                w + (int64_t)t * k, gap ? gap + t : NULL, next ? next + t : NULL);
  return OR_OK;
}

int or_hash_route(int T, int H, int E, int k, const uint16_t* x, const int32_t* tids,
                  const int32_t* tid2eid, int V, const float* gate_w, double scale, int32_t* ids,
                  double* w) {
  if (T < 0 || H <= 0 || E <= 0 || k <= 0 || k > 64 || V <= 0) return OR_EINVAL;
  for (int t = 0; t < T; ++t)
    if (tids[t] < 0 || tids[t] >= V) return OR_EINVAL;
  for (int64_t i = 0; i < (int64_t)V * k; ++i)
    if (tid2eid[i] < 0 || tid2eid[i] >= E) return OR_EINVAL;
#pragma omp parallel for schedule(dynamic, 1)
  for (int t = 0; t < T; ++t)
    hash_route_token(x + (int64_t)t * H, H, k, gate_w, tid2eid + (int64_t)tids[t] * k, scale,
                     ids + (int64_t)t * k, w + (int64_t)t * k);
  return OR_OK;
}

/* ---- permutation --------------------------------------------------------- */

/* Counting sort of the T*k slots (slot = t*k + j) by expert, stable:
 * offsets[e] = first position of expert e (offsets[E] = T*k),
 * sorted_slots[p] = slot at position p, slot_pos[slot] = its position. */
int or_permute(int T, int k, int E, const int32_t* ids, int32_t* offsets, int32_t* sorted_slots,
               int32_t* slot_pos) {
  if (T < 0 || k <= 0 || E <= 0) return OR_EINVAL;
  int64_t n = (int64_t)T * k;
  for (int64_t i = 0; i < n; ++i)
    if (ids[i] < 0 || ids[i] >= E) return OR_EINVAL;
  int32_t* cursor = (int32_t*)calloc((size_t)E + 1, sizeof(int32_t));
  if (!cursor) return OR_EINVAL;
  for (int64_t i = 0; i < n; ++i) cursor[ids[i] + 1]++;
  for (int e = 0; e < E; ++e) cursor[e + 1] += cursor[e];
  memcpy(offsets, cursor, ((size_t)E + 1) * sizeof(int32_t));
  for (int64_t i = 0; i < n; ++i) {
    int32_t p = cursor[ids[i]]++;
    sorted_slots[p] = (int32_t)i;
    slot_pos[i] = p;
  }
  free(cursor);
  return OR_OK;
}

/* ---- expert feed-forward ------------------------------------------------- */

/* One routed expert on one token: y = W2 * swiglu(W13 * x), MXFP4 weights.
 * w13: codes [2I][H/2], scales [2I][H/32]; w2: codes [H][I/2], scales [H][I/32].
 * The inner loops run over whole 32-weight groups so that the group's
 * exponent is decoded once per group. */
static void routed_expert(int H, int I, const double* xd, const uint8_t* c13, const uint8_t* s13,
                          const uint8_t* c2, const uint8_t* s2, const uint16_t* s2q3, int w2q3,
                          const float* levels, double limit, int round_h, double* hbuf, double* y) {
#pragma omp parallel for schedule(static)
  for (int i = 0; i < I; ++i) {
    double g = 0.0, u = 0.0;
    for (int k0 = 0; k0 < H; k0 += 32) {
      double sg = or_e8m0(s13[(int64_t)i * (H / 32) + k0 / 32]);
      double su = or_e8m0(s13[(int64_t)(I + i) * (H / 32) + k0 / 32]);
      for (int k = k0; k < k0 + 32; ++k) {
        uint8_t bg = c13[(int64_t)i * (H / 2) + k / 2];
        uint8_t bu = c13[(int64_t)(I + i) * (H / 2) + k / 2];
        int cg = (k & 1) ? (bg >> 4) : (bg & 15);
        int cu = (k & 1) ? (bu >> 4) : (bu & 15);
        g += or_e2m1(cg) * sg * xd[k];
        u += or_e2m1(cu) * su * xd[k];
      }
    }
    double h = or_swiglu(g, u, limit);
    hbuf[i] = round_h ? or_round_bf16(h) : h;
  }
  if (w2q3) { /* down projection in 3-bit blocks: d * level[code] */
#pragma omp parallel for schedule(static)
    for (int n = 0; n < H; ++n) {
      double acc = 0.0;
      for (int i0 = 0; i0 < I; i0 += 32) {
        double d = or_fp16_value(s2q3[(int64_t)n * (I / 32) + i0 / 32]);
        const uint8_t* blk = c2 + ((int64_t)n * (I / 32) + i0 / 32) * 12;
        for (int i = i0; i < i0 + 32; ++i) acc += d * or_q3_level(levels, or_q3_code(blk, i - i0)) * hbuf[i];
      }
      y[n] = acc;
    }
    return;
  }
#pragma omp parallel for schedule(static)
  for (int n = 0; n < H; ++n) {
    double acc = 0.0;
    for (int i0 = 0; i0 < I; i0 += 32) {
      double sc = or_e8m0(s2[(int64_t)n * (I / 32) + i0 / 32]);
      for (int i = i0; i < i0 + 32; ++i) {
        uint8_t b = c2[(int64_t)n * (I / 2) + i / 2];
        int c = (i & 1) ? (b >> 4) : (b & 15);
        acc += or_e2m1(c) * sc * hbuf[i];
      }
    }
    y[n] = acc;
  }
}

/* The shared expert on one token, int8 weights with per-output-row scales:
 * g_i = s13[i] * sum_h q13[i][h] x_h (likewise u from row I+i),
 * z_n = s2[n] * sum_i q2[n][i] h_i. */
static void shared_expert(int H, int I, const double* xd, const int8_t* q13, const float* s13,
                          const int8_t* q2, const float* s2, double limit, int round_h,
                          double* hbuf, double* z) {
#pragma omp parallel for schedule(static)
  for (int i = 0; i < I; ++i) {
    double g = 0.0, u = 0.0;
    for (int h = 0; h < H; ++h) {
      g += (double)q13[(int64_t)i * H + h] * xd[h];
      u += (double)q13[(int64_t)(I + i) * H + h] * xd[h];
    }
    g *= (double)s13[i];
    u *= (double)s13[I + i];
    double hv = or_swiglu(g, u, limit);
    hbuf[i] = round_h ? or_round_bf16(hv) : hv;
  }
#pragma omp parallel for schedule(static)
  for (int n = 0; n < H; ++n) {
    double acc = 0.0;
    for (int i = 0; i < I; ++i) acc += (double)q2[(int64_t)n * I + i] * hbuf[i];
    z[n] = (double)s2[n] * acc;
  }
}

typedef struct {
  int H, E, k, I;
  const uint8_t *w13c, *w13s, *w2c, *w2s;
  double limit;
  int round_h;
  /* w2 in 3-bit blocks: w2c [E][H][I/32][12], w2s16 [E][H][I/32], w2lv [E][8] or NULL */
  int w2q3;
  const uint16_t* w2s16;
  const float* w2lv;
} routed_args;

/* out[n] = sum_j w_j * y_j[n] for one token, slots in order j = 0..k-1. */
static int routed_token(const routed_args* a, const double* xd, const int32_t* ids, const double* w,
                        double* out) {
  int H = a->H, I = a->I;
  double* hbuf = (double*)malloc(sizeof(double) * (size_t)I);
  double* y = (double*)malloc(sizeof(double) * (size_t)H);
  if (!hbuf || !y) {
    free(hbuf);
    free(y);
    return OR_EINVAL;
  }
  for (int n = 0; n < H; ++n) out[n] = 0.0;
  for (int j = 0; j < a->k; ++j) {
    int e = ids[j];
    if (a->w2q3)
      routed_expert(H, I, xd, a->w13c + (int64_t)e * 2 * I * (H / 2), a->w13s + (int64_t)e * 2 * I * (H / 32),
                    a->w2c + (int64_t)e * H * (I / 32) * 12, NULL, a->w2s16 + (int64_t)e * H * (I / 32), 1,
                    a->w2lv ? a->w2lv + (int64_t)e * 8 : NULL, a->limit, a->round_h, hbuf, y);
    else
      routed_expert(H, I, xd, a->w13c + (int64_t)e * 2 * I * (H / 2), a->w13s + (int64_t)e * 2 * I * (H / 32),
                    a->w2c + (int64_t)e * H * (I / 2), a->w2s + (int64_t)e * H * (I / 32), NULL, 0, NULL,
                    a->limit, a->round_h, hbuf, y);
    for (int n = 0; n < H; ++n) out[n] += w[j] * y[n];
  }
  free(hbuf);
  free(y);
  return OR_OK;
}

static void bf16_row_to_double(const uint16_t* xt, int H, double* xd) {
  for (int h = 0; h < H; ++h) xd[h] = or_bf16_value(xt[h]);
}

/* Routed experts only: routed_out[t] = sum_j w[t][j] * expert_{ids[t][j]}(x_t). */
int or_expert_ffn(int T, int H, int E, int k, int I, const uint16_t* x, const int32_t* ids,
                  const double* w, const uint8_t* w13c, const uint8_t* w13s, const uint8_t* w2c,
                  const uint8_t* w2s, double limit, int round_h, double* routed_out) {
  if (T < 0 || H <= 0 || H % 32 || I <= 0 || I % 32 || E <= 0 || k <= 0) return OR_EINVAL;
  for (int64_t i = 0; i < (int64_t)T * k; ++i)
    if (ids[i] < 0 || ids[i] >= E) return OR_EINVAL;
  routed_args a = {H, E, k, I, w13c, w13s, w2c, w2s, limit, round_h, 0, NULL, NULL};
  double* xd = (double*)malloc(sizeof(double) * (size_t)H);
  if (!xd) return OR_EINVAL;
  int rc = OR_OK;
  for (int t = 0; t < T && rc == OR_OK; ++t) {
    bf16_row_to_double(x + (int64_t)t * H, H, xd);
    rc = routed_token(&a, xd, ids + (int64_t)t * k, w + (int64_t)t * k, routed_out + (int64_t)t * H);
  }
  free(xd);
  return rc;
}

/* Shared expert only: z[t] for every token. */
int or_shared_ffn(int T, int H, int I, const uint16_t* x, const int8_t* q13, const float* s13,
                  const int8_t* q2, const float* s2, double limit, int round_h, double* z) {
  if (T < 0 || H <= 0 || I <= 0) return OR_EINVAL;
  double* xd = (double*)malloc(sizeof(double) * (size_t)H);
  double* hbuf = (double*)malloc(sizeof(double) * (size_t)I);
  if (!xd || !hbuf) {
    free(xd);
    free(hbuf);
    return OR_EINVAL;
  }
  for (int t = 0; t < T; ++t) {
    bf16_row_to_double(x + (int64_t)t * H, H, xd);
    shared_expert(H, I, xd, q13, s13, q2, s2, limit, round_h, hbuf, z + (int64_t)t * H);
  }
  free(xd);
  free(hbuf);
  return OR_OK;
}

/* The whole layer for the tokens listed in rows[0..n_rows) (all T tokens if
 * rows is NULL; n_rows is then T):
 *   route (learned router, or the hash table when tids is given),
 *   out[r] = sum_j w_j * expert_{e_j}(x_t) + shared(x_t).
 * force_ids [n_rows][k], if given, replaces the learned top-k selection
 * (weights are still the renormalised scores of those experts).
 * Per-row outputs: ids [n_rows][k], w [n_rows][k], gap [n_rows] (learned
 * router only; +inf for hash), next [n_rows], out [n_rows][H]. */
static int forward_impl(const routed_args* ra, int T, const uint16_t* x, const float* gate_w,
                        const float* bias, const float* offset, const int32_t* tids, const int32_t* tid2eid,
                        int V, const int8_t* q13, const float* s13, const int8_t* q2, const float* s2,
                        double scale, const int32_t* rows, int n_rows, const int32_t* force_ids, int32_t* ids,
                        double* w, double* gap, int32_t* next, double* out) {
  const int H = ra->H, E = ra->E, k = ra->k, I = ra->I, round_h = ra->round_h;
  const double limit = ra->limit;
  if (T < 0 || H <= 0 || H % 32 || I <= 0 || I % 32 || E <= 0 || E > 4096 || k <= 0 || k > E ||
      k > 64)
    return OR_EINVAL;
  if (!rows) n_rows = T;
  for (int r = 0; r < n_rows; ++r) {
    int t = rows ? rows[r] : r;
    if (t < 0 || t >= T) return OR_EINVAL;
    if (tids && (tids[t] < 0 || tids[t] >= V)) return OR_EINVAL;
  }
  const routed_args a = *ra;
  double* xd = (double*)malloc(sizeof(double) * (size_t)H);
  double* z = (double*)malloc(sizeof(double) * (size_t)H);
  double* hbuf = (double*)malloc(sizeof(double) * (size_t)I);
  if (!xd || !z || !hbuf) {
    free(xd);
    free(z);
    free(hbuf);
    return OR_EINVAL;
  }
  int rc = OR_OK;
  for (int r = 0; r < n_rows && rc == OR_OK; ++r) {
    int t = rows ? rows[r] : r;
    const uint16_t* xt = x + (int64_t)t * H;
    int32_t* idr = ids + (int64_t)r * k;
    double* wr = w + (int64_t)r * k;
    if (tids) {
      hash_route_token(xt, H, k, gate_w, tid2eid + (int64_t)tids[t] * k, scale, idr, wr);
      if (gap) gap[r] = INFINITY;
      if (next) next[r] = -1;
    } else {
      route_token(xt, H, E, k, gate_w, bias, offset, scale, force_ids ? force_ids + (int64_t)r * k : NULL,
                  idr, wr, gap ? gap + r : NULL, next ? next + r : NULL);
    }
    for (int j = 0; j < k; ++j)
      if (idr[j] < 0 || idr[j] >= E) rc = OR_EINVAL;
    if (rc != OR_OK) break;
    bf16_row_to_double(xt, H, xd);
    rc = routed_token(&a, xd, idr, wr, out + (int64_t)r * H);
    if (rc != OR_OK) break;
    shared_expert(H, I, xd, q13, s13, q2, s2, limit, round_h, hbuf, z);
    for (int n = 0; n < H; ++n) out[(int64_t)r * H + n] += z[n];
  }
  free(xd);
  free(z);
  free(hbuf);
  return rc;
}

int or_forward(int T, int H, int E, int k, int I, const uint16_t* x, const float* gate_w,
               const float* bias, const float* offset, const int32_t* tids, const int32_t* tid2eid,
               int V, const uint8_t* w13c, const uint8_t* w13s, const uint8_t* w2c, const uint8_t* w2s,
               const int8_t* q13, const float* s13, const int8_t* q2, const float* s2, double scale,
               double limit, int round_h, const int32_t* rows, int n_rows, const int32_t* force_ids,
               int32_t* ids, double* w, double* gap, int32_t* next, double* out) {
  routed_args a = {H, E, k, I, w13c, w13s, w2c, w2s, limit, round_h, 0, NULL, NULL};
  return forward_impl(&a, T, x, gate_w, bias, offset, tids, tid2eid, V, q13, s13, q2, s2, scale, rows, n_rows,
                      force_ids, ids, w, gap, next, out);
}

/* or_forward with the routed experts' down projection (w2) in 3-bit blocks:
 * w2c [E][H][I/32][12] codes, w2s [E][H][I/32] binary16 scales, w2_levels
 * [E][8] fp32 (one table per expert) or NULL for the uniform code book. */
int or_forward_w2q3(int T, int H, int E, int k, int I, const uint16_t* x, const float* gate_w,
                    const float* bias, const float* offset, const int32_t* tids, const int32_t* tid2eid,
                    int V, const uint8_t* w13c, const uint8_t* w13s, const uint8_t* w2c, const uint16_t* w2s,
                    const float* w2_levels, const int8_t* q13, const float* s13, const int8_t* q2,
                    const float* s2, double scale, double limit, int round_h, const int32_t* rows, int n_rows,
                    const int32_t* force_ids, int32_t* ids, double* w, double* gap, int32_t* next,
                    double* out) {
  routed_args a = {H, E, k, I, w13c, w13s, w2c, NULL, limit, round_h, 1, w2s, w2_levels};
  return forward_impl(&a, T, x, gate_w, bias, offset, tids, tid2eid, V, q13, s13, q2, s2, scale, rows, n_rows,
                      force_ids, ids, w, gap, next, out);
}

/* ---- int8 per-channel linear layers ("w8a16") --------------------------- */

/* The attention projections of the model are int8, symmetric, one scale per
 * output channel, with 16-bit activations (page "deepseek-v4-mxfp4-int8
 * config.json", quantization_config, config group linears_w8a16: targets
 * fused_wqa_wkv, wq_b, wo_a, wo_b, indexer.wq_b, indexer.compressor.wkv).
 * groups > 1 is a block-diagonal (grouped) projection: group g maps input
 * features [g*K, (g+1)*K) to output features [g*N, (g+1)*N) with its own
 * weights.
 *   x [T][groups*K] bf16, q [groups][N][K] int8, s [groups][N] fp32
 *   out[t][g*N + n] = s[g][n] * sum_k q[g][n][k] * x[t][g*K + k]   (fp64) */
int or_linear_w8a16(int T, int K, int N, int groups, const uint16_t* x, const int8_t* q, const float* s,
                    double* out) {
  if (T < 0 || K <= 0 || N <= 0 || groups <= 0) return OR_EINVAL;
#pragma omp parallel for schedule(dynamic, 1)
  for (int t = 0; t < T; ++t) {
    for (int g = 0; g < groups; ++g) {
      const uint16_t* xt = x + ((int64_t)t * groups + g) * K;
      for (int n = 0; n < N; ++n) {
        const int8_t* row = q + ((int64_t)g * N + n) * K;
        double acc = 0.0;
        for (int k = 0; k < K; ++k) acc += (double)row[k] * or_bf16_value(xt[k]);
        out[((int64_t)t * groups + g) * N + n] = (double)s[(int64_t)g * N + n] * acc;
      }
    }
  }
  return OR_OK;
}
