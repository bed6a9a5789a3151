/*
 * Seeded synthetic inputs for the DeepSeek-V4-Flash MoE layer.
 *
 * This module only makes inputs: Gaussian tensors, their MXFP4 and int8
 * encodings, bf16 tokens, Zipf token ids and a token-id -> expert table.
 * It holds none of the layer's arithmetic (no decode, no routing, no
 * GEMM, no SwiGLU); the CPU oracle and the GPU library each implement those
 * on their own and both consume what this file writes.
 *
 * Random numbers: a counter-based generator. Every value is a pure
 * function of (seed, stream, sub, index), so any slice of any tensor can be
 * regenerated independently and in parallel. The mixing function is the
 * SplitMix64 output function (Steele, Lea & Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014); Gaussians come from the
 * Box-Muller transform (Box & Muller 1958) evaluated in fp32, one pair of
 * normals per two counters (normal 2p uses the cosine, 2p+1 the sine).
 *
 * Encodings written here (inputs to the layer, not part of it):
 *  - MXFP4: per 32 consecutive weights along K, an E8M0 exponent byte
 *    X + 127 with X = floor(log2(max|w|)) - 2, and E2M1 codes of w / 2^X
 *    rounded to nearest, ties to the even code, saturating at 6. Nibble
 *    2i is the low half of byte i. (OCP Microscaling Formats v1.0, E2M1
 *    and E8M0; group size 32 from the checkpoint's quantization_config.)
 *  - int8: symmetric, one fp32 scale per output row, s = max|w| / 127,
 *    q = round-half-even(w / s) in [-127, 127]; all-zero rows get s = 1.
 *  - bf16: round to nearest even from fp32.
 *  - 3-bit blocks (14 bytes per 32 weights; the byte count is the one page
 *    "Geometric-AI/DeepSeek-V4-Flash-0731-ROCmFP3-MIX" gives for its
 *    uniform and adaptive down-expert formats; the bit layout is this
 *    library's own): per 32 consecutive weights along K, an IEEE binary16
 *    scale d = max|w| / max|level| (rounded to nearest even) and 3-bit codes
 *    c = the level nearest w / d (ties to the lower code), packed in 12
 *    bytes b[0..11]: byte j + 4q (j < 4, q < 3) holds the code of weight
 *    8q + j in bits 0..2 and of weight 8q + 4 + j in bits 3..5; weight 24 + j
 *    takes bits 6..7 of byte j as its code bits 0..1 and bit 6 of byte 8 + j
 *    as its bit 2; weight 28 + j takes bits 6..7 of byte 4 + j and bit 7 of
 *    byte 8 + j. Levels: 8 per table; no table means c - 4 (the uniform
 *    code book).
 */
#define _GNU_SOURCE
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GOLDEN_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* Key of one (seed, stream, sub) sequence. */
static inline uint64_t seq_key(uint64_t seed, uint64_t stream, uint64_t sub) {
  uint64_t k = mix64(seed + GOLDEN_GAMMA);
  k = mix64(k + (stream + 1) * GOLDEN_GAMMA);
  k = mix64(k + (sub + 1) * GOLDEN_GAMMA);
  return k;
}

static inline uint64_t ctr_u64(uint64_t key, uint64_t i) {
  return mix64(key + (i + 1) * GOLDEN_GAMMA);
}

/* Uniform in the open interval (0, 1) with 53 bits (used for sampling ids). */
static inline double ctr_unif(uint64_t key, uint64_t i) {
  return ((double)(ctr_u64(key, i) >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

/* Uniform in (0, 1) with 24 bits, exactly representable in fp32. */
static inline float ctr_unif24(uint64_t key, uint64_t i) {
  return ((float)(ctr_u64(key, i) >> 40) + 0.5f) * (1.0f / 16777216.0f);
}

/* Standard normals 2p and 2p+1 of the sequence: Box-Muller on counters 2p
 * and 2p+1, evaluated in fp32. */
static inline void ctr_normal_pair(uint64_t key, uint64_t p, float* z0, float* z1) {
  float u1 = ctr_unif24(key, 2 * p);
  float u2 = ctr_unif24(key, 2 * p + 1);
  float r = sqrtf(-2.0f * logf(u1));
  float sn, cs;
  sincosf(6.28318530717958647692f * u2, &sn, &cs);
  *z0 = r * cs;
  *z1 = r * sn;
}

static inline float ctr_normal(uint64_t key, uint64_t i) {
  float z0, z1;
  ctr_normal_pair(key, i >> 1, &z0, &z1);
  return (i & 1) ? z1 : z0;
}

/* out[m] = fp32(mean + sigma * N_{first+m}), m in [0, n). */
static void fill_normal(uint64_t key, uint64_t first, int64_t n, double mean, double sigma,
                        float* out) {
  int64_t m = 0;
  uint64_t i = first;
  if (n > 0 && (i & 1)) {
    out[m++] = (float)(mean + sigma * (double)ctr_normal(key, i++));
  }
  for (; m + 1 < n; m += 2, i += 2) {
    float z0, z1;
    ctr_normal_pair(key, i >> 1, &z0, &z1);
    out[m] = (float)(mean + sigma * (double)z0);
    out[m + 1] = (float)(mean + sigma * (double)z1);
  }
  if (m < n) out[m] = (float)(mean + sigma * (double)ctr_normal(key, i));
}

uint64_t synth_u64(uint64_t seed, uint64_t stream, uint64_t sub, uint64_t i) {
  return ctr_u64(seq_key(seed, stream, sub), i);
}

double synth_normal_at(uint64_t seed, uint64_t stream, uint64_t sub, uint64_t i) {
  return (double)ctr_normal(seq_key(seed, stream, sub), i);
}

/* out[i] = (float)(sigma * N_i) + mean, i in [0, n). */
void synth_normal_f32(uint64_t seed, uint64_t stream, uint64_t sub, double mean,
                      double sigma, int64_t n, float* out) {
  uint64_t key = seq_key(seed, stream, sub);
  const int64_t chunk = 1 << 14;
#pragma omp parallel for schedule(static)
  for (int64_t c = 0; c < (n + chunk - 1) / chunk; ++c) {
    int64_t b = c * chunk, m = (n - b < chunk) ? n - b : chunk;
    fill_normal(key, (uint64_t)b, m, mean, sigma, out + b);
  }
}

/* fp32 -> bf16 bits, round to nearest even (finite inputs). */
static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFF) ? 0x40 : 0));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

void synth_f32_to_bf16(const float* in, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_rne(in[i]);
}

/* bf16 tokens: out[i] = bf16(fp32(sigma * N_i)). */
void synth_normal_bf16(uint64_t seed, uint64_t stream, uint64_t sub, double sigma, int64_t n,
                       uint16_t* out) {
  uint64_t key = seq_key(seed, stream, sub);
  const int64_t chunk = 1 << 14;
#pragma omp parallel
  {
    float buf[1 << 14];
#pragma omp for schedule(static)
    for (int64_t c = 0; c < (n + chunk - 1) / chunk; ++c) {
      int64_t b = c * chunk, m = (n - b < chunk) ? n - b : chunk;
      fill_normal(key, (uint64_t)b, m, 0.0, sigma, buf);
      for (int64_t j = 0; j < m; ++j) out[b + j] = f32_to_bf16_rne(buf[j]);
    }
  }
}

/* ---- MXFP4 encoder (input preparation only) ---------------------------- */

/* |v| (already divided by the block scale) -> 3-bit E2M1 magnitude code,
 * round to nearest with ties to the even code, saturating at 6.0. The
 * representable magnitudes are 0, .5, 1, 1.5, 2, 3, 4, 6 for codes 0..7. */
static inline uint8_t e2m1_mag_code(double a) {
  if (a <= 0.25) return 0;
  if (a < 0.75) return 1;
  if (a <= 1.25) return 2;
  if (a < 1.75) return 3;
  if (a <= 2.5) return 4;
  if (a < 3.5) return 5;
  if (a <= 5.0) return 6;
  return 7;
}

/* Encode one row of K fp32 weights (K % 32 == 0). */
static void encode_mxfp4_row(const float* w, int64_t K, uint8_t* codes, uint8_t* scales) {
  for (int64_t g = 0; g < K / 32; ++g) {
    const float* wg = w + g * 32;
    double amax = 0.0;
    for (int j = 0; j < 32; ++j) {
      double a = fabs((double)wg[j]);
      if (a > amax) amax = a;
    }
    int X = 0;
    if (amax > 0.0) {
      int e;
      frexp(amax, &e); /* amax = m * 2^e, m in [0.5, 1): floor(log2(amax)) = e - 1 */
      X = (e - 1) - 2;
      if (X < -127) X = -127;
      if (X > 127) X = 127;
    } else {
      X = -127;
    }
    scales[g] = (uint8_t)(X + 127);
    const double inv = ldexp(1.0, -X); /* exact power of two */
    for (int j = 0; j < 32; j += 2) {
      uint8_t c[2];
      for (int h = 0; h < 2; ++h) {
        double v = (double)wg[j + h] * inv;
        uint8_t m = e2m1_mag_code(fabs(v));
        c[h] = (uint8_t)(m | (signbit(v) ? 8 : 0));
      }
      codes[g * 16 + j / 2] = (uint8_t)(c[0] | (c[1] << 4));
    }
  }
}

void synth_quant_mxfp4(const float* w, int64_t rows, int64_t K, uint8_t* codes, uint8_t* scales) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    encode_mxfp4_row(w + r * K, K, codes + r * (K / 2), scales + r * (K / 32));
}

/* rows x K Gaussian weights N(0, sigma^2), element (r, k) = number r*K + k of
 * the sequence, rounded to fp32 and encoded as MXFP4 without keeping the
 * fp32 tensor. */
void synth_mxfp4_normal(uint64_t seed, uint64_t stream, uint64_t sub, double sigma, int64_t rows,
                        int64_t K, uint8_t* codes, uint8_t* scales) {
  uint64_t key = seq_key(seed, stream, sub);
#pragma omp parallel
  {
    float* buf = (float*)malloc((size_t)K * sizeof(float));
#pragma omp for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
      fill_normal(key, (uint64_t)(r * K), K, 0.0, sigma, buf);
      encode_mxfp4_row(buf, K, codes + r * (K / 2), scales + r * (K / 32));
    }
    free(buf);
  }
}

/* ---- 3-bit block encoder (input preparation only) ----------------------- */

/* fp32 -> IEEE binary16 bits, round to nearest even, saturating at 65504
 * (finite inputs only). */
static uint16_t f32_to_f16_rne(double v) {
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (a == 0.0) return sign;
  if (a >= 65504.0) return (uint16_t)(sign | 0x7BFF);
  int e;
  frexp(a, &e); /* a = m 2^e, m in [0.5, 1) */
  int E = e - 1; /* a in [2^E, 2^(E+1)) */
  if (E < -14) { /* subnormal: multiples of 2^-24 */
    double q = nearbyint(ldexp(a, 24));
    if (q >= 1024.0) return (uint16_t)(sign | 0x0400);
    return (uint16_t)(sign | (uint16_t)q);
  }
  double q = nearbyint(ldexp(a, 10 - E)); /* 1024 .. 2048 */
  if (q >= 2048.0) {
    q = 1024.0;
    E += 1;
  }
  if (E > 15) return (uint16_t)(sign | 0x7BFF);
  return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)((int)q - 1024));
}

static double f16_bits_to_double(uint16_t h) {
  int s = h >> 15, E = (h >> 10) & 31, m = h & 1023;
  double v = E == 0 ? ldexp((double)m, -24) : ldexp(1024.0 + m, E - 25);
  return s ? -v : v;
}

static const float kQ3Uniform[8] = {-4.f, -3.f, -2.f, -1.f, 0.f, 1.f, 2.f, 3.f};

static void q3_put_code(uint8_t* b, int i, int c) {
  int j = i & 3;
  if (i < 24) {
    int q = i >> 3, hi = (i >> 2) & 1;
    b[4 * q + j] |= (uint8_t)(c << (hi ? 3 : 0));
  } else if (i < 28) {
    b[j] |= (uint8_t)((c & 3) << 6);
    b[8 + j] |= (uint8_t)(((c >> 2) & 1) << 6);
  } else {
    b[4 + j] |= (uint8_t)((c & 3) << 6);
    b[8 + j] |= (uint8_t)(((c >> 2) & 1) << 7);
  }
}

static void encode_q3_row(const float* w, int64_t K, const float* lv, uint8_t* codes, uint16_t* scales) {
  double lmax = 0.0;
  for (int c = 0; c < 8; ++c)
    if (fabs((double)lv[c]) > lmax) lmax = fabs((double)lv[c]);
  for (int64_t g = 0; g < K / 32; ++g) {
    const float* wg = w + g * 32;
    double amax = 0.0;
    for (int j = 0; j < 32; ++j)
      if (fabs((double)wg[j]) > amax) amax = fabs((double)wg[j]);
    uint16_t dh = (amax > 0.0 && lmax > 0.0) ? f32_to_f16_rne(amax / lmax) : 0;
    scales[g] = dh;
    double d = f16_bits_to_double(dh);
    uint8_t* b = codes + g * 12;
    memset(b, 0, 12);
    for (int i = 0; i < 32; ++i) {
      int best = 0;
      double be = INFINITY;
      for (int c = 0; c < 8; ++c) {
        double err = fabs((double)wg[i] - d * (double)lv[c]);
        if (err < be) {
          be = err;
          best = c;
        }
      }
      q3_put_code(b, i, best);
    }
  }
}

/* rows x K fp32 weights -> codes [rows][K/32 * 12], scales [rows][K/32]
 * (binary16 bits). tables [n][8] levels, row r using table r / rows_per_table,
 * or NULL for the uniform code book. */
void synth_quant_q3(const float* w, int64_t rows, int64_t K, const float* tables, int64_t rows_per_table,
                    uint8_t* codes, uint16_t* scales) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    encode_q3_row(w + r * K, K, tables ? tables + (r / rows_per_table) * 8 : kQ3Uniform, codes + r * (K / 32) * 12,
                  scales + r * (K / 32));
}

/* Gaussian rows N(0, sigma^2) (element (r, k) = number r*K + k of the
 * sequence) encoded as 3-bit blocks. */
void synth_q3_normal(uint64_t seed, uint64_t stream, uint64_t sub, double sigma, int64_t rows, int64_t K,
                     const float* tables, int64_t rows_per_table, uint8_t* codes, uint16_t* scales) {
  uint64_t key = seq_key(seed, stream, sub);
#pragma omp parallel
  {
    float* buf = (float*)malloc((size_t)K * sizeof(float));
#pragma omp for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
      fill_normal(key, (uint64_t)(r * K), K, 0.0, sigma, buf);
      encode_q3_row(buf, K, tables ? tables + (r / rows_per_table) * 8 : kQ3Uniform, codes + r * (K / 32) * 12,
                    scales + r * (K / 32));
    }
    free(buf);
  }
}

/* n per-expert code books of 8 ascending levels: the normal quantiles at
 * (c + 1/2) / 8, each times (1 + 0.15 u) with u uniform in (-1, 1), sorted. */
void synth_q3_tables(uint64_t seed, uint64_t stream, uint64_t sub, int64_t n, float* out) {
  static const double base[8] = {-1.5341205443525463, -0.8871465590189700, -0.4887764111146695,
                                 -0.1573106846101707, 0.1573106846101707,  0.4887764111146695,
                                 0.8871465590189700,  1.5341205443525463};
  uint64_t key = seq_key(seed, stream, sub);
  for (int64_t e = 0; e < n; ++e) {
    float* t = out + e * 8;
    for (int c = 0; c < 8; ++c) t[c] = (float)(base[c] * (1.0 + 0.15 * (2.0 * ctr_unif(key, (uint64_t)(e * 8 + c)) - 1.0)));
    for (int a = 1; a < 8; ++a)
      for (int b = a; b > 0 && t[b - 1] > t[b]; --b) {
        float x = t[b];
        t[b] = t[b - 1];
        t[b - 1] = x;
      }
  }
}

/* ---- int8 per-row symmetric encoder ------------------------------------ */

static void encode_int8_row(const float* w, int64_t K, int8_t* q, float* s) {
  double amax = 0.0;
  for (int64_t k = 0; k < K; ++k) {
    double a = fabs((double)w[k]);
    if (a > amax) amax = a;
  }
  float sc = amax > 0.0 ? (float)(amax / 127.0) : 1.0f;
  *s = sc;
  for (int64_t k = 0; k < K; ++k) {
    double v = nearbyint((double)w[k] / (double)sc); /* default mode: ties to even */
    if (v > 127.0) v = 127.0;
    if (v < -127.0) v = -127.0;
    q[k] = (int8_t)v;
  }
}

void synth_quant_int8(const float* w, int64_t rows, int64_t K, int8_t* q, float* s) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) encode_int8_row(w + r * K, K, q + r * K, s + r);
}

void synth_int8_normal(uint64_t seed, uint64_t stream, uint64_t sub, double sigma, int64_t rows,
                       int64_t K, int8_t* q, float* s) {
  uint64_t key = seq_key(seed, stream, sub);
#pragma omp parallel
  {
    float* buf = (float*)malloc((size_t)K * sizeof(float));
#pragma omp for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
      fill_normal(key, (uint64_t)(r * K), K, 0.0, sigma, buf);
      encode_int8_row(buf, K, q + r * K, s + r);
    }
    free(buf);
  }
}

/* ---- token ids and the hash table -------------------------------------- */

/* n token ids drawn from Zipf(s) over ranks 1..V by inverse CDF; id = rank-1. */
int synth_zipf_ids(uint64_t seed, uint64_t stream, uint64_t sub, double s, int64_t V, int64_t n,
                   int32_t* out) {
  double* cdf = (double*)malloc((size_t)V * sizeof(double));
  if (!cdf) return -1;
  double acc = 0.0;
  for (int64_t r = 0; r < V; ++r) {
    acc += pow((double)(r + 1), -s);
    cdf[r] = acc;
  }
  uint64_t key = seq_key(seed, stream, sub);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    double u = ctr_unif(key, (uint64_t)i) * acc;
    int64_t lo = 0, hi = V - 1; /* first r with cdf[r] >= u */
    while (lo < hi) {
      int64_t mid = (lo + hi) / 2;
      if (cdf[mid] >= u) hi = mid; else lo = mid + 1;
    }
    out[i] = (int32_t)lo;
  }
  free(cdf);
  return 0;
}

/* V rows of k distinct experts in [0, E), uniform: a partial Fisher-Yates
 * shuffle of 0..E-1 per row, draws from counters row*k + j. */
int synth_tid2eid(uint64_t seed, uint64_t stream, uint64_t sub, int64_t V, int32_t E, int32_t k,
                  int32_t* out) {
  if (k > E || E <= 0 || E > 4096) return -1;
  uint64_t key = seq_key(seed, stream, sub);
#pragma omp parallel
  {
    int32_t perm[4096];
#pragma omp for schedule(static)
    for (int64_t v = 0; v < V; ++v) {
      for (int32_t e = 0; e < E; ++e) perm[e] = e;
      for (int32_t j = 0; j < k; ++j) {
        uint64_t u = ctr_u64(key, (uint64_t)(v * k + j));
        int32_t pick = j + (int32_t)(((u >> 32) * (uint64_t)(E - j)) >> 32);
        int32_t t = perm[j];
        perm[j] = perm[pick];
        perm[pick] = t;
        out[v * k + j] = perm[j];
      }
    }
  }
  return 0;
}
