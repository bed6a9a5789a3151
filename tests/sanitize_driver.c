/* Host sanitizer run of the seeded input generator (synth/synth.c) and the
 * CPU oracle (oracle/oracle.c): a tiny layer generated and evaluated through
 * every oracle entry point, built with AddressSanitizer and
 * UndefinedBehaviorSanitizer by tests/test_sanitizers.py. Any out-of-bounds
 * access, leak or undefined operation aborts with a report. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void synth_normal_f32(uint64_t, uint64_t, uint64_t, double, double, int64_t, float*);
void synth_normal_bf16(uint64_t, uint64_t, uint64_t, double, int64_t, uint16_t*);
void synth_mxfp4_normal(uint64_t, uint64_t, uint64_t, double, int64_t, int64_t, uint8_t*, uint8_t*);
void synth_int8_normal(uint64_t, uint64_t, uint64_t, double, int64_t, int64_t, int8_t*, float*);
int synth_zipf_ids(uint64_t, uint64_t, uint64_t, double, int64_t, int64_t, int32_t*);
int synth_tid2eid(uint64_t, uint64_t, uint64_t, int64_t, int32_t, int32_t, int32_t*);
int or_route(int, int, int, int, const uint16_t*, const float*, const float*, const float*, double, int32_t*,
             double*, double*, int32_t*);
int or_hash_route(int, int, int, int, const uint16_t*, const int32_t*, const int32_t*, int, const float*, double,
                  int32_t*, double*);
int or_permute(int, int, int, const int32_t*, int32_t*, int32_t*, int32_t*);
int or_expert_ffn(int, int, int, int, int, const uint16_t*, const int32_t*, const double*, const uint8_t*,
                  const uint8_t*, const uint8_t*, const uint8_t*, double, int, double*);
int or_shared_ffn(int, int, int, const uint16_t*, const int8_t*, const float*, const int8_t*, const float*, double,
                  int, double*);
int or_forward(int, int, int, int, int, const uint16_t*, const float*, const float*, const float*, const int32_t*,
               const int32_t*, int, const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*, const int8_t*,
               const float*, const int8_t*, const float*, double, double, int, const int32_t*, int,
               const int32_t*, int32_t*, double*, double*, int32_t*, double*);

#define CHECK(x)                                              \
  do {                                                        \
    if (!(x)) {                                               \
      fprintf(stderr, "check failed line %d: %s\n", __LINE__, #x); \
      return 1;                                               \
    }                                                         \
  } while (0)

int main(void) {
  const int T = 9, H = 64, E = 8, k = 3, I = 32, V = 40;
  uint8_t* c13 = malloc((size_t)E * 2 * I * H / 2);
  uint8_t* s13 = malloc((size_t)E * 2 * I * H / 32);
  uint8_t* c2 = malloc((size_t)E * H * I / 2);
  uint8_t* s2 = malloc((size_t)E * H * I / 32);
  int8_t* q13 = malloc((size_t)2 * I * H);
  float* sc13 = malloc(sizeof(float) * 2 * I);
  int8_t* q2 = malloc((size_t)H * I);
  float* sc2 = malloc(sizeof(float) * H);
  float* gate = malloc(sizeof(float) * E * H);
  float* bias = malloc(sizeof(float) * E);
  float* off = malloc(sizeof(float) * E);
  uint16_t* x = malloc(sizeof(uint16_t) * T * H);
  int32_t* tids = malloc(sizeof(int32_t) * T);
  int32_t* t2e = malloc(sizeof(int32_t) * V * k);
  for (int e = 0; e < E; ++e) {
    synth_mxfp4_normal(0, 1, e, 0.02, 2 * I, H, c13 + (size_t)e * 2 * I * H / 2, s13 + (size_t)e * 2 * I * H / 32);
    synth_mxfp4_normal(0, 2, e, 0.02, H, I, c2 + (size_t)e * H * I / 2, s2 + (size_t)e * H * I / 32);
  }
  synth_int8_normal(0, 3, 0, 0.02, 2 * I, H, q13, sc13);
  synth_int8_normal(0, 4, 0, 0.02, H, I, q2, sc2);
  synth_normal_f32(0, 5, 0, 0.0, 0.02, E * H, gate);
  synth_normal_f32(0, 6, 0, 0.0, 0.01, E, bias);
  synth_normal_f32(0, 7, 0, 0.0, 0.5, E, off);
  synth_normal_bf16(0, 8, 0, 1.0, T * H, x);
  CHECK(synth_zipf_ids(0, 9, 0, 1.1, V, T, tids) == 0);
  CHECK(synth_tid2eid(0, 10, 0, V, E, k, t2e) == 0);

  int32_t ids[T * k], nxt[T], offs[E + 1], sorted[T * k], spos[T * k], fids[3 * k];
  double w[T * k], gap[T], y[T * H], z[T * H], out[T * H];
  CHECK(or_route(T, H, E, k, x, gate, bias, off, 1.5, ids, w, gap, nxt) == 0);
  CHECK(or_hash_route(T, H, E, k, x, tids, t2e, V, gate, 1.5, ids, w) == 0);
  CHECK(or_permute(T, k, E, ids, offs, sorted, spos) == 0);
  CHECK(offs[E] == T * k);
  CHECK(or_expert_ffn(T, H, E, k, I, x, ids, w, c13, s13, c2, s2, 10.0, 1, y) == 0);
  CHECK(or_shared_ffn(T, H, I, x, q13, sc13, q2, sc2, 10.0, 1, z) == 0);
  CHECK(or_forward(T, H, E, k, I, x, gate, bias, off, NULL, NULL, 0, c13, s13, c2, s2, q13, sc13, q2, sc2, 1.5, 10.0,
                   1, NULL, T, NULL, ids, w, gap, nxt, out) == 0);
  int32_t rows[3] = {8, 0, 4};
  for (int j = 0; j < 3 * k; ++j) fids[j] = (j * 5) % E;
  fids[1] = 1; fids[2] = 2; fids[4] = 4; fids[5] = 6; fids[7] = 7; fids[8] = 3;
  CHECK(or_forward(T, H, E, k, I, x, gate, bias, off, NULL, NULL, 0, c13, s13, c2, s2, q13, sc13, q2, sc2, 1.5, 10.0,
                   1, rows, 3, fids, ids, w, gap, nxt, out) == 0);
  CHECK(or_forward(T, H, E, k, I, x, gate, bias, off, tids, t2e, V, c13, s13, c2, s2, q13, sc13, q2, sc2, 1.5, 10.0,
                   0, rows, 3, NULL, ids, w, gap, nxt, out) == 0);
  for (int i = 0; i < 3 * H; ++i) CHECK(isfinite(out[i]));
  /* argument errors return an error code without touching memory */
  int32_t bad[3] = {0, E, 1};
  CHECK(or_permute(1, 3, E, bad, offs, sorted, spos) != 0);
  free(c13); free(s13); free(c2); free(s2); free(q13); free(sc13); free(q2); free(sc2);
  free(gate); free(bias); free(off); free(x); free(tids); free(t2e);
  printf("sanitized oracle and generator run: ok\n");
  return 0;
}
