/* Drives every function of the oracle (oracle/moe_oracle.c) once per dtype on small
 * random inputs, including the argument checks, so that a build with AddressSanitizer
 * and UndefinedBehaviorSanitizer sees each of its loops.  Test infrastructure: built
 * and run by tests/test_oracle_sanitized.py.  Exit status 0 when every call returned
 * what it should. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_num_threads(void);
int oracle_set_num_threads(int32_t n);
int oracle_round_to_dtype(int64_t n, const float* in, float* out, int dtype);
int oracle_rmsnorm(int64_t T, int32_t d, int32_t dtype, float eps, const void* x, const void* w,
                   float* h);
int oracle_router_scores(int64_t T, int32_t d, int32_t E, int32_t dtype, const float* h,
                         const void* router_w, float* logits, float* scores);
int oracle_select(int64_t T, int32_t E, int32_t k, const float* scores, const float* corr_bias,
                  double routed_scale, int32_t* idx, double* w, double* margin);
int oracle_counts(int64_t T, int32_t E, int32_t k, const int32_t* idx, int32_t* counts,
                  int64_t* offsets);
int oracle_experts(int64_t n_tok, const int64_t* tokens, int32_t d, int32_t E, int32_t I,
                   int32_t Is, int32_t k, int32_t dtype, const void* x, const float* h,
                   const int32_t* idx, const double* w, const void* const* gate_up,
                   const void* const* down, const void* shared_gate, const void* shared_up,
                   const void* shared_down, double* delta, float* out, double* act_dbg,
                   double* y_dbg, double* act_s_dbg, double* s_dbg);
int oracle_dense_mlp(int64_t T, int32_t d, int32_t Id, int32_t dtype, const void* x,
                     const float* h, const void* gate, const void* up, const void* down,
                     double* delta, float* out, double* act_dbg);

static uint64_t state = 0x9e3779b97f4a7c15ull;
static double uniform(void) { /* xorshift64*, in [-1, 1) */
  state ^= state >> 12;
  state ^= state << 25;
  state ^= state >> 27;
  return (double)((state * 0x2545f4914f6cdd1dull) >> 11) / 4503599627370496.0 - 1.0;
}

/* n elements of dtype (0: fp32, 1: bf16 bits) with values scale * U(-1, 1) */
static void* draw(int64_t n, int dtype, double scale) {
  if (dtype == 0) {
    float* p = malloc((size_t)n * sizeof(float));
    for (int64_t i = 0; i < n; ++i) p[i] = (float)(scale * uniform());
    return p;
  }
  uint16_t* p = malloc((size_t)n * sizeof(uint16_t));
  for (int64_t i = 0; i < n; ++i) {
    const float f = (float)(scale * uniform());
    uint32_t u;
    memcpy(&u, &f, 4);
    p[i] = (uint16_t)(u >> 16);
  }
  return p;
}

#define CHECK(cond)                                              \
  do {                                                           \
    if (!(cond)) {                                               \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      return 1;                                                  \
    }                                                            \
  } while (0)

static int run(int dtype) {
  const int64_t T = 7;
  const int32_t d = 40, E = 9, I = 24, Is = 16, k = 3, Id = 32;
  void* x = draw(T * d, dtype, 1.0);
  void* nw = draw(d, dtype, 1.0);
  void* rw = draw((int64_t)E * d, dtype, 0.2);
  float* bias = draw(E, 0, 0.05);
  void* gu[9];
  void* dn[9];
  for (int e = 0; e < E; ++e) {
    gu[e] = draw((int64_t)d * 2 * I, dtype, 0.1);
    dn[e] = draw((int64_t)I * d, dtype, 0.1);
  }
  void* sg = draw((int64_t)Is * d, dtype, 0.1);
  void* su = draw((int64_t)Is * d, dtype, 0.1);
  void* sd = draw((int64_t)d * Is, dtype, 0.1);
  float* h = malloc(sizeof(float) * T * d);
  float* logits = malloc(sizeof(float) * T * E);
  float* scores = malloc(sizeof(float) * T * E);
  int32_t* idx = malloc(sizeof(int32_t) * T * k);
  double* w = malloc(sizeof(double) * T * k);
  double* margin = malloc(sizeof(double) * T);
  int32_t* counts = malloc(sizeof(int32_t) * E);
  int64_t* offsets = malloc(sizeof(int64_t) * (E + 1));
  int64_t* tokens = malloc(sizeof(int64_t) * T);
  double* delta = malloc(sizeof(double) * T * d);
  float* out = malloc(sizeof(float) * T * d);
  double* act = malloc(sizeof(double) * T * k * I);
  double* y = malloc(sizeof(double) * T * k * d);
  double* act_s = malloc(sizeof(double) * T * Is);
  double* s_out = malloc(sizeof(double) * T * d);
  float* rin = draw(T * d, 0, 3.0);
  float* rout = malloc(sizeof(float) * T * d);
  for (int64_t t = 0; t < T; ++t) tokens[t] = T - 1 - t; /* any order */

  CHECK(oracle_round_to_dtype(T * d, rin, rout, dtype) == 0);
  CHECK(oracle_rmsnorm(T, d, dtype, 1e-6f, x, nw, h) == 0);
  CHECK(oracle_rmsnorm(T, 0, dtype, 1e-6f, x, nw, h) != 0);
  CHECK(oracle_router_scores(T, d, E, dtype, h, rw, logits, scores) == 0);
  CHECK(oracle_router_scores(T, d, E, dtype, h, rw, NULL, scores) == 0);
  CHECK(oracle_select(T, E, k, scores, bias, 2.5, idx, w, margin) == 0);
  CHECK(oracle_select(T, E, E, scores, bias, 1.0, NULL, w, NULL) != 0);
  CHECK(oracle_counts(T, E, k, idx, counts, offsets) == 0);
  CHECK(offsets[E] == T * k);
  CHECK(oracle_experts(T, tokens, d, E, I, Is, k, dtype, x, h, idx, w, (const void* const*)gu,
                       (const void* const*)dn, sg, su, sd, delta, out, act, y, act_s,
                       s_out) == 0);
  CHECK(oracle_experts(T, tokens, d, E, I, 0, k, dtype, x, h, idx, w, (const void* const*)gu,
                       (const void* const*)dn, NULL, NULL, NULL, delta, out, NULL, NULL, NULL,
                       NULL) == 0);
  CHECK(oracle_experts(0, tokens, d, E, I, Is, k, dtype, x, h, idx, w, NULL, NULL, NULL, NULL,
                       NULL, NULL, NULL, NULL, NULL, NULL, NULL) == 0);
  {
    void* g = draw((int64_t)Id * d, dtype, 0.1);
    void* u = draw((int64_t)Id * d, dtype, 0.1);
    void* dd = draw((int64_t)d * Id, dtype, 0.1);
    double* act_d = malloc(sizeof(double) * T * Id);
    CHECK(oracle_dense_mlp(T, d, Id, dtype, x, h, g, u, dd, delta, out, act_d) == 0);
    CHECK(oracle_dense_mlp(T, d, Id, dtype, x, h, g, u, dd, delta, out, NULL) == 0);
    free(g); free(u); free(dd); free(act_d);
  }
  for (int64_t i = 0; i < T * d; ++i) CHECK(isfinite(out[i]));

  free(x); free(nw); free(rw); free(bias);
  for (int e = 0; e < E; ++e) { free(gu[e]); free(dn[e]); }
  free(sg); free(su); free(sd); free(h); free(logits); free(scores); free(idx); free(w);
  free(margin); free(counts); free(offsets); free(tokens); free(delta); free(out); free(act);
  free(y); free(act_s); free(s_out); free(rin); free(rout);
  return 0;
}

int main(void) {
  CHECK(oracle_set_num_threads(2) == 0 || oracle_num_threads() >= 1);
  for (int dtype = 0; dtype < 2; ++dtype)
    if (run(dtype) != 0) return 1;
  printf("oracle driver: all calls ok\n");
  return 0;
}
