/*
 * moe_oracle.c -- plain, slow CPU oracle for the MoE feed-forward sublayer of a
 * GLM-style MoE block (RMSNorm -> sigmoid router with correction-bias top-k ->
 * routed SwiGLU experts in the grouped layout + one SwiGLU shared expert ->
 * weighted combine + residual).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark load this library.  It shares no code, header,
 * table or helper with the GPU library and must never be used as a fallback
 * for it.
 *
 * Sources (web pages; cited by title and section):
 *   [RMS]  "GLM-5 · Input features" (OpenModelAtlas), excerpt "rmsnorm"
 *          (GlmMoeDsaRMSNorm): one gain per feature; normalise in float32 with
 *          the mean of squares (no centring), cast back to the input dtype,
 *          then multiply by the gain; default epsilon 1e-6.  The same excerpt
 *          appears on "GLM-5 · Query latent".
 *   [MLP]  same page, excerpt "mlp" (GlmMoeDsaMLP): the feed-forward network is
 *          down(silu(gate x) * up x) with three bias-free linear maps.
 *   [BLK]  same page, excerpt "block" (GlmMoeDsaDecoderLayer): the residual is
 *          the pre-norm hidden state; out = residual + mlp(norm(residual)).
 *   [LAY]  "nemo_automodel.components.models.glm4_moe.state_dict_adapter", class
 *          Glm4MoeStateDictAdapter: the grouped native layout
 *          gate_and_up_projs [n_experts, dim, 2*moe_inter_dim] and
 *          down_projs [n_experts, moe_inter_dim, dim]; the shared expert keeps
 *          separate gate/up/down nn.Linear weights ([out, in]).
 *   [PAR]  "GLM-5 · MoE transformer block", Parameters table and the note under
 *          it: the router keeps one correction-bias value per expert as a buffer.
 *   The router rule itself (sigmoid scores, bias added for selection only,
 *   renormalised unbiased scores times a routed scale) is not printed on the
 *   pages; it is the workload definition this oracle is written against.
 *
 * Precision.  Storage dtype D is fp32 (dtype 0) or bfloat16 (dtype 1, passed as
 * raw uint16 bit patterns).  RMSNorm follows the page's fp32 arithmetic: the
 * mean of squares is the correctly rounded fp32 value (accumulated in double),
 * r = 1/sqrt(ms + eps) with IEEE fp32 sqrt and divide, n = fp32(x*r) rounded to
 * D, h = fp32(w*n) rounded to D.  Router scores and the biased selection key
 * are fp32 (the precision in which the selection decision is taken); every
 * other accumulation (logits, expert matmuls, combine) is fp64 with no
 * intermediate rounding, and the output is rounded once to D.
 *
 * Error behaviour: functions return 0 on success, -1 on a bad argument.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_API __attribute__((visibility("default")))

enum { OR_F32 = 0, OR_BF16 = 1 };

/* bfloat16 <-> float by bit manipulation (round to nearest even). */
static float bf16_bits_to_float(uint16_t b) {
  uint32_t u = ((uint32_t)b) << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static uint16_t float_to_bf16_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x40); /* NaN */
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* Round a float to the storage dtype and return it as float. */
static float round_to_dtype(float f, int dtype) {
  if (dtype == OR_BF16) return bf16_bits_to_float(float_to_bf16_bits(f));
  return f;
}

static float load_elem(const void* p, int64_t i, int dtype) {
  if (dtype == OR_BF16) return bf16_bits_to_float(((const uint16_t*)p)[i]);
  return ((const float*)p)[i];
}

/* Threads an OpenMP parallel region of this library uses. */
ORACLE_API int oracle_num_threads(void) { return omp_get_max_threads(); }

/* Threads of the parallel loops that follow on the calling thread (timing only). */
ORACLE_API int oracle_set_num_threads(int32_t n) {
  if (n < 1) return -1;
  omp_set_num_threads(n);
  return 0;
}

ORACLE_API int oracle_round_to_dtype(int64_t n, const float* in, float* out, int dtype) {
  if (n < 0 || (n > 0 && (!in || !out))) return -1;
  for (int64_t i = 0; i < n; ++i) out[i] = round_to_dtype(in[i], dtype);
  return 0;
}

/* ---- O1: RMSNorm [RMS] ------------------------------------------------------
 * x [T, d] (dtype), w [d] (dtype) -> h [T, d] as float holding dtype values. */
ORACLE_API int oracle_rmsnorm(int64_t T, int32_t d, int32_t dtype, float eps, const void* x,
                              const void* w, float* h) {
  if (T < 0 || d <= 0 || (T > 0 && (!x || !w || !h))) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    double ss = 0.0;
    for (int32_t i = 0; i < d; ++i) {
      double v = (double)load_elem(x, t * d + i, dtype);
      ss += v * v;
    }
    float ms = (float)(ss / (double)d);      /* mean of squares, fp32 */
    float r = 1.0f / sqrtf(ms + eps);        /* fp32 sqrt and divide */
    for (int32_t i = 0; i < d; ++i) {
      float xi = load_elem(x, t * d + i, dtype);
      float n = round_to_dtype(xi * r, dtype);            /* cast back to input dtype */
      float wi = load_elem(w, i, dtype);
      h[t * d + i] = round_to_dtype(wi * n, dtype);       /* gain, result in dtype */
    }
  }
  return 0;
}

/* ---- O2: router scores -----------------------------------------------------
 * logit[t,e] = sum_i h[t,i] * router_w[e,i]   (fp64 accumulation, then fp32)
 * score[t,e] = sigmoid(logit) in fp32 (computed in double, rounded once).
 * router_w is [E, d] in the nn.Linear [out, in] orientation. */
ORACLE_API int oracle_router_scores(int64_t T, int32_t d, int32_t E, int32_t dtype, const float* h,
                                    const void* router_w, float* logits, float* scores) {
  if (T < 0 || d <= 0 || E <= 0 || (T > 0 && (!h || !router_w || !scores))) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    for (int32_t e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int32_t i = 0; i < d; ++i)
        acc += (double)h[t * d + i] * (double)load_elem(router_w, (int64_t)e * d + i, dtype);
      float l = (float)acc;
      if (logits) logits[t * E + e] = l;
      scores[t * E + e] = (float)(1.0 / (1.0 + exp(-(double)l)));
    }
  }
  return 0;
}

/* ---- O3 + O4: selection and weights ----------------------------------------
 * key[e] = score[e] + corr_bias[e] (fp32 add).  The k selected experts are the
 * first k in the order (key descending, expert index ascending); idx lists them
 * in that order.  margin[t] = key of the k-th pick minus key of the (k+1)-th
 * (infinity when k == E).  w_j = routed_scale * score[idx_j] / sum_j' score[idx_j'],
 * in fp64; the bias never enters the weights. */
ORACLE_API int oracle_select(int64_t T, int32_t E, int32_t k, const float* scores,
                             const float* corr_bias, double routed_scale, int32_t* idx, double* w,
                             double* margin) {
  if (T < 0 || E <= 0 || k < 1 || k > E || (T > 0 && (!scores || !corr_bias || !idx || !w)))
    return -1;
  int ok = 0;
#pragma omp parallel
  {
    float* key = (float*)malloc(sizeof(float) * (size_t)E);
    unsigned char* taken = (unsigned char*)malloc((size_t)E);
    if (!key || !taken) {
#pragma omp atomic write
      ok = -1;
    }
    /* every thread reaches the worksharing loop; one without buffers skips work */
#pragma omp for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
      if (!key || !taken) continue;
      {
        for (int32_t e = 0; e < E; ++e) {
          key[e] = scores[t * E + e] + corr_bias[e];
          taken[e] = 0;
        }
        float kth = 0.0f;
        for (int32_t j = 0; j < k; ++j) {
          int32_t best = -1;
          for (int32_t e = 0; e < E; ++e) {
            if (taken[e]) continue;
            if (best < 0 || key[e] > key[best]) best = e; /* strict '>' keeps the lower index on ties */
          }
          taken[best] = 1;
          idx[t * k + j] = best;
          kth = key[best];
        }
        if (margin) {
          if (k == E) {
            margin[t] = INFINITY;
          } else {
            int32_t next = -1;
            for (int32_t e = 0; e < E; ++e)
              if (!taken[e] && (next < 0 || key[e] > key[next])) next = e;
            margin[t] = (double)kth - (double)key[next];
          }
        }
        double ssum = 0.0;
        for (int32_t j = 0; j < k; ++j) ssum += (double)scores[t * E + idx[t * k + j]];
        for (int32_t j = 0; j < k; ++j)
          w[t * k + j] = routed_scale * (double)scores[t * E + idx[t * k + j]] / ssum;
      }
    }
    free(key);
    free(taken);
  }
  return ok;
}

/* ---- O5: per-expert counts and segment offsets ----------------------------- */
ORACLE_API int oracle_counts(int64_t T, int32_t E, int32_t k, const int32_t* idx, int32_t* counts,
                             int64_t* offsets /* [E+1] or NULL */) {
  if (T < 0 || E <= 0 || k < 1 || !counts || (T > 0 && !idx)) return -1;
  for (int32_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t a = 0; a < T * k; ++a) {
    int32_t e = idx[a];
    if (e < 0 || e >= E) return -1;
    counts[e]++;
  }
  if (offsets) {
    offsets[0] = 0;
    for (int32_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  }
  return 0;
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* ---- O6 - O8: experts, shared expert, combine ------------------------------
 * For each listed token s (tokens[s] indexes the full batch):
 *   routed expert e = idx[t, j] (grouped layout [LAY]):
 *     g_n = sum_i h_i * gate_up[e][i][n],  u_n = sum_i h_i * gate_up[e][i][I + n]
 *     a_n = silu(g_n) * u_n                 ([MLP]: gate half first, then up)
 *     y_m = sum_n a_n * down[e][n][m]
 *   shared expert (nn.Linear [out, in] weights [LAY], [MLP]):
 *     gs_n = sum_i shared_gate[n][i] h_i,  us_n = sum_i shared_up[n][i] h_i
 *     as_n = silu(gs_n) * us_n,  s_m = sum_n shared_down[m][n] as_n
 *   delta_m = s_m + sum_j w_j y_{j,m}  (shared first, then j ascending)
 *   out_m   = D(x_m + delta_m)          ([BLK]: residual is the pre-norm input)
 * gate_up / down are arrays of E per-expert pointers; an expert no listed token
 * selects may be NULL.  Shared pointers may be NULL when Is == 0.
 * Optional outputs: act [n_tok*k*I] and y [n_tok*k*d] (fp64, per (s, j)),
 * act_s [n_tok*Is], s_out [n_tok*d]. */
ORACLE_API int oracle_experts(int64_t n_tok, const int64_t* tokens, int32_t d, int32_t E, int32_t I,
                              int32_t Is, int32_t k, int32_t dtype, const void* x, const float* h,
                              const int32_t* idx, const double* w, const void* const* gate_up,
                              const void* const* down, const void* shared_gate,
                              const void* shared_up, const void* shared_down, double* delta,
                              float* out, double* act_dbg, double* y_dbg, double* act_s_dbg,
                              double* s_dbg) {
  if (n_tok < 0 || d <= 0 || E <= 0 || I <= 0 || Is < 0 || k < 1 || k > E) return -1;
  if (n_tok == 0) return 0;
  if (!tokens || !x || !h || !idx || !w || !gate_up || !down || !delta || !out) return -1;
  if (Is > 0 && (!shared_gate || !shared_up || !shared_down)) return -1;
  for (int64_t s = 0; s < n_tok; ++s)
    for (int32_t j = 0; j < k; ++j) {
      int32_t e = idx[tokens[s] * k + j];
      if (e < 0 || e >= E || !gate_up[e] || !down[e]) return -1;
    }

  const int64_t n_asg = n_tok * k;
  double* y = (double*)calloc((size_t)n_asg * (size_t)d, sizeof(double));
  double* sh = (double*)calloc((size_t)n_tok * (size_t)d, sizeof(double));
  if (!y || !sh) {
    free(y);
    free(sh);
    return -1;
  }
  int status = 0;

  /* Routed experts, one expert at a time; the assignments of one expert share
   * each streamed weight row. */
#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t e = 0; e < E; ++e) {
    int64_t na = 0;
    for (int64_t a = 0; a < n_asg; ++a)
      if (idx[tokens[a / k] * k + (a % k)] == e) na++;
    if (na == 0) continue;
    int64_t* list = (int64_t*)malloc(sizeof(int64_t) * (size_t)na);
    double* gu = (double*)calloc((size_t)na * 2 * (size_t)I, sizeof(double));
    double* av = (double*)malloc(sizeof(double) * (size_t)na * (size_t)I);
    float* row = (float*)malloc(sizeof(float) * (size_t)(2 * I > d ? 2 * I : d));
    if (!list || !gu || !av || !row) {
#pragma omp atomic write
      status = -1;
      free(list); free(gu); free(av); free(row);
      continue;
    }
    int64_t c = 0;
    for (int64_t a = 0; a < n_asg; ++a)
      if (idx[tokens[a / k] * k + (a % k)] == e) list[c++] = a;

    /* gate and up: contraction over dim (rows of gate_up[e]) */
    for (int32_t i = 0; i < d; ++i) {
      for (int32_t n = 0; n < 2 * I; ++n)
        row[n] = load_elem(gate_up[e], (int64_t)i * 2 * I + n, dtype);
      for (int64_t q = 0; q < na; ++q) {
        double hi = (double)h[tokens[list[q] / k] * d + i];
        double* acc = gu + q * 2 * I;
        for (int32_t n = 0; n < 2 * I; ++n) acc[n] += hi * (double)row[n];
      }
    }
    for (int64_t q = 0; q < na; ++q)
      for (int32_t n = 0; n < I; ++n) {
        double g = gu[q * 2 * I + n], u = gu[q * 2 * I + I + n];
        av[q * I + n] = silu(g) * u;
        if (act_dbg) act_dbg[list[q] * I + n] = av[q * I + n];
      }
    /* down: contraction over moe_inter (rows of down[e]) */
    for (int32_t n = 0; n < I; ++n) {
      for (int32_t m = 0; m < d; ++m) row[m] = load_elem(down[e], (int64_t)n * d + m, dtype);
      for (int64_t q = 0; q < na; ++q) {
        double an = av[q * I + n];
        double* acc = y + list[q] * d;
        for (int32_t m = 0; m < d; ++m) acc[m] += an * (double)row[m];
      }
    }
    free(list); free(gu); free(av); free(row);
  }

  /* Shared expert, one token at a time. */
  if (Is > 0) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t s = 0; s < n_tok; ++s) {
      const float* hs = h + tokens[s] * d;
      double* as = (double*)malloc(sizeof(double) * (size_t)Is);
      if (!as) {
#pragma omp atomic write
        status = -1;
        continue;
      }
      for (int32_t n = 0; n < Is; ++n) {
        double g = 0.0, u = 0.0;
        for (int32_t i = 0; i < d; ++i) {
          g += (double)load_elem(shared_gate, (int64_t)n * d + i, dtype) * (double)hs[i];
          u += (double)load_elem(shared_up, (int64_t)n * d + i, dtype) * (double)hs[i];
        }
        as[n] = silu(g) * u;
        if (act_s_dbg) act_s_dbg[s * Is + n] = as[n];
      }
      for (int32_t m = 0; m < d; ++m) {
        double acc = 0.0;
        for (int32_t n = 0; n < Is; ++n)
          acc += (double)load_elem(shared_down, (int64_t)m * Is + n, dtype) * as[n];
        sh[s * d + m] = acc;
      }
      free(as);
    }
  }

  /* Combine: shared output, then routed outputs in j order, then residual. */
  for (int64_t s = 0; s < n_tok; ++s) {
    int64_t t = tokens[s];
    for (int32_t m = 0; m < d; ++m) {
      double acc = sh[s * d + m];
      for (int32_t j = 0; j < k; ++j) acc += w[t * k + j] * y[(s * k + j) * d + m];
      delta[s * d + m] = acc;
      double xm = (double)load_elem(x, t * d + m, dtype);
      out[s * d + m] = round_to_dtype((float)(xm + acc), dtype);
    }
  }
  if (y_dbg) memcpy(y_dbg, y, sizeof(double) * (size_t)n_asg * (size_t)d);
  if (s_dbg) memcpy(s_dbg, sh, sizeof(double) * (size_t)n_tok * (size_t)d);
  free(y);
  free(sh);
  return status;
}

/* ---- O9: dense SwiGLU MLP block ---------------------------------------------
 * The blocks before the first MoE block use a dense MLP instead of the MoE
 * ([BLK]: the first first_k_dense_replace blocks; [MLP]: GlmMoeDsaMLP, three
 * bias-free nn.Linear maps [out, in], down(silu(gate x) * up x)).  For every
 * token t of the batch, with h the RMSNorm output (O1):
 *   g_n = sum_i gate[n][i] h_i,  u_n = sum_i up[n][i] h_i,  a_n = silu(g_n) * u_n
 *   y_m = sum_n down[m][n] a_n
 *   out_m = D(x_m + y_m)            ([BLK]: the residual is the pre-norm input)
 * fp64 accumulation, no intermediate rounding; optional act [T*Id] and y [T*d]. */
ORACLE_API int oracle_dense_mlp(int64_t T, int32_t d, int32_t Id, int32_t dtype, const void* x,
                                const float* h, const void* gate, const void* up,
                                const void* down, double* delta, float* out, double* act_dbg) {
  if (T < 0 || d <= 0 || Id <= 0) return -1;
  if (T == 0) return 0;
  if (!x || !h || !gate || !up || !down || !delta || !out) return -1;
  int status = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t t = 0; t < T; ++t) {
    const float* ht = h + t * d;
    double* a = (double*)malloc(sizeof(double) * (size_t)Id);
    if (!a) {
#pragma omp atomic write
      status = -1;
      continue;
    }
    for (int32_t n = 0; n < Id; ++n) {
      double g = 0.0, u = 0.0;
      for (int32_t i = 0; i < d; ++i) {
        g += (double)load_elem(gate, (int64_t)n * d + i, dtype) * (double)ht[i];
        u += (double)load_elem(up, (int64_t)n * d + i, dtype) * (double)ht[i];
      }
      a[n] = silu(g) * u;
      if (act_dbg) act_dbg[t * Id + n] = a[n];
    }
    for (int32_t m = 0; m < d; ++m) {
      double y = 0.0;
      for (int32_t n = 0; n < Id; ++n) y += (double)load_elem(down, (int64_t)m * Id + n, dtype) * a[n];
      delta[t * d + m] = y;
      out[t * d + m] = round_to_dtype((float)((double)load_elem(x, t * d + m, dtype) + y), dtype);
    }
    free(a);
  }
  return status;
}
