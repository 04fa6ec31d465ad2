/*
 * Plain fp64 CPU oracle for the routed-expert MoE FFN layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the GPU library, and the GPU library never
 * calls it.
 *
 * Every result is the plain definition written out as loops in double
 * precision; stored fp16/bf16/fp32/int8 inputs are taken exactly into fp64.
 *
 * Sources (the pages describing the method):
 *  - BigMoeOnEdge (onecrewdev), section "every token is re-routed at every
 *    layer": per token and layer a router scores the experts, the top-K are
 *    chosen with coefficients, and the output is the coefficient-weighted sum
 *    of the chosen experts' FFN outputs; the shared expert is not among the K.
 *  - Same page, section "from the real routing to the GGUF weight slice":
 *    an expert has gate, up and down projections.
 *  - Rockchip-NPU MoE streaming plan (cnblogs), §2.1/§2.5: affine 4-bit
 *    weights in groups of 64 for routed and shared experts, router at 8 bits;
 *    §2.4: the shared expert's output is fused with the routed outputs.
 *  - Same plan, §8.4: prefill is processed in 128-token chunks so one fetched
 *    expert serves every row of the chunk that chose it (the token->expert
 *    grouping computed by oracle_sort).
 * Readings where the pages are silent (activation = SiLU-gated, softmax over
 * all experts then renormalise over the chosen K, lower index wins ties,
 * unit-weight shared expert, int8 router with one fp16 scale per row plus an
 * fp32 logit bias) are listed with the design notes of the repository.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "moe_oracle.h"

#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads the OpenMP loops of this library will use. */
int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Set that number (n >= 1); used to time the oracle on one core. */
void oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* ---- exact storage-format decoding ------------------------------------- */

double oracle_f16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1;
  int ex = (h >> 10) & 0x1F;
  int man = h & 0x3FF;
  double v;
  if (ex == 0)
    v = ldexp((double)man, -24); /* subnormal: man * 2^-24 */
  else if (ex == 31)
    v = man ? NAN : INFINITY;
  else
    v = ldexp((double)(man | 0x400), ex - 25); /* (1024+man) * 2^(ex-15-10) */
  return sign ? -v : v;
}

double oracle_bf16_to_f64(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Round a double to the nearest bf16 (ties to even), directly from fp64. */
uint16_t oracle_f64_to_bf16(double v) {
  if (isnan(v)) return 0x7FC0;
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);            /* a = m * 2^e, m in [0.5, 1) */
  int ulp_e = e - 8;       /* bf16 keeps 8 significant bits */
  if (ulp_e < -133) ulp_e = -133; /* subnormal spacing 2^-133 */
  double ulp = ldexp(1.0, ulp_e);
  double q = a / ulp;      /* exact: scaling by a power of two */
  double r = nearbyint(q); /* default rounding mode: ties to even */
  double rv = r * ulp;
  float f = (float)rv;     /* rv is representable in bf16, hence in fp32 */
  if (isinf(f) || rv > 3.3895313892515355e38) return sign | 0x7F80;
  uint32_t u;
  memcpy(&u, &f, 4);
  return sign | (uint16_t)(u >> 16);
}

/* ---- dequantisation ----------------------------------------------------- */

/* q[r][c] is nibble (c % 8) of word c/8 of row r, low nibble first; the
 * weight is scale*q + bias with (scale, bias) of group c/64 of row r. */
double oracle_weight(const uint32_t* q, const uint16_t* s, const uint16_t* b, int cols, int r, int c) {
  uint32_t word = q[(size_t)r * (cols / 8) + c / 8];
  int nib = (int)((word >> (4 * (c % 8))) & 0xFu);
  size_t g = (size_t)r * (cols / 64) + c / 64;
  return oracle_f16_to_f64(s[g]) * (double)nib + oracle_f16_to_f64(b[g]);
}

void oracle_dequant(const uint32_t* q, const uint16_t* s, const uint16_t* b, int rows, int cols, double* W) {
  for (int r = 0; r < rows; ++r)
    for (int c = 0; c < cols; ++c) W[(size_t)r * cols + c] = oracle_weight(q, s, b, cols, r, c);
}

/* out[r] = sum_c W[r][c] * x[c] */
static void matvec(const uint32_t* q, const uint16_t* s, const uint16_t* b, int rows, int cols,
                   const double* x, double* out) {
#pragma omp parallel for schedule(static)
  for (int r = 0; r < rows; ++r) {
    double acc = 0.0;
    for (int c = 0; c < cols; ++c) acc += oracle_weight(q, s, b, cols, r, c) * x[c];
    out[r] = acc;
  }
}

/* ---- router ------------------------------------------------------------- */

/* l[t][e] = s_e * sum_c Wr[e][c] * x[t][c] + b_e */
void oracle_router_logits(const oracle_layer* L, const double* x, int T, double* logits) {
  for (int t = 0; t < T; ++t)
    for (int e = 0; e < L->E; ++e) {
      double acc = 0.0;
      for (int c = 0; c < L->d; ++c) acc += (double)L->router_w[(size_t)e * L->d + c] * x[(size_t)t * L->d + c];
      double l = oracle_f16_to_f64(L->router_scale[e]) * acc;
      if (L->router_bias) l += (double)L->router_bias[e];
      logits[(size_t)t * L->E + e] = l;
    }
}

/* ---- selection ---------------------------------------------------------- */

/* a ranks before b: larger logit first, lower index on equal logits */
static int ranks_before(double la, int a, double lb, int b) { return la > lb || (la == lb && a < b); }

/* Choose the K best experts of one token (order: logit descending, index
 * ascending), report them in ascending index order with weights
 * w_e = exp(l_e - max) / sum over the chosen set, i.e. a softmax over all
 * experts renormalised to the chosen ones.  margin = l_(K) - l_(K+1)
 * (INFINITY when K == E). */
void oracle_select_one(const double* l, int E, int K, int32_t* ids, double* w, double* margin) {
  int* order = (int*)malloc(sizeof(int) * E);
  for (int e = 0; e < E; ++e) order[e] = e;
  /* insertion sort: plain and stable enough for E <= 1024 */
  for (int i = 1; i < E; ++i) {
    int v = order[i], j = i - 1;
    while (j >= 0 && ranks_before(l[v], v, l[order[j]], order[j])) {
      order[j + 1] = order[j];
      --j;
    }
    order[j + 1] = v;
  }
  if (margin) *margin = (K < E) ? l[order[K - 1]] - l[order[K]] : INFINITY;
  /* ascending ids */
  int32_t* sel = (int32_t*)malloc(sizeof(int32_t) * K);
  for (int k = 0; k < K; ++k) sel[k] = order[k];
  for (int i = 1; i < K; ++i) {
    int32_t v = sel[i];
    int j = i - 1;
    while (j >= 0 && sel[j] > v) {
      sel[j + 1] = sel[j];
      --j;
    }
    sel[j + 1] = v;
  }
  oracle_weights_for_set(l, sel, K, w);
  for (int k = 0; k < K; ++k) ids[k] = sel[k];
  free(sel);
  free(order);
}

void oracle_weights_for_set(const double* l, const int32_t* sel, int K, double* w) {
  double mx = -INFINITY;
  for (int k = 0; k < K; ++k)
    if (l[sel[k]] > mx) mx = l[sel[k]];
  double den = 0.0;
  for (int k = 0; k < K; ++k) den += exp(l[sel[k]] - mx);
  for (int k = 0; k < K; ++k) w[k] = exp(l[sel[k]] - mx) / den;
}

/* ---- experts ------------------------------------------------------------ */

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* out[d] = W_down * (silu(W_gate x) (.) (W_up x)); expert < 0 selects the
 * shared expert. */
void oracle_expert(const oracle_layer* L, int expert, const double* x, double* out) {
  int d = L->d;
  int f = expert < 0 ? L->fs : L->f;
  const uint32_t *gq, *uq, *dq;
  const uint16_t *gs, *gb, *us, *ub, *ds, *db;
  if (expert < 0) {
    gq = L->sh_gate_q; gs = L->sh_gate_s; gb = L->sh_gate_b;
    uq = L->sh_up_q;   us = L->sh_up_s;   ub = L->sh_up_b;
    dq = L->sh_down_q; ds = L->sh_down_s; db = L->sh_down_b;
  } else {
    size_t e = (size_t)expert;
    size_t gu_w = (size_t)f * d / 8, gu_g = (size_t)f * d / 64;
    gq = L->gate_q + e * gu_w; gs = L->gate_s + e * gu_g; gb = L->gate_b + e * gu_g;
    uq = L->up_q + e * gu_w;   us = L->up_s + e * gu_g;   ub = L->up_b + e * gu_g;
    dq = L->down_q + e * gu_w; ds = L->down_s + e * gu_g; db = L->down_b + e * gu_g;
  }
  double* g = (double*)malloc(sizeof(double) * f);
  double* u = (double*)malloc(sizeof(double) * f);
  matvec(gq, gs, gb, f, d, x, g);
  matvec(uq, us, ub, f, d, x, u);
  for (int r = 0; r < f; ++r) g[r] = silu(g[r]) * u[r];
  matvec(dq, ds, db, d, f, g, out);
  free(g);
  free(u);
}

/* ---- whole layer -------------------------------------------------------- */

/* y[t] = shared(x_t) + sum_{e in S_t} w_e * expert_e(x_t).
 * forced (nullable, [T][K] ascending ids): use that set instead of the top-K,
 * with weights renormalised from the current logits over it.
 * ids/w/margin (nullable) receive the selection. */
int oracle_layer_forward(const oracle_layer* L, const double* x, int T, const int32_t* forced, double* y,
                         int32_t* ids_out, double* w_out, double* margin_out) {
  int d = L->d, E = L->E, K = L->K;
  if (K < 1 || K > E || d % 64 || L->f % 64 || (L->fs % 64)) return 1;
  double* logits = (double*)malloc(sizeof(double) * (size_t)T * E);
  double* o = (double*)malloc(sizeof(double) * d);
  int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * K);
  double* w = (double*)malloc(sizeof(double) * K);
  oracle_router_logits(L, x, T, logits);
  for (int t = 0; t < T; ++t) {
    const double* lt = logits + (size_t)t * E;
    double margin = INFINITY;
    if (forced) {
      for (int k = 0; k < K; ++k) ids[k] = forced[(size_t)t * K + k];
      oracle_weights_for_set(lt, ids, K, w);
    } else {
      oracle_select_one(lt, E, K, ids, w, &margin);
    }
    double* yt = y + (size_t)t * d;
    for (int c = 0; c < d; ++c) yt[c] = 0.0;
    if (L->fs > 0) {
      oracle_expert(L, -1, x + (size_t)t * d, o);
      for (int c = 0; c < d; ++c) yt[c] += o[c];
    }
    for (int k = 0; k < K; ++k) {
      oracle_expert(L, ids[k], x + (size_t)t * d, o);
      for (int c = 0; c < d; ++c) yt[c] += w[k] * o[c];
    }
    if (ids_out)
      for (int k = 0; k < K; ++k) ids_out[(size_t)t * K + k] = ids[k];
    if (w_out)
      for (int k = 0; k < K; ++k) w_out[(size_t)t * K + k] = w[k];
    if (margin_out) margin_out[t] = margin;
  }
  free(w);
  free(ids);
  free(o);
  free(logits);
  return 0;
}

/* ---- token -> expert grouping (prefill) --------------------------------- */

/* Stable grouping of the T*K (token, slot) pairs by expert: pairs of expert e
 * occupy perm[offsets[e] .. offsets[e+1]) in ascending token order; perm holds
 * t*K + k, and inv[t*K + k] is that pair's position in perm. */
void oracle_sort(const int32_t* ids, int T, int K, int E, int32_t* counts, int32_t* offsets, int32_t* perm,
                 int32_t* inv) {
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int i = 0; i < T * K; ++i) counts[ids[i]]++;
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int pos = 0;
  for (int e = 0; e < E; ++e)
    for (int t = 0; t < T; ++t)
      for (int k = 0; k < K; ++k)
        if (ids[t * K + k] == e) {
          perm[pos] = t * K + k;
          inv[t * K + k] = pos;
          ++pos;
        }
}

/* ---- stack glue --------------------------------------------------------- */

/* n = bf16(h / sqrt(mean(h^2) + eps)) with unit gain */
void oracle_rmsnorm_bf16(const uint16_t* h, int d, double eps, uint16_t* n_out) {
  double ss = 0.0;
  for (int c = 0; c < d; ++c) {
    double v = oracle_bf16_to_f64(h[c]);
    ss += v * v;
  }
  double inv = 1.0 / sqrt(ss / d + eps);
  for (int c = 0; c < d; ++c) n_out[c] = oracle_f64_to_bf16(oracle_bf16_to_f64(h[c]) * inv);
}

/* h_out = bf16(h + y) */
void oracle_residual_bf16(const uint16_t* h, const double* y, int d, uint16_t* h_out) {
  for (int c = 0; c < d; ++c) h_out[c] = oracle_f64_to_bf16(oracle_bf16_to_f64(h[c]) + y[c]);
}

/* One stack step through n_layers layers for one token:
 * h <- bf16(h + MoE_l(bf16(rmsnorm(h)))) for l = 0..n_layers-1.
 * forced (nullable): [n_layers][K] expert sets (row of -1s = route normally). */
int oracle_stack_step(const oracle_layer* layers, int n_layers, double eps, uint16_t* h, const int32_t* forced,
                      int32_t* ids_out) {
  int d = layers[0].d;
  uint16_t* n = (uint16_t*)malloc(sizeof(uint16_t) * d);
  double* xn = (double*)malloc(sizeof(double) * d);
  double* y = (double*)malloc(sizeof(double) * d);
  int rc = 0;
  for (int l = 0; l < n_layers && rc == 0; ++l) {
    const oracle_layer* L = &layers[l];
    oracle_rmsnorm_bf16(h, d, eps, n);
    for (int c = 0; c < d; ++c) xn[c] = oracle_bf16_to_f64(n[c]);
    const int32_t* fl = NULL;
    if (forced && forced[(size_t)l * L->K] >= 0) fl = forced + (size_t)l * L->K;
    rc = oracle_layer_forward(L, xn, 1, fl, y, ids_out ? ids_out + (size_t)l * L->K : NULL, NULL, NULL);
    oracle_residual_bf16(h, y, d, h);
  }
  free(y);
  free(xn);
  free(n);
  return rc;
}
