/*
 * oracle.c -- plain fp64 CPU reference of the per-token MoE expert block.
 * TEST INFRASTRUCTURE ONLY (see oracle.h). Shares no code with the fmoe library.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

int oracle_code(const uint8_t* codes, int cols, int bits, int r, int c) {
  size_t row_bytes = (size_t)cols * (size_t)bits / 8;
  const uint8_t* row = codes + (size_t)r * row_bytes;
  if (bits == 4) {
    uint8_t byte = row[c / 2];
    return (c % 2 == 0) ? (byte & 0x0f) : (byte >> 4);
  }
  if (bits == 3) {
    /* 8 columns per 3 bytes: column 8j+t is bits 3t..3t+2 of the little-endian 24-bit
     * word of bytes 3j..3j+2 */
    const uint8_t* p = row + 3 * (size_t)(c / 8);
    uint32_t w = (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16);
    return (int)((w >> (3 * (c % 8))) & 0x07u);
  }
  /* bits == 2 */
  uint8_t byte = row[c / 4];
  return (byte >> (2 * (c % 4))) & 0x03;
}

double oracle_bf16(uint16_t b) {
  uint32_t bits = (uint32_t)b << 16;
  float f;
  memcpy(&f, &bits, 4);
  return (double)f;
}

double oracle_weight(const uint8_t* codes, const uint16_t* scale, const uint16_t* bias, int cols,
                     int bits, int group, int r, int c) {
  int q = oracle_code(codes, cols, bits, r, c);
  size_t g = (size_t)r * (size_t)(cols / group) + (size_t)(c / group);
  /* q*s+b is exact in fp64: q has at most 4 bits, s and b have 8 significant bits. */
  return (double)q * oracle_bf16(scale[g]) + oracle_bf16(bias[g]);
}

void oracle_matvec(const uint8_t* codes, const uint16_t* scale, const uint16_t* bias, int rows, int cols,
                   int bits, int group, const double* x, double* y) {
#pragma omp parallel for schedule(static)
  for (int r = 0; r < rows; ++r) {
    double acc = 0.0;
    for (int c = 0; c < cols; ++c) acc += oracle_weight(codes, scale, bias, cols, bits, group, r, c) * x[c];
    y[r] = acc;
  }
}

/* a ranks before b: larger logit first, lower index on equal logits, NaN last. */
static int ranks_before(double la, int ia, double lb, int ib) {
  int na = isnan(la), nb = isnan(lb);
  if (na != nb) return nb;
  if (na && nb) return ia < ib;
  if (la != lb) return la > lb;
  return ia < ib;
}

void oracle_route(const float* router, const double* v, int n_experts, int hidden, int k, int* idx,
                  double* w, double* logits, double* margin) {
  if (k < 1 || k > 16 || k > n_experts) {
    for (int j = 0; j < k && j < 16; ++j) {
      idx[j] = -1;
      w[j] = 0.0;
    }
    if (margin) *margin = NAN;
    return;
  }
  double* l = (double*)malloc(sizeof(double) * (size_t)n_experts);
  char* taken = (char*)calloc((size_t)n_experts, 1);
#pragma omp parallel for schedule(static)
  for (int e = 0; e < n_experts; ++e) {
    double acc = 0.0;
    for (int i = 0; i < hidden; ++i) acc += (double)router[(size_t)e * hidden + i] * v[i];
    l[e] = acc;
  }
  /* selection of the first k+1 in rank order (k+1 only for the margin) */
  int nsel = (k < n_experts) ? k + 1 : k;
  int order[17];
  double ord_l[17];
  for (int j = 0; j < nsel; ++j) {
    int best = -1;
    for (int e = 0; e < n_experts; ++e) {
      if (taken[e]) continue;
      if (best < 0 || ranks_before(l[e], e, l[best], best)) best = e;
    }
    taken[best] = 1;
    order[j] = best;
    ord_l[j] = l[best];
  }
  /* softmax over the selected logits, shifted by the largest */
  double denom = 0.0;
  for (int j = 0; j < k; ++j) denom += exp(ord_l[j] - ord_l[0]);
  for (int j = 0; j < k; ++j) {
    idx[j] = order[j];
    w[j] = exp(ord_l[j] - ord_l[0]) / denom;
  }
  if (margin) {
    double m = INFINITY;
    for (int j = 0; j + 1 < nsel; ++j) {
      double gap = ord_l[j] - ord_l[j + 1];
      if (gap < m) m = gap;
    }
    *margin = m;
  }
  if (logits)
    for (int e = 0; e < n_experts; ++e) logits[e] = l[e];
  free(l);
  free(taken);
}

void oracle_rmsnorm(const double* h, int n, double eps, double* v) {
  double ss = 0.0;
  for (int i = 0; i < n; ++i) ss += h[i] * h[i];
  double inv = 1.0 / sqrt(ss / n + eps);
  for (int i = 0; i < n; ++i) v[i] = h[i] * inv;
}

double oracle_swiglu(double g, double u) { return g / (1.0 + exp(-g)) * u; }

void oracle_expert_ffn(const uint8_t* const* codes, const uint16_t* const* scale,
                       const uint16_t* const* bias, int hidden, int inter, int bits, int group,
                       const double* x, double* y, double* a_out) {
  double* g = (double*)malloc(sizeof(double) * (size_t)inter);
  double* u = (double*)malloc(sizeof(double) * (size_t)inter);
  double* a = (double*)malloc(sizeof(double) * (size_t)inter);
  oracle_matvec(codes[0], scale[0], bias[0], inter, hidden, bits, group, x, g);
  oracle_matvec(codes[1], scale[1], bias[1], inter, hidden, bits, group, x, u);
  for (int j = 0; j < inter; ++j) a[j] = oracle_swiglu(g[j], u[j]);
  oracle_matvec(codes[2], scale[2], bias[2], hidden, inter, bits, group, a, y);
  if (a_out) memcpy(a_out, a, sizeof(double) * (size_t)inter);
  free(g);
  free(u);
  free(a);
}

/* Weight of the shared expert: the logistic function of the gate vector's dot product with
 * v (reading of [hada] "Model mimarisi", one shared expert per layer, and "Metal Compute
 * Shaders", a gate in the combine; the gate's form is not on the pages). */
static double shared_weight(const float* gate, const double* v, int hidden) {
  double z = 0.0;
  for (int i = 0; i < hidden; ++i) z += (double)gate[i] * v[i];
  return 1.0 / (1.0 + exp(-z));
}

int oracle_moe_layer(oracle_provider_fn provide, void* ctx, int layer, const float* router,
                     const double* h, int hidden, int inter, int n_experts, int k, int bits, int group,
                     int prenorm, double eps, double* out, int* idx, double* w, double* margin,
                     const float* shared_gate, double* shared_w) {
  double* v = (double*)malloc(sizeof(double) * (size_t)hidden);
  double* y = (double*)malloc(sizeof(double) * (size_t)hidden);
  double* acc = (double*)calloc((size_t)hidden, sizeof(double));
  if (prenorm)
    oracle_rmsnorm(h, hidden, eps, v);
  else
    memcpy(v, h, sizeof(double) * (size_t)hidden);
  oracle_route(router, v, n_experts, hidden, k, idx, w, NULL, margin);
  int rc = 0;
  for (int j = 0; j < k; ++j) {
    const uint8_t* codes[3];
    const uint16_t* scale[3];
    const uint16_t* bias[3];
    if (provide(ctx, layer, idx[j], codes, scale, bias) != 0) {
      rc = -1;
      break;
    }
    oracle_expert_ffn(codes, scale, bias, hidden, inter, bits, group, v, y, NULL);
    for (int i = 0; i < hidden; ++i) acc[i] += w[j] * y[i];
  }
  if (rc == 0 && shared_gate) {
    /* the shared expert (provider index n_experts) on every token, weighted by its gate */
    const uint8_t* codes[3];
    const uint16_t* scale[3];
    const uint16_t* bias[3];
    if (provide(ctx, layer, n_experts, codes, scale, bias) != 0) {
      rc = -1;
    } else {
      const double sw = shared_weight(shared_gate, v, hidden);
      if (shared_w) *shared_w = sw;
      oracle_expert_ffn(codes, scale, bias, hidden, inter, bits, group, v, y, NULL);
      for (int i = 0; i < hidden; ++i) acc[i] += sw * y[i];
    }
  }
  for (int i = 0; i < hidden; ++i) out[i] = h[i] + acc[i];
  free(v);
  free(y);
  free(acc);
  return rc;
}

int oracle_stack(oracle_provider_fn provide, void* ctx, const float* const* routers, int n_layers,
                 const float* x, int hidden, int inter, int n_experts, int k, int bits, int group, double eps,
                 double stop_margin, double* out, int* idx, double* w, double* margins, double* h_all,
                 const float* const* shared_gates, double* shared_ws) {
  double* h = (double*)malloc(sizeof(double) * (size_t)hidden);
  double* hn = (double*)malloc(sizeof(double) * (size_t)hidden);
  for (int i = 0; i < hidden; ++i) h[i] = (double)x[i];
  int done = 0;
  for (int l = 0; l < n_layers; ++l) {
    double m;
    int rc = oracle_moe_layer(provide, ctx, l, routers[l], h, hidden, inter, n_experts, k, bits, group, 1, eps,
                              hn, idx + (size_t)l * k, w + (size_t)l * k, &m, shared_gates ? shared_gates[l] : NULL,
                              shared_ws ? shared_ws + l : NULL);
    if (rc != 0) {
      free(h);
      free(hn);
      return -1;
    }
    if (margins) margins[l] = m;
    memcpy(h, hn, sizeof(double) * (size_t)hidden);
    if (h_all) memcpy(h_all + (size_t)l * hidden, h, sizeof(double) * (size_t)hidden);
    done = l + 1;
    if (stop_margin > 0.0 && m < stop_margin) break;
  }
  memcpy(out, h, sizeof(double) * (size_t)hidden);
  free(h);
  free(hn);
  return done;
}

double oracle_round_bf16(double v) {
  float f = (float)v; /* round to nearest even fp32 */
  uint32_t bits;
  memcpy(&bits, &f, 4);
  if ((bits & 0x7f800000u) == 0x7f800000u) return (double)f;
  uint32_t rounding = ((bits >> 16) & 1u) + 0x7fffu;
  bits = ((bits + rounding) >> 16) << 16;
  memcpy(&f, &bits, 4);
  return (double)f;
}

/* bf16 sum of w16 * x16 along one row, products and sum in fp64. */
/* One row of exact weights against a bf16-rounded vector, summed in fp64. */
static double row_dot_x16(const uint8_t* codes, const uint16_t* scale, const uint16_t* bias, int cols, int bits,
                          int group, int r, const double* x16) {
  double acc = 0.0;
  for (int c = 0; c < cols; ++c) acc += oracle_weight(codes, scale, bias, cols, bits, group, r, c) * x16[c];
  return acc;
}

int oracle_layer_bf16(oracle_provider_fn provide, void* ctx, int layer, const float* router, const float* x,
                      int T, int hidden, int inter, int n_experts, int k, int bits, int group, int prenorm,
                      double eps, double* out, int* idx, double* w, double* margins, const float* a16_force,
                      float* a16_out, double* g_out, double* u_out, const float* shared_gate, double* shared_w,
                      const float* shared_a16_force, float* shared_a16_out) {
  double* xv = (double*)malloc(sizeof(double) * (size_t)hidden);
  double* vv = (double*)malloc(sizeof(double) * (size_t)hidden);
  double* x16 = (double*)malloc(sizeof(double) * (size_t)T * hidden);
  double* ys = (double*)malloc(sizeof(double) * (size_t)T * k * hidden);
  double* sws = (double*)malloc(sizeof(double) * (size_t)T);
  double* yshared = shared_gate ? (double*)malloc(sizeof(double) * (size_t)T * hidden) : NULL;
  int rc = 0;
  /* v = rmsnorm(x) or x; routing on v; the experts see v rounded to bf16 */
  for (int t = 0; t < T; ++t) {
    for (int i = 0; i < hidden; ++i) xv[i] = (double)x[(size_t)t * hidden + i];
    if (prenorm) oracle_rmsnorm(xv, hidden, eps, vv);
    else memcpy(vv, xv, sizeof(double) * (size_t)hidden);
    for (int i = 0; i < hidden; ++i) x16[(size_t)t * hidden + i] = oracle_round_bf16(vv[i]);
    double m;
    oracle_route(router, vv, n_experts, hidden, k, idx + (size_t)t * k, w + (size_t)t * k, NULL, &m);
    if (margins) margins[t] = m;
    sws[t] = shared_gate ? shared_weight(shared_gate, vv, hidden) : 0.0;
    if (shared_w) shared_w[t] = sws[t];
  }
  /* every (token, slot) FFN; experts fetched once each (independent computations) */
  double* a16 = (double*)malloc(sizeof(double) * (size_t)inter);
  for (int e = 0; e < n_experts && rc == 0; ++e) {
    int used = 0;
    for (int s = 0; s < T * k; ++s) used |= (idx[s] == e);
    if (!used) continue;
    const uint8_t* codes[3];
    const uint16_t* scale[3];
    const uint16_t* bias[3];
    if (provide(ctx, layer, e, codes, scale, bias) != 0) {
      rc = -1;
      break;
    }
    for (int s = 0; s < T * k; ++s) {
      if (idx[s] != e) continue;
      int t = s / k;
      const double* xt = x16 + (size_t)t * hidden;
#pragma omp parallel for schedule(static)
      for (int j = 0; j < inter; ++j) {
        double g = row_dot_x16(codes[0], scale[0], bias[0], hidden, bits, group, j, xt);
        double u = row_dot_x16(codes[1], scale[1], bias[1], hidden, bits, group, j, xt);
        if (g_out) g_out[(size_t)s * inter + j] = g;
        if (u_out) u_out[(size_t)s * inter + j] = u;
        double a = oracle_swiglu(g, u);
        double r16 = oracle_round_bf16(a);
        if (a16_out) a16_out[(size_t)s * inter + j] = (float)r16;
        a16[j] = a16_force ? (double)a16_force[(size_t)s * inter + j] : r16;
      }
#pragma omp parallel for schedule(static)
      for (int i = 0; i < hidden; ++i)
        ys[(size_t)s * hidden + i] = row_dot_x16(codes[2], scale[2], bias[2], inter, bits, group, i, a16);
    }
  }
  /* the shared expert on every token under the same contract */
  if (rc == 0 && shared_gate) {
    const uint8_t* codes[3];
    const uint16_t* scale[3];
    const uint16_t* bias[3];
    if (provide(ctx, layer, n_experts, codes, scale, bias) != 0) rc = -1;
    for (int t = 0; t < T && rc == 0; ++t) {
      const double* xt = x16 + (size_t)t * hidden;
#pragma omp parallel for schedule(static)
      for (int j = 0; j < inter; ++j) {
        double g = row_dot_x16(codes[0], scale[0], bias[0], hidden, bits, group, j, xt);
        double u = row_dot_x16(codes[1], scale[1], bias[1], hidden, bits, group, j, xt);
        double r16 = oracle_round_bf16(oracle_swiglu(g, u));
        if (shared_a16_out) shared_a16_out[(size_t)t * inter + j] = (float)r16;
        a16[j] = shared_a16_force ? (double)shared_a16_force[(size_t)t * inter + j] : r16;
      }
#pragma omp parallel for schedule(static)
      for (int i = 0; i < hidden; ++i)
        yshared[(size_t)t * hidden + i] = row_dot_x16(codes[2], scale[2], bias[2], inter, bits, group, i, a16);
    }
  }
  /* combine + residual per token, slots in rank order, the shared expert last */
  if (rc == 0) {
    for (int t = 0; t < T; ++t) {
      for (int i = 0; i < hidden; ++i) {
        double acc = 0.0;
        for (int j = 0; j < k; ++j) acc += w[(size_t)t * k + j] * ys[((size_t)t * k + j) * hidden + i];
        if (yshared) acc += sws[t] * yshared[(size_t)t * hidden + i];
        out[(size_t)t * hidden + i] = (double)x[(size_t)t * hidden + i] + acc;
      }
    }
  }
  free(sws);
  free(yshared);
  free(a16);
  free(xv);
  free(vv);
  free(x16);
  free(ys);
  return rc;
}
