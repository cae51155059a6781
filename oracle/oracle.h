/*
 * oracle.h -- plain CPU reference of the per-token MoE expert block (test infrastructure).
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load this library. The product path (the fmoe C-ABI library)
 * never links, loads or calls it, and it shares no code with that library: it reads
 * only the canonical layout produced by the synthetic-input module (synth.h).
 *
 * Everything is accumulated in fp64 with plain loops; OpenMP splits only independent
 * output rows. Sources (web pages about the Flash-MoE engine):
 *   [aibit]   aibit.im, "397B MoE sur MacBook : 4,4 t/s Moteur Flash-MoE"
 *   [hada]    tr.news.hada.io topic 27758, "Flash-MoE - Dizustunde 397 milyar parametreli
 *             modeli calistirma"
 *   [radar]   openclawradar.com, "Autoresearch pousse Qwen3.5-397B a 20,34 tok/s sur M5 Max
 *             via le streaming SSD"
 *   [veille]  grafana.dev.probatiovault.com veille note on Flash-MoE ("Metal pur")
 * Each function names the passage it follows. Where the pages are silent the reading
 * used is stated at the function.
 */
#ifndef FMOE_ORACLE_H
#define FMOE_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Expert provider: fills codes/scale/bias pointers for matrices gate(0), up(1), down(2)
 * of expert `expert` in layer `layer`, canonical layout. Pointers stay valid until the
 * next call. Returns 0 on success. */
typedef int (*oracle_provider_fn)(void* ctx, int layer, int expert, const uint8_t** codes,
                                  const uint16_t** scale, const uint16_t** bias);

/* Code q[r][c] from the canonical layout: each row is a little-endian bit stream in which
 * column c occupies bits bits*c .. bits*c + bits - 1. 4-bit: element 2c low nibble; 2-bit:
 * element 4c+t in bits 2t..2t+1; 3-bit (openclawradar.com "Optimisations efficaces": 3-bit
 * experts, 23% smaller than 4-bit): 8 columns per 3 bytes, column 8j+t in bits 3t..3t+2 of
 * the little-endian 24-bit word of bytes 3j..3j+2. */
int oracle_code(const uint8_t* codes, int cols, int bits, int r, int c);

/* bf16 bit pattern -> value (exact widening). */
double oracle_bf16(uint16_t b);

/* O1: dequantized weight q*s+b of group floor(c/group) ([aibit] "Techniques de rupture"
 * item 2 and [hada] "FMA optimize dequant cekirdegi": the affine form nibble*scale+bias). */
double oracle_weight(const uint8_t* codes, const uint16_t* scale, const uint16_t* bias, int cols,
                     int bits, int group, int r, int c);

/* O2: y[r] = sum_c (q*s+b) * x[c], fp64 ([aibit] item 4: the 4-/2-bit dequantized matvec). */
void oracle_matvec(const uint8_t* codes, const uint16_t* scale, const uint16_t* bias, int rows, int cols,
                   int bits, int group, const double* x, double* y);

/* O3: router logits l = R v (fp64), top-k by (logit desc, index asc; NaN last), softmax
 * over the k selected logits, and the margin min_{j<k} (l_(j) - l_(j+1)) over the first
 * k+1 ordered logits (+inf if n_experts == k == 1). [aibit] item 1 and [hada] "Model
 * mimarisi": k = 4 of 512 experts chosen per token per layer; the router itself is the
 * engine's CPU routing step ([aibit] item 3). logits and margin may be NULL. */
void oracle_route(const float* router, const double* v, int n_experts, int hidden, int k, int* idx,
                  double* w, double* logits, double* margin);

/* RMSNorm without a learned weight: v = h / sqrt(mean(h^2) + eps) ([aibit] item 4 lists
 * an RMS norm kernel; the form and eps are the plainest reading). */
void oracle_rmsnorm(const double* h, int n, double eps, double* v);

/* silu(z) * u with silu(z) = z / (1 + exp(-z)) ([aibit] item 4: fused SwiGLU). */
double oracle_swiglu(double g, double u);

/* O4: y = Wd (silu(Wg x) * (Wu x)). codes/scale/bias: [3] arrays (gate, up, down);
 * gate/up are [inter][hidden], down is [hidden][inter]. a_out (nullable) gets the SwiGLU
 * vector [inter]. */
void oracle_expert_ffn(const uint8_t* const* codes, const uint16_t* const* scale,
                       const uint16_t* const* bias, int hidden, int inter, int bits, int group,
                       const double* x, double* y, double* a_out);

/* O5: one MoE layer for one token: v = prenorm ? rmsnorm(h) : h; route on v; out = h +
 * sum_k w_k FFN_{idx_k}(v) ([aibit] item 3 / [hada] "Deferred GPU Expert Compute": the
 * combine + residual (+ norm for the next layer) step). idx, w: [k]; margin nullable.
 * shared_gate (nullable, fp32 [hidden]): the layer also has a shared expert (provider index
 * n_experts) that every token runs, added with weight s = 1 / (1 + exp(-gate . v)) (reading
 * of [hada] "Model mimarisi": one shared expert, and "Metal Compute Shaders": a gate in the
 * combine); shared_w (nullable) receives s. O6 and O7 take the same per layer. */
int oracle_moe_layer(oracle_provider_fn provide, void* ctx, int layer, const float* router,
                     const double* h, int hidden, int inter, int n_experts, int k, int bits, int group,
                     int prenorm, double eps, double* out, int* idx, double* w, double* margin,
                     const float* shared_gate, double* shared_w);

/* O6: n_layers layers applied in order to x, pre-normed ([hada] "Model mimarisi": 60
 * layers). routers[l] is layer l's router. idx/w: [n_layers][k]; margins: [n_layers];
 * h_all (nullable): [n_layers][hidden] = output of every layer. out = last layer output.
 * stop_margin > 0 stops early (returning the number of layers done) at the first layer
 * whose margin is below it; otherwise returns n_layers. Negative on provider error. */
int oracle_stack(oracle_provider_fn provide, void* ctx, const float* const* routers, int n_layers,
                 const float* x, int hidden, int inter, int n_experts, int k, int bits, int group, double eps,
                 double stop_margin, double* out, int* idx, double* w, double* margins, double* h_all,
                 const float* const* shared_gates, double* shared_ws);

/* Round-to-nearest-even fp64 -> fp32 -> bf16 value (as double). */
double oracle_round_bf16(double v);

/* O7: the batched bf16 contract for one layer over T tokens:
 *   v = rmsnorm(x) (prenorm != 0) or x, in fp64; routing is O3 on v;
 *   x16 = bf16(fp32(v)); weights exact (q*s+b); gate/up sums of w*x16 in fp64;
 *   a = silu(g)*u in fp64, a16 = bf16(fp32(a)); down sums of w*a16 in fp64;
 *   out = x + sum_k w_k y_k in fp64.
 * Only the two activation vectors are rounded to bf16: the codes are small integers and
 * the affine terms apply per group, so the weights themselves need no rounding.
 * x: [T][hidden]. out: [T][hidden]. idx, w: [T][k]. margins: [T] (nullable).
 * a16_force (nullable) [T][k][inter]: use these a16 values instead of the oracle's own
 * (teacher forcing of the down stage). a16_out (nullable) [T][k][inter]: the oracle's a16.
 * g_out/u_out (nullable) [T][k][inter]: gate/up sums. */
int oracle_layer_bf16(oracle_provider_fn provide, void* ctx, int layer, const float* router, const float* x,
                      int T, int hidden, int inter, int n_experts, int k, int bits, int group, int prenorm,
                      double eps, double* out, int* idx, double* w, double* margins, const float* a16_force,
                      float* a16_out, double* g_out, double* u_out, const float* shared_gate, double* shared_w,
                      const float* shared_a16_force, float* shared_a16_out);

#ifdef __cplusplus
}
#endif
#endif
