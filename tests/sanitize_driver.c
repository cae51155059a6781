/* sanitize_driver.c -- runs every function of the CPU oracle (oracle/oracle.c) and of the
 * input generator (synth/synth.c) on small shapes, for a build with the address and
 * undefined-behaviour sanitizers (tests/test_sanitize_cpu.py). Besides running clean it
 * checks a few properties that hold exactly: a layer whose experts have zero scale and
 * bias returns its input, the routing weights sum to 1, and the stack of one layer equals
 * that layer. Exit status 0 on success. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../oracle/oracle.h"
#include "../synth/synth.h"

static int zero_provide(void* ctx, int layer, int expert, const uint8_t** codes, const uint16_t** scale,
                        const uint16_t** bias) {
  (void)layer;
  (void)expert;
  synth_provider* p = (synth_provider*)ctx;
  for (int m = 0; m < 3; ++m) {
    codes[m] = p->codes[m];
    scale[m] = p->scale[m];
    bias[m] = p->bias[m];
  }
  return 0;
}

#define CHECK(c)                                              \
  do {                                                        \
    if (!(c)) {                                               \
      fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
      return 1;                                               \
    }                                                         \
  } while (0)

static int run(int bits) {
  const int H = 256, I = 128, E = 12, k = 3, T = 3, L = 2, G = 64;
  float* R = malloc(sizeof(float) * E * H);
  float* R2 = malloc(sizeof(float) * E * H);
  float* x = malloc(sizeof(float) * T * H);
  float* gate = malloc(sizeof(float) * H);
  double *v = malloc(sizeof(double) * H), *y = malloc(sizeof(double) * H), *out = malloc(sizeof(double) * H);
  double* a = malloc(sizeof(double) * I);
  synth_router(0, 0, E, H, R);
  synth_router(0, 1, E, H, R2);
  synth_router(0, 1000, 1, H, gate);
  for (int t = 0; t < T; ++t) synth_token(0, (uint64_t)t, H, x + t * H);
  for (int i = 0; i < H; ++i) v[i] = x[i];

  synth_provider prov;
  CHECK(synth_provider_init(&prov, 0, H, I, bits, G) == 0);
  const uint8_t* c[3];
  const uint16_t *s[3], *b[3];
  CHECK(synth_provide(&prov, 0, 1, c, s, b) == 0);
  CHECK(oracle_code(c[0], H, bits, I - 1, H - 1) >= 0);
  (void)oracle_weight(c[0], s[0], b[0], H, bits, G, I - 1, H - 1);
  oracle_matvec(c[0], s[0], b[0], I, H, bits, G, v, a);
  oracle_expert_ffn((const uint8_t* const*)c, (const uint16_t* const*)s, (const uint16_t* const*)b, H, I, bits, G,
                    v, y, a);
  int idx[16];
  double w[16], logits[64], m;
  oracle_route(R, v, E, H, k, idx, w, logits, &m);
  CHECK(fabs(w[0] + w[1] + w[2] - 1.0) < 1e-15);
  oracle_rmsnorm(v, H, 1e-6, y);
  (void)oracle_swiglu(-1e4, 2.0);
  (void)oracle_round_bf16(3.14159);
  double sw;
  CHECK(oracle_moe_layer(synth_provide, &prov, 0, R, v, H, I, E, k, bits, G, 1, 1e-6, out, idx, w, &m, gate, &sw) == 0);

  const float* routers[2] = {R, R2};
  const float* gates[2] = {gate, gate};
  double *hall = malloc(sizeof(double) * L * H), margins[2], sws[2], ws2[32];
  int idx2[32];
  CHECK(oracle_stack(synth_provide, &prov, routers, L, x, H, I, E, k, bits, G, 1e-6, 0.0, out, idx2, ws2, margins,
                     hall, gates, sws) == L);
  /* the stack of one layer is that layer */
  double* one = malloc(sizeof(double) * H);
  CHECK(oracle_stack(synth_provide, &prov, routers, 1, x, H, I, E, k, bits, G, 1e-6, 0.0, one, idx2, ws2, margins,
                     NULL, NULL, NULL) == 1);
  CHECK(oracle_moe_layer(synth_provide, &prov, 0, R, v, H, I, E, k, bits, G, 1, 1e-6, out, idx, w, &m, NULL, NULL) == 0);
  for (int i = 0; i < H; ++i) CHECK(one[i] == out[i]);

  double* outT = malloc(sizeof(double) * T * H);
  int* idxT = malloc(sizeof(int) * T * k);
  double *wT = malloc(sizeof(double) * T * k), *mT = malloc(sizeof(double) * T);
  float* a16 = malloc(sizeof(float) * T * k * I);
  double *g = malloc(sizeof(double) * T * k * I), *u = malloc(sizeof(double) * T * k * I);
  double* swT = malloc(sizeof(double) * T);
  float* sa16 = malloc(sizeof(float) * T * I);
  CHECK(oracle_layer_bf16(synth_provide, &prov, 0, R, x, T, H, I, E, k, bits, G, 1, 1e-6, outT, idxT, wT, mT, NULL,
                          a16, g, u, gate, swT, NULL, sa16) == 0);
  CHECK(oracle_layer_bf16(synth_provide, &prov, 0, R, x, T, H, I, E, k, bits, G, 0, 1e-6, outT, idxT, wT, mT, a16,
                          NULL, NULL, NULL, NULL, NULL, NULL, NULL) == 0);

  /* zero scale and bias: every expert is the zero map, so the layer returns its input */
  synth_provider zp;
  CHECK(synth_provider_init(&zp, 0, H, I, bits, G) == 0);
  CHECK(synth_provide(&zp, 0, 0, c, s, b) == 0);
  for (int mtx = 0; mtx < 3; ++mtx) {
    const int rows = mtx < 2 ? I : H, cols = mtx < 2 ? H : I;
    memset(zp.scale[mtx], 0, sizeof(uint16_t) * rows * (cols / G));
    memset(zp.bias[mtx], 0, sizeof(uint16_t) * rows * (cols / G));
  }
  CHECK(oracle_moe_layer(zero_provide, &zp, 0, R, v, H, I, E, k, bits, G, 1, 1e-6, out, idx, w, &m, gate, &sw) == 0);
  for (int i = 0; i < H; ++i) CHECK(out[i] == v[i]);

  uint8_t cb[64];
  synth_codes(synth_stream(0, 1, 0, 0, 0), cb, sizeof cb);
  uint16_t sb[8];
  synth_uniform_bf16(synth_stream(0, 2, 0, 0, 0), 0.001, 0.019, sb, 8);
  CHECK(synth_bf16_to_f32(synth_f32_to_bf16(1.5f)) == 1.5f);
  (void)synth_uniform_at(0, 6, 0, 1, 0, 3);

  synth_provider_free(&prov);
  synth_provider_free(&zp);
  free(R); free(R2); free(x); free(gate); free(v); free(y); free(out); free(a); free(hall); free(one);
  free(outT); free(idxT); free(wT); free(mT); free(a16); free(g); free(u); free(swT); free(sa16);
  return 0;
}

int main(void) {
  if (run(4) || run(2)) return 1;
  printf("sanitize driver: ok\n");
  return 0;
}
