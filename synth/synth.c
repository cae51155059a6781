/* synth.c -- CPU side of the counter-based synthetic input generator (see synth.h). */
#include "synth.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

uint64_t synth_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}

uint64_t synth_stream(uint64_t seed, uint32_t tag, uint32_t layer, uint32_t expert, uint32_t matrix) {
  uint64_t s = synth_mix64(seed + SYNTH_GAMMA);
  s = synth_mix64(s + ((uint64_t)tag + 1) * SYNTH_GAMMA);
  s = synth_mix64(s + ((uint64_t)layer + 1) * SYNTH_GAMMA);
  s = synth_mix64(s + ((uint64_t)expert + 1) * SYNTH_GAMMA);
  s = synth_mix64(s + ((uint64_t)matrix + 1) * SYNTH_GAMMA);
  return s;
}

uint64_t synth_hash(uint64_t stream, uint64_t idx) { return synth_mix64(stream + (idx + 1) * SYNTH_GAMMA); }

double synth_u01(uint64_t hash) { return (double)(hash >> 40) * (1.0 / 16777216.0); }

uint16_t synth_f32_to_bf16(float f) {
  uint32_t bits;
  memcpy(&bits, &f, 4);
  if ((bits & 0x7f800000u) == 0x7f800000u && (bits & 0x007fffffu)) return (uint16_t)((bits >> 16) | 0x40u);
  uint32_t rounding = ((bits >> 16) & 1u) + 0x7fffu;
  return (uint16_t)((bits + rounding) >> 16);
}

float synth_bf16_to_f32(uint16_t b) {
  uint32_t bits = (uint32_t)b << 16;
  float f;
  memcpy(&f, &bits, 4);
  return f;
}

void synth_codes(uint64_t stream, uint8_t* out, size_t nbytes) {
  size_t nw = nbytes / 8;
#pragma omp parallel for schedule(static) if (nw > 65536)
  for (long long w = 0; w < (long long)nw; ++w) {
    uint64_t h = synth_hash(stream, (uint64_t)w);
    for (int j = 0; j < 8; ++j) out[8 * w + j] = (uint8_t)(h >> (8 * j));
  }
}

void synth_uniform_bf16(uint64_t stream, double lo, double width, uint16_t* out, size_t n) {
#pragma omp parallel for schedule(static) if (n > 65536)
  for (long long i = 0; i < (long long)n; ++i) {
    double u = synth_u01(synth_hash(stream, (uint64_t)i));
    volatile double t = width * u; /* one rounding for the product ... */
    double v = lo + t;             /* ... and one for the sum */
    out[i] = synth_f32_to_bf16((float)v);
  }
}

void synth_normal_f32(uint64_t stream, double sigma, float* out, size_t n) {
  const double two_pi = 6.283185307179586476925286766559;
#pragma omp parallel for schedule(static) if (n > 16384)
  for (long long i = 0; i < (long long)n; ++i) {
    uint64_t h = synth_hash(stream, (uint64_t)i);
    double u1 = ((double)(h >> 40) + 1.0) * (1.0 / 16777216.0);
    double u2 = (double)((h >> 16) & 0xffffffull) * (1.0 / 16777216.0);
    double z = sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
    out[i] = (float)(sigma * z);
  }
}

void synth_matrix(uint64_t seed, int layer, int expert, int matrix, int rows, int cols, int bits,
                  int group, uint8_t* codes, uint16_t* scale, uint16_t* bias) {
  size_t ncode = (size_t)rows * (size_t)cols * (size_t)bits / 8;
  size_t ngrp = (size_t)rows * (size_t)(cols / group);
  if (codes) synth_codes(synth_stream(seed, SYNTH_TAG_CODES, layer, expert, matrix), codes, ncode);
  if (scale)
    synth_uniform_bf16(synth_stream(seed, SYNTH_TAG_SCALE, layer, expert, matrix), SYNTH_SCALE_LO,
                       SYNTH_SCALE_WIDTH, scale, ngrp);
  if (bias)
    synth_uniform_bf16(synth_stream(seed, SYNTH_TAG_BIAS, layer, expert, matrix), SYNTH_BIAS_LO,
                       SYNTH_BIAS_WIDTH, bias, ngrp);
}

void synth_router(uint64_t seed, int layer, int n_experts, int hidden, float* out) {
  synth_normal_f32(synth_stream(seed, SYNTH_TAG_ROUTER, layer, 0, 0), SYNTH_ROUTER_SIGMA, out,
                   (size_t)n_experts * (size_t)hidden);
}

void synth_token(uint64_t seed, uint64_t draw, int hidden, float* out) {
  /* the draw index is split over two 32-bit coordinates */
  synth_normal_f32(synth_stream(seed, SYNTH_TAG_TOKEN, (uint32_t)(draw >> 32), (uint32_t)draw, 0), 1.0,
                   out, (size_t)hidden);
}

double synth_uniform_at(uint64_t seed, uint32_t tag, uint32_t a, uint32_t b, uint32_t c, uint64_t i) {
  return synth_u01(synth_hash(synth_stream(seed, tag, a, b, c), i));
}

int synth_provider_init(synth_provider* p, uint64_t seed, int hidden, int inter, int bits, int group) {
  memset(p, 0, sizeof(*p));
  p->seed = seed;
  p->hidden = hidden;
  p->inter = inter;
  p->bits = bits;
  p->group = group;
  size_t ncode = (size_t)hidden * (size_t)inter * (size_t)bits / 8;
  size_t ngrp = (size_t)hidden * (size_t)inter / (size_t)group;
  for (int m = 0; m < 3; ++m) {
    p->codes[m] = (uint8_t*)malloc(ncode);
    p->scale[m] = (uint16_t*)malloc(ngrp * 2);
    p->bias[m] = (uint16_t*)malloc(ngrp * 2);
    if (!p->codes[m] || !p->scale[m] || !p->bias[m]) {
      synth_provider_free(p);
      return -1;
    }
  }
  return 0;
}

void synth_provider_free(synth_provider* p) {
  for (int m = 0; m < 3; ++m) {
    free(p->codes[m]);
    free(p->scale[m]);
    free(p->bias[m]);
    p->codes[m] = NULL;
    p->scale[m] = NULL;
    p->bias[m] = NULL;
  }
}

int synth_provide(void* ctx, int layer, int expert, const uint8_t** codes, const uint16_t** scale,
                  const uint16_t** bias) {
  synth_provider* p = (synth_provider*)ctx;
  for (int m = 0; m < 3; ++m) {
    int rows = (m == SYNTH_DOWN) ? p->hidden : p->inter;
    int cols = (m == SYNTH_DOWN) ? p->inter : p->hidden;
    synth_matrix(p->seed, layer, expert, m, rows, cols, p->bits, p->group, p->codes[m], p->scale[m], p->bias[m]);
    codes[m] = p->codes[m];
    scale[m] = p->scale[m];
    bias[m] = p->bias[m];
  }
  return 0;
}
