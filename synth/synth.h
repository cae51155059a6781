/*
 * synth.h -- seeded, counter-based synthetic inputs for the quantized MoE expert block.
 *
 * This module is shared by the oracle (CPU) and by the GPU-side tests and benchmark.
 * It holds none of the method's arithmetic: it only produces input bytes (4-bit or
 * 2-bit codes, bf16 scales and biases, fp32 router weights and fp32 token vectors)
 * in the canonical layout below, from a seed and a coordinate.
 *
 * Generator: the SplitMix64 output function ("mix64", Steele, Lea & Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014, with the
 * variant-13 constants of the Java 8 SplittableRandom) applied to a 64-bit counter.
 * A stream is keyed by (seed, tag, layer, expert, matrix) by folding each
 * coordinate into the state with one mix64 step; element i of a stream is
 * mix64(state + (i + 1) * GAMMA). The GPU fixture (synth_gpu.hip) implements the
 * same definition and the two agree byte for byte on every integer and on every
 * value derived from a hash by exact IEEE operations (codes, scales, biases).
 * Normals use libm (log, sqrt, cos) and are produced on the CPU only.
 *
 * Canonical layout (what the oracle reads):
 *   4-bit codes  uint8 [rows][cols/2]; element 2c in bits 0-3, element 2c+1 in bits 4-7.
 *   2-bit codes  uint8 [rows][cols/4]; element 4c+t in bits 2t..2t+1.
 *   scale, bias  bf16 (uint16 bit patterns) [rows][cols/group].
 *   router       fp32 [n_experts][hidden], row-major.
 *   token        fp32 [hidden].
 * The canonical code bytes of one matrix are the little-endian bytes of the hash
 * stream: byte 8w+j is bits 8j..8j+7 of element w.
 *
 * Distributions (uniform u = (hash >> 40) * 2^-24, exact in fp64):
 *   codes: every bit uniform, so codes are uniform over 0..15 (0..3 at 2 bits);
 *   scale = bf16(float(0.001 + 0.019 * u)), bias = bf16(float(-0.1 + 0.2 * u)),
 *   the fp64 sum and product rounded one at a time (no fused multiply-add);
 *   router ~ N(0, 0.02^2), token ~ N(0, 1) by Box-Muller from one hash each.
 */
#ifndef SYNTH_H
#define SYNTH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SYNTH_GAMMA 0x9e3779b97f4a7c15ull

/* Stream tags. */
enum {
  SYNTH_TAG_CODES = 1,
  SYNTH_TAG_SCALE = 2,
  SYNTH_TAG_BIAS = 3,
  SYNTH_TAG_ROUTER = 4,
  SYNTH_TAG_TOKEN = 5,
  SYNTH_TAG_PLANT = 6,
  SYNTH_TAG_NOISE = 7
};

/* Matrix ids within an expert. */
enum { SYNTH_GATE = 0, SYNTH_UP = 1, SYNTH_DOWN = 2 };

/* Ranges of the affine parameters. */
#define SYNTH_SCALE_LO 0.001
#define SYNTH_SCALE_WIDTH 0.019
#define SYNTH_BIAS_LO (-0.1)
#define SYNTH_BIAS_WIDTH 0.2
#define SYNTH_ROUTER_SIGMA 0.02

uint64_t synth_mix64(uint64_t z);
uint64_t synth_stream(uint64_t seed, uint32_t tag, uint32_t layer, uint32_t expert, uint32_t matrix);
uint64_t synth_hash(uint64_t stream, uint64_t idx);
double synth_u01(uint64_t hash);
uint16_t synth_f32_to_bf16(float f);
float synth_bf16_to_f32(uint16_t b);

/* Canonical code bytes of one matrix: nbytes must be a multiple of 8. */
void synth_codes(uint64_t stream, uint8_t* out, size_t nbytes);
/* n bf16 values lo + width * u. */
void synth_uniform_bf16(uint64_t stream, double lo, double width, uint16_t* out, size_t n);
/* n fp32 values sigma * N(0,1). */
void synth_normal_f32(uint64_t stream, double sigma, float* out, size_t n);

/* One matrix of expert (layer, expert): canonical codes + scale + bias.
 * matrix is SYNTH_GATE/UP (rows = inter, cols = hidden) or SYNTH_DOWN
 * (rows = hidden, cols = inter). */
void synth_matrix(uint64_t seed, int layer, int expert, int matrix, int rows, int cols, int bits,
                  int group, uint8_t* codes, uint16_t* scale, uint16_t* bias);

/* Router of a layer, fp32 [n_experts][hidden] ~ N(0, 0.02^2). */
void synth_router(uint64_t seed, int layer, int n_experts, int hidden, float* out);

/* Token vector of draw index `draw`, fp32 [hidden] ~ N(0,1). */
void synth_token(uint64_t seed, uint64_t draw, int hidden, float* out);

/* Uniform in [0,1) from stream (seed, tag, a, b, c) at index i (for planting draws). */
double synth_uniform_at(uint64_t seed, uint32_t tag, uint32_t a, uint32_t b, uint32_t c, uint64_t i);

/* Expert provider used by callers that need experts on demand (same signature as the
 * oracle's provider callback). ctx points at a synth_provider. The buffers are owned
 * by the provider and stay valid until the next call. Returns 0 on success. */
typedef struct {
  uint64_t seed;
  int hidden, inter, bits, group;
  uint8_t* codes[3];
  uint16_t* scale[3];
  uint16_t* bias[3];
} synth_provider;

int synth_provider_init(synth_provider* p, uint64_t seed, int hidden, int inter, int bits, int group);
void synth_provider_free(synth_provider* p);
int synth_provide(void* ctx, int layer, int expert, const uint8_t** codes, const uint16_t** scale,
                  const uint16_t** bias);

#ifdef __cplusplus
}
#endif
#endif
