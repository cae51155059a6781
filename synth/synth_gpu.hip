// synth_gpu.hip -- device-side fixture of the counter-based synthetic input generator.
//
// Implements the same definition as synth.c (SplitMix64 output function over a counter,
// streams keyed by (seed, tag, layer, expert, matrix)) for the quantized weights only:
// canonical code bytes and bf16 scales/biases, so that a whole expert stack can be filled
// in device memory and spot-checked byte for byte against the CPU generator. Uniform
// values use only exact IEEE operations with explicit rounding (no contraction), so the
// device and the host produce identical bits. Holds none of the method's arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "synth.h"

namespace {

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t stream_key(uint64_t seed, uint32_t tag, uint32_t layer, uint32_t expert,
                                               uint32_t matrix) {
  uint64_t s = mix64(seed + SYNTH_GAMMA);
  s = mix64(s + ((uint64_t)tag + 1) * SYNTH_GAMMA);
  s = mix64(s + ((uint64_t)layer + 1) * SYNTH_GAMMA);
  s = mix64(s + ((uint64_t)expert + 1) * SYNTH_GAMMA);
  s = mix64(s + ((uint64_t)matrix + 1) * SYNTH_GAMMA);
  return s;
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t bits = __float_as_uint(f);
  uint32_t rounding = ((bits >> 16) & 1u) + 0x7fffu;
  return (uint16_t)((bits + rounding) >> 16);
}

__device__ __forceinline__ uint16_t uniform_bf16(uint64_t h, double lo, double width) {
  double u = (double)(h >> 40) * (1.0 / 16777216.0);
  double t = __dmul_rn(width, u);
  double v = __dadd_rn(lo, t);
  return f32_to_bf16(__double2float_rn(v));
}

__global__ void codes_kernel(uint64_t seed, int layer, int expert0, int which, uint64_t* dst, size_t stride_words,
                             size_t n_words) {
  const int e = blockIdx.y;
  const uint64_t key = stream_key(seed, SYNTH_TAG_CODES, (uint32_t)layer, (uint32_t)(expert0 + e), (uint32_t)which);
  uint64_t* out = dst + (size_t)e * stride_words;
  for (size_t w = blockIdx.x * (size_t)blockDim.x + threadIdx.x; w < n_words; w += (size_t)gridDim.x * blockDim.x)
    out[w] = mix64(key + (w + 1) * SYNTH_GAMMA);
}

__global__ void sb_kernel(uint64_t seed, int layer, int expert0, int which, uint16_t* scale, uint16_t* bias,
                          size_t stride_halves, size_t n) {
  const int e = blockIdx.y;
  const uint64_t ks = stream_key(seed, SYNTH_TAG_SCALE, (uint32_t)layer, (uint32_t)(expert0 + e), (uint32_t)which);
  const uint64_t kb = stream_key(seed, SYNTH_TAG_BIAS, (uint32_t)layer, (uint32_t)(expert0 + e), (uint32_t)which);
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    if (scale) scale[(size_t)e * stride_halves + i] = uniform_bf16(mix64(ks + (i + 1) * SYNTH_GAMMA), SYNTH_SCALE_LO, SYNTH_SCALE_WIDTH);
    if (bias) bias[(size_t)e * stride_halves + i] = uniform_bf16(mix64(kb + (i + 1) * SYNTH_GAMMA), SYNTH_BIAS_LO, SYNTH_BIAS_WIDTH);
  }
}

}  // namespace

// Returns 0 or the hipError_t of the failed launch. Strides in bytes; codes_stride and the
// codes pointer must be 8-byte aligned, sb_stride and the scale/bias pointers 2-byte aligned.
extern "C" int synth_gpu_matrix(uint64_t seed, int layer, int expert0, int n_experts, int which, int rows, int cols,
                                int bits, int group, void* codes, size_t codes_stride, uint16_t* scale,
                                uint16_t* bias, size_t sb_stride, hipStream_t stream) {
  if (n_experts < 1 || n_experts > 65535) return (int)hipErrorInvalidValue;
  const size_t n_words = (size_t)rows * cols * bits / 8 / 8;
  if (codes) {
    if (((uintptr_t)codes % 8) || (codes_stride % 8)) return (int)hipErrorInvalidValue;
    size_t blocks = (n_words + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(codes_kernel, dim3((unsigned)blocks, n_experts), dim3(256), 0, stream, seed, layer, expert0,
                       which, (uint64_t*)codes, codes_stride / 8, n_words);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
  }
  if (scale || bias) {
    if (sb_stride % 2) return (int)hipErrorInvalidValue;
    const size_t n = (size_t)rows * (cols / group);
    size_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(sb_kernel, dim3((unsigned)blocks, n_experts), dim3(256), 0, stream, seed, layer, expert0, which,
                       scale, bias, sb_stride / 2, n);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
  }
  return 0;
}
