// fmoe_device.h -- device building blocks shared by the fmoe kernels (gfx950, wave64).
//
// Quantized rows are read in 16-byte "chunks": 32 codes at 4 bits or 64 codes at 2 bits,
// always inside one 64-weight group (4-bit: two chunks per group, 2-bit: one). A lane
// holds the activation values of the columns of the chunks it reads, in registers, in the
// order in which the codes sit in the chunk, pre-scaled so that a code can be converted
// to float straight from its byte lane (v_cvt_f32_ubyte0..3) without a shift:
//   4-bit dword t of a chunk holds columns 8t..8t+7 as nibbles (even column in the low
//   nibble of each byte); (w & 0x0F0F0F0F) has the even-column codes in its bytes and
//   (w & 0xF0F0F0F0) has 16x the odd-column codes, so odd-column x values are kept / 16.
//   2-bit dword t holds columns 16t..16t+15, byte i = columns 16t+4i+{0..3} in bit pairs;
//   (w & (3 << 2p)) per byte holds 4^p x the code of column 16t+4i+p, so those x values
//   are kept / 4^p.
// All scalings are powers of two, so the products equal the unscaled ones exactly.
//
// A chunk's contribution to a row dot product uses the per-group factorisation
//   sum_j (q_j s + b) x_j = s * sum_j q_j x_j + b * sum_j x_j
// (the affine dequantization of the Flash-MoE pages, aibit.im "Techniques de rupture"
// item 2), with sum_j x_j precomputed per chunk.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fmoe {

constexpr int kWave = 64;

// AND that the optimizer cannot fold into later byte extractions, so that each byte is
// converted with a single v_cvt_f32_ubyteN.
__device__ __forceinline__ uint32_t and_opaque(uint32_t a, uint32_t m) {
  uint32_t r;
  asm volatile("v_and_b32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(m));
  return r;
}

__device__ __forceinline__ float ub0(uint32_t v) { return (float)(v & 0xffu); }
__device__ __forceinline__ float ub1(uint32_t v) { return (float)((v >> 8) & 0xffu); }
__device__ __forceinline__ float ub2(uint32_t v) { return (float)((v >> 16) & 0xffu); }
__device__ __forceinline__ float ub3(uint32_t v) { return (float)(v >> 24); }

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

template <int BITS>
struct Chunk {
  static constexpr int kCodes = BITS == 4 ? 32 : 64;  // columns per 16-byte chunk
  static constexpr int kPerGroup = 64 / kCodes;       // chunks per 64-weight group
};

// Register image of the activation values of one chunk (see header comment).
template <int BITS>
struct XChunk {
  float v[Chunk<BITS>::kCodes];
  float sum;  // plain sum of the chunk's x values
};

// Fill an XChunk from x[c0 .. c0 + kCodes) (any address space readable by the lane).
template <int BITS>
__device__ __forceinline__ void load_xchunk(XChunk<BITS>& xc, const float* x) {
  float s = 0.f;
  if constexpr (BITS == 4) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        float e = x[8 * t + 2 * b], o = x[8 * t + 2 * b + 1];
        xc.v[8 * t + b] = e;              // even columns, slot 8t+b
        xc.v[8 * t + 4 + b] = o * 0.0625f;  // odd columns / 16, slot 8t+4+b
        s += e + o;
      }
    }
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float sc = p == 0 ? 1.f : p == 1 ? 0.25f : p == 2 ? 0.0625f : 0.015625f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float e = x[16 * t + 4 * i + p];
          xc.v[16 * t + 4 * p + i] = e * sc;
          s += e;
        }
      }
    }
  }
  xc.sum = s;
}

// sum_j q_j x_j over one chunk (codes in w), fp32.
template <int BITS>
__device__ __forceinline__ float chunk_qx(const uint4& w, const XChunk<BITS>& xc) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  float a0 = 0.f, a1 = 0.f;
  if constexpr (BITS == 4) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      uint32_t lo = and_opaque(ws[t], 0x0F0F0F0Fu);
      uint32_t hi = and_opaque(ws[t], 0xF0F0F0F0u);
      a0 = fmaf(ub0(lo), xc.v[8 * t + 0], a0);
      a1 = fmaf(ub0(hi), xc.v[8 * t + 4], a1);
      a0 = fmaf(ub1(lo), xc.v[8 * t + 1], a0);
      a1 = fmaf(ub1(hi), xc.v[8 * t + 5], a1);
      a0 = fmaf(ub2(lo), xc.v[8 * t + 2], a0);
      a1 = fmaf(ub2(hi), xc.v[8 * t + 6], a1);
      a0 = fmaf(ub3(lo), xc.v[8 * t + 3], a0);
      a1 = fmaf(ub3(hi), xc.v[8 * t + 7], a1);
    }
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        uint32_t m = and_opaque(ws[t], 0x03030303u << (2 * p));
        float& acc = (p & 1) ? a1 : a0;
        acc = fmaf(ub0(m), xc.v[16 * t + 4 * p + 0], acc);
        acc = fmaf(ub1(m), xc.v[16 * t + 4 * p + 1], acc);
        acc = fmaf(ub2(m), xc.v[16 * t + 4 * p + 2], acc);
        acc = fmaf(ub3(m), xc.v[16 * t + 4 * p + 3], acc);
      }
    }
  }
  return a0 + a1;
}

// Contribution of one chunk to its row: s * sum(q x) + b * sum(x).
template <int BITS>
__device__ __forceinline__ float chunk_dot(const uint4& w, uint32_t sb, const XChunk<BITS>& xc) {
  float qx = chunk_qx<BITS>(w, xc);
  return fmaf(bf16_lo(sb), qx, bf16_hi(sb) * xc.sum);
}

// Sum over groups of `width` consecutive lanes (width a power of two <= 64); every lane
// of the group gets the total.
__device__ __forceinline__ float group_sum(float v, int width) {
  for (int m = width >> 1; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}

// Rank order of the router: a before b when its logit is larger, or equal with a lower
// index; NaN ranks after every number.
__device__ __forceinline__ bool ranks_before(float la, int ia, float lb, int ib) {
  bool na = la != la, nb = lb != lb;
  if (na != nb) return nb;
  if (na) return ia < ib;
  if (la != lb) return la > lb;
  return ia < ib;
}

// silu(g) * u with silu(g) = g / (1 + exp(-g)); for very negative g, exp(-g) is +inf
// and the quotient is -0 (never NaN).
__device__ __forceinline__ float swiglu(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// Coherent (device-scope) scalar accesses used for data exchanged between workgroups
// of one kernel: they are performed at the device coherence point, so no cache
// write-back or invalidation is needed around them.
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev_u32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_dev_u32(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev_u64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev_u64(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until every vector memory operation this wave issued has completed (stores
// acknowledged by the coherence point). Also a compiler barrier for memory.
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

}  // namespace fmoe
