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
//
// 3-bit codes (two planes, fmoe_layout.h): a chunk is the 16 bytes of the low plane for 64
// columns (as a 2-bit chunk) plus the two high-plane words of the same group.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fmoe_layout.h"

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
  static constexpr int kCodes = BITS == 4 ? 32 : 64;  // columns per 16-byte (low-plane) chunk
  static constexpr int kPerGroup = 64 / kCodes;       // chunks per 64-weight group
  static constexpr int kLoBits = BITS == 3 ? 2 : BITS;  // code width of the (low) plane's layout
};

// The code bytes of one chunk as loaded: 16 bytes, plus the two high-plane words at 3 bits.
template <int BITS>
struct CChunk {
  uint4 w;
};
template <>
struct CChunk<3> {
  uint4 w;
  uint2 h;
};

// Load chunk `c` (16-byte chunk index along the row) of row r of a packed matrix whose codes
// start at `mat` (rows x cols).
template <int BITS>
__device__ __forceinline__ void load_cchunk(CChunk<BITS>& cc, const uint8_t* mat, int rows, int cols, int r, int c) {
  constexpr int LB = Chunk<BITS>::kLoBits;
  const size_t row_bytes = (size_t)cols * LB / 8;
  cc.w = *reinterpret_cast<const uint4*>(mat + code_offset<LB>(rows, row_bytes, r, (size_t)c * 16));
  if constexpr (BITS == 3) {
    const uint32_t* hp = reinterpret_cast<const uint32_t*>(mat + lo_plane_bytes(rows, cols));
    cc.h = *reinterpret_cast<const uint2*>(hp + hi_offset(rows, cols / 64, r, c, 0));
  }
}

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

// 3-bit: the low plane's dword t holds columns 16t..16t+15 in bit pairs, (w >> 2p) &
// 0x03030303 has column 16t + 4m + p in byte m; the high-plane word of the dword's 32-column
// half, shifted by 2 (t % 2), has that column's third bit at 8m + 4 (p / 2) + p % 2
// (fmoe_layout.h, hi_bit), which one shift and mask move to bit 2 of byte m. The register
// image of x is kept unscaled in that order: v[16t + 4p + m] = x[16t + 4m + p].
__device__ __forceinline__ uint32_t hi_bytes3(uint32_t hs, int p) {
  const int b = 4 * (p / 2) + (p % 2);  // the bit of byte m, before the move to bit 2
  return (b >= 2 ? (hs >> (b - 2)) : (hs << (2 - b))) & 0x04040404u;
}
template <>
__device__ __forceinline__ void load_xchunk<3>(XChunk<3>& xc, const float* x) {
  float s = 0.f;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const float e = x[16 * t + 4 * m + p];
        xc.v[16 * t + 4 * p + m] = e;
        s += e;
      }
  xc.sum = s;
}
__device__ __forceinline__ float chunk_qx3(const CChunk<3>& cc, const XChunk<3>& xc) {
  const uint32_t ws[4] = {cc.w.x, cc.w.y, cc.w.z, cc.w.w};
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint32_t hs = (t < 2 ? cc.h.x : cc.h.y) >> (2 * (t % 2));
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t q = ((ws[t] >> (2 * p)) & 0x03030303u) | hi_bytes3(hs, p);
      float& acc = (p & 1) ? a1 : a0;
      acc = fmaf(ub0(q), xc.v[16 * t + 4 * p + 0], acc);
      acc = fmaf(ub1(q), xc.v[16 * t + 4 * p + 1], acc);
      acc = fmaf(ub2(q), xc.v[16 * t + 4 * p + 2], acc);
      acc = fmaf(ub3(q), xc.v[16 * t + 4 * p + 3], acc);
    }
  }
  return a0 + a1;
}

// Contribution of one chunk to its row: s * sum(q x) + b * sum(x).
template <int BITS>
__device__ __forceinline__ float chunk_dot(const CChunk<BITS>& cc, uint32_t sb, const XChunk<BITS>& xc) {
  float qx;
  if constexpr (BITS == 3) qx = chunk_qx3(cc, xc);
  else qx = chunk_qx<BITS>(cc.w, xc);
  return fmaf(bf16_lo(sb), qx, bf16_hi(sb) * xc.sum);
}

// Cross-lane data movement with DPP (no LDS round trip). Controls (GFX9 encoding):
// quad_perm [1,0,3,2] = 0xB1, quad_perm [2,3,0,1] = 0x4E, row_half_mirror = 0x141,
// row_mirror = 0x140, row_ror:4 = 0x124, row_ror:8 = 0x128, row_bcast:15 = 0x142,
// row_bcast:31 = 0x143.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}
__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Sum over groups of `width` consecutive lanes (width a power of two <= 64); every lane
// of the group gets the group's total.
__device__ __forceinline__ float group_sum(float v, int width) {
  if (width >= 2) v += dpp_f<0xB1>(v);
  if (width >= 4) v += dpp_f<0x4E>(v);
  if (width >= 8) v += dpp_f<0x141>(v);
  if (width >= 16) v += dpp_f<0x140>(v);
  if (width == 32) {
    const float r0 = readlane_f(v, 0), r1 = readlane_f(v, 16), r2 = readlane_f(v, 32), r3 = readlane_f(v, 48);
    v = (threadIdx.x & 32) ? (r2 + r3) : (r0 + r1);
  } else if (width >= 64) {
    // rows 1 and 3 add lane 15 of the row before (row_bcast:15), then rows 2 and 3 add
    // lane 31 (row_bcast:31): lane 63 ends with the total
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));
    v = readlane_f(v, 63);
  }
  return v;
}

__device__ __forceinline__ float wave_sum(float v) { return group_sum(v, 64); }

// The value of the lane at distance D in the pairing used by reduce_transposed: D = 1, 2
// exchange with lane ^ D (quad_perm), D = 4 and 8 rotate each 16-lane row by 4 and 8
// (row_ror), D = 16 exchanges with lane ^ 16 (ds_swizzle, bit mode), D = 32 with
// lane ^ 32 (ds_bpermute).
template <int D>
__device__ __forceinline__ float xlane(float v) {
  if constexpr (D == 1) return dpp_f<0xB1>(v);
  else if constexpr (D == 2) return dpp_f<0x4E>(v);
  else if constexpr (D == 4) return dpp_f<0x124>(v);
  else if constexpr (D == 8) return dpp_f<0x128>(v);
  else if constexpr (D == 16) return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
  else return __int_as_float(__builtin_amdgcn_ds_bpermute((int)((threadIdx.x & 63) ^ 32) << 2, __float_as_int(v)));
}

// One halving step of a transposed reduction: a lane whose bit D is set keeps the upper
// half of its values and sends the lower half to its partner, and the other way round, so
// that after the step each lane holds NV/2 values summed over the pair.
template <int D, int NV>
__device__ __forceinline__ void transpose_step(float (&v)[8]) {
  const bool up = (threadIdx.x & D) != 0;
#pragma unroll
  for (int k = 0; k < NV / 2; ++k) {
    const float keep = up ? v[NV / 2 + k] : v[k];
    const float send = up ? v[k] : v[NV / 2 + k];
    v[k] = keep + xlane<D>(send);
  }
}

// Sum NV values (NV = 1, 2, 4 or 8) each over its group of W consecutive lanes (W = 16,
// 32 or 64) in one pass: the first log2(NV) steps split the values between partner lanes
// instead of reducing each one separately, so NV sums cost about as many cross-lane
// operations as 2 single ones. Afterwards every lane of a group holds the total of value
// transposed_index<NV>(lane). The rotation at distance 4 pairs quad q of a row with quad
// q - 1; the rotation at distance 8 then adds the remaining two quads, so every quad of
// the row is counted once.
template <int NV, int W>
__device__ __forceinline__ float reduce_transposed(const float (&in)[NV]) {
  static_assert(NV == 1 || NV == 2 || NV == 4 || NV == 8, "NV must be 1, 2, 4 or 8");
  static_assert(W == 16 || W == 32 || W == 64, "W must be 16, 32 or 64");
  float v[8];
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] = in[i];
  if constexpr (NV >= 2) transpose_step<1, NV>(v);
  else v[0] += xlane<1>(v[0]);
  if constexpr (NV >= 4) transpose_step<2, NV / 2>(v);
  else v[0] += xlane<2>(v[0]);
  if constexpr (NV >= 8) transpose_step<4, 2>(v);
  else v[0] += xlane<4>(v[0]);
  v[0] += xlane<8>(v[0]);
  if constexpr (W >= 32) v[0] += xlane<16>(v[0]);
  if constexpr (W >= 64) v[0] += xlane<32>(v[0]);
  return v[0];
}

// Which of the NV values a lane holds after reduce_transposed<NV, W>.
template <int NV>
__device__ __forceinline__ int transposed_index(int lane) {
  if constexpr (NV == 8) return 4 * (lane & 1) + 2 * ((lane >> 1) & 1) + ((lane >> 2) & 1);
  else if constexpr (NV == 4) return 2 * (lane & 1) + ((lane >> 1) & 1);
  else if constexpr (NV == 2) return lane & 1;
  else return 0;
}

// Maximum over groups of `width` consecutive lanes (width 2, 4, 8 or 16).
__device__ __forceinline__ float group_max(float v, int width) {
  if (width >= 2) v = fmaxf(v, dpp_f<0xB1>(v));
  if (width >= 4) v = fmaxf(v, dpp_f<0x4E>(v));
  if (width >= 8) v = fmaxf(v, dpp_f<0x141>(v));
  if (width >= 16) v = fmaxf(v, dpp_f<0x140>(v));
  return v;
}

// Maximum of a 64-bit key over the wave, returned in every lane.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t k) {
  uint32_t hi = (uint32_t)(k >> 32), lo = (uint32_t)k;
#define FMOE_MAXSTEP(CTRL)                                             \
  {                                                                    \
    uint32_t oh = dpp_u<CTRL>(hi), ol = dpp_u<CTRL>(lo);               \
    bool take = (oh > hi) || (oh == hi && ol > lo);                    \
    hi = take ? oh : hi;                                               \
    lo = take ? ol : lo;                                               \
  }
  FMOE_MAXSTEP(0xB1) FMOE_MAXSTEP(0x4E) FMOE_MAXSTEP(0x141) FMOE_MAXSTEP(0x140)
#undef FMOE_MAXSTEP
  uint64_t best = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    uint64_t c = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)hi, 16 * r) << 32) |
                 (uint32_t)__builtin_amdgcn_readlane((int)lo, 16 * r);
    best = c > best ? c : best;
  }
  return best;
}

// Rank key of a router logit: larger key = earlier in rank order (larger logit first,
// lower index on equal logits, NaN after every number). Keys of different experts are
// distinct and never 0.
__device__ __forceinline__ uint64_t rank_key(float logit, int e) {
  uint32_t b = logit == 0.f ? 0u : __float_as_uint(logit);  // -0 ranks as +0
  uint32_t ord = (logit != logit) ? 0u : ((b & 0x80000000u) ? ~b : (b | 0x80000000u));
  return ((uint64_t)ord << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
}
__device__ __forceinline__ int rank_key_index(uint64_t key) { return (int)(0xFFFFFFFFu - (uint32_t)key); }
__device__ __forceinline__ float rank_key_logit(uint64_t key) {
  uint32_t ord = (uint32_t)(key >> 32);
  uint32_t b = (ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord;
  return __uint_as_float(b);
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

// Top-k progress published to the other waves of the workgroup (LDS word): r after
// round r, and k + 1 once the softmax weights are written.
__device__ __forceinline__ void topk_progress(int* ready, int r) {
  if (ready && (threadIdx.x & 63) == 0) __hip_atomic_store(ready, r, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Top-k of n ranked keys held in LDS (one wave; keys are consumed). Round r takes the
// wave-wide maximum key; its owner lane clears it and rescans its own keys. Lane 0 writes
// isel[r] (expert index) and lsel[r] (logit); then lanes < k turn the logits into the
// softmax over the selected experts, shifted by the largest: wsel[j] = e^(l_j - l_0) /
// sum_j' e^(l_j' - l_0).
__device__ __forceinline__ void wave_topk_keys(uint64_t* keys, int n, int k, int* isel, float* lsel,
                                               float* wsel, int* ready = nullptr) {
  const int lane = threadIdx.x & 63;
  uint64_t best = 0;
  for (int e = lane; e < n; e += 64) best = keys[e] > best ? keys[e] : best;
  for (int r = 0; r < k; ++r) {
    const uint64_t w = wave_max_u64(best);
    if (lane == 0) {
      isel[r] = rank_key_index(w);
      lsel[r] = rank_key_logit(w);
    }
    topk_progress(ready, r + 1);
    if (best == w && w != 0) {
      best = 0;
      for (int e = lane; e < n; e += 64) {
        uint64_t kv = keys[e];
        if (kv == w) keys[e] = 0;
        else best = kv > best ? kv : best;
      }
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
  float ex = 0.f;
  if (lane < k) ex = expf(lsel[lane] - lsel[0]);
  const float denom = wave_sum(ex);
  if (lane < k) wsel[lane] = ex / denom;
  topk_progress(ready, k + 1);
}

// Maximum of a 32-bit value over the wave (every lane gets it; wave-uniform).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u<0xB1>(v));
  v = max(v, dpp_u<0x4E>(v));
  v = max(v, dpp_u<0x141>(v));
  v = max(v, dpp_u<0x140>(v));
  // across rows as in group_sum (row_bcast:15, then row_bcast:31); lanes outside the row
  // mask keep their own value
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x142, 0xA, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x143, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// The wave-wide maximum of one rank key per lane (0 = no key): the 32-bit maximum of the
// high words (the ordered logits), then, only when several lanes hold that logit, the
// maximum of their low words (lower index first). Wave-uniform result.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t key) {
  const uint32_t hi = (uint32_t)(key >> 32), lo = (uint32_t)key;
  const uint32_t m = wave_max_u32(hi);
  const uint64_t tied = __ballot(hi == m);
  uint32_t lw;
  if (__popcll(tied) == 1) lw = (uint32_t)__builtin_amdgcn_readlane((int)lo, (int)__ffsll((long long)tied) - 1);
  else lw = wave_max_u32(hi == m ? lo : 0u);
  return ((uint64_t)m << 32) | lw;
}

// One round of a top-k over per-lane key lists sorted in descending order: the wave
// maximum of the heads; the lane holding it drops its head. Returns the winner.
template <int KPL>
__device__ __forceinline__ uint64_t topk_round(uint64_t (&kr)[KPL]) {
  const uint64_t w = wave_max_key(kr[0]);
  if (kr[0] == w) {
#pragma unroll
    for (int j = 0; j + 1 < KPL; ++j) kr[j] = kr[j + 1];
    kr[KPL - 1] = 0;
  }
  return w;
}

template <int N>
__device__ __forceinline__ void cmp_swap_desc(uint64_t (&k)[N], int i, int j) {
  const uint64_t a = k[i], b = k[j];
  const bool sw = b > a;
  k[i] = sw ? b : a;
  k[j] = sw ? a : b;
}

// k rounds of topk_round over sorted per-lane lists, recording each winner (index and
// logit, lane 0) and releasing progress r + 1 after round r; then the softmax over the k
// selected logits (max-subtracted) and progress k + 1.
template <int KPL>
__device__ __forceinline__ void topk_select(uint64_t (&kr)[KPL], int k, int* isel, float* lsel, float* wsel,
                                            int* ready) {
  const int lane = threadIdx.x & 63;
  for (int r = 0; r < k; ++r) {
    const uint64_t w = topk_round(kr);
    if (lane == 0) {
      isel[r] = rank_key_index(w);
      lsel[r] = rank_key_logit(w);
    }
    topk_progress(ready, r + 1);
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
  float ex = 0.f;
  if (lane < k) ex = expf(lsel[lane] - lsel[0]);
  const float denom = wave_sum(ex);
  if (lane < k) wsel[lane] = ex / denom;
  topk_progress(ready, k + 1);
}

// Top-k of at most 64 * KPL ranked keys held in registers (key j of a lane is element
// lane + 64 j; absent elements hold key 0). Same contract as wave_topk_keys; the keys are
// consumed. Each lane first sorts its keys (descending); a round then takes the wave-wide
// maximum of the lanes' heads: the 32-bit maximum of the high words (the ordered logits),
// then, only when several lanes hold that logit, the maximum of their low words (lower
// index first); the winning lane drops its head.
template <int KPL>
__device__ __forceinline__ void wave_topk_regs(uint64_t (&kr)[KPL], int k, int* isel, float* lsel, float* wsel,
                                               int* ready = nullptr) {
  static_assert(KPL == 8, "sorting network for 8 keys per lane");
  const int lane = threadIdx.x & 63;
  // Batcher's odd-even merge sort, 8 inputs (19 compare-exchanges)
  cmp_swap_desc(kr, 0, 1); cmp_swap_desc(kr, 2, 3); cmp_swap_desc(kr, 4, 5); cmp_swap_desc(kr, 6, 7);
  cmp_swap_desc(kr, 0, 2); cmp_swap_desc(kr, 1, 3); cmp_swap_desc(kr, 4, 6); cmp_swap_desc(kr, 5, 7);
  cmp_swap_desc(kr, 1, 2); cmp_swap_desc(kr, 5, 6);
  cmp_swap_desc(kr, 0, 4); cmp_swap_desc(kr, 1, 5); cmp_swap_desc(kr, 2, 6); cmp_swap_desc(kr, 3, 7);
  cmp_swap_desc(kr, 2, 4); cmp_swap_desc(kr, 3, 5);
  cmp_swap_desc(kr, 1, 2); cmp_swap_desc(kr, 3, 4); cmp_swap_desc(kr, 5, 6);
  topk_select(kr, k, isel, lsel, wsel, ready);
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
