// fmoe_intdot.h -- integer dot products of 4-bit / 3-bit / 2-bit codes with block-fixed-point
// activations (gfx950 v_dot8_u32_u4: eight 4-bit x 4-bit products summed into 32 bits).
//
// Per chunk of activation values (the columns one 16-byte code chunk covers: 32 at 4
// bits, 64 at 2 bits) the values are put on a common fixed-point grid:
//   step = 2^(e - 22) with max|x| < 2^e,   X_j = rint(x_j / step),  |X_j| < 2^22,
// and stored as U_j = X_j + 2^22 (0 <= U_j < 2^23) in six 4-bit digits d_k(U_j). For a
// row with codes q_j, sum_j q_j x_j ~= step * sum_j q_j X_j, and
//   sum_j q_j X_j = sum_k 16^k D_k - 2^22 N,  D_k = sum_j q_j d_k(U_j),  N = sum_j q_j,
// where every D_k and N is one v_dot8 chain per code dword (exact integers). The only
// rounding is that of x to the grid (at most step/2 = 2^-23 of the chunk's largest
// magnitude) and the final conversion to fp32; the per-group affine form is then
//   s * step * sum_j q_j X_j + b * sum_j x_j
// (the nibble*scale+bias dequantization of aibit.im "Techniques de rupture" item 2,
// factored per group). This replaces a float convert + FMA per weight by ~7/8 of an
// integer dot instruction per weight.
//
// Digit dword layout (must match the code nibble order): a 4-bit code dword holds the 8
// consecutive columns 8t..8t+7, column 8t+p in nibble p, so digit dword (t, k) holds
// d_k of column 8t+p in nibble p. A 2-bit code dword holds 16 columns 16t+i (bits 2i);
// (w & 0x33333333) keeps the even columns 16t+2p in nibble p and ((w >> 2) & 0x33333333)
// the odd columns 16t+2p+1, so a 2-bit dword has two digit sets (even, odd).
#pragma once

#include "fmoe_device.h"

namespace fmoe {

template <int BITS>
struct Digits {
  static constexpr int kCodes = Chunk<BITS>::kCodes;       // columns per chunk
  static constexpr int kSets = BITS == 4 ? 4 : 8;           // 8-column digit sets per chunk
  static constexpr int kWords = kSets * 6;                  // digit dwords per chunk
};

// Register image of one chunk's digits.
template <int BITS>
struct DChunk {
  uint32_t d[Digits<BITS>::kWords];
  float step;  // grid step of the chunk
  float xsum;  // plain fp32 sum of the chunk's values
};

// LDS digit store for a vector of n_chunks chunks, structure-of-arrays so that lanes
// reading consecutive chunks touch consecutive words: word q of chunk c at q * n_chunks + c.
struct DigitStore {
  uint32_t* words;  // [kWords][n_chunks]
  float* step;      // [n_chunks]
  float* xsum;      // [n_chunks]
  int n_chunks;
};

template <int BITS>
__device__ __forceinline__ void load_dchunk(DChunk<BITS>& dc, const DigitStore& st, int c) {
#pragma unroll
  for (int q = 0; q < Digits<BITS>::kWords; ++q) dc.d[q] = st.words[q * st.n_chunks + c];
  dc.step = st.step[c];
  dc.xsum = st.xsum[c];
}

// sum_j q_j x_j of one chunk of codes, via the digit image. 3 bits: the code dwords are the
// low plane's (2-bit order) and the high-plane word of a dword's 32-column half, shifted by
// 2 (t % 2), has the third bit of nibble n of the even operand at bit 4n and of the odd one
// at 4n + 1 (fmoe_layout.h, hi_bit): one shift and an and-or make each operand's nibbles the
// full 3-bit codes, and the digit sets are those of 2 bits.
template <int BITS>
__device__ __forceinline__ float chunk_qx_int(const CChunk<BITS>& cc, const DChunk<BITS>& dc) {
  const uint4& w = cc.w;
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  uint32_t D[6] = {0, 0, 0, 0, 0, 0};
  uint32_t N = 0;
  if constexpr (BITS == 4) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int k = 0; k < 6; ++k) D[k] = __builtin_amdgcn_udot8(ws[t], dc.d[t * 6 + k], D[k], false);
      N = __builtin_amdgcn_udot8(ws[t], 0x11111111u, N, false);
    }
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      uint32_t ev = and_opaque(ws[t], 0x33333333u);
      uint32_t od = (ws[t] >> 2) & 0x33333333u;
      if constexpr (BITS == 3) {
        const uint32_t hs = (t < 2 ? cc.h.x : cc.h.y) >> (2 * (t % 2));
        ev |= (hs << 2) & 0x44444444u;
        od |= (hs << 1) & 0x44444444u;
      }
#pragma unroll
      for (int k = 0; k < 6; ++k) {
        D[k] = __builtin_amdgcn_udot8(ev, dc.d[(2 * t) * 6 + k], D[k], false);
        D[k] = __builtin_amdgcn_udot8(od, dc.d[(2 * t + 1) * 6 + k], D[k], false);
      }
      N = __builtin_amdgcn_udot8(ev, 0x11111111u, N, false);
      N = __builtin_amdgcn_udot8(od, 0x11111111u, N, false);
    }
  }
  const int lo = (int)(D[0] + (D[1] << 4) + (D[2] << 8));
  const int hi = (int)(D[3] + (D[4] << 4) + (D[5] << 8)) - (int)(N << 10);
  return fmaf(4096.f, (float)hi, (float)lo) * dc.step;
}

template <int BITS>
__device__ __forceinline__ float chunk_dot_int(const CChunk<BITS>& cc, uint32_t sb, const DChunk<BITS>& dc) {
  return fmaf(bf16_lo(sb), chunk_qx_int<BITS>(cc, dc), bf16_hi(sb) * dc.xsum);
}

// Six 4-bit digit words of 8 values: word k holds nibble k of u[p] in nibble p (an 8 x 8
// nibble transpose of which rows 0..5 are kept; nibbles 6 and 7 of the inputs are
// ignored). Three block-swap stages: 4-nibble and 2-nibble blocks move as whole bytes
// (v_perm_b32), single nibbles with a bit-field insert.
__device__ __forceinline__ void nibble_transpose6(const uint32_t (&u)[8], uint32_t (&d)[6]) {
  uint32_t r[8];
  // stage 1: nibbles 4..7 of row p <-> nibbles 0..3 of row p + 4
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    r[p] = __builtin_amdgcn_perm(u[p + 4], u[p], 0x05040100u);      // [a0 a1 b0 b1]
    r[p + 4] = __builtin_amdgcn_perm(u[p + 4], u[p], 0x07060302u);  // [a2 a3 b2 b3]
  }
  // stage 2: bytes 1, 3 of row p <-> bytes 0, 2 of row p + 2
#pragma unroll
  for (int p : {0, 1, 4, 5}) {
    const uint32_t a = r[p], b = r[p + 2];
    r[p] = __builtin_amdgcn_perm(b, a, 0x06020400u);      // [a0 b0 a2 b2]
    r[p + 2] = __builtin_amdgcn_perm(b, a, 0x07030501u);  // [a1 b1 a3 b3]
  }
  // stage 3: odd nibbles of row p <-> even nibbles of row p + 1 (rows 6, 7 not needed)
#pragma unroll
  for (int p = 0; p < 6; p += 2) {
    const uint32_t a = r[p], b = r[p + 1];
    d[p] = (a & 0x0F0F0F0Fu) | ((b << 4) & 0xF0F0F0F0u);
    d[p + 1] = ((a >> 4) & 0x0F0F0F0Fu) | (b & 0xF0F0F0F0u);
  }
}

// Build the digit store entries of chunks c0 .. c0 + n / CC of an fp32 vector (n a
// multiple of the chunk size), whose column i is read through xat(i); the stored step and
// sum are multiplied by `scale` (a vector v = scale * x is digitised through x). Work
// items are 8-column digit sets; the sets of one chunk sit on consecutive lanes, which
// share the chunk's maximum and sum through DPP. Run by `nthreads` threads (a multiple of
// 64) with thread index t; no barrier inside.
//
// Rounding to the grid: with |x / step| < 2^22, fma(x, 1/step, 1.5 * 2^23) lies in
// [2^23, 2^24), where fp32 has unit spacing, so the single rounding of the fma is the
// round-to-nearest-even of x / step and the low 23 bits of the result are
// rint(x / step) + 2^22 = U.
template <int BITS, typename XAt>
__device__ __forceinline__ void build_digits(const DigitStore& st, int c0, int n, XAt xat, int nthreads, int t,
                                             float scale = 1.f) {
  constexpr int CC = Digits<BITS>::kCodes;
  constexpr int SETS = Digits<BITS>::kSets;
  const int n_sets = (n / CC) * SETS;
  for (int it = t; it < n_sets; it += nthreads) {
    const int c = c0 + it / SETS, set = it % SETS;
    float x[8];
    float m = 0.f, s = 0.f;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      int col;
      if constexpr (BITS == 4) col = c * CC + set * 8 + p;
      else col = c * CC + (set / 2) * 16 + 2 * p + (set & 1);
      x[p] = xat(col);
      m = fmaxf(m, fabsf(x[p]));
      s += x[p];
    }
    m = group_max(m, SETS);
    s = group_sum(s, SETS);
    int e = 0;
    frexpf(m, &e);  // m < 2^e
    const bool tiny = !(m >= 1e-30f);
    const float step = tiny ? 1.f : ldexpf(1.f, e - 22);
    const float inv = tiny ? 0.f : ldexpf(1.f, 22 - e);
    if (set == 0) {
      st.step[c] = step * scale;
      st.xsum[c] = s * scale;
    }
    uint32_t u[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) u[p] = __float_as_uint(fmaf(x[p], inv, 12582912.0f));
    uint32_t d[6];
    nibble_transpose6(u, d);
#pragma unroll
    for (int k = 0; k < 6; ++k) st.words[(set * 6 + k) * st.n_chunks + c] = d[k];
  }
}

}  // namespace fmoe
