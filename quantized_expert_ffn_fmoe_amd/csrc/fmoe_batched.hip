// fmoe_batched.hip -- the multi-token path of fmoe_moe_layer: tokens grouped by expert,
// each expert's gate/up and down projections as bf16 matrix-core products (gfx950
// v_mfma_f32_16x16x32_bf16) with fp32 accumulation.
//
// Per layer (the same block as the decode path: route, run the selected experts, combine
// with the residual; aibit.im "Techniques de rupture" items 3-4, tr.news.hada.io "Model
// mimarisi"), with the batch of tokens sorted by expert so that every expert's weights
// are read once per call:
//   1. route: fp32 router logits of the raw h (fp32 matrix cores), as column-slice partials;
//   2. per token: 1 / rms(h) under the pre-norm, the logits (partials summed, times that
//      factor), top-k with softmax; v = h / rms(h) (or h) as its bf16 image v16 in operand
//      order and, per group of 64 columns, the fp32 sum of the bf16 values;
//   3. sort (by the last workgroup of step 2): counting sort of the (token, slot) pairs by
//      expert; the list of work units (16 pairs of one expert each);
//   4. gate/up: per (active expert, block of 128 rows): g and u for all of the expert's
//      tokens, a = silu(g) * u, rounded to bf16 (a16) in the down operand's order, plus
//      the group sums of a16;
//   5. down: per (active expert, block of 256 rows): y = Wd a16 for the expert's tokens,
//      one fp32 row per (token, slot) pair;
//   6. combine: h' = h + sum_j w_j y_j in slot order.
//
// Matrix-core form of the affine dequantization. A weight is q*s + b with (s, b) per
// group of 64 columns of a row (the nibble*scale+bias form of aibit.im "Techniques de
// rupture" item 2). The codes enter the bf16 matrix core as the exact values c = o + u*q:
// q sits in the top mantissa bits of a bf16 whose exponent is fixed and even (4 bits:
// bits 0x4200 | q << 3, c = 32 + 2q; 3 and 2 bits: 0x4100 | q << 4, c = 8 + q), so a
// shift and an AND place a dword's codes byte-wise and one byte permute pairs two of them
// with the fixed high bytes, per bf16 pair. For one group, with X = sum of the group's
// bf16 activations and P = sum x*c from the matrix core,
//   u * sum x (q s + b) = s P + (u b - o s) X
// (the per-group factorisation s*sum(q x) + b*sum(x)), and the factor u (a power of two) is
// divided out once at the end. The first term is applied once per group to the fp32
// partial product; the second, summed over the groups of a stage, is itself a small
// product (tokens x groups times groups x rows), done as one fp32 matrix-core product per
// tile and stage (v_mfma_f32_16x16x4f32, operands in fp32). The offset cancels between the
// two terms, so the partial sums hold up to ~o/u times the magnitude of sum x q; o/u is
// kept at 16 or below. No weight is rounded; only v and a are (to bf16).
// Operand order. For 16x16x32 bf16 products lane l holds, for the A operand, row l % 16
// and the 8 consecutive K indices 8*(l/16)..+7; the same for B with column l % 16; the
// result holds D[4*(l/16) + i][l % 16] in element i. Tokens are the rows (A), weight rows
// the columns (B). Within one group of 64 K indices, lane block kb = l/16 takes the 16
// columns 16*kb..+15 (two products of 8), so a lane reads 8 (4-bit) or 4 (2-bit) code
// bytes of its row per group. Because the pairs of codes come out of a code dword as
// (q_j, q_j+4) (4-bit) or (q_j, q_j+8) (2-bit), the activation operands are stored
// permuted within every block of 16 columns the same way (perm_col / perm_pos).
#include <stdint.h>

#include "fmoe_batched.h"
#include "fmoe_device.h"
#include "fmoe_internal.h"
#include "fmoe_layout.h"

namespace fmoe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBT = 256;          // threads per workgroup
constexpr int kGuRowsWave = 32;   // rows of gate (and of up) per wave
constexpr int kGuRowsWg = 128;
constexpr int kDnRowsWave = 64;   // rows of down per wave
constexpr int kDnRowsWg = 256;

// Column (0..15) of a 16-column block held at operand position p.
template <int BITS>
__host__ __device__ constexpr int perm_col(int p) {
  return BITS == 4 ? 8 * (p >> 3) + ((p & 7) >> 1) + 4 * (p & 1) : 4 * (p >> 3) + ((p & 7) >> 1) + 8 * (p & 1);
}
// Operand position of column c (inverse of perm_col).
template <int BITS>
__host__ __device__ constexpr int perm_pos(int c) {
  return BITS == 4 ? 8 * (c >> 3) + 2 * (c & 3) + ((c & 7) >> 2) : 8 * ((c & 7) >> 2) + 2 * (c & 3) + (c >> 3);
}

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ float bf16_val(uint32_t b) { return __uint_as_float(b << 16); }

template <int SH>
__device__ __forceinline__ uint32_t shift(uint32_t w) {
  if constexpr (SH >= 0) return w >> SH;
  else return w << (-SH);
}

// The two 8-element B operands of one group from this lane's code bytes (see header).
// v_perm_b32 byte selectors: 0-3 take bytes of the second operand, 4 the fixed high byte.
template <int BITS>
constexpr uint32_t kHiBytes = BITS == 4 ? 0x42424242u : 0x41414141u;
template <int BITS>
constexpr float kCodeOffset = BITS == 4 ? 32.f : 8.f;  // o
template <int BITS>
constexpr float kCodeUnit = BITS == 4 ? 2.f : 1.f;  // u
constexpr uint32_t kSelEven = 0x04020400u;  // [x.b0, hi, x.b2, hi]
constexpr uint32_t kSelOdd = 0x04030401u;   // [x.b1, hi, x.b3, hi]
template <int BITS>
__device__ __forceinline__ void build_b(const uint32_t* w, u32x4& b0, u32x4& b1) {
  if constexpr (BITS == 4) {
    // w[h] holds columns 8h..8h+7 of the lane's 16, nibble p = column 8h + p; pair j of
    // half h is (8h + j, 8h + j + 4): the even nibbles go to bits 3-6 of the bytes of ev,
    // the odd ones to those of od
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t ev = (w[h] << 3) & 0x78787878u, od = (w[h] >> 1) & 0x78787878u;
      u32x4& b = h ? b1 : b0;
      b.x = __builtin_amdgcn_perm(kHiBytes<4>, ev, kSelEven);
      b.y = __builtin_amdgcn_perm(kHiBytes<4>, od, kSelEven);
      b.z = __builtin_amdgcn_perm(kHiBytes<4>, ev, kSelOdd);
      b.w = __builtin_amdgcn_perm(kHiBytes<4>, od, kSelOdd);
    }
  } else {
    // w[0] holds the lane's 16 columns, column i in bits 2i; byte m of t_r holds column
    // 4m + r in bits 4-5, and half h, pair r takes columns 4h + r and 4h + r + 8
    const uint32_t d = w[0];
    const uint32_t t0 = (d << 4) & 0x30303030u, t1 = (d << 2) & 0x30303030u;
    const uint32_t t2 = d & 0x30303030u, t3 = (d >> 2) & 0x30303030u;
    b0.x = __builtin_amdgcn_perm(kHiBytes<2>, t0, kSelEven);
    b0.y = __builtin_amdgcn_perm(kHiBytes<2>, t1, kSelEven);
    b0.z = __builtin_amdgcn_perm(kHiBytes<2>, t2, kSelEven);
    b0.w = __builtin_amdgcn_perm(kHiBytes<2>, t3, kSelEven);
    b1.x = __builtin_amdgcn_perm(kHiBytes<2>, t0, kSelOdd);
    b1.y = __builtin_amdgcn_perm(kHiBytes<2>, t1, kSelOdd);
    b1.z = __builtin_amdgcn_perm(kHiBytes<2>, t2, kSelOdd);
    b1.w = __builtin_amdgcn_perm(kHiBytes<2>, t3, kSelOdd);
  }
}

// 3 bits: the lane's low-plane dword as at 2 bits, plus the high-plane word of its 32-column
// half (kb / 2), shifted by 2 (kb % 2): the low bits of column 4m + r sit at bits 8m + 2r,
// + 1 of the dword and its third bit at 8m + 4 (r / 2) + r % 2 of the shifted word
// (fmoe_layout.h, hi_bit); byte m of t_r gets the code in bits 4-6.
__device__ __forceinline__ void build_b3(uint32_t d, uint32_t hw, int kb, u32x4& b0, u32x4& b1) {
  const uint32_t hs = hw >> (2 * (kb & 1));
  const uint32_t t0 = ((d << 4) & 0x30303030u) | ((hs << 6) & 0x40404040u);
  const uint32_t t1 = ((d << 2) & 0x30303030u) | ((hs << 5) & 0x40404040u);
  const uint32_t t2 = (d & 0x30303030u) | ((hs << 2) & 0x40404040u);
  const uint32_t t3 = ((d >> 2) & 0x30303030u) | ((hs << 1) & 0x40404040u);
  b0.x = __builtin_amdgcn_perm(kHiBytes<3>, t0, kSelEven);
  b0.y = __builtin_amdgcn_perm(kHiBytes<3>, t1, kSelEven);
  b0.z = __builtin_amdgcn_perm(kHiBytes<3>, t2, kSelEven);
  b0.w = __builtin_amdgcn_perm(kHiBytes<3>, t3, kSelEven);
  b1.x = __builtin_amdgcn_perm(kHiBytes<3>, t0, kSelOdd);
  b1.y = __builtin_amdgcn_perm(kHiBytes<3>, t1, kSelOdd);
  b1.z = __builtin_amdgcn_perm(kHiBytes<3>, t2, kSelOdd);
  b1.w = __builtin_amdgcn_perm(kHiBytes<3>, t3, kSelOdd);
}
__device__ __forceinline__ f32x4 mfma(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

struct BParams {
  const uint8_t* experts;
  size_t stride;
  int H, I, k;
  const int32_t* pairs;    // [P] pair ids (t * k + j) sorted by expert
  const int32_t* act_e;    // [n_act] expert of each work unit
  const int32_t* act_off;  // [n_act] first position of the unit in pairs
  const int32_t* act_cnt;  // [n_act] number of pairs of the unit (1..16)
  const int32_t* n_act;
  const uint16_t* v16;  // [T][H] bf16, operand order
  const float* xg;      // [T][H/64] group sums of v16
  uint16_t* a16;        // [P][I] bf16, operand order (pair-id rows)
  float* ag;            // [P][I/64] group sums of a16
  float* ys;            // [P][H] down outputs (pair-id rows)
};

// ---------------------------------------------------------------- 1. stage (one token)
// x = h * inv (inv = 1 / rms(h), or 1 without the pre-norm) as bf16 in operand order (v16)
// and, per group of 64 columns, the fp32 sum of the bf16 values (xg). One 16-column block
// per thread step; the 4 blocks of a group sit on 4 consecutive lanes (nthreads and the
// first thread's index are multiples of 64, so every group's lanes are active together).
template <int BITS>
__device__ __forceinline__ void stage_token(const float* __restrict__ hr, int H, float inv, uint16_t* __restrict__ v16r,
                                            float* __restrict__ xgr, int tid, int nthreads) {
  for (int blk = tid; blk < H / 16; blk += nthreads) {
    float x[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 f = reinterpret_cast<const float4*>(hr + blk * 16)[q];
      x[4 * q] = f.x * inv;
      x[4 * q + 1] = f.y * inv;
      x[4 * q + 2] = f.z * inv;
      x[4 * q + 3] = f.w * inv;
    }
    uint32_t r[16];
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      r[c] = bf16_rne(x[c]);
      s += bf16_val(r[c]);
    }
    uint32_t o[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) o[q] = r[perm_col<BITS>(2 * q)] | (r[perm_col<BITS>(2 * q + 1)] << 16);
    u32x4* dst = reinterpret_cast<u32x4*>(v16r + blk * 16);
    dst[0] = u32x4{o[0], o[1], o[2], o[3]};
    dst[1] = u32x4{o[4], o[5], o[6], o[7]};
    s = group_sum(s, 4);
    if ((blk & 3) == 0) xgr[blk / 4] = s;
  }
}

// ---------------------------------------------------------------- 2. route
// Router logits as an fp32 matrix-core product on the raw h (the pre-norm's 1 / rms is a
// per-token factor, applied to the summed logits by route_stage_kernel), with
// v_mfma_f32_16x16x4f32 (lane l holds A[l % 16][l / 16], B[l / 16][l % 16], result as above).
// Workgroup (e-tile, slice): 16 experts x one 512-column slice of K, for up to 64 tokens at a
// time, wave w taking the 16-token tile w; its partial logits part[slice][t][e] are written
// directly. The operands go through LDS in 128-column chunks: the global loads are in lane
// order (consecutive threads read consecutive 16-byte pieces of one row, so every lane quad
// reads one piece of a cache line; loaded in matrix-core order instead, a quad would span 4
// rows), and each row's 32 pieces sit in LDS as 8 blocks of 4 pieces plus one pad piece per
// row, so the 16-byte operand reads (16 rows, same block) fall on distinct banks. The next
// chunk's loads are in flight while the current one is multiplied.
constexpr int kRtSlice = 512;
constexpr int kRtChunk = 128;                     // columns per LDS chunk
constexpr int kRtBlocks = kRtChunk / 16;          // 16-column blocks per chunk
constexpr int kRtPad = 5;                         // 16-byte pieces per row and block slot (4 + pad)
constexpr int kRtTok = 64;                        // tokens per pass (4 waves x 16)
constexpr int kRtLoadsA = kRtTok * kRtChunk / 4 / kBT;  // float4 loads per thread per chunk
constexpr int kRtLoadsB = 16 * kRtChunk / 4 / kBT;
constexpr int kRtMaxParts = 16;  // slices of a hidden size up to 8192
static_assert(kRtLoadsA * kBT * 4 == kRtTok * kRtChunk && kRtLoadsB * kBT * 4 == 16 * kRtChunk, "chunk loads");

__device__ __forceinline__ f32x4 mfma4(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Lane-order loads of one chunk (columns k0 .. k0 + 127): item i = tid + kBT * u is the
// 16-byte piece i % 32 of row i / 32 (token rows past T and expert rows past E repeat the
// last one; their products are not stored).
__device__ __forceinline__ void rt_load_chunk(f32x4 (&ra)[kRtLoadsA], f32x4 (&rb)[kRtLoadsB],
                                              const float* __restrict__ R, const float* __restrict__ v, int tid,
                                              int t0, int T, int e0, int E, int H, int k0) {
#pragma unroll
  for (int u = 0; u < kRtLoadsA; ++u) {
    const int i = tid + kBT * u, t = min(t0 + i / 32, T - 1);
    ra[u] = reinterpret_cast<const f32x4*>(v + (size_t)t * H + k0)[i % 32];
  }
#pragma unroll
  for (int u = 0; u < kRtLoadsB; ++u) {
    const int i = tid + kBT * u, e = min(e0 + i / 32, E - 1);
    rb[u] = reinterpret_cast<const f32x4*>(R + (size_t)e * H + k0)[i % 32];
  }
}

__global__ void __launch_bounds__(kBT) router_kernel_mfma(const float* __restrict__ R, const float* __restrict__ v,
                                                          int T, int E, int H, float* __restrict__ part) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nl = lane & 15, kb = lane >> 4;
  const int e0 = blockIdx.x * 16, ks = blockIdx.y;
  const int k_lo = ks * kRtSlice, k_hi = min(H, k_lo + kRtSlice);
  const int n_chunks = (k_hi - k_lo) / kRtChunk;  // H % 128 == 0 (batched shapes)
  __shared__ f32x4 sA[kRtBlocks][kRtTok][kRtPad];  // [block][token][piece]
  __shared__ f32x4 sB[kRtBlocks][16][kRtPad];      // [block][expert][piece]
  for (int t0 = 0; t0 < T; t0 += kRtTok) {
    f32x4 ra[kRtLoadsA], rb[kRtLoadsB];
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    rt_load_chunk(ra, rb, R, v, tid, t0, T, e0, E, H, k_lo);
    for (int c = 0; c < n_chunks; ++c) {
      __syncthreads();  // the previous chunk's operand reads are done
#pragma unroll
      for (int u = 0; u < kRtLoadsA; ++u) {
        const int i = tid + kBT * u;
        sA[(i % 32) / 4][i / 32][i % 4] = ra[u];
      }
#pragma unroll
      for (int u = 0; u < kRtLoadsB; ++u) {
        const int i = tid + kBT * u;
        sB[(i % 32) / 4][i / 32][i % 4] = rb[u];
      }
      __syncthreads();
      // the next chunk (unconditional: after the last one, the last again, unused)
      rt_load_chunk(ra, rb, R, v, tid, t0, T, e0, E, H, k_lo + min(c + 1, n_chunks - 1) * kRtChunk);
      // tile of wave w: tokens t0 + 16 w + nl; block j's columns 16 j + 4 kb + (0..3)
#pragma unroll
      for (int j = 0; j < kRtBlocks; ++j) {
        const f32x4 a = sA[j][16 * wave + nl][kb];
        const f32x4 b = sB[j][nl][kb];
        acc = mfma4(a[0], b[0], acc);
        acc = mfma4(a[1], b[1], acc);
        acc = mfma4(a[2], b[2], acc);
        acc = mfma4(a[3], b[3], acc);
      }
    }
    // lane holds tokens t0 + 16 w + 4 kb + i, expert e0 + nl
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = t0 + 16 * wave + 4 * kb + i, e = e0 + nl;
      if (tok < T && e < E) part[((size_t)ks * T + tok) * E + e] = acc[i];
    }
  }
}

// ---------------------------------------------------------------- 3. sort by expert
// Pair s = t * k + j goes to expert idx[s]; pairs of one expert are contiguous in `pairs`
// (their order inside an expert does not affect any result: every token's rows are
// computed independently). The work list holds one unit per 16 pairs of an expert
// (expert, first position, count), so a hot expert's passes run in parallel. Run by the
// NT threads of one workgroup; cnt and cur are E ints of LDS each, sc 2 * NT ints.
template <int NT>
__device__ void sort_pairs(const int32_t* __restrict__ idx, int P, int E, int32_t* __restrict__ pairs,
                           int32_t* __restrict__ act_e, int32_t* __restrict__ act_off, int32_t* __restrict__ act_cnt,
                           int32_t* __restrict__ n_act, int* cnt, int* cur, int* sc) {
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += NT) cnt[e] = 0;
  __syncthreads();
  for (int s = tid; s < P; s += NT) atomicAdd(&cnt[ld_dev_u32(reinterpret_cast<const uint32_t*>(idx) + s)], 1);
  __syncthreads();
  const int per = (E + NT - 1) / NT;
  const int lo = min(tid * per, E), hi = min(lo + per, E);
  int c = 0, a = 0;
  for (int e = lo; e < hi; ++e) {
    c += cnt[e];
    a += (cnt[e] + 15) / 16;
  }
  // inclusive scans of (c, a) over the threads (Hillis-Steele)
  sc[tid] = c;
  sc[NT + tid] = a;
  __syncthreads();
  for (int d = 1; d < NT; d <<= 1) {
    const int vc = sc[tid] + (tid >= d ? sc[tid - d] : 0);
    const int va = sc[NT + tid] + (tid >= d ? sc[NT + tid - d] : 0);
    __syncthreads();
    sc[tid] = vc;
    sc[NT + tid] = va;
    __syncthreads();
  }
  int off = sc[tid] - c, act = sc[NT + tid] - a;
  for (int e = lo; e < hi; ++e) {
    cur[e] = off;
    for (int u = 0; 16 * u < cnt[e]; ++u) {  // one work unit per 16 pairs of the expert
      act_e[act] = e;
      act_off[act] = off + 16 * u;
      act_cnt[act] = min(16, cnt[e] - 16 * u);
      ++act;
    }
    off += cnt[e];
  }
  if (tid == NT - 1) *n_act = sc[NT + tid];
  __syncthreads();
  for (int s = tid; s < P; s += NT) pairs[atomicAdd(&cur[ld_dev_u32(reinterpret_cast<const uint32_t*>(idx) + s)], 1)] = s;
}

// Per token t (one workgroup): 1 / rms(h_t) under the pre-norm; the logits (slice partials
// summed in slice order, times that factor) written out and ranked; wave 0 takes the top-k
// and the softmax over the selected logits while waves 1-3 write the token's v16 and group
// sums. The selected experts are stored at the device coherence point; once they are
// acknowledged the workgroup counts itself on a device-scope counter, and the workgroup
// that finishes last reads all T * k selections back from the coherence point, sorts the
// pairs by expert and resets the counter for the next call. (A device-scope fence instead
// would write back this XCD's whole L2.) With a shared expert (gate != null) every token has
// ks = k + 1 slots: slot k is expert E with weight 1 / (1 + exp(-gate . v)).
template <int BITS>
__global__ void __launch_bounds__(kBT) route_stage_kernel(const float* __restrict__ h, int prenorm, float eps,
                                                          const float* __restrict__ part, int n_part, int T, int E,
                                                          int H, int k, const float* __restrict__ gate, int ks,
                                                          float* __restrict__ logits,
                                                          int32_t* __restrict__ idx, float* __restrict__ w,
                                                          uint16_t* __restrict__ v16, float* __restrict__ xg,
                                                          int32_t* __restrict__ pairs, int32_t* __restrict__ act_e,
                                                          int32_t* __restrict__ act_off, int32_t* __restrict__ act_cnt,
                                                          int32_t* __restrict__ n_act, uint32_t* __restrict__ done) {
  const int t = blockIdx.x, lane = threadIdx.x & 63;
  const float* hr = h + (size_t)t * H;
  __shared__ uint64_t keys[4096];  // also the sort's two E-int arrays
  __shared__ int sc[2 * kBT];
  __shared__ float lsel[16], wsel[16], red[kBT / 64];
  __shared__ int isel[16];
  __shared__ int is_last;
  __shared__ float gred[kBT / 64];
  float inv = 1.f, gdot = 0.f;
  if (prenorm || gate) {
    float ss = 0.f, gd = 0.f;
    for (int i = threadIdx.x; i < H / 4; i += kBT) {
      const float4 q = reinterpret_cast<const float4*>(hr)[i];
      ss = fmaf(q.x, q.x, ss);
      ss = fmaf(q.y, q.y, ss);
      ss = fmaf(q.z, q.z, ss);
      ss = fmaf(q.w, q.w, ss);
      if (gate) {
        const float4 g4 = reinterpret_cast<const float4*>(gate)[i];
        gd = fmaf(g4.x, q.x, gd);
        gd = fmaf(g4.y, q.y, gd);
        gd = fmaf(g4.z, q.z, gd);
        gd = fmaf(g4.w, q.w, gd);
      }
    }
    ss = wave_sum(ss);
    gd = wave_sum(gd);
    if (lane == 0) {
      red[threadIdx.x >> 6] = ss;
      gred[threadIdx.x >> 6] = gd;
    }
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int q = 0; q < kBT / 64; ++q) {
      tot += red[q];
      gdot += gred[q];
    }
    if (prenorm) inv = 1.0f / sqrtf(tot / (float)H + eps);
  }
  for (int e = threadIdx.x; e < E; e += kBT) {
    // all slices' loads first (clamped, unconditional), then the sum in slice order
    float x[kRtMaxParts];
#pragma unroll
    for (int q = 0; q < kRtMaxParts; ++q) x[q] = part[((size_t)min(q, n_part - 1) * T + t) * E + e];
    float l = 0.f;
#pragma unroll
    for (int q = 0; q < kRtMaxParts; ++q) l = q < n_part ? l + x[q] : l;
    l *= inv;
    logits[(size_t)t * E + e] = l;
    keys[e] = rank_key(l, e);
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    if (E <= 512) {
      uint64_t kr[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) kr[j] = lane + 64 * j < E ? keys[lane + 64 * j] : 0ull;
      wave_topk_regs<8>(kr, k, isel, lsel, wsel);
    } else {
      wave_topk_keys(keys, E, k, isel, lsel, wsel);
    }
  } else {
    stage_token<BITS>(hr, H, inv, v16 + (size_t)t * H, xg + (size_t)t * (H / 64), threadIdx.x - 64, kBT - 64);
  }
  __syncthreads();
  if (threadIdx.x < k) {
    st_dev_u32(reinterpret_cast<uint32_t*>(idx) + (size_t)t * ks + threadIdx.x, (uint32_t)isel[threadIdx.x]);
    w[(size_t)t * ks + threadIdx.x] = wsel[threadIdx.x];
  } else if (gate && (int)threadIdx.x == k) {  // the shared expert's slot (gate . v = inv * gate . h)
    st_dev_u32(reinterpret_cast<uint32_t*>(idx) + (size_t)t * ks + k, (uint32_t)E);
    w[(size_t)t * ks + k] = 1.0f / (1.0f + expf(-gdot * inv));
  }
  wait_vmem();  // idx acknowledged at the device coherence point (read by the last workgroup)
  __syncthreads();
  if (threadIdx.x == 0) is_last = atomicAdd(done, 1u) == (uint32_t)(T - 1);
  __syncthreads();
  if (!is_last) return;  // uniform over the workgroup
  int* cnt = reinterpret_cast<int*>(keys);
  const int EB = E + (gate ? 1 : 0);  // expert buckets of the sort
  sort_pairs<kBT>(idx, T * ks, EB, pairs, act_e, act_off, act_cnt, n_act, cnt, cnt + EB, sc);
  if (threadIdx.x == 0) st_dev_u32(done, 0u);
}

// ---------------------------------------------------------------- 4./5. expert products
// Stage the per-group activation sums of the pass's m-tiles: xs[mt][g][m].
__device__ __forceinline__ void stage_sums(float* xs, const BParams& p, const float* sums, int G, int off, int cnt,
                                           int m0, int nmt, bool by_token) {
  for (int i = threadIdx.x; i < nmt * G * 16; i += kBT) {
    const int m = i & 15, g = (i >> 4) % G, mt = (i >> 4) / G;
    const int r = m0 + mt * 16 + m;
    float val = 0.f;
    if (r < cnt) {
      const int s = p.pairs[off + r];
      const int row = by_token ? s / p.k : s;
      val = sums[(size_t)row * G + g];
    }
    xs[(mt * G + g) * 16 + m] = val;
  }
}

// Each wave owns 64 weight rows (4 tiles of 16) and streams them through a private,
// double-buffered LDS region in stages of GC groups: one 16-byte LDS-DMA
// (global_load_lds) per lane moves 1 KB of whole row segments per instruction, so every
// memory line is fetched once, in full (a direct fragment load would touch 16 rows x 32
// bytes per instruction). The scale/bias words of a stage arrive as one 16-byte load per
// tile, and the token operands as two 16-byte loads per group; both go to registers.
// Stage layout in LDS: instruction j carries rows j * RPI .. + RPI - 1; lane i of it
// brings 16-byte segment i / RPI of row j * RPI + i % RPI, stored at j * 1024 + 16 i.
//
// Waits. The LDS-DMA is issued from asm and the stage buffers are read from asm, so the
// compiler neither sees the DMA in flight nor places waits of its own for it: with an
// LDS-DMA pending it would wait for every outstanding load before the first use of any
// loaded register, which serialises the stages. The compiler's waits for the register
// loads stay correct (it counts only the loads it knows of, which can only make a wait
// stricter). A wave's vector loads, LDS-DMA included, complete in issue order, so the
// explicit wait before a stage is read lets exactly the loads of the stages issued after
// it stay in flight.
constexpr int kWaveRows = 64;

template <int BITS, int GC>
struct StageGeom {
  static constexpr int kLB = BITS == 3 ? 2 : BITS;  // code width of the (low) plane's layout
  static constexpr int kBPG = kLB * 8;           // (low-plane) code bytes per row per group
  static constexpr int kRS = GC * kBPG;          // bytes per row per stage
  static constexpr int kRPI = 1024 / kRS;        // rows per DMA instruction
  static constexpr int kNJ = kWaveRows / kRPI;   // DMA instructions per stage
  static constexpr int kLoBytes = kWaveRows * kRS;
  // 3 bits: the high plane's two words per (row, group) follow in the stage buffer, one KB
  // per DMA instruction (4-group stages: 32 rows' whole pieces; 2-group stages: 16 bytes of
  // each of the 64 rows)
  static constexpr int kHRS = BITS == 3 ? 8 * GC : 0;        // high-plane bytes per row per stage
  static constexpr int kNJH = kWaveRows * kHRS / 1024;       // its DMA instructions
  static constexpr int kBytes = kLoBytes + kWaveRows * kHRS;  // LDS bytes of one stage
  static constexpr int kLoads = 4 + 2 * GC + kNJ + kNJH;  // vector memory instructions per stage
};

// b in the lanes of `lanes` (a constant lane mask), a elsewhere: one v_cndmask with the mask
// in scalar registers (written as asm so that a chain of them over one register array is not
// turned into a dynamically indexed copy of the array in scratch memory).
__device__ __forceinline__ uint32_t lane_pick(uint32_t a, uint32_t b, uint64_t lanes) {
  uint32_t r;
  asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "s"(lanes));
  return r;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// 16 bytes per lane from global memory to LDS: lane i's bytes land at lds + 16 i (lds is
// the wave-uniform LDS byte address, passed through M0). The weights are read once per pass,
// so the load carries the non-temporal policy (measured on a read-only 4 GiB stream through
// LDS-DMA: 6.75 TB/s against 6.11 TB/s without it).
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off nt" ::"v"(g),
      "s"(__builtin_amdgcn_readfirstlane(lds))
      : "memory", "m0");
}
// Wait until at most N of this wave's vector memory instructions are outstanding (the
// compiler does not wait for LDS-DMA data by itself).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lgkm() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Register part of one stage: scale/bias words of its GC groups for the 4 tiles, and the
// token operand of each group (two 8-element halves).
template <int GC>
struct StageRegs {
  uint32_t sb[4][GC];
  u32x4 a[GC][2];
};

// src(j, g0): the lane's 16 source bytes for DMA instruction j of the stage at group g0;
// sbs(t, g0): the lane's scale/bias words of tile t for groups g0 .. g0 + GC - 1.
template <int BITS, int GC, typename Src, typename HSrc, typename SbSrc>
__device__ __forceinline__ void issue_stage(char* buf, StageRegs<GC>& r, Src src, HSrc hsrc, SbSrc sbs,
                                            const uint16_t* tp, int g0, int lane) {
  using SG = StageGeom<BITS, GC>;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    if constexpr (GC == 4) {
      const uint4 q = *reinterpret_cast<const uint4*>(sbs(t, g0));
      r.sb[t][0] = q.x;
      r.sb[t][1] = q.y;
      r.sb[t][2] = q.z;
      r.sb[t][3] = q.w;
    } else {
      const uint2 q = *reinterpret_cast<const uint2*>(sbs(t, g0));
      r.sb[t][0] = q.x;
      r.sb[t][1] = q.y;
    }
  }
#pragma unroll
  for (int gl = 0; gl < GC; ++gl) {
    const u32x4* ap = reinterpret_cast<const u32x4*>(tp + (size_t)(g0 + gl) * 64);
    r.a[gl][0] = ap[0];
    r.a[gl][1] = ap[1];
  }
  const uint32_t lb = lds_addr(buf);
#pragma unroll
  for (int j = 0; j < SG::kNJ; ++j) dma16(src(j, g0), lb + j * 1024);
#pragma unroll
  for (int j = 0; j < SG::kNJH; ++j) dma16(hsrc(j, g0), lb + SG::kLoBytes + j * 1024);
}

// Byte offset in a stage buffer of weight row R's code bytes at offset `off` of its stage
// segment (layout above). For R = 16 t + nl and off = gl * kBPG + lane part it is the sum of
// a per-lane term, a per-tile term and a per-group term.
template <int BITS, int GC>
__host__ __device__ constexpr int stage_off(int R, int off) {
  using SG = StageGeom<BITS, GC>;
  return (R / SG::kRPI) * 1024 + ((off / 16) * SG::kRPI + R % SG::kRPI) * 16 + off % 16;
}

// One group's LDS operands: the lane's code bytes of the 4 tiles (at base + T1 * t) and,
// with WX (the stage's first group), the lane's activation group sum X[token nl][g0 + kb]
// for the stage's bias product (at xaddr), read in one asm block that also waits for them.
// The reads are written in asm because the compiler, unable to tell them apart from the
// stage buffers that LDS-DMA is still filling, would otherwise wait for every load in flight
// before them.
template <bool WX, int T1, int T2, int T3>
__device__ __forceinline__ void read_group4(uint32_t base, uint32_t xaddr, uint32_t (&w)[4][2], float& xa) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  u32x2 q0, q1, q2, q3;
  if constexpr (WX) {
    asm volatile(
        "ds_read_b64 %0, %5\n"
        "ds_read_b64 %1, %5 offset:%7\n"
        "ds_read_b64 %2, %5 offset:%8\n"
        "ds_read_b64 %3, %5 offset:%9\n"
        "ds_read_b32 %4, %6\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(q0), "=&v"(q1), "=&v"(q2), "=&v"(q3), "=&v"(xa)
        : "v"(base), "v"(xaddr), "n"(T1), "n"(T2), "n"(T3)
        : "memory");
  } else {
    asm volatile(
        "ds_read_b64 %0, %4\n"
        "ds_read_b64 %1, %4 offset:%5\n"
        "ds_read_b64 %2, %4 offset:%6\n"
        "ds_read_b64 %3, %4 offset:%7\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(q0), "=&v"(q1), "=&v"(q2), "=&v"(q3)
        : "v"(base), "n"(T1), "n"(T2), "n"(T3)
        : "memory");
  }
  w[0][0] = q0.x, w[0][1] = q0.y, w[1][0] = q1.x, w[1][1] = q1.y;
  w[2][0] = q2.x, w[2][1] = q2.y, w[3][0] = q3.x, w[3][1] = q3.y;
}
template <bool WX, int T1, int T2, int T3>
__device__ __forceinline__ void read_group2(uint32_t base, uint32_t xaddr, uint32_t (&w)[4][2], float& xa) {
  uint32_t q0, q1, q2, q3;
  if constexpr (WX) {
    asm volatile(
        "ds_read_b32 %0, %5\n"
        "ds_read_b32 %1, %5 offset:%7\n"
        "ds_read_b32 %2, %5 offset:%8\n"
        "ds_read_b32 %3, %5 offset:%9\n"
        "ds_read_b32 %4, %6\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(q0), "=&v"(q1), "=&v"(q2), "=&v"(q3), "=&v"(xa)
        : "v"(base), "v"(xaddr), "n"(T1), "n"(T2), "n"(T3)
        : "memory");
  } else {
    asm volatile(
        "ds_read_b32 %0, %4\n"
        "ds_read_b32 %1, %4 offset:%5\n"
        "ds_read_b32 %2, %4 offset:%6\n"
        "ds_read_b32 %3, %4 offset:%7\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(q0), "=&v"(q1), "=&v"(q2), "=&v"(q3)
        : "v"(base), "n"(T1), "n"(T2), "n"(T3)
        : "memory");
  }
  w[0][0] = q0, w[1][0] = q1, w[2][0] = q2, w[3][0] = q3;
  w[0][1] = w[1][1] = w[2][1] = w[3][1] = 0;
}

// 3 bits: the 2-bit read plus the lane's high-plane word of each tile (at hbase + H1 * t).
template <bool WX, int T1, int T2, int T3, int H1, int H2, int H3>
__device__ __forceinline__ void read_group3(uint32_t base, uint32_t hbase, uint32_t xaddr, uint32_t (&w)[4][2],
                                            uint32_t (&hw)[4], float& xa) {
  uint32_t q0, q1, q2, q3, g0, g1, g2, g3;
  if constexpr (WX) {
    asm volatile(
        "ds_read_b32 %0, %9\n"
        "ds_read_b32 %1, %9 offset:%12\n"
        "ds_read_b32 %2, %9 offset:%13\n"
        "ds_read_b32 %3, %9 offset:%14\n"
        "ds_read_b32 %4, %10\n"
        "ds_read_b32 %5, %10 offset:%15\n"
        "ds_read_b32 %6, %10 offset:%16\n"
        "ds_read_b32 %7, %10 offset:%17\n"
        "ds_read_b32 %8, %11\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(q0), "=&v"(q1), "=&v"(q2), "=&v"(q3), "=&v"(g0), "=&v"(g1), "=&v"(g2), "=&v"(g3), "=&v"(xa)
        : "v"(base), "v"(hbase), "v"(xaddr), "n"(T1), "n"(T2), "n"(T3), "n"(H1), "n"(H2), "n"(H3)
        : "memory");
  } else {
    asm volatile(
        "ds_read_b32 %0, %8\n"
        "ds_read_b32 %1, %8 offset:%10\n"
        "ds_read_b32 %2, %8 offset:%11\n"
        "ds_read_b32 %3, %8 offset:%12\n"
        "ds_read_b32 %4, %9\n"
        "ds_read_b32 %5, %9 offset:%13\n"
        "ds_read_b32 %6, %9 offset:%14\n"
        "ds_read_b32 %7, %9 offset:%15\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(q0), "=&v"(q1), "=&v"(q2), "=&v"(q3), "=&v"(g0), "=&v"(g1), "=&v"(g2), "=&v"(g3)
        : "v"(base), "v"(hbase), "n"(T1), "n"(T2), "n"(T3), "n"(H1), "n"(H2), "n"(H3)
        : "memory");
  }
  w[0][0] = q0, w[1][0] = q1, w[2][0] = q2, w[3][0] = q3;
  w[0][1] = w[1][1] = w[2][1] = w[3][1] = 0;
  hw[0] = g0, hw[1] = g1, hw[2] = g2, hw[3] = g3;
}

// acc[tile] += u times the affine group products of the GC groups of one stage (see the
// header: codes enter the matrix core as the exact bf16 values o + u q; per group s P, and
// per stage one fp32 product of the group sums X with u b - o s).
// Stage buffer layouts. 4-group stages hold the code layout's own bytes (fmoe_layout.h):
// instruction j's KB holds rows j * kRPI .. + kRPI - 1, each row's piece contiguous with
// its 16-byte chunks rotated by rot(row). 2-group stages use the layout of stage_off.
template <int BITS, int GC>
__device__ __forceinline__ void compute_stage(f32x4 (&acc)[4], const char* buf, const StageRegs<GC>& r,
                                              const float* xs, int g0, int nl, int kb) {
  using SG = StageGeom<BITS, GC>;
  using CL = CodeLayout<SG::kLB>;
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  constexpr bool kPiece = GC == 4;  // the stage is one piece of the code layout
  const int lane_part = kb * (SG::kLB * 2);  // the lane's code bytes within a group's kBPG
  // 3 bits: the lane's high-plane word of group gl, tile 0 (row nl), word kb / 2; 4-group
  // stages hold 32 rows' pieces (32 bytes per row) per KB, 2-group stages 16 bytes per row
  const uint32_t h_base = lds_addr(buf) + SG::kLoBytes + (kPiece ? nl * 32 : nl * 16) + (kb >> 1) * 4;
  const uint32_t lane_base = kPiece ? lds_addr(buf) + (nl / SG::kRPI) * 1024 + (nl % SG::kRPI) * SG::kRS + lane_part % 16
                                    : lds_addr(buf) + stage_off<BITS, GC>(nl, lane_part);
  // A operand of the bias product: X[token nl][group g0 + kb] (zero for kb >= GC; the read
  // stays inside the LDS: xs is followed by the stage buffers)
  const uint32_t x_addr = lds_addr(xs + (g0 + kb) * 16 + nl);
  float xa = 0.f;
#pragma unroll
  for (int gl = 0; gl < GC; ++gl) {
    uint32_t w[4][2];
    uint32_t gbase;
    if constexpr (kPiece) {
      const int k = (gl * SG::kBPG + lane_part) / 16;  // the lane's chunk of the row's piece
      gbase = lane_base + ((k + CL::rot(nl)) % (SG::kRS / 16)) * 16;
    } else {
      gbase = lane_base + stage_off<BITS, GC>(0, gl * SG::kBPG);
    }
    constexpr int T1 = kPiece ? (16 / SG::kRPI) * 1024 : stage_off<BITS, GC>(16, 0);
    constexpr int T2 = kPiece ? 2 * T1 : stage_off<BITS, GC>(32, 0);
    constexpr int T3 = kPiece ? 3 * T1 : stage_off<BITS, GC>(48, 0);
    uint32_t hw[4] = {0u, 0u, 0u, 0u};
    if (gl == 0) {
      if constexpr (BITS == 4) read_group4<true, T1, T2, T3>(gbase, x_addr, w, xa);
      else if constexpr (BITS == 3)
        read_group3<true, T1, T2, T3, kPiece ? 512 : 256, kPiece ? 1024 : 512, kPiece ? 1536 : 768>(gbase, h_base,
                                                                                               x_addr, w, hw, xa);
      else read_group2<true, T1, T2, T3>(gbase, x_addr, w, xa);
      if (kb >= GC) xa = 0.f;
    } else {
      if constexpr (BITS == 4) read_group4<false, T1, T2, T3>(gbase, 0u, w, xa);
      else if constexpr (BITS == 3)
        read_group3<false, T1, T2, T3, kPiece ? 512 : 256, kPiece ? 1024 : 512, kPiece ? 1536 : 768>(
            gbase, h_base + gl * 8, 0u, w, hw, xa);
      else read_group2<false, T1, T2, T3>(gbase, 0u, w, xa);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      u32x4 b0, b1;
      if constexpr (BITS == 3) build_b3(w[t][0], hw[t], kb, b0, b1);
      else build_b<BITS>(w[t], b0, b1);
      const float cs = bf16_lo(r.sb[t][gl]);
      f32x4 P = mfma(r.a[gl][0], b0, zero);
      P = mfma(r.a[gl][1], b1, P);
      acc[t][0] = fmaf(cs, P[0], acc[t][0]);
      acc[t][1] = fmaf(cs, P[1], acc[t][1]);
      acc[t][2] = fmaf(cs, P[2], acc[t][2]);
      acc[t][3] = fmaf(cs, P[3], acc[t][3]);
    }
    __builtin_amdgcn_sched_barrier(0);  // one group at a time: bounds the live fragments
  }
  // the stage's bias term: tile t += X (tokens x groups) times (u b - o s) (groups x rows);
  // last in the stage, so that its latency passes while the next stage's first group is
  // read and unpacked
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    // the lane's own group's word (group g0 + kb; the X operand is zero for kb >= GC)
    uint32_t wk = lane_pick(r.sb[t][0], r.sb[t][1], 0x00000000FFFF0000ull);
    if constexpr (GC == 4) {
      wk = lane_pick(wk, r.sb[t][2], 0x0000FFFF00000000ull);
      wk = lane_pick(wk, r.sb[t][3], 0xFFFF000000000000ull);
    }
    acc[t] = mfma4(xa, fmaf(-kCodeOffset<BITS>, bf16_lo(wk), kCodeUnit<BITS> * bf16_hi(wk)), acc[t]);
  }
}

// All G groups of a pass (GC * U divides G): blocks of U stages, two stages in flight
// inside a block (stage u + 2 is requested once stage u is read). A block issues and
// consumes all of its own loads, so nothing is in flight across the loop's back edge. With
// U = G / GC (the stage counts of the common shapes) the pass is one block: the loads never
// drain between stages.
template <int BITS, int GC, int U, typename Src, typename HSrc, typename SbSrc>
__device__ __forceinline__ void expert_pass(f32x4 (&acc)[4], char* wbuf, Src src, HSrc hsrc, SbSrc sptr,
                                            const uint16_t* tp, const float* xs, int G, int lane, int nl, int kb) {
  using SG = StageGeom<BITS, GC>;
  for (int s0 = 0; s0 < G / GC; s0 += U) {
    StageRegs<GC> r[2];
    issue_stage<BITS, GC>(wbuf, r[0], src, hsrc, sptr, tp, s0 * GC, lane);
    if constexpr (U > 1) issue_stage<BITS, GC>(wbuf + SG::kBytes, r[1], src, hsrc, sptr, tp, (s0 + 1) * GC, lane);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (u + 1 < U) wait_vmcnt<SG::kLoads>();
      else wait_vmcnt<0>();
      compute_stage<BITS, GC>(acc, wbuf + (u % 2) * SG::kBytes, r[u % 2], xs, (s0 + u) * GC, nl, kb);
      if (u + 2 < U) {
        wait_lgkm();  // the stage's reads of this buffer are done before the DMA refills it
        issue_stage<BITS, GC>(wbuf + (u % 2) * SG::kBytes, r[u % 2], src, hsrc, sptr, tp, (s0 + u + 2) * GC, lane);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// The pass with the largest block that divides the stage count: the whole pass for 16 and
// 8 stages (hidden or inter 4096 and 2048 with 4-group stages; 1024 is one block of 4),
// else blocks of 4, 2 or 1 stages.
template <int BITS, int GC, typename Src, typename HSrc, typename SbSrc>
__device__ __forceinline__ void expert_pass_any_u(f32x4 (&acc)[4], char* wbuf, Src src, HSrc hsrc, SbSrc sptr,
                                                  const uint16_t* tp, const float* xs, int G, int lane, int nl,
                                                  int kb) {
  const int NS = G / GC;
  if (NS == 16) expert_pass<BITS, GC, 16>(acc, wbuf, src, hsrc, sptr, tp, xs, G, lane, nl, kb);
  else if (NS == 8) expert_pass<BITS, GC, 8>(acc, wbuf, src, hsrc, sptr, tp, xs, G, lane, nl, kb);
  else if (NS % 4 == 0) expert_pass<BITS, GC, 4>(acc, wbuf, src, hsrc, sptr, tp, xs, G, lane, nl, kb);
  else if (NS % 2 == 0) expert_pass<BITS, GC, 2>(acc, wbuf, src, hsrc, sptr, tp, xs, G, lane, nl, kb);
  else expert_pass<BITS, GC, 1>(acc, wbuf, src, hsrc, sptr, tp, xs, G, lane, nl, kb);
}

// Stage width for G groups (G even for every accepted shape). Wave row R
// lives in the matrix at mat_of(R) (rows_of rows of row_bytes bytes), row row_of(R).
// With 4-group stages every stage is one piece of the code layout (fmoe_layout.h): the
// instructions of a 32-row half read one contiguous run of it, and a lane's source is its
// base for stage 0 plus one run per stage; 2-group stages (G % 4 == 2, where a row ends in
// a half piece) take the general offset.
template <int BITS, typename MatOf, typename RowOf>
__device__ __forceinline__ void expert_pass_any(f32x4 (&acc)[4], char* wbuf, MatOf mat_of, RowOf row_of,
                                                int rows_of, size_t row_bytes, const uint32_t* const (&sbm)[4],
                                                const int (&sbr)[4],
                                                const uint16_t* tp, const float* xs, int G, int lane, int nl, int kb) {
  constexpr int LB = BITS == 3 ? 2 : BITS;
  // 3 bits: the high plane (two words per (row, group), blocked in 32-row blocks, fmoe_layout.h)
  // starts after the low plane of each matrix
  auto hi_of = [&](int R) {
    return reinterpret_cast<const uint32_t*>(mat_of(R) + lo_plane_bytes(rows_of, G * 64));
  };
  if (G % 4 == 0) {
    using SG = StageGeom<BITS, 4>;
    static_assert(SG::kRPI == CodeLayout<LB>::kSubRows && SG::kRS == CodeLayout<LB>::kPieceBytes,
                  "a 4-group stage instruction is one contiguous KB of the code layout");
    const uint8_t* dmarow[SG::kNJ];
    int run[SG::kNJ];  // bytes from one piece of the instruction's rows to the next
#pragma unroll
    for (int j = 0; j < SG::kNJ; ++j) {  // rows j * kRPI .. (consecutive, kRPI-aligned): lane l takes byte 16 l
      const int R = j * SG::kRPI;
      const size_t o0 = code_offset<LB>(rows_of, row_bytes, row_of(R), 0);
      dmarow[j] = mat_of(R) + o0 + 16 * lane;
      run[j] = (int)(code_offset<LB>(rows_of, row_bytes, row_of(R), SG::kRS) - o0);
    }
    auto src = [&](int j, int g0) { return dmarow[j] + (size_t)(g0 / 4) * run[j]; };
    // high plane: instruction j takes the piece of wave rows 32 j .. 32 j + 31 (one 32-row
    // block of one matrix: the wave's row halves start at multiples of 32), one KB per
    // piece, lane l bytes 16 l .. 16 l + 15
    const uint8_t* hrow[SG::kNJH > 0 ? SG::kNJH : 1];
#pragma unroll
    for (int j = 0; j < SG::kNJH; ++j)
      hrow[j] = reinterpret_cast<const uint8_t*>(hi_of(32 * j) + hi_offset(rows_of, G, row_of(32 * j), 0, 0)) +
                16 * lane;
    auto hsrc = [&](int j, int g0) { return hrow[j] + (size_t)(g0 / 4) * 1024; };
    const uint32_t* sp[4];  // the lane's scale/bias piece at stage 0; a stage is 32 rows x 4 words further
#pragma unroll
    for (int t = 0; t < 4; ++t) sp[t] = sbm[t] + sb_offset(rows_of, G, sbr[t], 0);
    auto sptr = [&](int t, int g0) { return sp[t] + (g0 / 4) * 128; };
    expert_pass_any_u<BITS, 4>(acc, wbuf, src, hsrc, sptr, tp, xs, G, lane, nl, kb);
  } else {
    using SG = StageGeom<BITS, 2>;
    const uint8_t* mat[SG::kNJ];
    int row[SG::kNJ];
#pragma unroll
    for (int j = 0; j < SG::kNJ; ++j) {
      const int R = j * SG::kRPI + lane % SG::kRPI;
      mat[j] = mat_of(R);
      row[j] = row_of(R);
    }
    const int seg = 16 * (lane / SG::kRPI);
    auto src = [&](int j, int g0) {
      return mat[j] + code_offset<LB>(rows_of, row_bytes, row[j], (size_t)g0 * SG::kBPG + seg);
    };
    // high plane: one instruction, lane l the 16 bytes (groups g0, g0 + 1) of wave row l
    const uint32_t* hl = hi_of(lane);
    const int hr = row_of(lane);
    auto hsrc = [&](int, int g0) { return hl + hi_offset(rows_of, G, hr, g0, 0); };
    auto sptr = [&](int t, int g0) { return sbm[t] + sb_offset(rows_of, G, sbr[t], g0); };
    expert_pass<BITS, 2, 1>(acc, wbuf, src, hsrc, sptr, tp, xs, G, lane, nl, kb);
  }
}

// LDS of one wave's stage buffers (the larger of the two stage widths).
template <int BITS>
constexpr int wave_stage_bytes() {
  return 2 * (StageGeom<BITS, 4>::kBytes > StageGeom<BITS, 2>::kBytes ? StageGeom<BITS, 4>::kBytes
                                                                       : StageGeom<BITS, 2>::kBytes);
}

// Token operand row of the lane for the pass's 16-token tile: rows past the expert's count
// point at its last pair (their products land in output rows that are never stored).
__device__ __forceinline__ const uint16_t* token_row(const uint16_t* base, const BParams& p, int off, int cnt, int m0,
                                                     int nl, int kb, size_t row_len, bool by_token) {
  const int r = min(m0 + nl, cnt - 1);
  const int s = p.pairs[off + r];
  return base + (size_t)(by_token ? s / p.k : s) * row_len + kb * 16;
}

// Dynamic LDS of the expert kernels: group sums of the pass's tokens, then the waves'
// stage buffers.
template <int BITS>
size_t expert_smem_bytes(int G) {
  return (size_t)G * 16 * 4 + (size_t)(kBT / 64) * wave_stage_bytes<BITS>();
}

template <int BITS>
__global__ void __launch_bounds__(kBT, 2) gate_up_kernel(BParams p) {
  const int item = blockIdx.y;
  if (item >= *p.n_act) return;
  const int e = p.act_e[item], off = p.act_off[item], cnt = p.act_cnt[item];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nl = lane & 15, kb = lane >> 4;
  const int H = p.H, I = p.I, G = H / 64;
  const uint8_t* blob = p.experts + (size_t)e * p.stride;
  const size_t cbytes = (size_t)I * H * BITS / 8, sbytes = (size_t)I * G * 4;
  const size_t rowb = (size_t)H * (BITS == 3 ? 2 : BITS) / 8;  // (low-plane) code bytes per row
  const int row0 = blockIdx.x * kGuRowsWg + wave * kGuRowsWave;
  // tiles 0, 1: gate rows row0 .. row0 + 31; tiles 2, 3: the same rows of up
  const uint32_t* sbm[4];  // scale/bias matrix and row of each tile (blocked layout, fmoe_layout.h)
  int sbr[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    sbr[t] = row0 + 16 * (t & 1) + nl;
    sbm[t] = reinterpret_cast<const uint32_t*>(blob + 3 * cbytes + (t < 2 ? 0 : sbytes));
  }
  // wave row R: tile R / 16 (0, 1 gate; 2, 3 up), row R % 16 of it
  auto mat_of = [&](int R) { return blob + (R < 32 ? 0 : cbytes); };
  auto row_of = [&](int R) { return row0 + 16 * ((R / 16) & 1) + R % 16; };
  extern __shared__ float smem_f[];
  float* xs = smem_f;  // [G][16]
  char* wbuf = reinterpret_cast<char*>(smem_f + G * 16) + wave * wave_stage_bytes<BITS>();
  __shared__ float agp[kBT / 64][16];  // per-wave sums of a16 over its 32 rows
  const int Gd = I / 64;
  for (int m0 = 0; m0 < cnt; m0 += 16) {
    __syncthreads();
    stage_sums(xs, p, p.xg, G, off, cnt, m0, 1, true);
    __syncthreads();
    const uint16_t* tp = token_row(p.v16, p, off, cnt, m0, nl, kb, (size_t)H, true);
    f32x4 acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    expert_pass_any<BITS>(acc, wbuf, mat_of, row_of, I, rowb, sbm, sbr, tp, xs, G, lane, nl, kb);
    // epilogue: a = silu(g) * u -> bf16 in the down operand's order; group sums of the
    // rounded values
    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int n = row0 + 16 * t + nl;
      const int col = (n & ~15) + perm_pos<BITS>(n & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = m0 + 4 * kb + i;
        const uint32_t b = bf16_rne(swiglu(acc[t][i] / kCodeUnit<BITS>, acc[t + 2][i] / kCodeUnit<BITS>));
        if (r < cnt) {
          p.a16[(size_t)p.pairs[off + r] * I + col] = (uint16_t)b;
          part[i] += bf16_val(b);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) part[i] = group_sum(part[i], 16);
    if (nl == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) agp[wave][4 * kb + i] = part[i];
    }
    __syncthreads();
    // waves 2q and 2q+1 cover the 64 rows of down group 2 * blockIdx.x + q
    for (int i = threadIdx.x; i < 2 * 16; i += kBT) {
      const int q = i / 16, m = i % 16;
      const int r = m0 + m;
      if (r < cnt) p.ag[(size_t)p.pairs[off + r] * Gd + 2 * blockIdx.x + q] = agp[2 * q][m] + agp[2 * q + 1][m];
    }
  }
}

template <int BITS>
__global__ void __launch_bounds__(kBT, 2) down_kernel(BParams p) {
  const int item = blockIdx.y;
  if (item >= *p.n_act) return;
  const int e = p.act_e[item], off = p.act_off[item], cnt = p.act_cnt[item];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nl = lane & 15, kb = lane >> 4;
  const int H = p.H, I = p.I, G = I / 64;
  const uint8_t* blob = p.experts + (size_t)e * p.stride;
  const size_t cbytes = (size_t)I * H * BITS / 8, sbytes = (size_t)H * G * 4;
  const size_t rowb = (size_t)I * (BITS == 3 ? 2 : BITS) / 8;  // (low-plane) code bytes per row
  const int row0 = blockIdx.x * kDnRowsWg + wave * kDnRowsWave;
  const uint32_t* sbm[4];
  int sbr[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    sbr[t] = row0 + 16 * t + nl;
    sbm[t] = reinterpret_cast<const uint32_t*>(blob + 3 * cbytes + 2 * sbytes);
  }
  auto mat_of = [&](int) { return blob + 2 * cbytes; };
  auto row_of = [&](int R) { return row0 + R; };
  extern __shared__ float smem_f[];
  float* xs = smem_f;  // [G][16]
  char* wbuf = reinterpret_cast<char*>(smem_f + G * 16) + wave * wave_stage_bytes<BITS>();
  for (int m0 = 0; m0 < cnt; m0 += 16) {
    __syncthreads();
    stage_sums(xs, p, p.ag, G, off, cnt, m0, 1, false);
    __syncthreads();
    const uint16_t* tp = token_row(p.a16, p, off, cnt, m0, nl, kb, (size_t)I, false);
    f32x4 acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    expert_pass_any<BITS>(acc, wbuf, mat_of, row_of, H, rowb, sbm, sbr, tp, xs, G, lane, nl, kb);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = m0 + 4 * kb + i;
      if (r < cnt) {
        float* y = p.ys + (size_t)p.pairs[off + r] * H + row0 + nl;
#pragma unroll
        for (int t = 0; t < 4; ++t) y[16 * t] = acc[t][i] / kCodeUnit<BITS>;
      }
    }
  }
}

// ---------------------------------------------------------------- 6. combine
__global__ void __launch_bounds__(kBT) combine_kernel(const float* __restrict__ h, const float* __restrict__ ys,
                                                      const int32_t* __restrict__ idx, const float* __restrict__ w,
                                                      int H, int k, int kr, float* __restrict__ h_next,
                                                      int32_t* __restrict__ idx_out, float* __restrict__ w_out,
                                                      int layer, int n_layers) {
  // k slots per token (the kr routed ones, then the shared expert's if any). The loads of h
  // and of up to 4 slots' rows are issued together (one memory round trip per 4 slots, not
  // one per slot); the sum still runs in slot order.
  const int t = blockIdx.y;
  const int i4 = blockIdx.x * kBT + threadIdx.x;
  if (i4 < H / 4) {
    const float4 hv = reinterpret_cast<const float4*>(h + (size_t)t * H)[i4];
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j0 = 0; j0 < k; j0 += 4) {
      float4 y[4];
      float wj[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = min(j0 + u, k - 1);  // past the last slot: a repeated row, weight 0
        y[u] = reinterpret_cast<const float4*>(ys + ((size_t)t * k + j) * H)[i4];
        wj[u] = j0 + u < k ? w[t * k + j] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (j0 + u < k) {
          s.x = fmaf(wj[u], y[u].x, s.x);
          s.y = fmaf(wj[u], y[u].y, s.y);
          s.z = fmaf(wj[u], y[u].z, s.z);
          s.w = fmaf(wj[u], y[u].w, s.w);
        }
      }
    }
    reinterpret_cast<float4*>(h_next + (size_t)t * H)[i4] = make_float4(hv.x + s.x, hv.y + s.y, hv.z + s.z, hv.w + s.w);
  }
  if (blockIdx.x == 0 && (int)threadIdx.x < kr) {
    const size_t o = ((size_t)t * n_layers + layer) * kr + threadIdx.x;
    if (idx_out) idx_out[o] = idx[t * k + threadIdx.x];
    if (w_out) w_out[o] = w[t * k + threadIdx.x];
  }
}

// a16 (operand order, pair-id rows) -> natural column order.
template <int BITS>
__global__ void __launch_bounds__(kBT) a16_natural_kernel(const uint16_t* __restrict__ a16, int P, int I,
                                                          uint16_t* __restrict__ out) {
  const size_t n = (size_t)P * I;
  for (size_t i = blockIdx.x * (size_t)kBT + threadIdx.x; i < n; i += (size_t)gridDim.x * kBT) {
    const size_t row = i / I;
    const int c = (int)(i % I);
    out[i] = a16[row * I + (c & ~15) + perm_pos<BITS>(c & 15)];
  }
}

// ---------------------------------------------------------------- workspace
// Work units of the expert kernels: 16 pairs of one expert each (at most one partial unit
// per active expert).
inline size_t max_units(int P, int E) { return (size_t)(E < P ? E : P) + (size_t)P / 16; }

struct BatchedWs {
  float* h[2];
  uint16_t* v16;
  float* xg;
  float* logits;
  float* part;
  int32_t* idx;
  float* w;
  int32_t* pairs;
  int32_t* act_e;
  int32_t* act_off;
  int32_t* act_cnt;
  int32_t* n_act;
  uint32_t* done;  // workgroups of route_stage_kernel finished (0 between calls; in the control block)
  uint16_t* a16;
  float* ag;
  float* ys;
  size_t bytes;
};

size_t up256(size_t b) { return (b + 255) / 256 * 256; }

BatchedWs carve(void* base, int T, int H, int I, int E, int k) {
  BatchedWs w;
  char* p = static_cast<char*>(base);
  size_t o = 0;
  auto take = [&](size_t b) {
    char* q = p ? p + o : nullptr;
    o += up256(b);
    return q;
  };
  const size_t P = (size_t)T * k;
  w.h[0] = reinterpret_cast<float*>(take((size_t)T * H * 4));
  w.h[1] = reinterpret_cast<float*>(take((size_t)T * H * 4));
  w.v16 = reinterpret_cast<uint16_t*>(take((size_t)T * H * 2));
  w.xg = reinterpret_cast<float*>(take((size_t)T * (H / 64) * 4));
  w.logits = reinterpret_cast<float*>(take((size_t)T * E * 4));
  w.part = reinterpret_cast<float*>(take((size_t)((H + kRtSlice - 1) / kRtSlice) * T * E * 4));
  w.idx = reinterpret_cast<int32_t*>(take(P * 4));
  w.w = reinterpret_cast<float*>(take(P * 4));
  w.pairs = reinterpret_cast<int32_t*>(take(P * 4));
  const size_t units = max_units(P, E);
  w.act_e = reinterpret_cast<int32_t*>(take(units * 4));
  w.act_off = reinterpret_cast<int32_t*>(take(units * 4));
  w.act_cnt = reinterpret_cast<int32_t*>(take(units * 4));
  w.n_act = reinterpret_cast<int32_t*>(take(4));
  w.done = nullptr;  // set by the caller: a fixed word of the workspace's control block
  w.a16 = reinterpret_cast<uint16_t*>(take(P * I * 2));
  w.ag = reinterpret_cast<float*>(take(P * (I / 64) * 4));
  w.ys = reinterpret_cast<float*>(take(P * H * 4));
  w.bytes = o;
  return w;
}

template <int BITS>
int run_layers(const fmoe_layer* layers, int n_layers, const float* x_in, float* h_out, int T, int k, float eps,
               unsigned flags, int32_t* idx_out, float* w_out, const BatchedWs& ws, hipStream_t s) {
  const fmoe_layer& L0 = layers[0];
  const int hs = L0.shared_gate != nullptr;
  const int H = L0.hidden, I = L0.inter, E = L0.n_experts, ks = k + hs, P = T * ks;
  const int max_items = (int)max_units(P, E + hs);
  const size_t sm_gu = expert_smem_bytes<BITS>(H / 64), sm_dn = expert_smem_bytes<BITS>(I / 64);
  // the stage buffers take the expert kernels past the default 64 KB of dynamic LDS
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(&gate_up_kernel<BITS>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm_gu) != hipSuccess ||
      hipFuncSetAttribute(reinterpret_cast<const void*>(&down_kernel<BITS>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm_dn) != hipSuccess)
    return FMOE_ERR_HIP;
  for (int l = 0; l < n_layers; ++l) {
    const float* hin = l == 0 ? x_in : ws.h[(l - 1) & 1];
    float* hnext = l == n_layers - 1 ? h_out : ws.h[l & 1];
    const fmoe_layer& L = layers[l];
    const int n_part = (H + kRtSlice - 1) / kRtSlice;
    hipLaunchKernelGGL(router_kernel_mfma, dim3((E + 15) / 16, n_part), dim3(kBT), 0, s, L.router, hin, T, E, H,
                       ws.part);
    if (hipGetLastError() != hipSuccess) return FMOE_ERR_HIP;
    hipLaunchKernelGGL(route_stage_kernel<BITS>, dim3(T), dim3(kBT), 0, s, hin, (flags & FMOE_PRENORM) ? 1 : 0, eps,
                       ws.part, n_part, T, E, H, k, L.shared_gate, ks, ws.logits, ws.idx, ws.w, ws.v16, ws.xg,
                       ws.pairs, ws.act_e,
                       ws.act_off, ws.act_cnt, ws.n_act, ws.done);
    if (hipGetLastError() != hipSuccess) return FMOE_ERR_HIP;
    BParams bp;
    bp.experts = static_cast<const uint8_t*>(L.experts);
    bp.stride = L.expert_stride;
    bp.H = H;
    bp.I = I;
    bp.k = ks;
    bp.pairs = ws.pairs;
    bp.act_e = ws.act_e;
    bp.act_off = ws.act_off;
    bp.act_cnt = ws.act_cnt;
    bp.n_act = ws.n_act;
    bp.v16 = ws.v16;
    bp.xg = ws.xg;
    bp.a16 = ws.a16;
    bp.ag = ws.ag;
    bp.ys = ws.ys;
    hipLaunchKernelGGL(gate_up_kernel<BITS>, dim3(I / kGuRowsWg, max_items), dim3(kBT), sm_gu, s, bp);
    if (hipGetLastError() != hipSuccess) return FMOE_ERR_HIP;
    hipLaunchKernelGGL(down_kernel<BITS>, dim3(H / kDnRowsWg, max_items), dim3(kBT), sm_dn, s, bp);
    if (hipGetLastError() != hipSuccess) return FMOE_ERR_HIP;
    hipLaunchKernelGGL(combine_kernel, dim3((H / 4 + kBT - 1) / kBT, T), dim3(kBT), 0, s, hin, ws.ys, ws.idx, ws.w,
                       H, ks, k, hnext, idx_out, w_out, l, n_layers);
    if (hipGetLastError() != hipSuccess) return FMOE_ERR_HIP;
  }
  return FMOE_OK;
}

}  // namespace

bool batched_shape_ok(int hidden, int inter) { return hidden % kDnRowsWg == 0 && inter % kGuRowsWg == 0; }
bool batched_bits_ok(int bits) { return bits == 2 || bits == 3 || bits == 4; }

// The scratch is carved for n_experts + 1 sort buckets (a shared expert's) and the call's
// slots; the size query covers k + 1 slots.
size_t batched_workspace_bytes(int n_tokens, int hidden, int inter, int n_experts, int k) {
  return carve(nullptr, n_tokens, hidden, inter, n_experts + 1, k + 1).bytes;
}

size_t batched_region_bytes(int n_tokens, int hidden, int inter, int n_experts, int k_slots) {
  return carve(nullptr, n_tokens, hidden, inter, n_experts + 1, k_slots).bytes;
}

int launch_batched(const fmoe_layer* layers, int n_layers, const float* x_in, float* h_out, int n_tokens, int k,
                   float eps, unsigned flags, int32_t* idx_out, float* w_out, void* ws, size_t ws_bytes,
                   uint32_t* done, hipStream_t s) {
  const fmoe_layer& L0 = layers[0];
  if (!batched_shape_ok(L0.hidden, L0.inter)) return FMOE_ERR_SHAPE;
  const int ks = k + (L0.shared_gate != nullptr ? 1 : 0);
  BatchedWs w = carve(ws, n_tokens, L0.hidden, L0.inter, L0.n_experts + 1, ks);
  if (w.bytes > ws_bytes) return FMOE_ERR_WORKSPACE;
  w.done = done;
  if (L0.bits == 4) return run_layers<4>(layers, n_layers, x_in, h_out, n_tokens, k, eps, flags, idx_out, w_out, w, s);
  if (L0.bits == 3) return run_layers<3>(layers, n_layers, x_in, h_out, n_tokens, k, eps, flags, idx_out, w_out, w, s);
  return run_layers<2>(layers, n_layers, x_in, h_out, n_tokens, k, eps, flags, idx_out, w_out, w, s);
}

int launch_batched_a16(const void* ws, int n_tokens, int hidden, int inter, int n_experts, int k, int bits,
                       uint16_t* out, hipStream_t s) {
  const BatchedWs w = carve(const_cast<void*>(ws), n_tokens, hidden, inter, n_experts + 1, k);
  const int P = n_tokens * k;
  const size_t n = (size_t)P * inter;
  size_t blocks = (n + kBT - 1) / kBT;
  if (blocks > 4096) blocks = 4096;
  if (bits == 4)
    hipLaunchKernelGGL(a16_natural_kernel<4>, dim3((unsigned)blocks), dim3(kBT), 0, s, w.a16, P, inter, out);
  else  // 3 bits: the operand order of 2 bits
    hipLaunchKernelGGL(a16_natural_kernel<2>, dim3((unsigned)blocks), dim3(kBT), 0, s, w.a16, P, inter, out);
  return hipGetLastError() == hipSuccess ? FMOE_OK : FMOE_ERR_HIP;
}

}  // namespace fmoe
