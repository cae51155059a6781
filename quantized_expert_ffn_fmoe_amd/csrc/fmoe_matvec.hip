// fmoe_matvec.hip -- standalone dequantized matvec, packing, and router/top-k kernels.
//
// Dequantized matvec: the 4-bit / 2-bit "dequant matvec" kernel of the Flash-MoE pages
// (aibit.im "Techniques de rupture" item 4), redesigned for gfx950: a 64-lane wave
// covers LPR lanes per row (LPR = a power of two, up to 64) and 64/LPR rows at a time;
// each lane reads CPL 16-byte chunks of its row(s) (16-byte coalesced loads) and keeps
// the matching activation values in registers for every row it visits.
#include "fmoe_device.h"
#include "fmoe_internal.h"
#include "fmoe_layout.h"

namespace fmoe {

// One wave pass over R row blocks (R * 64/lpr rows) of one matrix starting at row rb0:
// mv_load issues all of the pass's loads, mv_reduce forms the dots and the cross-lane sums
// (one transposed reduction for the R rows when a row spans the wave). A lane keeps x in
// registers, so taking several row blocks per pass spreads that load over more weights.
template <int BITS, int CPL, int R>
struct MvPass {
  CChunk<BITS> w[R][CPL];
  uint32_t s[R][CPL];
};

template <int BITS, int CPL, int R>
__device__ __forceinline__ void mv_load(MvPass<BITS, CPL, R>& P, const uint8_t* __restrict__ codes,
                                        const uint32_t* __restrict__ sb, int rows, int cols, int lpr, int rb0) {
  using C = Chunk<BITS>;
  const int lane = threadIdx.x & 63;
  const int rpw = kWave / lpr, sub = lane & (lpr - 1), rsel = lane / lpr;
  const int n_chunks = cols / C::kCodes, ngroups = cols / 64;
#pragma unroll
  for (int u = 0; u < R; ++u) {
    const int r = rb0 + u * rpw + rsel;
    if (r < rows) {
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        int c = sub + lpr * j;
        if (c < n_chunks) {
          load_cchunk<BITS>(P.w[u][j], codes, rows, cols, r, c);
          P.s[u][j] = sb[sb_offset(rows, ngroups, r, c / C::kPerGroup)];
        }
      }
    }
  }
}

template <int BITS, int CPL, int R>
__device__ __forceinline__ void mv_reduce(const MvPass<BITS, CPL, R>& P, float* __restrict__ yv, int rows, int cols,
                                          int lpr, int rb0, const XChunk<BITS> (&xc)[CPL]) {
  using C = Chunk<BITS>;
  const int lane = threadIdx.x & 63;
  const int rpw = kWave / lpr, sub = lane & (lpr - 1), rsel = lane / lpr;
  const int n_chunks = cols / C::kCodes;
  float acc[R];
#pragma unroll
  for (int u = 0; u < R; ++u) {
    const int r = rb0 + u * rpw + rsel;
    acc[u] = 0.f;
    if (r < rows) {
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        int c = sub + lpr * j;
        if (c < n_chunks) acc[u] += chunk_dot<BITS>(P.w[u][j], P.s[u][j], xc[j]);
      }
    }
  }
  if (lpr == kWave) {
    // afterwards lane i < R holds the total of row rb0 + transposed_index<R>(i)
    const float sum = reduce_transposed<R, 64>(acc);
    const int r = rb0 + transposed_index<R>(lane);
    if (lane < R && r < rows) yv[r] = sum;
  } else {
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int r = rb0 + u * rpw + rsel;
      const float a = group_sum(acc[u], lpr);
      if (r < rows && sub == 0) yv[r] = a;
    }
  }
}

// Row blocks per wave pass (fewer when a lane holds 4 chunks of x, to stay within the
// register file).
template <int CPL> constexpr int mv_pass_blocks() { return CPL >= 4 ? 2 : 4; }

// Load and reduce one pass. (Measured against alternatives on a fused 4096 + 512 + 512-row
// projection: issuing the first pass's loads before reading x, or keeping the pass
// registers across loop iterations with the matrix fields in a struct, took 14.7-16.6 us
// against 10.1 us for this form.)
template <int BITS, int CPL, int R>
__device__ __forceinline__ void matvec_pass(const uint8_t* __restrict__ codes, const uint32_t* __restrict__ sb,
                                            float* __restrict__ yv, int rows, int cols, int lpr, int rb0,
                                            const XChunk<BITS> (&xc)[CPL]) {
  MvPass<BITS, CPL, R> P;
  mv_load<BITS, CPL, R>(P, codes, sb, rows, cols, lpr, rb0);
  mv_reduce<BITS, CPL, R>(P, yv, rows, cols, lpr, rb0, xc);
}
template <int BITS, int CPL, int RB = 0>
__global__ void __launch_bounds__(256) matvec_kernel(const uint8_t* __restrict__ codes,
                                                     const uint32_t* __restrict__ sb, const float* __restrict__ x,
                                                     float* __restrict__ y, int rows, int cols, int lpr) {
  using C = Chunk<BITS>;
  constexpr int R = RB ? RB : mv_pass_blocks<CPL>();
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int sub = lane & (lpr - 1);
  const int n_chunks = cols / C::kCodes;
  const int span = R * (kWave / lpr);
  const float* xv = x + (size_t)blockIdx.y * cols;
  float* yv = y + (size_t)blockIdx.y * rows;
  const int waves_total = gridDim.x * (blockDim.x >> 6);
  const int rb0 = (blockIdx.x * (blockDim.x >> 6) + wave) * span;
  if (rb0 >= rows) return;  // uniform over the wave
  XChunk<BITS> xc[CPL];
  if (rb0 + waves_total * span >= rows) {
    // one pass for this wave (small matrices): its weight loads go out before x is read,
    // so the two memory latencies overlap instead of adding up
    MvPass<BITS, CPL, R> P;
    mv_load<BITS, CPL, R>(P, codes, sb, rows, cols, lpr, rb0);
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      int c = sub + lpr * j;
      if (c < n_chunks) load_xchunk<BITS>(xc[j], xv + (size_t)c * C::kCodes);
    }
    mv_reduce<BITS, CPL, R>(P, yv, rows, cols, lpr, rb0, xc);
    return;
  }
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    int c = sub + lpr * j;
    if (c < n_chunks) load_xchunk<BITS>(xc[j], xv + (size_t)c * C::kCodes);
  }
  for (int rb = rb0; rb < rows; rb += waves_total * span)
    matvec_pass<BITS, CPL, R>(codes, sb, yv, rows, cols, lpr, rb, xc);
}
// Several matrices applied to one input (openclawradar.com "Optimisations efficaces": the
// fused Q/K/V projection reads the input vector once instead of once per matrix). Every
// wave loads its share of x into registers once and walks wave passes over all matrices;
// the row space of matrix m starts at prow[m], each matrix padded to whole passes, so a
// pass never spans two matrices and m is uniform over the wave. The matrix fields are
// picked by a select chain (no dynamic indexing of the kernel-argument arrays).
template <int BITS, int CPL>
__global__ void __launch_bounds__(256) matvec_multi_kernel(MultiMat P, const float* __restrict__ x, int cols,
                                                           int lpr) {
  using C = Chunk<BITS>;
  constexpr int R = mv_pass_blocks<CPL>();
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int sub = lane & (lpr - 1);
  const int n_chunks = cols / C::kCodes;
  const int span = R * (kWave / lpr);
  const float* xv = x + (size_t)blockIdx.y * cols;
  XChunk<BITS> xc[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    int c = sub + lpr * j;
    if (c < n_chunks) load_xchunk<BITS>(xc[j], xv + (size_t)c * C::kCodes);
  }
  const int waves_total = gridDim.x * (blockDim.x >> 6);
  const int total = P.prow[P.n_mats];
  for (int rb = (blockIdx.x * (blockDim.x >> 6) + wave) * span; rb < total; rb += waves_total * span) {
    int m = 0;
#pragma unroll
    for (int i = 1; i < kMaxMulti; ++i)
      if (i < P.n_mats && rb >= P.prow[i]) m = i;
    const uint8_t* codes = P.codes[0];
    const uint32_t* sb = P.sb[0];
    float* y = P.y[0];
    int rows = P.rows[0], r0 = P.prow[0];
#pragma unroll
    for (int i = 1; i < kMaxMulti; ++i)
      if (m == i) {
        codes = P.codes[i];
        sb = P.sb[i];
        y = P.y[i];
        rows = P.rows[i];
        r0 = P.prow[i];
      }
    matvec_pass<BITS, CPL, R>(codes, sb, y + (size_t)blockIdx.y * rows, rows, cols, lpr, rb - r0, xc);
  }
}

// Canonical (row-major) codes -> the packed layout of fmoe_layout.h, one 16-byte chunk per
// thread step (chunks never straddle a piece); scale and bias interleaved into sb words,
// placed in the blocked sb order of the same header.
template <int BITS>
__global__ void pack_kernel(const uint8_t* __restrict__ codes_in, const uint16_t* __restrict__ scale,
                            const uint16_t* __restrict__ bias, uint8_t* __restrict__ codes_out,
                            uint32_t* __restrict__ sb_out, int rows, size_t row_bytes, size_t n_groups) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  const int groups = (int)(n_groups / rows);
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n_groups; i += stride)
    sb_out[sb_offset(rows, groups, (int)(i / groups), (int)(i % groups))] =
        (uint32_t)scale[i] | ((uint32_t)bias[i] << 16);
  const size_t per_row = row_bytes / 16, n_code16 = (size_t)rows * per_row;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n_code16; i += stride) {
    const int r = (int)(i / per_row);
    const size_t b = (i % per_row) * 16;
    *reinterpret_cast<uint4*>(codes_out + code_offset<BITS>(rows, row_bytes, r, b)) =
        reinterpret_cast<const uint4*>(codes_in)[i];
  }
}

// Router logits for a tile of up to 8 tokens: logits[t][e] = sum_i R[e][i] x[t][i] (fp32).
// One wave per expert row; the row is streamed once per token tile in 16-byte loads.
constexpr int kRouteTile = 8;
__global__ void __launch_bounds__(256) router_kernel(const float* __restrict__ R, const float* __restrict__ x,
                                                     float* __restrict__ logits, int n_tokens, int n_experts,
                                                     int hidden) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int t0 = blockIdx.y * kRouteTile;
  if (e >= n_experts) return;
  const int nt = min(kRouteTile, n_tokens - t0);
  float acc[kRouteTile];
#pragma unroll
  for (int t = 0; t < kRouteTile; ++t) acc[t] = 0.f;
  const float4* row = reinterpret_cast<const float4*>(R + (size_t)e * hidden);
  for (int c = lane; c < hidden / 4; c += kWave) {
    float4 r = row[c];
#pragma unroll
    for (int t = 0; t < kRouteTile; ++t) {
      if (t < nt) {
        float4 v = reinterpret_cast<const float4*>(x + (size_t)(t0 + t) * hidden)[c];
        acc[t] = fmaf(r.x, v.x, acc[t]);
        acc[t] = fmaf(r.y, v.y, acc[t]);
        acc[t] = fmaf(r.z, v.z, acc[t]);
        acc[t] = fmaf(r.w, v.w, acc[t]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kRouteTile; ++t) {
    float s = wave_sum(acc[t]);
    if (lane == 0 && t < nt) logits[(size_t)(t0 + t) * n_experts + e] = s;
  }
}

// One wave per token: the logits become rank keys in LDS, then k rounds of a wave-wide
// maximum select the experts (larger logit first, lower index on equal logits, NaN last)
// and the softmax over the k selected logits gives their weights.
__global__ void __launch_bounds__(64) topk_kernel(const float* __restrict__ logits, int n_tokens, int n_experts,
                                                  int k, int32_t* __restrict__ idx, float* __restrict__ w) {
  const int t = blockIdx.x;
  const int lane = threadIdx.x;
  const float* l = logits + (size_t)t * n_experts;
  __shared__ uint64_t keys[4096];
  __shared__ float lsel[16], wsel[16];
  __shared__ int isel[16];
  for (int e = lane; e < n_experts; e += kWave) keys[e] = rank_key(l[e], e);
  __syncthreads();
  wave_topk_keys(keys, n_experts, k, isel, lsel, wsel);
  __syncthreads();
  if (lane < k) {
    idx[(size_t)t * k + lane] = isel[lane];
    w[(size_t)t * k + lane] = wsel[lane];
  }
}

// ------------------------------------------------------------------ host launchers
// Launch shape of the matvec kernels (any multiple of 64 threads up to 256 per workgroup;
// a wave walks its passes by its global wave index). A call with fewer waves than about
// four per compute unit uses one-wave workgroups, so that its waves spread over all the
// compute units instead of filling a quarter of them with four-wave workgroups (a
// 1024 x 4096 4-bit matrix is 256 waves of one pass each).
void mv_grid(int total_waves, int waves_per_vec, int* threads, int* blocks) {
  const int per_wg = total_waves < 1024 ? 1 : 4;
  *threads = 64 * per_wg;
  int b = (waves_per_vec + per_wg - 1) / per_wg;
  const int cap = per_wg == 1 ? 8192 : 2048;
  *blocks = b > cap ? cap : b;
}

int launch_matvec(const QMat& W, const float* x, float* y, int n_vec, hipStream_t s) {
  const int n_chunks = W.cols / (W.bits == 4 ? 32 : 64);  // 16-byte (low-plane) chunks per row
  int lpr = 1;
  while (lpr < n_chunks && lpr < 64) lpr <<= 1;
  const int cpl = (n_chunks + lpr - 1) / lpr;
  // A matrix of at most 4096 row blocks (of 64 / lpr rows) gets two row blocks per wave, in
  // two-wave workgroups: for 1024 x 4096 at 4 bits, 512 waves over 256 workgroups, so that two
  // SIMDs of every compute unit take part and each copy of x read from L2 serves two rows
  // (measured against one row block per wave in four-wave workgroups, two in one-wave
  // workgroups and one in two-wave workgroups: 4.86 against 5.07, 4.96 and 5.23 us per call);
  // larger ones take mv_pass_blocks row blocks per wave pass.
  const int one = (W.rows + 64 / lpr - 1) / (64 / lpr);
  const bool single = one * n_vec <= 4096;
  const int span = (single ? 2 : cpl >= 3 ? 2 : 4) * (64 / lpr);  // rows of a wave pass
  const int waves_needed = (W.rows + span - 1) / span;
  int threads = 0, blocks = 0;
  if (single) {
    threads = 128;
    blocks = (waves_needed + 1) / 2;
  } else {
    mv_grid(waves_needed * n_vec, waves_needed, &threads, &blocks);
  }
  dim3 grid(blocks, n_vec);
  const uint8_t* codes = static_cast<const uint8_t*>(W.codes);
#define FMOE_MV(B, C)                                                                                         \
  do {                                                                                                        \
    if (single)                                                                                               \
      hipLaunchKernelGGL((matvec_kernel<B, C, 2>), grid, dim3(threads), 0, s, codes, W.sb, x, y, W.rows, W.cols, \
                         lpr);                                                                                \
    else                                                                                                      \
      hipLaunchKernelGGL((matvec_kernel<B, C>), grid, dim3(threads), 0, s, codes, W.sb, x, y, W.rows, W.cols, lpr); \
  } while (0)
  if (W.bits == 4) {
    if (cpl == 1) FMOE_MV(4, 1);
    else if (cpl == 2) FMOE_MV(4, 2);
    else if (cpl <= 4) FMOE_MV(4, 4);
    else return FMOE_ERR_SHAPE;
  } else if (W.bits == 3) {
    if (cpl == 1) FMOE_MV(3, 1);
    else if (cpl == 2) FMOE_MV(3, 2);
    else if (cpl <= 4) FMOE_MV(3, 4);
    else return FMOE_ERR_SHAPE;
  } else {
    if (cpl == 1) FMOE_MV(2, 1);
    else if (cpl == 2) FMOE_MV(2, 2);
    else if (cpl <= 4) FMOE_MV(2, 4);
    else return FMOE_ERR_SHAPE;
  }
#undef FMOE_MV
  return hipGetLastError() == hipSuccess ? FMOE_OK : FMOE_ERR_HIP;
}

int launch_matvec_multi(const QMat* W, int n_mats, const float* x, float* const* y, int n_vec, hipStream_t s) {
  const int cols = W[0].cols, bits = W[0].bits;
  const int n_chunks = cols / (bits == 4 ? 32 : 64);
  int lpr = 1;
  while (lpr < n_chunks && lpr < 64) lpr <<= 1;
  const int cpl = (n_chunks + lpr - 1) / lpr;
  const int span = (cpl >= 3 ? 2 : 4) * (64 / lpr);  // rows of a wave pass (mv_pass_blocks of the CPL run)
  MultiMat P;
  P.n_mats = n_mats;
  P.prow[0] = 0;
  for (int i = 0; i < kMaxMulti; ++i) {
    const int m = i < n_mats ? i : n_mats - 1;  // unused slots repeat the last matrix
    P.codes[i] = static_cast<const uint8_t*>(W[m].codes);
    P.sb[i] = W[m].sb;
    P.y[i] = y[m];
    P.rows[i] = W[m].rows;
    P.prow[i + 1] = P.prow[i] + (i < n_mats ? (W[i].rows + span - 1) / span * span : 0);
  }
  const int waves_needed = P.prow[n_mats] / span;
  int threads = 0, blocks = 0;
  mv_grid(waves_needed * n_vec, waves_needed, &threads, &blocks);
  dim3 grid(blocks, n_vec);
#define FMOE_MV(B, C) hipLaunchKernelGGL((matvec_multi_kernel<B, C>), grid, dim3(threads), 0, s, P, x, cols, lpr)
  if (bits == 4) {
    if (cpl == 1) FMOE_MV(4, 1);
    else if (cpl == 2) FMOE_MV(4, 2);
    else if (cpl <= 4) FMOE_MV(4, 4);
    else return FMOE_ERR_SHAPE;
  } else if (bits == 3) {
    if (cpl == 1) FMOE_MV(3, 1);
    else if (cpl == 2) FMOE_MV(3, 2);
    else if (cpl <= 4) FMOE_MV(3, 4);
    else return FMOE_ERR_SHAPE;
  } else {
    if (cpl == 1) FMOE_MV(2, 1);
    else if (cpl == 2) FMOE_MV(2, 2);
    else if (cpl <= 4) FMOE_MV(2, 4);
    else return FMOE_ERR_SHAPE;
  }
#undef FMOE_MV
  return hipGetLastError() == hipSuccess ? FMOE_OK : FMOE_ERR_HIP;
}

// 3-bit canonical codes -> the two planes of fmoe_layout.h: one (row, group) per thread
// step. The group's 24 canonical bytes hold its 64 codes as a little-endian bit stream
// (column c at bits 3c..3c+2); the low 2 bits go to the low plane's 16-byte chunk in the
// 2-bit order (column c at bits 2c), the third bits to the group's two high-plane words at
// hi_bit(c % 32) of word c / 32. Scale and bias words as for the other widths.
__global__ void pack3_kernel(const uint8_t* __restrict__ codes_in, const uint16_t* __restrict__ scale,
                             const uint16_t* __restrict__ bias, uint8_t* __restrict__ codes_out,
                             uint32_t* __restrict__ sb_out, int rows, int cols) {
  const int groups = cols / 64;
  const size_t n_groups = (size_t)rows * groups;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  const size_t row_bytes = (size_t)cols * 3 / 8, lo_row_bytes = (size_t)cols / 4;
  uint32_t* hi = reinterpret_cast<uint32_t*>(codes_out + lo_plane_bytes(rows, cols));
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n_groups; i += stride) {
    const int r = (int)(i / groups), g = (int)(i % groups);
    sb_out[sb_offset(rows, groups, r, g)] = (uint32_t)scale[i] | ((uint32_t)bias[i] << 16);
    const uint64_t* src = reinterpret_cast<const uint64_t*>(codes_in + (size_t)r * row_bytes + (size_t)g * 24);
    const uint64_t s0 = src[0], s1 = src[1], s2 = src[2];
    uint32_t lo[4] = {0u, 0u, 0u, 0u}, hw[2] = {0u, 0u};
#pragma unroll
    for (int c = 0; c < 64; ++c) {
      const int b = 3 * c;  // first bit of column c in the 192-bit stream s0 | s1 << 64 | s2 << 128
      uint32_t q;
      if (b + 3 <= 64) q = (uint32_t)(s0 >> b);
      else if (b < 64) q = (uint32_t)((s0 >> b) | (s1 << (64 - b)));
      else if (b + 3 <= 128) q = (uint32_t)(s1 >> (b - 64));
      else if (b < 128) q = (uint32_t)((s1 >> (b - 64)) | (s2 << (128 - b)));
      else q = (uint32_t)(s2 >> (b - 128));
      q &= 7u;
      lo[c / 16] |= (q & 3u) << (2 * (c % 16));
      hw[c / 32] |= (q >> 2) << hi_bit(c % 32);
    }
    *reinterpret_cast<uint4*>(codes_out + code_offset<2>(rows, lo_row_bytes, r, (size_t)g * 16)) =
        make_uint4(lo[0], lo[1], lo[2], lo[3]);
    *reinterpret_cast<uint2*>(hi + hi_offset(rows, groups, r, g, 0)) = make_uint2(hw[0], hw[1]);
  }
}

int launch_pack(const uint8_t* codes_in, const uint16_t* scale, const uint16_t* bias, int rows, int cols, int bits,
                void* codes_out, uint32_t* sb_out, hipStream_t s) {
  if (bits == 3) {
    const size_t n_groups = (size_t)rows * (cols / 64);
    size_t blocks = (n_groups + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(pack3_kernel, dim3((unsigned)blocks), dim3(256), 0, s, codes_in, scale, bias,
                       static_cast<uint8_t*>(codes_out), sb_out, rows, cols);
    return hipGetLastError() == hipSuccess ? FMOE_OK : FMOE_ERR_HIP;
  }
  size_t n_code16 = (size_t)rows * cols * bits / 8 / 16;
  size_t n_groups = (size_t)rows * (cols / 64);
  size_t work = n_code16 > n_groups ? n_code16 : n_groups;
  size_t blocks = (work + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  const size_t row_bytes = (size_t)cols * bits / 8;
  if (bits == 4)
    hipLaunchKernelGGL(pack_kernel<4>, dim3((unsigned)blocks), dim3(256), 0, s, codes_in, scale, bias,
                       static_cast<uint8_t*>(codes_out), sb_out, rows, row_bytes, n_groups);
  else
    hipLaunchKernelGGL(pack_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, s, codes_in, scale, bias,
                       static_cast<uint8_t*>(codes_out), sb_out, rows, row_bytes, n_groups);
  return hipGetLastError() == hipSuccess ? FMOE_OK : FMOE_ERR_HIP;
}

int launch_route(const float* R, const float* x, int n_tokens, int n_experts, int hidden, int k, int32_t* idx,
                 float* w, float* logits, hipStream_t s) {
  dim3 g1((n_experts + 3) / 4, (n_tokens + kRouteTile - 1) / kRouteTile);
  hipLaunchKernelGGL(router_kernel, g1, dim3(256), 0, s, R, x, logits, n_tokens, n_experts, hidden);
  if (hipGetLastError() != hipSuccess) return FMOE_ERR_HIP;
  hipLaunchKernelGGL(topk_kernel, dim3(n_tokens), dim3(64), 0, s, logits, n_tokens, n_experts, k, idx, w);
  return hipGetLastError() == hipSuccess ? FMOE_OK : FMOE_ERR_HIP;
}

}  // namespace fmoe
