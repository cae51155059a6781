// fmoe_decode.hip -- single-token decode through a stack of MoE layers in ONE persistent
// kernel (one workgroup per compute unit, all co-resident).
//
// Per layer (aibit.im "Techniques de rupture" item 3 and tr.news.hada.io "Deferred GPU
// Expert Compute": route, run the k selected experts, combine with the residual, and
// normalize for the next layer; the pages route on the CPU, here routing stays on the
// device):
//   1. v = h * inv_rms(h) (or v = h without pre-norm), staged in LDS by every workgroup;
//   2. router: workgroup g owns experts g, g+G, ...; its waves dot 1024-column slices of
//      those rows with v; the logits are published with a tag (value | layer << 32);
//   3. every workgroup polls the n_experts tagged logits, then selects the top-k and
//      their softmax weights itself (no extra round trip);
//   4. gate/up: (slot j, row i) items spread over all waves of all workgroups; each item
//      reads gate row i and up row i of expert idx[j] and stores a[j][i] = silu(g)*u;
//   5. grid barrier (dense arrival flags);
//   6. down + combine + residual: workgroup g owns a contiguous block of h rows and
//      computes h[r] += sum_j w_j * (Wd_j[r] . a_j) for them (fixed slot order);
//   7. grid barrier, next layer.
// Data exchanged between workgroups (h, a, logits, flags) is written and read with
// device-scope relaxed atomic accesses, which are performed at the device coherence
// point; a wave waits for its own stores (s_waitcnt) before its workgroup raises its
// flag, and reads exchanged data only after it has observed the flags.
#include "fmoe_decode.h"
#include "fmoe_device.h"
#include "fmoe_internal.h"

namespace fmoe {

constexpr int kDecodeThreads = 512;
constexpr int kDecodeWaves = kDecodeThreads / 64;
constexpr unsigned kSpinLimit = 1u << 21;

struct DecodeSmem {
  float* v;       // [hidden]
  float* logit;   // [n_experts]
  float* part;    // [router items per workgroup]
  float* a;       // [k][inter]
  float* y;       // [k][rows per workgroup]
  float* red;     // [kDecodeWaves]
  float* wsel;    // [16]
  int* isel;      // [16]
  int* fail;      // [1]
};

__device__ __forceinline__ bool spin_failed(const uint32_t* err) { return ld_dev_u32(err) != 0u; }

// Grid barrier: raise this workgroup's flag to `epoch`, wait until every flag reached it.
// Called by all threads of the workgroup. Returns false when the wait gave up.
__device__ bool grid_barrier(uint32_t* flags, int G, uint32_t epoch, uint32_t* err, int* fail) {
  wait_vmem();
  __syncthreads();
  if (threadIdx.x < 64) {
    if (threadIdx.x == 0) st_dev_u32(flags + blockIdx.x, epoch);
    unsigned spins = 0;
    while (true) {
      bool ok = true;
      for (int j = threadIdx.x; j < G; j += 64) ok &= ld_dev_u32(flags + j) >= epoch;
      if (__all(ok)) break;
      if (++spins > kSpinLimit || spin_failed(err)) {
        if (threadIdx.x == 0) {
          st_dev_u32(err, 1u);
          *fail = 1;
        }
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
  return *fail == 0;
}

template <int BITS, int CPL_G, int CPL_D>
__global__ void __launch_bounds__(kDecodeThreads) decode_kernel(DecodeParams p) {
  using C = Chunk<BITS>;
  extern __shared__ float smem_raw[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = gridDim.x, g = blockIdx.x;
  const int H = p.hidden, I = p.inter, E = p.n_experts, K = p.k;

  DecodeSmem sm;
  {
    float* q = smem_raw;
    sm.v = q; q += H;
    sm.logit = q; q += E;
    sm.part = q; q += p.router_items;
    sm.a = q; q += K * I;
    sm.y = q; q += K * p.rows_per_wg;
    sm.red = q; q += kDecodeWaves;
    sm.wsel = q; q += 16;
    sm.isel = reinterpret_cast<int*>(q); q += 16;
    sm.fail = reinterpret_cast<int*>(q);
  }
  if (tid == 0) *sm.fail = 0;
  __syncthreads();

  // geometry of the quantized rows
  const size_t cbH = (size_t)I * H * BITS / 8;  // bytes of gate (= up = down) codes
  const size_t sbb = (size_t)I * (H / 64) * 4;  // bytes of one sb array
  const int ngH = H / 64, ngI = I / 64;
  const size_t rowH = (size_t)H * BITS / 8, rowI = (size_t)I * BITS / 8;
  const int nchG = H / C::kCodes, nchD = I / C::kCodes;
  const int lprG = p.lpr_g, rpwG = 64 / lprG, subG = lane & (lprG - 1), rselG = lane / lprG;
  const int lprD = p.lpr_d, rpwD = 64 / lprD, subD = lane & (lprD - 1), rselD = lane / lprD;
  const int r0 = g * p.rows_per_wg;
  const int nr = max(0, min(H - r0, p.rows_per_wg));
  const int S = (H + 1023) / 1024;  // router slices per row
  const int my_experts = (E - g + G - 1) / G;

  for (int l = 0; l < p.n_layers; ++l) {
    const int lg = p.layer0 + l;
    const float* R = p.router[l];
    const uint8_t* X = p.experts[l];

    // ---- 1. v = rmsnorm(h) or h, in LDS
    float ss = 0.f;
    for (int i = tid; i < H; i += kDecodeThreads) {
      float hv = (lg == 0) ? p.x_in[i] : ld_dev(p.h + i);
      sm.v[i] = hv;
      ss = fmaf(hv, hv, ss);
    }
    ss = wave_sum(ss);
    if (lane == 0) sm.red[wave] = ss;
    __syncthreads();
    float inv = 1.f;
    if (p.flags & FMOE_PRENORM) {
      float tot = 0.f;
      for (int w2 = 0; w2 < kDecodeWaves; ++w2) tot += sm.red[w2];
      inv = 1.0f / sqrtf(tot / (float)H + p.eps);
    }
    for (int i = tid; i < H; i += kDecodeThreads) sm.v[i] *= inv;
    __syncthreads();

    // ---- 2. router rows of this workgroup's experts, 1024-column slices per wave
    for (int it = wave; it < my_experts * S; it += kDecodeWaves) {
      const int el = it / S, s = it % S;
      const int e = g + el * G;
      const int c0 = s * 1024, c1 = min(H, c0 + 1024);
      const float4* row = reinterpret_cast<const float4*>(R + (size_t)e * H);
      float acc = 0.f;
      for (int c = c0 / 4 + lane; c < c1 / 4; c += 64) {
        float4 r = row[c];
        acc = fmaf(r.x, sm.v[4 * c + 0], acc);
        acc = fmaf(r.y, sm.v[4 * c + 1], acc);
        acc = fmaf(r.z, sm.v[4 * c + 2], acc);
        acc = fmaf(r.w, sm.v[4 * c + 3], acc);
      }
      acc = wave_sum(acc);
      if (lane == 0) sm.part[it] = acc;
    }
    __syncthreads();
    const uint64_t tag = (uint64_t)(uint32_t)(lg + 1) << 32;
    for (int el = tid; el < my_experts; el += kDecodeThreads) {
      float lsum = 0.f;
      for (int s = 0; s < S; ++s) lsum += sm.part[el * S + s];
      st_dev_u64(p.logits + g + el * G, tag | __float_as_uint(lsum));
    }

    // ---- 3. gather all tagged logits (wave 0), top-k + softmax
    if (wave == 0) {
      unsigned spins = 0;
      while (true) {
        bool ok = true;
        for (int e = lane; e < E; e += 64) {
          uint64_t t = ld_dev_u64(p.logits + e);
          if ((t & 0xffffffff00000000ull) == tag) sm.logit[e] = __uint_as_float((uint32_t)t);
          else ok = false;
        }
        if (__all(ok)) break;
        if (++spins > kSpinLimit || spin_failed(p.err)) {
          if (lane == 0) {
            st_dev_u32(p.err, 1u);
            *sm.fail = 1;
          }
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      uint64_t taken = 0;
      for (int r = 0; r < K; ++r) {
        float best = 0.f;
        int bi = -1;
        for (int j = 0, e = lane; e < E; ++j, e += 64) {
          if ((taken >> j) & 1ull) continue;
          float v = sm.logit[e];
          if (bi < 0 || ranks_before(v, e, best, bi)) {
            best = v;
            bi = e;
          }
        }
        for (int m = 32; m >= 1; m >>= 1) {
          float ov = __shfl_xor(best, m, 64);
          int oi = __shfl_xor(bi, m, 64);
          if (oi >= 0 && (bi < 0 || ranks_before(ov, oi, best, bi))) {
            best = ov;
            bi = oi;
          }
        }
        if (bi >= 0 && (bi & 63) == lane) taken |= 1ull << (bi >> 6);
        if (lane == 0) {
          sm.isel[r] = bi;
          sm.wsel[r] = best;  // logit for now
        }
      }
      if (lane == 0) {
        float l0 = sm.wsel[0], denom = 0.f, ex[16];
        for (int j = 0; j < K; ++j) {
          ex[j] = expf(sm.wsel[j] - l0);
          denom += ex[j];
        }
        for (int j = 0; j < K; ++j) sm.wsel[j] = ex[j] / denom;
        if (*sm.fail) {
          for (int j = 0; j < K; ++j) sm.isel[j] = 0;
        }
      }
      if (g == 0 && lane < K) {
        size_t o = ((size_t)lg) * K + lane;
        if (p.idx_out) p.idx_out[o] = sm.isel[lane];
        if (p.w_out) p.w_out[o] = sm.wsel[lane];
      }
    }
    __syncthreads();
    if (*sm.fail) break;

    // ---- 4. gate/up + SwiGLU: items (j, i) in blocks of rpwG consecutive items
    {
      XChunk<BITS> xc[CPL_G];
#pragma unroll
      for (int j = 0; j < CPL_G; ++j) {
        int c = subG + lprG * j;
        if (c < nchG) load_xchunk<BITS>(xc[j], sm.v + c * C::kCodes);
      }
      const int n_items = K * I;
      const int n_blocks = (n_items + rpwG - 1) / rpwG;
      for (int b = g + G * wave; b < n_blocks; b += G * kDecodeWaves) {
        const int item = b * rpwG + rselG;
        float gs = 0.f, us = 0.f;
        const bool valid = item < n_items;
        if (valid) {
          const int j = item / I, i = item % I;
          const uint8_t* base = X + (size_t)sm.isel[j] * p.expert_stride;
          const uint4* gp = reinterpret_cast<const uint4*>(base + (size_t)i * rowH);
          const uint4* up = reinterpret_cast<const uint4*>(base + cbH + (size_t)i * rowH);
          const uint32_t* gsb = reinterpret_cast<const uint32_t*>(base + 3 * cbH) + (size_t)i * ngH;
          const uint32_t* usb = reinterpret_cast<const uint32_t*>(base + 3 * cbH + sbb) + (size_t)i * ngH;
          uint4 wg[CPL_G], wu[CPL_G];
          uint32_t sg[CPL_G], su[CPL_G];
#pragma unroll
          for (int q = 0; q < CPL_G; ++q) {
            int c = subG + lprG * q;
            if (c < nchG) {
              wg[q] = gp[c];
              wu[q] = up[c];
              sg[q] = gsb[c / C::kPerGroup];
              su[q] = usb[c / C::kPerGroup];
            }
          }
#pragma unroll
          for (int q = 0; q < CPL_G; ++q) {
            int c = subG + lprG * q;
            if (c < nchG) {
              gs += chunk_dot<BITS>(wg[q], sg[q], xc[q]);
              us += chunk_dot<BITS>(wu[q], su[q], xc[q]);
            }
          }
        }
        gs = group_sum(gs, lprG);
        us = group_sum(us, lprG);
        if (valid && subG == 0) st_dev(p.a + item, swiglu(gs, us));
      }
    }

    // ---- 5. all of a is published
    if (!grid_barrier(p.flags_arr, G, 2u * lg + 1u, p.err, sm.fail)) break;
    for (int i = tid; i < K * I; i += kDecodeThreads) sm.a[i] = ld_dev(p.a + i);
    __syncthreads();

    // ---- 6. down + combine + residual for rows [r0, r0 + nr)
    {
      const int n_rb = (nr + rpwD - 1) / rpwD;  // row blocks per slot
      int cur_j = -1;
      XChunk<BITS> xc[CPL_D];
      for (int it = wave; it < K * n_rb; it += kDecodeWaves) {
        const int j = it / n_rb, rb = it % n_rb;
        if (j != cur_j) {
#pragma unroll
          for (int q = 0; q < CPL_D; ++q) {
            int c = subD + lprD * q;
            if (c < nchD) load_xchunk<BITS>(xc[q], sm.a + j * I + c * C::kCodes);
          }
          cur_j = j;
        }
        const int rl = rb * rpwD + rselD;  // local row
        float acc = 0.f;
        if (rl < nr) {
          const int r = r0 + rl;
          const uint8_t* base = X + (size_t)sm.isel[j] * p.expert_stride;
          const uint4* dp = reinterpret_cast<const uint4*>(base + 2 * cbH + (size_t)r * rowI);
          const uint32_t* dsb = reinterpret_cast<const uint32_t*>(base + 3 * cbH + 2 * sbb) + (size_t)r * ngI;
          uint4 wd[CPL_D];
          uint32_t sd[CPL_D];
#pragma unroll
          for (int q = 0; q < CPL_D; ++q) {
            int c = subD + lprD * q;
            if (c < nchD) {
              wd[q] = dp[c];
              sd[q] = dsb[c / C::kPerGroup];
            }
          }
#pragma unroll
          for (int q = 0; q < CPL_D; ++q) {
            int c = subD + lprD * q;
            if (c < nchD) acc += chunk_dot<BITS>(wd[q], sd[q], xc[q]);
          }
        }
        acc = group_sum(acc, lprD);
        if (rl < nr && subD == 0) sm.y[j * p.rows_per_wg + rl] = acc;
      }
    }
    __syncthreads();
    const bool last = (l == p.n_layers - 1) && p.is_final;
    for (int rl = tid; rl < nr; rl += kDecodeThreads) {
      const int r = r0 + rl;
      float hv = (lg == 0) ? p.x_in[r] : ld_dev(p.h + r);
      float c = 0.f;
      for (int j = 0; j < K; ++j) c = fmaf(sm.wsel[j], sm.y[j * p.rows_per_wg + rl], c);
      float hn = hv + c;
      st_dev(p.h + r, hn);
      if (last) p.h_out[r] = hn;
    }
    // ---- 7. all of h is published
    if (l + 1 < p.n_layers) {
      if (!grid_barrier(p.flags_arr, G, 2u * lg + 2u, p.err, sm.fail)) break;
    }
  }
  if (*sm.fail && p.is_final) {
    for (int r = r0 + tid; r < r0 + nr; r += kDecodeThreads) p.h_out[r] = __uint_as_float(0x7fc00000u);
  }
}

__global__ void clear_kernel(uint32_t* p, size_t n_words) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n_words; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

int decode_geometry(int hidden, int inter, int bits, int* lpr_g, int* cpl_g, int* lpr_d, int* cpl_d) {
  const int cc = bits == 4 ? 32 : 64;
  int nG = hidden / cc, nD = inter / cc;
  int lg = 1, ld = 1;
  while (lg < nG && lg < 64) lg <<= 1;
  while (ld < nD && ld < 64) ld <<= 1;
  *lpr_g = lg;
  *lpr_d = ld;
  *cpl_g = (nG + lg - 1) / lg;
  *cpl_d = (nD + ld - 1) / ld;
  if (*cpl_g != 1 && *cpl_g != 2 && *cpl_g != 4) return FMOE_ERR_SHAPE;
  if (*cpl_d != 1 && *cpl_d != 2 && *cpl_d != 4) return FMOE_ERR_SHAPE;
  return FMOE_OK;
}

size_t decode_smem_bytes(int hidden, int inter, int n_experts, int k, int G, int rows_per_wg) {
  int my_experts = (n_experts + G - 1) / G;
  int S = (hidden + 1023) / 1024;
  size_t floats = (size_t)hidden + n_experts + (size_t)my_experts * S + (size_t)k * inter + (size_t)k * rows_per_wg +
                  kDecodeWaves + 16 + 16 + 1;
  return floats * 4;
}

int decode_grid(int* G_out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FMOE_ERR_HIP;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return FMOE_ERR_HIP;
  *G_out = cus;
  return FMOE_OK;
}

template <int BITS, int CG, int CD>
static int launch_decode_t(const DecodeParams& p, int G, size_t smem, hipStream_t s) {
  auto fn = decode_kernel<BITS, CG, CD>;
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fn, kDecodeThreads, smem) != hipSuccess) return FMOE_ERR_HIP;
  if (occ < 1) return FMOE_ERR_SHAPE;
  DecodeParams q = p;
  void* args[] = {&q};
  if (hipLaunchCooperativeKernel(reinterpret_cast<const void*>(fn), dim3(G), dim3(kDecodeThreads), args,
                                 (unsigned)smem, s) != hipSuccess)
    return FMOE_ERR_HIP;
  return FMOE_OK;
}

int launch_decode(const DecodeParams& p, int G, hipStream_t s) {
  const size_t smem = decode_smem_bytes(p.hidden, p.inter, p.n_experts, p.k, G, p.rows_per_wg);
  int cg = p.cpl_g, cd = p.cpl_d;
#define FMOE_DEC(B, X, Y) \
  if (p.bits == B && cg == X && cd == Y) return launch_decode_t<B, X, Y>(p, G, smem, s);
  FMOE_DEC(4, 1, 1) FMOE_DEC(4, 2, 1) FMOE_DEC(4, 4, 1) FMOE_DEC(4, 1, 2) FMOE_DEC(4, 2, 2) FMOE_DEC(4, 4, 2)
  FMOE_DEC(4, 1, 4) FMOE_DEC(4, 2, 4) FMOE_DEC(4, 4, 4)
  FMOE_DEC(2, 1, 1) FMOE_DEC(2, 2, 1) FMOE_DEC(2, 4, 1) FMOE_DEC(2, 1, 2) FMOE_DEC(2, 2, 2) FMOE_DEC(2, 4, 2)
  FMOE_DEC(2, 1, 4) FMOE_DEC(2, 2, 4) FMOE_DEC(2, 4, 4)
#undef FMOE_DEC
  return FMOE_ERR_SHAPE;
}

int launch_clear(uint32_t* p, size_t n_words, hipStream_t s) {
  unsigned blocks = (unsigned)((n_words + 255) / 256);
  if (blocks > 1024) blocks = 1024;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(clear_kernel, dim3(blocks), dim3(256), 0, s, p, n_words);
  return hipGetLastError() == hipSuccess ? FMOE_OK : FMOE_ERR_HIP;
}

}  // namespace fmoe
