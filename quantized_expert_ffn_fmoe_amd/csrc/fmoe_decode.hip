// fmoe_decode.hip -- single-token decode through a stack of MoE layers in ONE persistent
// kernel (one workgroup per compute unit, all co-resident).
//
// Per layer (aibit.im "Techniques de rupture" item 3 and tr.news.hada.io "Deferred GPU
// Expert Compute": route, run the k selected experts, combine with the residual, and
// normalize for the next layer; the pages route on the CPU, here routing stays on the
// device):
//   1. v = h * inv_rms(h) (or v = h without pre-norm), staged in LDS by every workgroup;
//   2. router: workgroup g owns experts g, g+G, ...; its waves dot 1024-column slices of
//      those rows with v; the logits are published with a tag (value | epoch << 32);
//   3. every workgroup polls the tagged logits, then selects the top-k and their softmax
//      weights itself (no extra round trip);
//   4. gate/up: (slot j, row i) items spread over all waves of all workgroups; each item
//      reads gate row i and up row i of expert idx[j] and publishes a[j][i] = silu(g)*u;
//      waves 1.. then issue the loads of their down-projection rows (prefetch);
//   5. grid barrier (arrival flags);
//   6. down + combine + residual: workgroup g owns a contiguous block of h rows and
//      computes h[r] += sum_j w_j * (Wd_j[r] . a_j) for them (fixed slot order);
//   7. grid barrier, next layer.
//
// Exchange between workgroups. Everything shared (h, a, logits, flags) is written and
// read with device-scope relaxed atomic accesses, which are performed at the device
// coherence point (no cache write-back or invalidation needed). A wave waits for its own
// stores (s_waitcnt) before its workgroup raises its flag, and reads exchanged data only
// after it has observed the flags. Each shared item is written to kRep replicas and
// workgroup g reads replica g % kRep, so that no memory line is polled by more than
// G / kRep workgroups at once (polling one line from all 256 workgroups serializes at the
// memory side and costs microseconds per round).
//
// Wave roles. Wave 0 is the communication wave: it raises the flags, polls, selects the
// top-k and combines; it never holds prefetch loads in flight, because a wave's loads
// return in issue order and a poll behind a prefetch would wait for it. Waves 1.. do the
// down-projection and may keep its loads in flight across the barrier.
//
// LDS layout. Activation vectors are stored with one padding word after every chunk of
// kCodes values, so that the 64 lanes of a wave, each reading its own chunk, hit 64
// different banks.
#include "fmoe_decode.h"
#include "fmoe_device.h"
#include "fmoe_internal.h"

namespace fmoe {

constexpr int kDecodeThreads = 256;
constexpr int kDecodeWaves = kDecodeThreads / 64;
constexpr int kDownWaves = kDecodeWaves - 1;  // waves 1.. run the down projection
constexpr unsigned kSpinLimit = 1u << 21;
// gate/up items and down row blocks whose loads are issued together (fewer when every
// lane holds more chunks per row, to stay within the register file)
template <int CPL> constexpr int batch_gu() { return CPL >= 4 ? 1 : 4; }
template <int CPL> constexpr int batch_d() { return CPL >= 4 ? 2 : (CPL == 2 ? 6 : 12); }
constexpr int kBatchN = 8;   // h values loaded together per thread

struct DecodeSmem {
  float* v;        // [hidden], padded
  uint64_t* key;   // [n_experts] rank keys
  float* part;     // [router items per workgroup]
  float* a;        // [k][inter], padded
  float* y;        // [k][rows per workgroup]
  float* red;      // [kDecodeWaves]
  float* wsel;     // [16]
  float* lsel;     // [16]
  int* isel;       // [16]
  int* fail;       // [1]
  uint32_t* base;  // [1]
};

template <int CC>
__device__ __forceinline__ int padded(int i) {
  return (i / CC) * (CC + 1) + (i % CC);
}

__device__ __forceinline__ bool spin_failed(unsigned spins, const uint32_t* err) {
  return spins > kSpinLimit || ((spins & 63u) == 63u && ld_dev_u32(err) != 0u);
}

// Wave 0 only: raise this workgroup's flag (every replica) to `epoch`, then wait until
// every flag of replica `rep` reached it. The caller has made sure that every wave's
// stores completed (s_waitcnt + workgroup barrier). Returns false when the wait gave up.
__device__ bool flag_arrive_and_wait(uint32_t* flags, int G, int rep, uint32_t epoch, uint32_t* err, int* fail) {
  const int lane = threadIdx.x & 63;
  if (lane < kRep) st_dev_u32(flags + (size_t)lane * kMaxGrid + blockIdx.x, epoch);
  const uint32_t* mine = flags + (size_t)rep * kMaxGrid;
  unsigned spins = 0;
  while (true) {
    bool ok = true;
    for (int j = lane; j < G; j += 64) ok &= (int32_t)(ld_dev_u32(mine + j) - epoch) >= 0;
    if (__all(ok)) return true;
    if (spin_failed(++spins, err)) {
      if (lane == 0) {
        st_dev_u32(err, 1u);
        *fail = 1;
      }
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// Fill XChunk registers from a padded LDS vector (chunk index c).
template <int BITS>
__device__ __forceinline__ void load_xchunk_padded(XChunk<BITS>& xc, const float* vpad, int c) {
  constexpr int CC = Chunk<BITS>::kCodes;
  load_xchunk<BITS>(xc, vpad + c * (CC + 1));
}

template <int BITS, int CPL_G, int CPL_D>
__global__ void __launch_bounds__(kDecodeThreads) decode_kernel(DecodeParams p) {
  constexpr int kBatchGU = batch_gu<CPL_G>();
  constexpr int kBatchD = batch_d<CPL_D>();
  using C = Chunk<BITS>;
  constexpr int CC = C::kCodes;
  extern __shared__ float smem_raw[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = gridDim.x, g = blockIdx.x, rep = g % kRep;
  const int H = p.hidden, I = p.inter, E = p.n_experts, K = p.k;

  DecodeSmem sm;
  {
    uint64_t* q64 = reinterpret_cast<uint64_t*>(smem_raw);
    sm.key = q64;
    float* q = reinterpret_cast<float*>(q64 + E);
    sm.v = q; q += H + H / CC;
    sm.part = q; q += p.router_items;
    sm.a = q; q += K * (I + I / CC);
    sm.y = q; q += K * p.rows_per_wg;
    sm.red = q; q += kDecodeWaves;
    sm.wsel = q; q += 16;
    sm.lsel = q; q += 16;
    sm.isel = reinterpret_cast<int*>(q); q += 16;
    sm.fail = reinterpret_cast<int*>(q); q += 1;
    sm.base = reinterpret_cast<uint32_t*>(q);
  }
  if (tid == 0) {
    *sm.fail = 0;
    // Every flag holds the same value F when a launch starts: 0 in a zero-filled
    // workspace, else the last epoch of the previous launch (all workgroups reach it).
    // This launch's epochs and logit tags are F + 1, F + 2, ...
    *sm.base = ld_dev_u32(p.flags_arr + (size_t)rep * kMaxGrid + blockIdx.x);
  }
  __syncthreads();
  const uint32_t F = *sm.base;

  // geometry of the quantized rows
  const size_t cbH = (size_t)I * H * BITS / 8;  // bytes of gate (= up = down) codes
  const size_t sbb = (size_t)I * (H / 64) * 4;  // bytes of one sb array
  const int ngH = H / 64, ngI = I / 64;
  const size_t rowH = (size_t)H * BITS / 8, rowI = (size_t)I * BITS / 8;
  const int nchG = H / CC, nchD = I / CC;
  const int lprG = p.lpr_g, rpwG = 64 / lprG, subG = lane & (lprG - 1), rselG = lane / lprG;
  const int lprD = p.lpr_d, rpwD = 64 / lprD, subD = lane & (lprD - 1), rselD = lane / lprD;
  const int r0 = g * p.rows_per_wg;
  const int nr = max(0, min(H - r0, p.rows_per_wg));
  const int n_rb = (nr + rpwD - 1) / rpwD;  // down row blocks per slot
  const int n_dit = (K * n_rb + kDownWaves - 1) / kDownWaves;  // down items per wave (waves 1..)
  const int S = (H + 1023) / 1024;  // router slices per row
  const int my_experts = (E - g + G - 1) / G;
  const size_t KI = (size_t)K * I;
  const float* h_rep = p.h + (size_t)rep * H;
  const float* a_rep = p.a + (size_t)rep * KI;
  const uint64_t* logits_rep = p.logits + (size_t)rep * E;

  for (int l = 0; l < p.n_layers; ++l) {
    const int lg = p.layer0 + l;
    const float* R = p.router[l];
    const uint8_t* X = p.experts[l];

    // ---- 1. v = rmsnorm(h) or h, in LDS (padded); loads issued kBatchN at a time
    float ss = 0.f;
    for (int i0 = tid; i0 < H; i0 += kDecodeThreads * kBatchN) {
      float hv[kBatchN];
#pragma unroll
      for (int u = 0; u < kBatchN; ++u) {
        const int i = i0 + u * kDecodeThreads;
        hv[u] = i < H ? ((lg == 0) ? p.x_in[i] : ld_dev(h_rep + i)) : 0.f;
      }
#pragma unroll
      for (int u = 0; u < kBatchN; ++u) {
        const int i = i0 + u * kDecodeThreads;
        if (i < H) sm.v[padded<CC>(i)] = hv[u];
        ss = fmaf(hv[u], hv[u], ss);
      }
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
    for (int i = tid; i < H; i += kDecodeThreads) sm.v[padded<CC>(i)] *= inv;
    __syncthreads();

    // ---- 2. router rows of this workgroup's experts, 1024-column slices per wave
    for (int it = wave; it < my_experts * S; it += kDecodeWaves) {
      const int el = it / S, s = it % S;
      const int e = g + el * G;
      const int c0 = s * 256, c1 = min(H / 4, c0 + 256);  // float4 columns of the slice
      const float4* row = reinterpret_cast<const float4*>(R + (size_t)e * H);
      float4 rv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = c0 + lane + 64 * u;
        if (c < c1) rv[u] = row[c];
      }
      float acc = 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = c0 + lane + 64 * u;
        if (c < c1) {
          const int pi = padded<CC>(4 * c);  // 4 consecutive values never straddle a chunk
          acc = fmaf(rv[u].x, sm.v[pi + 0], acc);
          acc = fmaf(rv[u].y, sm.v[pi + 1], acc);
          acc = fmaf(rv[u].z, sm.v[pi + 2], acc);
          acc = fmaf(rv[u].w, sm.v[pi + 3], acc);
        }
      }
      acc = wave_sum(acc);
      if (lane == 0) sm.part[it] = acc;
    }
    __syncthreads();
    const uint64_t tag = (uint64_t)(F + (uint32_t)l + 1u) << 32;

    // ---- 3. publish this workgroup's logits, gather all of them, top-k (wave 0)
    if (wave == 0) {
      for (int t = lane; t < my_experts * kRep; t += 64) {
        const int el = t / kRep, rr = t % kRep;
        float lsum = 0.f;
        for (int s = 0; s < S; ++s) lsum += sm.part[el * S + s];
        st_dev_u64(p.logits + (size_t)rr * E + g + el * G, tag | __float_as_uint(lsum));
      }
      unsigned spins = 0;
      while (true) {
        bool ok = true;
        for (int e = lane; e < E; e += 64) {
          uint64_t t = ld_dev_u64(logits_rep + e);
          if ((t & 0xffffffff00000000ull) == tag) sm.key[e] = rank_key(__uint_as_float((uint32_t)t), e);
          else ok = false;
        }
        if (__all(ok)) break;
        if (spin_failed(++spins, p.err)) {
          if (lane == 0) {
            st_dev_u32(p.err, 1u);
            *sm.fail = 1;
          }
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      if (*sm.fail) {
        if (lane < K) {
          sm.isel[lane] = 0;
          sm.wsel[lane] = 0.f;
        }
      } else {
        wave_topk_keys(sm.key, E, K, sm.isel, sm.lsel, sm.wsel);
      }
      if (g == 0 && lane < K) {
        size_t o = ((size_t)lg) * K + lane;
        if (p.idx_out) p.idx_out[o] = sm.isel[lane];
        if (p.w_out) p.w_out[o] = sm.wsel[lane];
      }
    }
    __syncthreads();
    if (*sm.fail) break;

    // ---- 4. gate/up + SwiGLU: items (j, i) in blocks of rpwG consecutive items; the
    // loads of kBatchGU blocks are issued before any of them is used
    {
      XChunk<BITS> xc[CPL_G];
#pragma unroll
      for (int q = 0; q < CPL_G; ++q) {
        int c = subG + lprG * q;
        if (c < nchG) load_xchunk_padded<BITS>(xc[q], sm.v, c);
      }
      const int n_items = K * I;
      const int n_blocks = (n_items + rpwG - 1) / rpwG;
      const int bstride = G * kDecodeWaves;
      for (int b0 = g + G * wave; b0 < n_blocks; b0 += bstride * kBatchGU) {
        uint4 wg[kBatchGU][CPL_G], wu[kBatchGU][CPL_G];
        uint32_t sg[kBatchGU][CPL_G], su[kBatchGU][CPL_G];
#pragma unroll
        for (int u = 0; u < kBatchGU; ++u) {
          const int item = (b0 + u * bstride) * rpwG + rselG;
          if (b0 + u * bstride < n_blocks && item < n_items) {
            const int j = item / I, i = item % I;
            const uint8_t* base = X + (size_t)sm.isel[j] * p.expert_stride;
            const uint4* gp = reinterpret_cast<const uint4*>(base + (size_t)i * rowH);
            const uint4* up = reinterpret_cast<const uint4*>(base + cbH + (size_t)i * rowH);
            const uint32_t* gsb = reinterpret_cast<const uint32_t*>(base + 3 * cbH) + (size_t)i * ngH;
            const uint32_t* usb = reinterpret_cast<const uint32_t*>(base + 3 * cbH + sbb) + (size_t)i * ngH;
#pragma unroll
            for (int q = 0; q < CPL_G; ++q) {
              int c = subG + lprG * q;
              if (c < nchG) {
                wg[u][q] = gp[c];
                wu[u][q] = up[c];
                sg[u][q] = gsb[c / C::kPerGroup];
                su[u][q] = usb[c / C::kPerGroup];
              }
            }
          }
        }
#pragma unroll
        for (int u = 0; u < kBatchGU; ++u) {
          if (b0 + u * bstride >= n_blocks) break;  // uniform over the wave
          const int item = (b0 + u * bstride) * rpwG + rselG;
          const bool valid = item < n_items;
          float gs = 0.f, us = 0.f;
          if (valid) {
#pragma unroll
            for (int q = 0; q < CPL_G; ++q) {
              int c = subG + lprG * q;
              if (c < nchG) {
                gs += chunk_dot<BITS>(wg[u][q], sg[u][q], xc[q]);
                us += chunk_dot<BITS>(wu[u][q], su[u][q], xc[q]);
              }
            }
          }
          gs = group_sum(gs, lprG);
          us = group_sum(us, lprG);
          if (valid && subG == 0) {
            const float av = swiglu(gs, us);
#pragma unroll
            for (int rr = 0; rr < kRep; ++rr) st_dev(p.a + (size_t)rr * KI + item, av);
          }
        }
      }
    }
    wait_vmem();  // this wave's a-stores are at the coherence point

    // ---- prefetch: waves 1.. issue the loads of their first kBatchD down items
    uint4 wd[kBatchD][CPL_D];
    uint32_t sd[kBatchD][CPL_D];
    auto down_item = [&](int m, int& j, int& rl) {
      const int t = (wave - 1) + kDownWaves * m;
      j = t / max(n_rb, 1);
      rl = (t % max(n_rb, 1)) * rpwD + rselD;
      return wave > 0 && m < n_dit && j < K;
    };
    auto down_load = [&](int m, int u) {
      int j, rl;
      if (down_item(m, j, rl) && rl < nr) {
        const int r = r0 + rl;
        const uint8_t* base = X + (size_t)sm.isel[j] * p.expert_stride;
        const uint4* dp = reinterpret_cast<const uint4*>(base + 2 * cbH + (size_t)r * rowI);
        const uint32_t* dsb = reinterpret_cast<const uint32_t*>(base + 3 * cbH + 2 * sbb) + (size_t)r * ngI;
#pragma unroll
        for (int q = 0; q < CPL_D; ++q) {
          int c = subD + lprD * q;
          if (c < nchD) {
            wd[u][q] = dp[c];
            sd[u][q] = dsb[c / C::kPerGroup];
          }
        }
      }
    };
#pragma unroll
    for (int u = 0; u < kBatchD; ++u) down_load(u, u);

    // ---- 5. all of a is published
    __syncthreads();
    if (wave == 0) flag_arrive_and_wait(p.flags_arr, G, rep, F + 2u * l + 1u, p.err, sm.fail);
    __syncthreads();
    if (*sm.fail) break;
    for (int i0 = tid; i0 < (int)KI; i0 += kDecodeThreads * kBatchN) {
      float av[kBatchN];
#pragma unroll
      for (int u = 0; u < kBatchN; ++u) {
        const int i = i0 + u * kDecodeThreads;
        av[u] = i < (int)KI ? ld_dev(a_rep + i) : 0.f;
      }
#pragma unroll
      for (int u = 0; u < kBatchN; ++u) {
        const int i = i0 + u * kDecodeThreads;
        if (i < (int)KI) sm.a[(i / I) * (I + I / CC) + padded<CC>(i % I)] = av[u];
      }
    }
    __syncthreads();

    // ---- 6. down (waves 1..), then combine + residual (wave 0)
    if (wave > 0) {
      int cur_j = -1;
      XChunk<BITS> xc[CPL_D];
      for (int m0 = 0; m0 < n_dit; m0 += kBatchD) {
        if (m0 > 0) {
#pragma unroll
          for (int u = 0; u < kBatchD; ++u) down_load(m0 + u, u);
        }
#pragma unroll
        for (int u = 0; u < kBatchD; ++u) {
          int j, rl;
          if (!down_item(m0 + u, j, rl)) continue;  // uniform over the wave
          if (j != cur_j) {
#pragma unroll
            for (int q = 0; q < CPL_D; ++q) {
              int c = subD + lprD * q;
              if (c < nchD) load_xchunk_padded<BITS>(xc[q], sm.a + j * (I + I / CC), c);
            }
            cur_j = j;
          }
          float acc = 0.f;
          if (rl < nr) {
#pragma unroll
            for (int q = 0; q < CPL_D; ++q) {
              int c = subD + lprD * q;
              if (c < nchD) acc += chunk_dot<BITS>(wd[u][q], sd[u][q], xc[q]);
            }
          }
          acc = group_sum(acc, lprD);
          if (rl < nr && subD == 0) sm.y[j * p.rows_per_wg + rl] = acc;
        }
      }
    }
    __syncthreads();
    const bool last = (l == p.n_layers - 1) && p.is_final;
    if (wave == 0) {
      for (int rl = lane; rl < nr; rl += 64) {
        const int r = r0 + rl;
        float hv = (lg == 0) ? p.x_in[r] : ld_dev(h_rep + r);
        float c = 0.f;
        for (int j = 0; j < K; ++j) c = fmaf(sm.wsel[j], sm.y[j * p.rows_per_wg + rl], c);
        float hn = hv + c;
#pragma unroll
        for (int rr = 0; rr < kRep; ++rr) st_dev(p.h + (size_t)rr * H + r, hn);
        if (last) p.h_out[r] = hn;
      }
      wait_vmem();
    }
    // ---- 7. all of h is published
    if (l + 1 < p.n_layers) {
      __syncthreads();
      if (wave == 0) flag_arrive_and_wait(p.flags_arr, G, rep, F + 2u * l + 2u, p.err, sm.fail);
      __syncthreads();
      if (*sm.fail) break;
    }
  }
  if (*sm.fail && p.is_final) {
    for (int r = r0 + tid; r < r0 + nr; r += kDecodeThreads) p.h_out[r] = __uint_as_float(0x7fc00000u);
  }
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

size_t decode_smem_bytes(int hidden, int inter, int n_experts, int k, int G, int rows_per_wg, int bits) {
  const int cc = bits == 4 ? 32 : 64;
  int my_experts = (n_experts + G - 1) / G;
  int S = (hidden + 1023) / 1024;
  size_t floats = (size_t)hidden + hidden / cc + (size_t)my_experts * S + (size_t)k * (inter + inter / cc) +
                  (size_t)k * rows_per_wg + kDecodeWaves + 16 + 16 + 16 + 2;
  return (size_t)n_experts * 8 + floats * 4;
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
  const size_t smem = decode_smem_bytes(p.hidden, p.inter, p.n_experts, p.k, G, p.rows_per_wg, p.bits);
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

}  // namespace fmoe
