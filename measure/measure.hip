// measure.hip -- measurement kernels of the benchmark (not part of the fmoe library).
//
// 1. A read-only streaming kernel: the attainable HBM read rate of plain streaming code on
//    this device, the bar beside the published 8 TB/s peak (plain, non-temporal, and
//    LDS-DMA loads). Each thread keeps U 16-byte
//    loads in flight over a grid-strided walk of the buffer; the loaded words are folded
//    into one register that is stored only if it equals an impossible value, so the kernel
//    writes nothing and no load can be removed.
// 2. An exchange-latency probe: a persistent grid (one workgroup per compute unit, all
//    resident) runs `rounds` chained exchanges of n_words tagged 64-bit words (value |
//    round << 32): in every round each workgroup publishes its share of the words, waits
//    for its stores, then polls all the words of its group until each carries the current
//    round (or a later one) and stamps the 100 MHz real-time clock. Round r + 1 starts
//    from the data of round r, so the spacing of the stamps is the latency of one exchange
//    including the spread between workgroups. Modes:
//      0  all workgroups, R replicas (replica g mod R), device-scope accesses (the decode
//         kernel's exchange uses R = 8);
//      1  the 32 workgroups of one XCD (workgroup g is dispatched to XCD g mod 8), device-
//         scope accesses;
//      2  the same groups with workgroup-scope accesses;
//      3  the same groups with plain stores (written through the compute unit's L1 into
//         the XCD's shared L2) and plain loads after an invalidation of the reader's L1
//         (buffer_inv at workgroup scope), so both sides meet in the XCD's L2;
//      4  the same groups with plain stores and non-temporal loads.
//    Modes 2-4 are only correct when a group shares one XCD, which the probe checks with
//    the XCC_ID hardware register; a mode whose loads cannot see the group's stores ends
//    at the spin limit with the error word set.
//    Every wait is bounded (spin limit, then the error word).
// 3. A row-stage read: the access pattern of the batched expert kernels' weight stages. Each
//    wave owns a block of 64 rows of row_bytes bytes and reads it through D 8-KB LDS stage
//    buffers with LDS-DMA (eight 1-KB instructions per stage, D stages in flight); a stage
//    covers 8192 / P rows x P bytes (P = 128: 128 bytes of each of the 64 rows, the batched
//    kernels' 4-group stages; P = row_bytes: whole consecutive rows, a contiguous 8 KB). Same
//    bytes, instructions and depth for every P, so the rates differ only by the pattern.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr unsigned kSpinLimit = 1u << 22;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int U, bool NT>
__global__ void __launch_bounds__(kThreads) stream_read_kernel(const u32x4* __restrict__ p, size_t n,
                                                               uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (U - 1) * stride < n; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = NT ? __builtin_nontemporal_load(p + i + u * stride) : p[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n; i += stride) {
    const u32x4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u && threadIdx.x == 0x3FF) sink[0] = acc;  // never true: threadIdx.x < 256
}

// The same read through LDS-DMA (global_load_lds_dwordx4, 16 bytes per lane into LDS, one KB
// per wave instruction): each wave streams its grid-strided KB-sized pieces into a private
// ring of U KB in LDS, keeping U instructions in flight, and folds one dword of each landed
// KB into a register (read back from LDS after the data has arrived).
template <int U, bool NT>
__global__ void __launch_bounds__(kThreads) stream_read_lds_kernel(const u32x4* __restrict__ p, size_t n,
                                                                   uint32_t* __restrict__ sink) {
  __shared__ uint32_t ring[kThreads / 64][U][256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const size_t n_kb = n / 64;  // KB pieces (64 lanes x 16 bytes)
  const size_t stride = (size_t)gridDim.x * (kThreads / 64);
  size_t kb = (size_t)blockIdx.x * (kThreads / 64) + wave;
  uint32_t acc = 0;
  for (; kb + (U - 1) * stride < n_kb; kb += U * stride) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const u32x4* src = p + (kb + u * stride) * 64 + lane;
      const uint32_t lds = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)&ring[wave][u][0];
      if (NT)
        asm volatile(
            "s_mov_b32 m0, %1\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %0, off nt" ::"v"(src),
            "s"(__builtin_amdgcn_readfirstlane(lds))
            : "memory", "m0");
      else
        asm volatile(
            "s_mov_b32 m0, %1\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %0, off" ::"v"(src),
            "s"(__builtin_amdgcn_readfirstlane(lds))
            : "memory", "m0");
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= ring[wave][u][lane * 4];
  }
  if (acc == 0x9E3779B9u && threadIdx.x == 0x3FF) sink[0] = acc;  // never true: threadIdx.x < 256
}

// Row-stage read (item 3 above). Stage s of a wave's block covers rows rg * Rs .. + Rs - 1
// (Rs = 8192 / P, rg = s / (row_bytes / P)) at bytes c * P .. + P - 1 of each (c = s mod
// row_bytes / P); byte e of the stage (e = 1024 j + 16 lane for instruction j) is byte e mod P
// of its row e / P. Requires row_bytes % P == 0 and P | 8192 (checked by the caller).
template <int P, int D>
__global__ void __launch_bounds__(kThreads) row_stage_kernel(const uint8_t* __restrict__ p, int row_bytes,
                                                             uint32_t* __restrict__ sink) {
  __shared__ uint32_t ring[kThreads / 64][D][2048];
  constexpr int Rs = 8192 / P;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint8_t* blk = p + ((size_t)blockIdx.x * (kThreads / 64) + wave) * 64 * (size_t)row_bytes;
  const int n_c = row_bytes / P, stages = row_bytes / 128;
  auto issue = [&](int s) {
    const int rg = s / n_c, c = s - rg * n_c;
    const uint8_t* base = blk + (size_t)rg * Rs * row_bytes + (size_t)c * P;
    const uint32_t lds = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)&ring[wave][s % D][0];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = j * 1024 + 16 * lane;
      const uint8_t* src = base + (size_t)(e / P) * row_bytes + (e % P);
      asm volatile(
          "s_mov_b32 m0, %1\n\t"
          "s_nop 0\n\t"
          "global_load_lds_dwordx4 %0, off nt" ::"v"(src),
          "s"(__builtin_amdgcn_readfirstlane(lds + j * 1024))
          : "memory", "m0");
    }
  };
  for (int s = 0; s < D && s < stages; ++s) issue(s);
  uint32_t acc = 0;
  for (int s = 0; s < stages; ++s) {
    if (s + D - 1 < stages)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(8 * (D - 1)) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    acc ^= ring[wave][s % D][lane * 32];
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (s + D < stages) issue(s + D);
  }
  if (acc == 0x9E3779B9u && threadIdx.x == 0x3FF) sink[0] = acc;  // never true: threadIdx.x < 256
}

__device__ __forceinline__ uint32_t xcc_id() { return __builtin_amdgcn_s_getreg((3 << 11) | 20); }

template <int MODE>
__device__ __forceinline__ void put(uint64_t* p, uint64_t v) {
  if (MODE == 2) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  else if (MODE >= 3) *p = v;  // plain store (kept in place by the asm wait that follows)
  else __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <int MODE>
__device__ __forceinline__ uint64_t get(const uint64_t* p) {
  if (MODE == 2) return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  if (MODE == 3) return *p;  // plain load (the asm invalidation before a pass forces a reload)
  if (MODE == 4) return __builtin_nontemporal_load(p);
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Mode 3: drop the reader's L1 copies before a pass of loads.
template <int MODE>
__device__ __forceinline__ void before_poll() {
  if (MODE == 3) asm volatile("buffer_inv sc0" ::: "memory");
}

// buf: mode 0: [reps][n_words]; modes 1-4: [8][n_words] (one region per XCD group).
// t_end: [rounds][G] stamps; xcc: [G] XCC_ID of each workgroup; err: set when a wait gave up.
template <int MODE>
__global__ void __launch_bounds__(kThreads) exchange_kernel(uint64_t* buf, int n_words, int rounds, uint32_t epoch0,
                                                            uint64_t* t_end, uint32_t* xcc, uint32_t* err, int reps,
                                                            int no_ack) {
  constexpr int kPoll = 16;
  const int G = gridDim.x, g = blockIdx.x, tid = threadIdx.x;
  const int grp = MODE == 0 ? g % reps : g % 8;  // replica (mode 0) or XCD group (modes 1-4)
  const int members = MODE == 0 ? G : G / 8;  // writers of one region
  const int rank = MODE == 0 ? g : g / 8;
  const int per = n_words / members;          // words owned by each writer
  __shared__ int failed;
  if (tid == 0) {
    failed = 0;
    xcc[g] = xcc_id();
  }
  __syncthreads();
  for (int r = 0; r < rounds && !failed; ++r) {
    const uint64_t tag = (uint64_t)(epoch0 + (uint32_t)r + 1u) << 32;
    for (int i = tid; i < per; i += kThreads) {
      const int w = rank * per + i;
      if (MODE == 0) {
        for (int rr = 0; rr < reps; ++rr) put<MODE>(buf + (size_t)rr * n_words + w, tag | (uint32_t)w);
      } else {
        put<MODE>(buf + (size_t)grp * n_words + w, tag | (uint32_t)w);
      }
    }
    if (!no_ack) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const uint64_t* src = buf + (size_t)grp * n_words;
    for (int i0 = tid; i0 < n_words; i0 += kThreads * kPoll) {
      uint64_t v[kPoll];
      before_poll<MODE>();
#pragma unroll
      for (int u = 0; u < kPoll; ++u) {
        const int i = i0 + u * kThreads;
        v[u] = i < n_words ? get<MODE>(src + i) : tag;
      }
      unsigned spins = 0;
      while (true) {
        bool ok = true;
#pragma unroll
        for (int u = 0; u < kPoll; ++u) ok &= (v[u] >> 32) >= (tag >> 32);
        if (ok) break;
        if (++spins > kSpinLimit || ((spins & 255u) == 255u && __hip_atomic_load(err, __ATOMIC_RELAXED,
                                                                                 __HIP_MEMORY_SCOPE_AGENT))) {
          __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          failed = 1;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
        before_poll<MODE>();
#pragma unroll
        for (int u = 0; u < kPoll; ++u) {
          const int i = i0 + u * kThreads;
          if ((v[u] >> 32) < (tag >> 32)) v[u] = get<MODE>(src + i);
        }
      }
    }
    __syncthreads();
    if (tid == 0) t_end[(size_t)r * G + g] = __builtin_amdgcn_s_memrealtime();
  }
}

template <typename K>
int coresident(K fn, int G) {
  int occ = 0, dev = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fn, kThreads, 0) != hipSuccess) return -8;
  if (hipGetDevice(&dev) != hipSuccess) return -8;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -8;
  return (occ >= 1 && G <= cus) ? 0 : -2;
}

}  // namespace

extern "C" {

// Number of compute units of the current device (the exchange probe's grid).
int measure_cus(void) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -8;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -8;
  return cus;
}

// Enqueue one read of nbytes (a multiple of 16; LDS-DMA: of 1024) at buf. variant: 0 plain
// loads, 1 non-temporal loads, 2 LDS-DMA, 3 non-temporal LDS-DMA; unroll 4 or 8 loads in flight per thread (LDS-DMA:
// KB pieces per wave); blocks: grid size.
int measure_stream_read(const void* buf, size_t nbytes, int variant, int unroll, int blocks, uint32_t* sink,
                        hipStream_t s) {
  if (!buf || !sink || nbytes % 16 || blocks < 1) return -1;
  const u32x4* p = static_cast<const u32x4*>(buf);
  const size_t n = nbytes / 16;
  if (variant == 0 && unroll == 4) hipLaunchKernelGGL((stream_read_kernel<4, false>), dim3(blocks), dim3(kThreads), 0, s, p, n, sink);
  else if (variant == 0 && unroll == 8) hipLaunchKernelGGL((stream_read_kernel<8, false>), dim3(blocks), dim3(kThreads), 0, s, p, n, sink);
  else if (variant == 1 && unroll == 4) hipLaunchKernelGGL((stream_read_kernel<4, true>), dim3(blocks), dim3(kThreads), 0, s, p, n, sink);
  else if (variant == 1 && unroll == 8) hipLaunchKernelGGL((stream_read_kernel<8, true>), dim3(blocks), dim3(kThreads), 0, s, p, n, sink);
  else if (variant == 2 && unroll == 4) hipLaunchKernelGGL((stream_read_lds_kernel<4, false>), dim3(blocks), dim3(kThreads), 0, s, p, n, sink);
  else if (variant == 2 && unroll == 8) hipLaunchKernelGGL((stream_read_lds_kernel<8, false>), dim3(blocks), dim3(kThreads), 0, s, p, n, sink);
  else if (variant == 3 && unroll == 4) hipLaunchKernelGGL((stream_read_lds_kernel<4, true>), dim3(blocks), dim3(kThreads), 0, s, p, n, sink);
  else if (variant == 3 && unroll == 8) hipLaunchKernelGGL((stream_read_lds_kernel<8, true>), dim3(blocks), dim3(kThreads), 0, s, p, n, sink);
  else return -2;
  return hipGetLastError() == hipSuccess ? 0 : -8;
}

// Enqueue one row-stage read (item 3 of the file comment) of nbytes at buf: nbytes a multiple
// of 256 * row_bytes (one workgroup per 4 blocks of 64 rows), row_bytes a multiple of 128 and
// of piece, piece (P) one of 128, 256, 512, 1024, 2048, depth (D) 2 or 4 stages in flight.
int measure_row_stages(const void* buf, size_t nbytes, int row_bytes, int piece, int depth, uint32_t* sink,
                       hipStream_t s) {
  if (!buf || !sink || row_bytes < 128 || row_bytes % 128 || piece < 128 || row_bytes % piece) return -1;
  if (nbytes % ((size_t)256 * row_bytes)) return -1;
  const size_t blocks = nbytes / ((size_t)256 * row_bytes);
  if (blocks < 1 || blocks > 0x7FFFFFFF) return -1;
  const uint8_t* p = static_cast<const uint8_t*>(buf);
  const dim3 g((unsigned)blocks), b(kThreads);
#define ROW_STAGES(P_, D_)                                                                   \
  if (piece == P_ && depth == D_) {                                                          \
    hipLaunchKernelGGL((row_stage_kernel<P_, D_>), g, b, 0, s, p, row_bytes, sink);         \
    return hipGetLastError() == hipSuccess ? 0 : -8;                                         \
  }
  ROW_STAGES(128, 2) ROW_STAGES(256, 2) ROW_STAGES(512, 2) ROW_STAGES(1024, 2) ROW_STAGES(2048, 2)
  ROW_STAGES(128, 4) ROW_STAGES(256, 4) ROW_STAGES(512, 4) ROW_STAGES(1024, 4) ROW_STAGES(2048, 4)
#undef ROW_STAGES
  return -2;
}

// Enqueue the exchange probe (see the file comment). reps: replicas of mode 0 (1..16; the
// XCD modes use 8 regions); no_ack: poll without first waiting for the own stores.
// buf: max(reps, 8) * n_words uint64 (zero-filled
// before the first call; epoch0 must exceed every round tag of earlier calls on buf);
// n_words a multiple of the writers of a region (G, or G / 8); t_end: rounds * G uint64;
// xcc: G uint32; err: one uint32 (0 before the call). G = measure_cus().
int measure_exchange(int mode, int n_words, int rounds, uint32_t epoch0, void* buf, uint64_t* t_end, uint32_t* xcc,
                     uint32_t* err, int reps, int no_ack, hipStream_t s) {
  if (reps < 1 || reps > 16) return -2;
  const int G = measure_cus();
  if (G < 8 || G % 8) return -2;
  if (!buf || !t_end || !xcc || !err || rounds < 1 || n_words < 1) return -1;
  const int members = mode == 0 ? G : G / 8;
  if (n_words % members) return -2;
  int rc;
  uint64_t* b = static_cast<uint64_t*>(buf);
  switch (mode) {
    case 0:
      if ((rc = coresident(exchange_kernel<0>, G))) return rc;
      hipLaunchKernelGGL(exchange_kernel<0>, dim3(G), dim3(kThreads), 0, s, b, n_words, rounds, epoch0, t_end, xcc, err,
                         reps, no_ack);
      break;
    case 1:
      if ((rc = coresident(exchange_kernel<1>, G))) return rc;
      hipLaunchKernelGGL(exchange_kernel<1>, dim3(G), dim3(kThreads), 0, s, b, n_words, rounds, epoch0, t_end, xcc, err,
                         8, no_ack);
      break;
    case 2:
      if ((rc = coresident(exchange_kernel<2>, G))) return rc;
      hipLaunchKernelGGL(exchange_kernel<2>, dim3(G), dim3(kThreads), 0, s, b, n_words, rounds, epoch0, t_end, xcc, err,
                         8, no_ack);
      break;
    case 3:
      if ((rc = coresident(exchange_kernel<3>, G))) return rc;
      hipLaunchKernelGGL(exchange_kernel<3>, dim3(G), dim3(kThreads), 0, s, b, n_words, rounds, epoch0, t_end, xcc, err,
                         8, no_ack);
      break;
    case 4:
      if ((rc = coresident(exchange_kernel<4>, G))) return rc;
      hipLaunchKernelGGL(exchange_kernel<4>, dim3(G), dim3(kThreads), 0, s, b, n_words, rounds, epoch0, t_end, xcc, err,
                         8, no_ack);
      break;
    default:
      return -2;
  }
  return hipGetLastError() == hipSuccess ? 0 : -8;
}

}  // extern "C"
