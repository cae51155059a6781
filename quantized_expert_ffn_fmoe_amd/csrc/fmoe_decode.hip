// fmoe_decode.hip -- single-token decode through a stack of MoE layers in ONE persistent
// kernel (one workgroup per compute unit, all co-resident; plain launch, see launch_decode_t).
//
// Per layer (aibit.im "Techniques de rupture" item 3 and tr.news.hada.io "Deferred GPU
// Expert Compute": route, run the k selected experts, combine with the residual, and
// normalize for the next layer; the pages route on the CPU, here routing stays on the
// device):
//   1. every workgroup gathers h (x on the first layer) into LDS and its sum of squares;
//      v = h * inv_rms(h) (or v = h without pre-norm) is never formed, inv_rms scales the
//      router sums and v's digit image instead;
//   2. router: workgroup g owns experts g, g+G, ...; its waves dot 1024-column slices of
//      those rows (loaded during the previous layer) with h; the logits are published;
//   3. every workgroup gathers the logits; wave 0 selects the top-k and the softmax
//      weights (no extra round trip) and releases the slots one by one, while the other
//      waves build the digit image of v (see fmoe_intdot.h);
//   4. gate/up: every workgroup takes 4 consecutive rows of every routed slot, slot j on
//      wave (j + 1) mod 4 once that slot's top-k round is out (compiled shapes; otherwise a
//      contiguous run of (slot, row) items per workgroup); each item reads gate row i and up
//      row i of expert idx[j] and publishes a[j][i] = silu(g)*u; every wave then issues the
//      loads of its down rows;
//   5. a: each wave gathers the a values of the slot(s) its down rows belong to and
//      builds their digit image;
//   6. down + combine + residual: workgroup g owns a contiguous block of h rows and
//      computes h[r] += sum_j w_j * (Wd_j[r] . a_j) for them (fixed slot order), published
//      for the next layer.
//
// Exchange between workgroups. h, a and the logits are exchanged as 64-bit words
// (fp32 value | epoch << 32), written and read with device-scope relaxed atomic accesses,
// which are performed at the device coherence point (no cache write-back or invalidation
// needed). A reader polls its words until each carries the epoch of the current layer, so
// no flag or barrier is needed: a value and its readiness arrive in one access. Epochs
// grow by 3 per layer and continue across launches (the last one is kept in the
// workspace), so an old word is never taken for a current one. Each word is written to
// kRep replicas and workgroup g reads replica g % kRep, so that no memory line is polled
// by more than G / kRep workgroups at once. Every wait is bounded (spin limit, then the
// error word and NaN outputs).
//
// Shapes. The template parameters HC, IC, EC, KC fix hidden, inter, n_experts and k at
// compile time (0 = read them from the parameters); the decode shapes of the 60-layer
// 512-expert stack get their own instantiations so that every index is a constant and the
// waves reduce all of their items together.
//
// LDS layout. fp32 vectors are stored with one padding word after every chunk of kCodes
// values, so that threads reading consecutive chunks hit different banks.
#include "fmoe_decode.h"
#include "fmoe_device.h"
#include "fmoe_internal.h"
#include "fmoe_intdot.h"
#include "fmoe_layout.h"

namespace fmoe {

constexpr int kDecodeThreads = 256;
constexpr int kDecodeWaves = kDecodeThreads / 64;
constexpr unsigned kSpinLimit = 1u << 21;
constexpr int kBatchN = 16;     // h / a values loaded together per thread
constexpr int kPollN = 8;       // tagged h / a words polled together per thread
constexpr int kPollA = 16;      // tagged a words of one slot polled together per lane
constexpr int kBatchR = 2;      // router slices per wave loaded ahead
constexpr int kKeysInRegs = 8;  // top-k from registers when n_experts <= 512

#ifdef FMOE_TRACE
// Phase trace (measurement builds only, compiled with -DFMOE_TRACE): lane 0 of the named wave
// of every workgroup stamps the device's constant-rate clock (s_memrealtime, 100 MHz) at each
// phase boundary of every layer into trace_stamps[(layer * kTracePhases + phase) * kMaxGrid +
// workgroup] (plain vector stores; set with fmoe_trace_set, null = off). Phases: 0 layer
// start, 1 h gathered, 2 logits published, 3 logits gathered, 4 top-k done (wave 0); 5 + w
// gate/up done, 9 + w a gathered, 13 + w down done (wave w); 17 h published (wave 0).
constexpr int kTracePhases = 18;
__device__ uint64_t* trace_stamps;
#define FMOE_STAMP(ph, who)                                                                     \
  do {                                                                                          \
    if ((who) && lane == 0 && tstamps != nullptr)                                               \
      tstamps[((size_t)lg * kTracePhases + (ph)) * kMaxGrid + g] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
#else
#define FMOE_STAMP(ph, who) \
  do {                      \
  } while (0)
#endif

// gate/up items and down row blocks whose loads are issued together (fewer when every
// lane holds more chunks per row, to stay within the register file)
template <int CPL> constexpr int batch_gu() { return CPL >= 4 ? 1 : 4; }
template <int CPL> constexpr int batch_d() { return CPL >= 4 ? 2 : (CPL == 2 ? 4 : 8); }

__host__ __device__ constexpr int lanes_per_row(int n_chunks) {
  int l = 1;
  while (l < n_chunks && l < 64) l <<= 1;
  return l;
}

template <int CC>
__device__ __forceinline__ int padded(int i) {
  return (i / CC) * (CC + 1) + (i % CC);
}

__device__ __forceinline__ bool spin_failed(unsigned spins, const uint32_t* err) {
  return spins > kSpinLimit || ((spins & 63u) == 63u && ld_dev_u32(err) != 0u);
}

// Tagged exchange words: value bits (low half) | epoch (high half).
__device__ __forceinline__ uint64_t tagged(float v, uint32_t epoch) {
  return ((uint64_t)epoch << 32) | __float_as_uint(v);
}

// Read n tagged values src[i0 + u * STRIDE] (u < N, i < n), waiting until each carries
// `epoch`; only stale words are read again. Returns false (after raising the error word)
// when the wait gave up.
template <int N, int STRIDE>
__device__ __forceinline__ bool poll_batch(const uint64_t* src, int n, int i0, uint32_t epoch, float (&out)[N],
                                           uint32_t* err) {
  uint64_t v[N];
#pragma unroll
  for (int u = 0; u < N; ++u) {
    const int i = i0 + u * STRIDE;
    v[u] = i < n ? ld_dev_u64(src + i) : tagged(0.f, epoch);
  }
  unsigned spins = 0;
  while (true) {
    bool ok = true;
#pragma unroll
    for (int u = 0; u < N; ++u) ok &= (uint32_t)(v[u] >> 32) == epoch;
    if (ok) break;
    if (spin_failed(++spins, err)) {
      st_dev_u32(err, 1u);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
#pragma unroll
    for (int u = 0; u < N; ++u) {
      const int i = i0 + u * STRIDE;
      if ((uint32_t)(v[u] >> 32) != epoch) v[u] = ld_dev_u64(src + i);
    }
  }
#pragma unroll
  for (int u = 0; u < N; ++u) out[u] = __uint_as_float((uint32_t)v[u]);
  return true;
}

// The same lane value, opaque to the optimizer: the code and scale offsets derived from it
// inside the layer loop are recomputed there (a few vector operations per layer) instead
// of being hoisted out of the loop and held in spill registers for its whole length (this
// halves the accumulation registers used as spill space in the compiled decode shapes).
__device__ __forceinline__ int opaque_lane(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Spread gate/up schedule (compiled top-4 shapes at 2 and 3 bits): a workgroup's 4 rows of each
// of the 4 slots go to its 4 waves so that no wave computes more than one row of the slot
// released last. Wave 1 + d (d < 3) takes rows 0 and 1 of slot d and one row of each other slot
// j < 3 (row 2 on wave 1 + (j + 1) % 3, row 3 on wave 1 + (j + 2) % 3); row w of slot 3 goes to
// wave w, so that wave 0, busy with the top-k, takes a single row. Item m of wave 1 + D
// (D = -1: wave 0) is row sp_row(m) of slot sp_slot(m), items in slot order.
template <int D>
constexpr int sp_items() {
  return D < 0 ? 1 : 5;
}
template <int D>
constexpr int sp_slot(int m) {
  if (D < 0) return 3;
  int first = 0;
  for (int j = 0; j < 3; ++j) {
    const int n = j == D ? 2 : 1;
    if (m < first + n) return j;
    first += n;
  }
  return 3;
}
template <int D>
constexpr int sp_row(int m) {
  if (D < 0) return 0;
  int first = 0;
  for (int j = 0; j < 3; ++j) {
    const int n = j == D ? 2 : 1;
    if (m < first + n) return j == D ? m - first : (D == (j + 1) % 3 ? 2 : 3);
    first += n;
  }
  return 1 + D;
}
template <int D>
constexpr int sp_first(int j) {  // the first item of slot j
  int m = 0;
  while (m < sp_items<D>() && sp_slot<D>(m) != j) ++m;
  return m;
}
template <int D>
constexpr int sp_count(int j) {  // items of slot j
  int n = 0;
  for (int m = 0; m < sp_items<D>(); ++m) n += sp_slot<D>(m) == j ? 1 : 0;
  return n;
}
template <int D>
constexpr void sp_mark(int (&seen)[4][4]) {
  for (int m = 0; m < sp_items<D>(); ++m) ++seen[sp_slot<D>(m)][sp_row<D>(m)];
}
// every (slot, row) of the workgroup's 16 goes to exactly one wave, and each wave's items are in
// slot order
constexpr bool sp_schedule_ok() {
  int seen[4][4] = {};
  sp_mark<-1>(seen);
  sp_mark<0>(seen);
  sp_mark<1>(seen);
  sp_mark<2>(seen);
  for (int j = 0; j < 4; ++j)
    for (int r = 0; r < 4; ++r)
      if (seen[j][r] != 1) return false;
  for (int m = 1; m < 5; ++m)
    if (sp_slot<0>(m) < sp_slot<0>(m - 1) || sp_slot<1>(m) < sp_slot<1>(m - 1) || sp_slot<2>(m) < sp_slot<2>(m - 1))
      return false;
  return true;
}
static_assert(sp_schedule_ok(), "the spread gate/up schedule covers each row of each slot once");

// Wait until wave 0's top-k progress word (LDS) reached r.
__device__ __forceinline__ void wait_ready(const int* ready, int r) {
  while (__hip_atomic_load(const_cast<int*>(ready), __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < r)
    __builtin_amdgcn_s_sleep(0);
}

template <int BITS, int CPL_G, int CPL_D, int HC, int IC, int EC, int KC, int SH>
__global__ void __launch_bounds__(kDecodeThreads) decode_kernel(DecodeParams p) {
  constexpr int kBatchGU = batch_gu<CPL_G>();
  using C = Chunk<BITS>;
  constexpr int CC = C::kCodes;
  // With the shape fixed at compile time, a wave reduces all of its gate/up or down items
  // in one transposed pass (reduce_transposed) instead of one cross-lane reduction each.
  constexpr int kLprG = HC ? lanes_per_row(HC / CC) : 0;
  constexpr int kLprD = IC ? lanes_per_row(IC / CC) : 0;
  // Down items per batch. The compiled shapes give each workgroup 16 rows of every slot (hidden
  // 4096 over 256 workgroups), i.e. kLprD / 4 items of 64 / kLprD rows: 8 at 4 bits, 4 at 2
  // and 3 bits (64 columns per chunk, so a wave pass covers 4 rows). The batch is sized to
  // that, since the unrolled item loop computes every item of a batch, present or not.
  constexpr int kBatchD =
      (HC && IC) ? (kLprD / 4 < 2 ? 2 : (kLprD / 4 > batch_d<CPL_D>() ? batch_d<CPL_D>() : kLprD / 4))
                 : batch_d<CPL_D>();
  constexpr bool kFastGU = kLprG == 64 && kBatchGU == 4;
  constexpr bool kFastD = kLprD >= 16 && kBatchD >= 2 && kBatchD <= 8;
  // Compiled shapes with a gated shared expert: its expert is fixed, so its gate/up rows run
  // while wave 0 waits for the logits and ranks them (waves 1-3, right after v's digit
  // image), its SwiGLU outputs are exchanged during the routed gate/up, and every
  // workgroup forms the gate logit itself from the gathered h (no router row, no logits
  // word for it).
  constexpr bool kSharedEarly = SH == 1;
  static_assert(!kSharedEarly || (HC && IC && EC && KC && kFastGU), "early shared expert: compiled shapes only");
  constexpr int NW = Digits<BITS>::kWords;
  extern __shared__ float smem_raw[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: per-wave indexing on the scalar unit
  const int G = gridDim.x, g = blockIdx.x, rep = g % kRep;
  const int H = HC ? HC : p.hidden;
  const int I = IC ? IC : p.inter;
  const int E = EC ? EC : p.n_experts;
  const int K = KC ? KC : p.k;  // routed experts per token
  // slots: the k routed experts, then the shared expert (index E) when the layers have one;
  // router rows: the E experts' rows, then the shared expert's gate (SH: compiled shapes
  // with a shared expert)
  const int KS = KC ? KC + SH : p.k + p.has_shared;
  const int ER = EC ? EC + (kSharedEarly ? 0 : SH) : p.n_experts + p.has_shared;
  const int KI = KS * I;
  const int vec_len = H > KI ? H : KI;
  const int max_chunks = vec_len / CC;

  // ---- LDS carve-up
  uint64_t* key = reinterpret_cast<uint64_t*>(smem_raw);  // [E] rank keys (large E)
  float* vec = reinterpret_cast<float*>(key + E);         // padded v, later padded a
  DigitStore dig;
  dig.words = reinterpret_cast<uint32_t*>(vec + vec_len + vec_len / CC);
  dig.step = reinterpret_cast<float*>(dig.words + (size_t)NW * max_chunks);
  dig.xsum = dig.step + max_chunks;
  dig.n_chunks = H / CC;
  float* part = dig.xsum + max_chunks;  // [router items]
  float* ybuf = part + p.router_items;  // [k][rows per workgroup]
  float* hraw = ybuf + KS * p.rows_per_wg;  // [rows per workgroup] this workgroup's rows of h
  float* red = hraw + p.rows_per_wg;  // per wave: sum of squares of h, then the shared gate's dot with h
  float* wsel = red + 2 * kDecodeWaves;
  float* lsel = wsel + 16;
  int* isel = reinterpret_cast<int*>(lsel + 16);
  int* fail = isel + 16;
  int* ready = fail + 1;
  uint32_t* base = reinterpret_cast<uint32_t*>(ready + 1);
  DigitStore dig_a;  // digit image of a (v keeps its own until the next layer)
  dig_a.n_chunks = KI / CC;
  dig_a.words = base + 4;
  dig_a.step = reinterpret_cast<float*>(dig_a.words + (size_t)NW * dig_a.n_chunks);
  dig_a.xsum = dig_a.step + dig_a.n_chunks;

#ifdef FMOE_TRACE
  uint64_t* const tstamps = trace_stamps;  // read once: the stamp sites then test a register
#endif
  if (tid == 0) {
    // a workspace whose error word is set (an earlier call gave up) fails at once
    *fail = ld_dev_u32(p.err) != 0u;
    base[1] = 0;  // digit-builder arrivals (3 per layer)
    // Epochs: every workgroup's slot holds the same value F when a launch starts (0 in a
    // zero-filled workspace, else the last epoch of the previous launch). Layer l of this
    // launch tags its logits F + 3l + 1, its a F + 3l + 2 and its output h F + 3l + 3.
    *base = ld_dev_u32(p.flags_arr + (size_t)rep * kMaxGrid + blockIdx.x);
    if (KS > K) isel[K] = E;  // the shared expert's slot never changes
  }
  __syncthreads();
  const uint32_t F = *base;

  // geometry of the quantized rows
  const size_t cbH = (size_t)I * H * BITS / 8;  // bytes of gate (= up = down) codes
  const size_t sbb = (size_t)I * (H / 64) * 4;  // bytes of one sb array
  const int ngH = H / 64, ngI = I / 64;
  const int nchG = H / CC, nchD = I / CC;
  const int lprG = HC ? lanes_per_row(HC / CC) : p.lpr_g, rpwG = 64 / lprG;
  const int lprD = IC ? lanes_per_row(IC / CC) : p.lpr_d, rpwD = 64 / lprD;
  int subG = lane & (lprG - 1), rselG = lane / lprG;  // recomputed per layer (opaque_lane)
  int subD = lane & (lprD - 1), rselD = lane / lprD;
  const int rows_wg = p.rows_per_wg;
  const int r0 = g * rows_wg;
  const int nr = max(0, min(H - r0, rows_wg));
  const int n_rb = (nr + rpwD - 1) / rpwD;  // down row blocks per slot
  // down items (j, rb) of this workgroup, a contiguous run per wave. With the early shared
  // expert, when every wave's run of the routed slots is one batch of one slot (sep_sh), the
  // shared slot's row blocks are dealt apart, at most two per wave, and computed first (their
  // a is exchanged before the routed a).
  const int dper_r = (K * n_rb + kDecodeWaves - 1) / kDecodeWaves;
  const int sd_per = (n_rb + kDecodeWaves - 1) / kDecodeWaves;
  const bool sep_sh = kSharedEarly && kFastD && dper_r > 0 && dper_r <= kBatchD && n_rb % dper_r == 0 && sd_per <= 2;
  const int sd_lo = min(n_rb, wave * sd_per), sd_hi = min(n_rb, sd_lo + sd_per);
  const int d_items = (sep_sh ? K : KS) * n_rb;
  const int d_per = (d_items + kDecodeWaves - 1) / kDecodeWaves;
  const int d_lo = wave * d_per, d_hi = min(d_items, d_lo + d_per);
  const int S = (H + 1023) / 1024;  // router slices per row
  const int my_experts = (ER - g + G - 1) / G;
  const int n_ritems = my_experts * S;
  // gate/up: a contiguous run of blocks (rpwG consecutive items each) per workgroup; the
  // last slot it touches is the top-k round the workgroup has to wait for. The early shared
  // expert's rows are dealt apart: rows sh_lo .. sh_hi - 1 (items K * I + row) per workgroup.
  const int KG = kSharedEarly ? K * I : KI;
  const int n_blocks = (KG + rpwG - 1) / rpwG;
  const int per_wg = (n_blocks + G - 1) / G;
  const int blk_lo = g * per_wg, blk_hi = min(n_blocks, blk_lo + per_wg);
  const int gu_last = min(blk_hi * rpwG, KG) - 1;
  const int sh_per = (I + G - 1) / G;
  const int sh_lo = kSharedEarly ? min(I, g * sh_per) : 0, sh_hi = kSharedEarly ? min(I, sh_lo + sh_per) : 0;
  // (a run inside the shared expert's slot needs no routing round: its expert is fixed)
  const int gu_first = blk_lo * rpwG / I, gu_lslot = gu_last / I;
  // Interleaved gate/up (compiled shapes, when G divides I in whole batches): every
  // workgroup takes the same rs = I / G rows (g * rs ..) of every routed slot, and slot j
  // goes to wave (j + 1) % 4, which waits for that slot's top-k round only; wave 0, busy with
  // the top-k, takes the slots released last. Each slot's rows are then spread over all
  // compute units, so the slot released last is streamed by all of them instead of by G / K
  // workgroups after the others are done.
  // (Not with the early shared expert: there the contiguous runs measured faster, 1,009
  // against 1,035 us per token.)
  const int rs = I / G;
  const bool gu_il =
      kFastGU && !kSharedEarly && kDecodeWaves == 4 && I % G == 0 && rs > 0 && rs % kBatchGU == 0;
  // the workgroup's row group: consecutive groups go to workgroups of one XCD (workgroup g
  // runs on XCD g mod 8), so that the 128-byte lines of blocked scale/bias words that two
  // 4-row groups share are fetched once into that XCD's L2 (with row group g they were
  // fetched by two XCDs: 1.097 against 1.041 bytes per algorithmic byte)
  const int gu_row0 = (G % 8 == 0 ? (g % 8) * (G / 8) + g / 8 : g) * rs;
  // The spread schedule above, at 2 and 3 bits: there each slot's rows arrive about a fixed
  // latency after its release, so the products of the slot released last set the end of the
  // gate/up phase. (At 4 bits the gate/up window streams near the HBM rate, so spreading the
  // products gains nothing, and the fifth row in flight on waves 1-3 costs registers.)
  constexpr bool kSpreadGU = kFastGU && !kSharedEarly && KC == 4 && kDecodeWaves == 4 && BITS != 4;
  const bool gu_sp = kSpreadGU && gu_il && rs == 4;
  const int gu_need =
      gu_il ? 0 : blk_lo >= blk_hi ? 0 : gu_lslot < K ? gu_lslot + 1 : gu_first < K ? K : 0;
  // What a workgroup takes part in. Router rows or gate/up items need all of v, hence the
  // h gather. A workgroup with only down rows needs just its own rows of h, which it wrote
  // itself in the previous layer's combine (kept in LDS): it reads no h word, so it never
  // waits on words that faster workgroups may already have overwritten with the next
  // layer's values (the next layer's h needs this workgroup's rows first). A workgroup
  // with none of the three skips every exchange. (Uniform over the workgroup; at the
  // 512-expert shapes every workgroup has all three.)
  const bool need_v = n_ritems > 0 || (gu_il ? K > 0 : blk_lo < blk_hi) || sh_lo < sh_hi;
  const int n_layers_run = (need_v || nr > 0) && !*fail ? p.n_layers : 0;
  const uint64_t* h_rep = p.h + (size_t)rep * H;
  const uint64_t* a_rep = p.a + (size_t)rep * KI;
  const uint64_t* logits_rep = p.logits + (size_t)rep * ER;

  // router slice `it` of layer `lr`: up to 4 float4 per lane. The loads are unconditional
  // (an index past the end is clamped to a valid row whose values go unused): a
  // conditional load would make the compiler wait for it on the spot to merge the old
  // register contents, instead of where the values are used.
  float4 rv[kBatchR][4];
  auto router_load = [&](int lr, int it, int u) {
    const int lc = min(lr, p.n_layers - 1);
    const int itc = max(0, min(it, n_ritems - 1));
    const int el = itc / S, s = itc % S;
    const int e = min(g + el * G, ER - 1);
    const int c0 = s * 256, c1 = min(H / 4, c0 + 256);
    const float4* row = reinterpret_cast<const float4*>(e < E ? p.router[lc] + (size_t)e * H : p.shared_gate[lc]);
#pragma unroll
    for (int q = 0; q < 4; ++q) rv[u][q] = row[min(c0 + lane + 64 * q, c1 - 1)];
  };
#pragma unroll
  for (int u = 0; u < kBatchR; ++u) router_load(0, wave + kDecodeWaves * u, u);

  for (int l = 0; l < n_layers_run; ++l) {
    const int lg = p.layer0 + l;
    const uint8_t* X = p.experts[l];
    const uint32_t ep = F + 3u * (uint32_t)l;
    FMOE_STAMP(0, wave == 0);
    {
      const int ln = opaque_lane(lane);
      subG = ln & (lprG - 1);
      rselG = ln / lprG;
      subD = ln & (lprD - 1);
      rselD = ln / lprD;
    }

    // ---- 1. h (the previous layer's tagged output, or x_in), v = rmsnorm(h) or h in LDS
    float ss = 0.f;
    // the first read of h waits for the router rows requested at the end of the previous
    // layer anyway (loads complete in order); issuing it after them samples h later
    if (lg != 0 && need_v) wait_vmem();
    if (!need_v && l == 0) {
      // own rows only: from the input, or (a later launch of a chunked stack) from the
      // previous launch's tagged output
      for (int i = tid; i < nr; i += kDecodeThreads) {
        float hv[1] = {0.f};
        if (lg == 0) hv[0] = p.x_in[r0 + i];
        else if (!poll_batch<1, 1>(h_rep + r0, nr, i, ep, hv, p.err)) *fail = 1;
        hraw[i] = hv[0];
      }
    }
    float gd = 0.f;  // early shared expert: this thread's part of the gate's dot with h
    for (int i0 = tid; need_v && i0 < H; i0 += kDecodeThreads * kPollN) {
      float hv[kPollN], gv[kPollN];
      if constexpr (kSharedEarly) {
#pragma unroll
        for (int u = 0; u < kPollN; ++u) gv[u] = p.shared_gate[l][min(i0 + u * kDecodeThreads, H - 1)];
      }
      if (lg == 0) {
#pragma unroll
        for (int u = 0; u < kPollN; ++u) {
          const int i = i0 + u * kDecodeThreads;
          hv[u] = i < H ? p.x_in[i] : 0.f;
        }
      } else if (!poll_batch<kPollN, kDecodeThreads>(h_rep, H, i0, ep, hv, p.err)) {
        *fail = 1;
      }
#pragma unroll
      for (int u = 0; u < kPollN; ++u) {
        const int i = i0 + u * kDecodeThreads;
        if (i < H) {
          vec[padded<CC>(i)] = hv[u];
          if (i >= r0 && i < r0 + nr) hraw[i - r0] = hv[u];
          ss = fmaf(hv[u], hv[u], ss);
          if constexpr (kSharedEarly) gd = fmaf(gv[u], hv[u], gd);
        }
      }
    }
    ss = wave_sum(ss);
    if (lane == 0) red[wave] = ss;
    if constexpr (kSharedEarly) {
      gd = wave_sum(gd);
      if (lane == 0) red[kDecodeWaves + wave] = gd;
    }
    if (tid == 0) *ready = 0;
    __syncthreads();
    if (*fail) break;
    FMOE_STAMP(1, wave == 0);
    // v = inv * h is never formed: the router sums are scaled by inv, and so are the
    // steps and sums of v's digit image
    float inv = 1.f;
    if (p.flags & FMOE_PRENORM) {
      float tot = 0.f;
      for (int w2 = 0; w2 < kDecodeWaves; ++w2) tot += red[w2];
      inv = 1.0f / sqrtf(tot / (float)H + p.eps);
    }
    if constexpr (kSharedEarly) {
      // the shared expert's weight: the logistic function of gate . v = inv * (gate . h)
      if (tid == 0) {
        float gdot = 0.f;
        for (int w2 = 0; w2 < kDecodeWaves; ++w2) gdot += red[kDecodeWaves + w2];
        wsel[K] = 1.0f / (1.0f + expf(-gdot * inv));
      }
    }

    // ---- 2. router: dot the loaded slices with v (the first two of a wave reduced together)
    int m_first = 0;
    if (kBatchR == 2 && wave + kDecodeWaves < n_ritems) {
      float acc2[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int s = (wave + kDecodeWaves * u) % S;
        const int c0 = s * 256, c1 = min(H / 4, c0 + 256);
        float acc = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = c0 + lane + 64 * q;
          if (c < c1) {
            const int pi = padded<CC>(4 * c);
            acc = fmaf(rv[u][q].x, vec[pi + 0], acc);
            acc = fmaf(rv[u][q].y, vec[pi + 1], acc);
            acc = fmaf(rv[u][q].z, vec[pi + 2], acc);
            acc = fmaf(rv[u][q].w, vec[pi + 3], acc);
          }
        }
        acc2[u] = acc;
      }
      const float sum = reduce_transposed<2, 64>(acc2);
      if (lane < 2) part[wave + kDecodeWaves * lane] = sum * inv;  // lane u holds slice u's total
      m_first = 2;
    }
    for (int m = m_first; wave + kDecodeWaves * m < n_ritems; ++m) {
      const int it = wave + kDecodeWaves * m;
      const int u = m < kBatchR ? m : kBatchR - 1;
      if (m >= kBatchR) router_load(l, it, u);
      const int s = it % S;
      const int c0 = s * 256, c1 = min(H / 4, c0 + 256);
      float acc = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = c0 + lane + 64 * q;
        if (c < c1) {
          const int pi = padded<CC>(4 * c);  // 4 consecutive values never straddle a chunk
          acc = fmaf(rv[u][q].x, vec[pi + 0], acc);
          acc = fmaf(rv[u][q].y, vec[pi + 1], acc);
          acc = fmaf(rv[u][q].z, vec[pi + 2], acc);
          acc = fmaf(rv[u][q].w, vec[pi + 3], acc);
        }
      }
      acc = wave_sum(acc);
      if (lane == 0) part[it] = acc * inv;
    }
    __syncthreads();
    const uint64_t tag = (uint64_t)(ep + 1u) << 32;

    // gate/up state (step 4); the early shared expert's rows run before the routing is known
    DChunk<BITS> dc[CPL_G];
    bool dc_loaded = false;  // the digits are read from LDS after the first loads are issued
    const uint64_t atag = (uint64_t)(ep + 2u) << 32;
    // items b0 .. b0 + kBatchGU - 1 (rows for rpwG > 1: blocks) for b0 = b_first, + b_step, ... < b_hi
    auto gu_run = [&](int b_first, int b_hi, int b_step) {
      for (int b0 = b_first; b0 < b_hi; b0 += b_step) {
        CChunk<BITS> wg[kBatchGU][CPL_G], wu[kBatchGU][CPL_G];
        uint32_t sg[kBatchGU][CPL_G], su[kBatchGU][CPL_G];
#pragma unroll
        for (int u = 0; u < kBatchGU; ++u) {
          // fast path: unconditional loads (an item past the run reads the run's last row,
          // whose result is not stored), so that each item waits only for its own loads
          const int item = kFastGU ? min(b0 + u, b_hi - 1) : (b0 + u) * rpwG + rselG;
          if (kFastGU || (b0 + u < b_hi && item < KI)) {
            const int j = item / I, i = item % I;
            const uint8_t* bp = X + (size_t)isel[j] * p.expert_stride;
            const uint8_t* gp = bp;  // gate codes; up codes follow at cbH
            const uint32_t* gsb = reinterpret_cast<const uint32_t*>(bp + 3 * cbH);  // blocked, fmoe_layout.h
            const uint32_t* usb = reinterpret_cast<const uint32_t*>(bp + 3 * cbH + sbb);
#pragma unroll
            for (int q = 0; q < CPL_G; ++q) {
              int c = subG + lprG * q;
              if (kFastGU || c < nchG) {  // the fast path covers exactly nchG chunks per row
                load_cchunk<BITS>(wg[u][q], gp, I, H, i, c);
                load_cchunk<BITS>(wu[u][q], gp + cbH, I, H, i, c);
                const size_t so = sb_offset(I, ngH, i, c / C::kPerGroup);
                sg[u][q] = gsb[so];
                su[u][q] = usb[so];
              }
            }
          }
        }
        if (!dc_loaded) {
#pragma unroll
          for (int q = 0; q < CPL_G; ++q) {
            int c = subG + lprG * q;
            if (c < nchG) load_dchunk<BITS>(dc[q], dig, c);
          }
          dc_loaded = true;
        }
        if constexpr (kFastGU) {
          static_assert(kRep == 8, "the 8 lane groups below store the 8 replicas of a");
          // one row per item (64 lanes per row): the 4 gate and 4 up sums of the batch are
          // reduced together; afterwards an even lane 8r + 2b1 + 4b2 holds the gate sum of
          // item 2b1 + b2 and its odd neighbour the up sum, and stores a to replica r.
          // Items past the run (uniform tail) were not loaded; their sums are not stored.
          float vals[8];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            float gs = 0.f, us = 0.f;
#pragma unroll
            for (int q = 0; q < CPL_G; ++q) {
              int c = lane + 64 * q;
              if (c < nchG) {
                gs += chunk_dot_int<BITS>(wg[u][q], sg[u][q], dc[q]);
                us += chunk_dot_int<BITS>(wu[u][q], su[u][q], dc[q]);
              }
            }
            vals[u] = gs;
            vals[4 + u] = us;
            // keep the items in load order, so each waits only for its own rows and its
            // arithmetic overlaps the arrival of the next ones
            __builtin_amdgcn_sched_barrier(0);
          }
          const float sum = reduce_transposed<8, 64>(vals);
          const float up_sum = xlane<1>(sum);
          const int u = 2 * ((lane >> 1) & 1) + ((lane >> 2) & 1);
          if (!(lane & 1) && b0 + u < b_hi)
            st_dev_u64(p.a + (size_t)(lane >> 3) * KI + (b0 + u), atag | __float_as_uint(swiglu(sum, up_sum)));
          continue;
        }
#pragma unroll
        for (int u = 0; u < kBatchGU; ++u) {
          if (b0 + u >= b_hi) break;  // uniform over the wave
          const int item = (b0 + u) * rpwG + rselG;
          const bool valid = item < KI;
          float gs = 0.f, us = 0.f;
          if (valid) {
#pragma unroll
            for (int q = 0; q < CPL_G; ++q) {
              int c = subG + lprG * q;
              if (c < nchG) {
                gs += chunk_dot_int<BITS>(wg[u][q], sg[u][q], dc[q]);
                us += chunk_dot_int<BITS>(wu[u][q], su[u][q], dc[q]);
              }
            }
          }
          gs = group_sum(gs, lprG);
          us = group_sum(us, lprG);
          if (valid && subG == 0) {
            const uint64_t av = atag | __float_as_uint(swiglu(gs, us));
#pragma unroll
            for (int rr = 0; rr < kRep; ++rr) st_dev_u64(p.a + (size_t)rr * KI + item, av);
          }
        }
      }
    };


    // ---- 3. publish this workgroup's logits and gather all of them (wave 0), then the
    // top-k, released round by round; the other waves build the digit image of v
    if (wave == 0) {
      for (int t = lane; t < my_experts * kRep; t += 64) {
        const int el = t / kRep, rr = t % kRep;
        float lsum = 0.f;
        for (int s = 0; s < S; ++s) lsum += part[el * S + s];
        st_dev_u64(p.logits + (size_t)rr * ER + g + el * G, tag | __float_as_uint(lsum));
      }
      // poll only once the own logits are acknowledged: a first read issued right behind
      // the stores samples memory too early (its result waits for the stores anyway) and
      // costs one more round trip
      wait_vmem();
      FMOE_STAMP(2, true);
      unsigned spins = 0;
      bool failed = false;
      const bool kGateWord = KS > K && !kSharedEarly;  // the gate logit comes with the others
      uint64_t kr[kKeysInRegs];  // E <= 64 * kKeysInRegs: keys stay in registers
      float gate_logit = 0.f;
      if (E <= 64 * kKeysInRegs) {
        // one poll batch in flight; words that arrived are kept, only stale ones are read
        // again
        uint64_t t[kKeysInRegs];
        uint32_t got = 0, want = 0;
        // the shared expert's gate logit (lane 0; others never wait for it)
        uint64_t tg = (kGateWord && lane == 0) ? ld_dev_u64(logits_rep + E) : tag;
#pragma unroll
        for (int j = 0; j < kKeysInRegs; ++j) {
          const int e = lane + 64 * j;
          kr[j] = 0;
          if (e < E) {
            want |= 1u << j;
            t[j] = ld_dev_u64(logits_rep + e);
          }
        }
        while (true) {
#pragma unroll
          for (int j = 0; j < kKeysInRegs; ++j) {
            const int e = lane + 64 * j;
            if (((want & ~got) >> j) & 1u) {
              if ((t[j] & 0xffffffff00000000ull) == tag) {
                kr[j] = rank_key(__uint_as_float((uint32_t)t[j]), e);
                got |= 1u << j;
              }
            }
          }
          const bool gok = (tg & 0xffffffff00000000ull) == tag;
          if (__all(got == want && gok)) break;
          if (spin_failed(++spins, p.err)) {
            failed = true;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
#pragma unroll
          for (int j = 0; j < kKeysInRegs; ++j)
            if (((want & ~got) >> j) & 1u) t[j] = ld_dev_u64(logits_rep + lane + 64 * j);
          if (!gok) tg = ld_dev_u64(logits_rep + E);
        }
        if (kGateWord && lane == 0) gate_logit = __uint_as_float((uint32_t)tg);
      } else {
        while (true) {
          bool ok = true;
          for (int e = lane; e < E; e += 64) {
            const uint64_t t = ld_dev_u64(logits_rep + e);
            ok &= (t & 0xffffffff00000000ull) == tag;
            key[e] = rank_key(__uint_as_float((uint32_t)t), e);
          }
          if (kGateWord && lane == 0) {
            const uint64_t t = ld_dev_u64(logits_rep + E);
            ok &= (t & 0xffffffff00000000ull) == tag;
            gate_logit = __uint_as_float((uint32_t)t);
          }
          if (__all(ok)) break;
          if (spin_failed(++spins, p.err)) {
            failed = true;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
      }
      if (failed) {
        if (lane == 0) {
          st_dev_u32(p.err, 1u);
          *fail = 1;
        }
        if (lane < KS) {
          isel[lane] = lane < K ? 0 : E;
          wsel[lane] = 0.f;
        }
        topk_progress(ready, K + 1);
      } else {
        FMOE_STAMP(3, true);
        // the shared expert's weight: the logistic function of its gate logit (written
        // before the top-k releases its last round)
        if (kGateWord && lane == 0) wsel[K] = 1.0f / (1.0f + expf(-gate_logit));
        if (E <= 64 * kKeysInRegs) wave_topk_regs<kKeysInRegs>(kr, K, isel, lsel, wsel, ready);
        else wave_topk_keys(key, E, K, isel, lsel, wsel, ready);
        FMOE_STAMP(4, true);
        if (g == 0 && lane < K) {
          size_t o = ((size_t)lg) * K + lane;
          if (p.idx_out) p.idx_out[o] = isel[lane];
          if (p.w_out) p.w_out[o] = wsel[lane];
        }
      }
    } else {
      if (need_v)
        build_digits<BITS>(dig, 0, H, [&](int i) { return vec[padded<CC>(i)]; }, kDecodeThreads - 64, tid - 64, inv);
      // the digit image is complete once every builder wave has passed this point
      if (lane == 0) __hip_atomic_fetch_add(base + 1, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      if constexpr (kSharedEarly) {
        // the shared expert's rows of this workgroup, once v's digit image is complete
        const int sb0 = sh_lo + (wave - 1) * kBatchGU;
        if (sb0 < sh_hi) {  // uniform over the wave
          while (__hip_atomic_load(base + 1, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < 3u * (uint32_t)(l + 1))
            __builtin_amdgcn_s_sleep(0);
          gu_run(K * I + sb0, K * I + sh_hi, (kDecodeWaves - 1) * kBatchGU);
        }
      }
      wait_ready(ready, gu_need);
    }
    // every wave (wave 0 included) waits for the three builder waves of this layer
    while (__hip_atomic_load(base + 1, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < 3u * (uint32_t)(l + 1))
      __builtin_amdgcn_s_sleep(0);
    if (*fail) break;  // set by wave 0 before it released the waiters

    // ---- 4. gate/up + SwiGLU over this workgroup's run of blocks, dealt to its waves in
    // runs of kBatchGU blocks whose loads are issued together; a is published tagged
    if (gu_sp) {
      if constexpr (kSpreadGU) {
        // the wave's items (sp_slot): loads issued slot by slot as the top-k releases them,
        // then the products slot by slot in arrival order, each slot's items reduced together
        // and their a published
        auto run_spread = [&](auto DS) {
          constexpr int D = decltype(DS)::value;
          constexpr int NI = sp_items<D>();
          CChunk<BITS> wg[NI][CPL_G], wu[NI][CPL_G];
          uint32_t sg[NI][CPL_G], su[NI][CPL_G];
#pragma unroll
          for (int m = 0; m < NI; ++m) {
            const int j = sp_slot<D>(m);
            if (m == 0 || j != sp_slot<D>(m - 1)) wait_ready(ready, j + 1);
            const int i = gu_row0 + sp_row<D>(m);
            const uint8_t* bp = X + (size_t)isel[j] * p.expert_stride;
            const uint32_t* gsb = reinterpret_cast<const uint32_t*>(bp + 3 * cbH);  // blocked, fmoe_layout.h
            const uint32_t* usb = reinterpret_cast<const uint32_t*>(bp + 3 * cbH + sbb);
#pragma unroll
            for (int q = 0; q < CPL_G; ++q) {
              const int c = lane + 64 * q;  // kFastGU: 64 lanes per row
              load_cchunk<BITS>(wg[m][q], bp, I, H, i, c);
              load_cchunk<BITS>(wu[m][q], bp + cbH, I, H, i, c);
              const size_t so = sb_offset(I, ngH, i, c / C::kPerGroup);
              sg[m][q] = gsb[so];
              su[m][q] = usb[so];
            }
            if (m == 0) {
#pragma unroll
              for (int q = 0; q < CPL_G; ++q) load_dchunk<BITS>(dc[q], dig, lane + 64 * q);
            }
          }
          static_assert(kRep == 8, "the lane groups below store the 8 replicas of a");
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int n = sp_count<D>(j), m0 = sp_first<D>(j);
            if (n == 0) continue;
            float gsum[2] = {0.f, 0.f}, usum[2] = {0.f, 0.f};
#pragma unroll
            for (int b = 0; b < 2; ++b) {
              if (b < n) {
#pragma unroll
                for (int q = 0; q < CPL_G; ++q) {
                  gsum[b] += chunk_dot_int<BITS>(wg[m0 + b][q], sg[m0 + b][q], dc[q]);
                  usum[b] += chunk_dot_int<BITS>(wu[m0 + b][q], su[m0 + b][q], dc[q]);
                }
              }
            }
            const size_t a0 = (size_t)j * I + gu_row0 + sp_row<D>(m0);
            if (n == 1) {
              // even lanes hold the gate sum, odd lanes the up sum; even lane 2 r stores replica r
              const float vals[2] = {gsum[0], usum[0]};
              const float sum = reduce_transposed<2, 64>(vals);
              const float up_sum = xlane<1>(sum);
              if (!(lane & 1) && (lane >> 1) < kRep)
                st_dev_u64(p.a + (size_t)(lane >> 1) * KI + a0, atag | __float_as_uint(swiglu(sum, up_sum)));
            } else {
              // lane 4 r + 2 b holds the gate sum of item b (rows 0, 1), its odd neighbour the
              // up sum; it stores replica r
              const float vals[4] = {gsum[0], gsum[1], usum[0], usum[1]};
              const float sum = reduce_transposed<4, 64>(vals);
              const float up_sum = xlane<1>(sum);
              if (!(lane & 1) && (lane >> 2) < kRep)
                st_dev_u64(p.a + (size_t)(lane >> 2) * KI + a0 + ((lane >> 1) & 1),
                           atag | __float_as_uint(swiglu(sum, up_sum)));
            }
            __builtin_amdgcn_sched_barrier(0);  // slots in arrival order
          }
        };
        if (wave == 0) run_spread(std::integral_constant<int, -1>{});
        else if (wave == 1) run_spread(std::integral_constant<int, 0>{});
        else if (wave == 2) run_spread(std::integral_constant<int, 1>{});
        else run_spread(std::integral_constant<int, 2>{});
      }
    } else if (gu_il) {
      for (int j = (wave + 3) % kDecodeWaves; j < K; j += kDecodeWaves) {
        wait_ready(ready, j + 1);
        gu_run(j * I + gu_row0, j * I + gu_row0 + rs, kBatchGU);
      }
    } else {
      gu_run(blk_lo + wave * kBatchGU, blk_hi, kDecodeWaves * kBatchGU);
    }
    FMOE_STAMP(5 + wave, true);

    // ---- prefetch: every wave issues the loads of its first kBatchD down items (all k
    // experts must be known)
    wait_ready(ready, K);
    CChunk<BITS> wd[kBatchD][CPL_D];
    uint32_t sd[kBatchD][CPL_D];
    auto down_load = [&](int m, int u) {
      const int t = d_lo + m;
      if (t < d_hi) {
        const int j = t / n_rb;
        const int rl = (t % n_rb) * rpwD + rselD;
        if (rl < nr) {
          const int r = r0 + rl;
          const uint8_t* bp = X + (size_t)isel[j] * p.expert_stride;
          const uint8_t* dp = bp + 2 * cbH;  // down codes
          const uint32_t* dsb = reinterpret_cast<const uint32_t*>(bp + 3 * cbH + 2 * sbb);  // blocked
#pragma unroll
          for (int q = 0; q < CPL_D; ++q) {
            int c = subD + lprD * q;
            if (c < nchD) {
              load_cchunk<BITS>(wd[u][q], dp, H, I, r, c);
              sd[u][q] = dsb[sb_offset(H, ngI, r, c / C::kPerGroup)];
            }
          }
        }
      }
    };
#pragma unroll
    for (int u = 0; u < kBatchD; ++u) down_load(u, u);
    // the shared slot's row blocks of this wave (sep_sh; a run of at most two, loaded
    // unconditionally: a block past the run repeats the run's last one, not stored)
    CChunk<BITS> wsh[2][CPL_D];
    uint32_t ssh[2][CPL_D];
    if (sep_sh && sd_lo < sd_hi) {
      const uint8_t* bp = X + (size_t)E * p.expert_stride;
      const uint8_t* dp = bp + 2 * cbH;
      const uint32_t* dsb = reinterpret_cast<const uint32_t*>(bp + 3 * cbH + 2 * sbb);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int r = r0 + min((min(sd_lo + u, sd_hi - 1)) * rpwD + rselD, nr - 1);
#pragma unroll
        for (int q = 0; q < CPL_D; ++q) {
          const int c = min(subD + lprD * q, nchD - 1);
          load_cchunk<BITS>(wsh[u][q], dp, H, I, r, c);
          ssh[u][q] = dsb[sb_offset(H, ngI, r, c / C::kPerGroup)];
        }
      }
    }

    // ---- 5a. the shared slot's down rows (sep_sh): its a was published while the routed
    // experts were being selected, so it is gathered and used while the routed a arrives
    if constexpr (kSharedEarly && kFastD) {
      if (sep_sh && sd_lo < sd_hi) {
        const uint64_t* a_s = a_rep + (size_t)K * I;
        wait_vmem();
        for (int i0 = lane; i0 < I; i0 += 64 * kPollA) {
          float av[kPollA];
          if (!poll_batch<kPollA, 64>(a_s, I, i0, ep + 2u, av, p.err)) *fail = 1;
#pragma unroll
          for (int u = 0; u < kPollA; ++u) {
            const int i = i0 + 64 * u;
            if (i < I) vec[padded<CC>(K * I + i)] = av[u];
          }
        }
        __builtin_amdgcn_wave_barrier();
        // every wave builds the same image of the shared slot's a (identical values)
        build_digits<BITS>(dig_a, K * nchD, I, [&](int i) { return vec[padded<CC>(i)]; }, 64, lane);
        __builtin_amdgcn_wave_barrier();
        DChunk<BITS> dcs[CPL_D];
#pragma unroll
        for (int q = 0; q < CPL_D; ++q) {
          int c = subD + kLprD * q;
          if (c < nchD) load_dchunk<BITS>(dcs[q], dig_a, K * nchD + c);
        }
        float acc[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          float a_ = 0.f;
#pragma unroll
          for (int q = 0; q < CPL_D; ++q) {
            int c = subD + kLprD * q;
            if (c < nchD) a_ += chunk_dot_int<BITS>(wsh[u][q], ssh[u][q], dcs[q]);
          }
          acc[u] = a_;
        }
        const float sum = reduce_transposed<2, kLprD>(acc);
        const int u = transposed_index<2>(lane);
        const int rl = (sd_lo + u) * rpwD + rselD;
        if (subD < 2 && sd_lo + u < sd_hi && rl < nr) ybuf[K * rows_wg + rl] = sum;
      }
    }

    // ---- 5./6. a, then down. When every wave's down items belong to one slot and fit one
    // batch (the compiled decode shapes), each wave gathers only its slot's a (written by
    // the workgroups that ran that slot's gate/up), builds that slot's digit image in its
    // own range of the store and reduces its items together, with no workgroup barrier
    // before the combine. Otherwise the workgroup gathers all of a, digitises it once and
    // reduces the down items one by one. (v's LDS image is free by now: the router and the
    // digit builders of v finished before any wave started gate/up.)
    const int j_lo = d_lo / n_rb;
    const bool fast_d = kFastD && d_per <= kBatchD && n_rb % d_per == 0;  // uniform over the workgroup
    if (fast_d) {
      if constexpr (kFastD) {
        if (d_lo < d_hi) {
          const uint64_t* a_j = a_rep + (size_t)j_lo * I;
          wait_vmem();  // as for h: the first read of a would wait for the down rows anyway
          for (int i0 = lane; i0 < I; i0 += 64 * kPollA) {
            float av[kPollA];
            if (!poll_batch<kPollA, 64>(a_j, I, i0, ep + 2u, av, p.err)) *fail = 1;
#pragma unroll
            for (int u = 0; u < kPollA; ++u) {
              const int i = i0 + 64 * u;
              if (i < I) vec[padded<CC>(j_lo * I + i)] = av[u];
            }
          }
          FMOE_STAMP(9 + wave, true);
          __builtin_amdgcn_wave_barrier();
          build_digits<BITS>(dig_a, j_lo * nchD, I, [&](int i) { return vec[padded<CC>(i)]; }, 64, lane);
          __builtin_amdgcn_wave_barrier();
          DChunk<BITS> dc[CPL_D];
#pragma unroll
          for (int q = 0; q < CPL_D; ++q) {
            int c = subD + kLprD * q;
            if (c < nchD) load_dchunk<BITS>(dc[q], dig_a, j_lo * nchD + c);
          }
          float acc[kBatchD];
#pragma unroll
          for (int u = 0; u < kBatchD; ++u) {
            float a_ = 0.f;
#pragma unroll
            for (int q = 0; q < CPL_D; ++q) {
              int c = subD + kLprD * q;
              if (c < nchD) a_ += chunk_dot_int<BITS>(wd[u][q], sd[u][q], dc[q]);
            }
            acc[u] = a_;
          }
          // lane i < kBatchD of a row group holds the sum of item transposed_index(i)
          const float sum = reduce_transposed<kBatchD, kLprD>(acc);
          const int u = transposed_index<kBatchD>(lane);
          const int rl = (d_lo - j_lo * n_rb + u) * rpwD + rselD;
          if (subD < kBatchD && d_lo + u < d_hi && rl < nr) ybuf[j_lo * rows_wg + rl] = sum;
          FMOE_STAMP(13 + wave, true);
        }
      }
    } else if (kFastD) {
      // compiled shapes whose waves' down items span several slots (top-k with large k):
      // the same per-wave scheme slot by slot. A slot shared by two waves is gathered and
      // digitised by both, which write identical values to the same LDS.
      if constexpr (kFastD) {
        for (int j = d_lo / n_rb; d_lo < d_hi && j * n_rb < d_hi; ++j) {  // slots < KS: items < KS * n_rb
          const int t_lo = max(d_lo, j * n_rb), t_hi = min(d_hi, (j + 1) * n_rb);
          const uint64_t* a_j = a_rep + (size_t)j * I;
          wait_vmem();
          for (int i0 = lane; i0 < I; i0 += 64 * kPollA) {
            float av[kPollA];
            if (!poll_batch<kPollA, 64>(a_j, I, i0, ep + 2u, av, p.err)) *fail = 1;
#pragma unroll
            for (int u = 0; u < kPollA; ++u) {
              const int i = i0 + 64 * u;
              if (i < I) vec[padded<CC>(j * I + i)] = av[u];
            }
          }
          __builtin_amdgcn_wave_barrier();
          build_digits<BITS>(dig_a, j * nchD, I, [&](int i) { return vec[padded<CC>(i)]; }, 64, lane);
          __builtin_amdgcn_wave_barrier();
          DChunk<BITS> dc[CPL_D];
#pragma unroll
          for (int q = 0; q < CPL_D; ++q) {
            int c = subD + kLprD * q;
            if (c < nchD) load_dchunk<BITS>(dc[q], dig_a, j * nchD + c);
          }
          for (int t0 = t_lo; t0 < t_hi; t0 += kBatchD) {
            if (t0 != d_lo) {  // the wave's first batch was requested before the gather
#pragma unroll
              for (int u = 0; u < kBatchD; ++u) down_load(t0 - d_lo + u, u);
            }
            float acc[kBatchD];
#pragma unroll
            for (int u = 0; u < kBatchD; ++u) {
              float a_ = 0.f;
              // Items past the slot's end are skipped (a wave-uniform branch) in the top-4
              // shapes, which take this path only on grids other than 256 workgroups. With
              // top-10 routing every wave takes it, and there the branch measured slower than
              // reducing the empty items.
              if (KC != 4 || t0 + u < t_hi) {
#pragma unroll
                for (int q = 0; q < CPL_D; ++q) {
                  int c = subD + kLprD * q;
                  if (c < nchD) a_ += chunk_dot_int<BITS>(wd[u][q], sd[u][q], dc[q]);
                }
              }
              acc[u] = a_;
            }
            // items past t_hi (another slot's or none) are reduced as zeros; their sums
            // are not stored
            const float sum = reduce_transposed<kBatchD, kLprD>(acc);
            const int u = transposed_index<kBatchD>(lane);
            const int t = t0 + u;
            const int rl = (t - j * n_rb) * rpwD + rselD;
            if (subD < kBatchD && t < t_hi && rl < nr) ybuf[j * rows_wg + rl] = sum;
          }
        }
      }
    } else {
      for (int i0 = tid; i0 < KI; i0 += kDecodeThreads * kPollN) {
        float av[kPollN];
        if (!poll_batch<kPollN, kDecodeThreads>(a_rep, KI, i0, ep + 2u, av, p.err)) *fail = 1;
#pragma unroll
        for (int u = 0; u < kPollN; ++u) {
          const int i = i0 + u * kDecodeThreads;
          if (i < KI) vec[padded<CC>(i)] = av[u];
        }
      }
      __syncthreads();
      if (*fail) break;
      build_digits<BITS>(dig_a, 0, KI, [&](int i) { return vec[padded<CC>(i)]; }, kDecodeThreads, tid);
      __syncthreads();
      int cur_j = -1;
      DChunk<BITS> dc[CPL_D];
      for (int m0 = 0; d_lo + m0 < d_hi; m0 += kBatchD) {
        if (m0 > 0) {
#pragma unroll
          for (int u = 0; u < kBatchD; ++u) down_load(m0 + u, u);
        }
#pragma unroll
        for (int u = 0; u < kBatchD; ++u) {
          const int t = d_lo + m0 + u;
          if (t >= d_hi) break;  // uniform over the wave
          const int j = t / n_rb;
          const int rl = (t % n_rb) * rpwD + rselD;
          if (j != cur_j) {
#pragma unroll
            for (int q = 0; q < CPL_D; ++q) {
              int c = subD + lprD * q;
              if (c < nchD) load_dchunk<BITS>(dc[q], dig_a, j * nchD + c);
            }
            cur_j = j;
          }
          float acc = 0.f;
          if (rl < nr) {
#pragma unroll
            for (int q = 0; q < CPL_D; ++q) {
              int c = subD + lprD * q;
              if (c < nchD) acc += chunk_dot_int<BITS>(wd[u][q], sd[u][q], dc[q]);
            }
          }
          acc = group_sum(acc, lprD);
          if (rl < nr && subD == 0) ybuf[j * rows_wg + rl] = acc;
        }
      }
    }
    // the next layer's router slices are requested now; their latency hides behind the
    // combine and the exchange of h
#pragma unroll
    for (int u = 0; u < kBatchR; ++u) router_load(l + 1, wave + kDecodeWaves * u, u);
    __syncthreads();
    if (*fail) break;
    const bool last = (l == p.n_layers - 1) && p.is_final;
    if (wave == 0) {
      // 16 rows at a time; the four lanes of a row (lane & 15) share its replica stores
      const uint32_t htag = ep + 3u;
      for (int rb = 0; rb < nr; rb += 16) {
        const int rl = rb + (lane & 15);
        if (rl < nr) {
          const int r = r0 + rl;
          float c = 0.f;
          for (int j = 0; j < KS; ++j) c = fmaf(wsel[j], ybuf[j * rows_wg + rl], c);
          const float hn = hraw[rl] + c;
          hraw[rl] = hn;  // this workgroup's rows of the next layer's h (read again only without need_v)
          const uint64_t hv = tagged(hn, htag);
#pragma unroll
          for (int rr = lane >> 4; rr < kRep; rr += 4) st_dev_u64(p.h + (size_t)rr * H + r, hv);
          if (last && lane < 16) p.h_out[r] = hn;
        }
      }
      FMOE_STAMP(17, true);
    }
  }
  __syncthreads();
  if (*fail) {
    if (p.is_final)
      for (int r = r0 + tid; r < r0 + nr; r += kDecodeThreads) p.h_out[r] = __uint_as_float(0x7fc00000u);
  } else if (tid == 0) {
    // the epoch the next launch starts from
    st_dev_u32(p.flags_arr + (size_t)rep * kMaxGrid + blockIdx.x, F + 3u * (uint32_t)p.n_layers);
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
  const int nw = bits == 4 ? Digits<4>::kWords : Digits<2>::kWords;  // (3 bits: the digit sets of 2)
  const size_t ki = (size_t)k * inter;
  const size_t vec_len = (size_t)hidden > ki ? (size_t)hidden : ki;
  const size_t max_chunks = vec_len / cc;
  int my_experts = (n_experts + G - 1) / G;
  int S = (hidden + 1023) / 1024;
  const size_t a_chunks = ki / cc;
  // after the padded vector and v's digit store: router partials, ybuf, hraw, red, wsel,
  // lsel, isel (16 each), fail, ready, base[4], then a's digit store
  size_t words = vec_len + vec_len / cc + (size_t)nw * max_chunks + 2 * max_chunks + (size_t)my_experts * S +
                 (size_t)k * rows_per_wg + rows_per_wg + 2 * kDecodeWaves + 16 + 16 + 16 + 6 + (size_t)nw * a_chunks +
                 2 * a_chunks;
  return (size_t)n_experts * 8 + words * 4;  // rank keys first
}

int decode_grid(int* G_out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FMOE_ERR_HIP;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return FMOE_ERR_HIP;
  *G_out = cus;
  return FMOE_OK;
}

template <int BITS, int CG, int CD, int HC, int IC, int EC, int KC, int SH = 0>
static int launch_decode_t(const DecodeParams& p, int G, size_t smem, hipStream_t s) {
  auto fn = decode_kernel<BITS, CG, CD, HC, IC, EC, KC, SH>;
  // Co-residency: G is the CU count and at least one workgroup fits per CU, so the whole
  // grid is resident once the device has room for it. A plain launch is enough for that;
  // every wait inside the kernel is bounded, so a grid that cannot be made resident (other
  // long kernels holding CUs) ends with the error flag and NaN output, not a hang.
  int occ = 0, dev = 0, cus = 0;
  // shapes whose LDS passes the 64 KB default (top-k with large k * inter) opt in
  if (smem > 64 * 1024 &&
      hipFuncSetAttribute(reinterpret_cast<const void*>(fn), hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem) !=
          hipSuccess)
    return FMOE_ERR_HIP;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fn, kDecodeThreads, smem) != hipSuccess) return FMOE_ERR_HIP;
  if (hipGetDevice(&dev) != hipSuccess) return FMOE_ERR_HIP;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return FMOE_ERR_HIP;
  if (occ < 1 || G > occ * cus) return FMOE_ERR_SHAPE;
  hipLaunchKernelGGL(fn, dim3(G), dim3(kDecodeThreads), smem, s, p);
  return hipGetLastError() == hipSuccess ? FMOE_OK : FMOE_ERR_HIP;
}

int launch_decode(const DecodeParams& p, int G, hipStream_t s) {
  const size_t smem = decode_smem_bytes(p.hidden, p.inter, p.n_experts + p.has_shared, p.k + p.has_shared, G,
                                        p.rows_per_wg, p.bits);
  int cg = p.cpl_g, cd = p.cpl_d;
  // the decode shapes of the 512-expert stack: hidden 4096, inter 1024, top-4 (and the
  // top-10 routing of the same layer), at 4, 3 and 2 bits
  // (and the top-4 routing with a gated shared expert; other shapes with a shared expert run
  // the generic kernel)
  if (p.hidden == 4096 && p.inter == 1024 && p.n_experts == 512 && p.k == 4 && p.has_shared) {
    if (p.bits == 4) return launch_decode_t<4, 2, 1, 4096, 1024, 512, 4, 1>(p, G, smem, s);
    if (p.bits == 3) return launch_decode_t<3, 1, 1, 4096, 1024, 512, 4, 1>(p, G, smem, s);
    return launch_decode_t<2, 1, 1, 4096, 1024, 512, 4, 1>(p, G, smem, s);
  }
  if (p.hidden == 4096 && p.inter == 1024 && p.n_experts == 512 && p.k == 4 && !p.has_shared) {
    if (p.bits == 4) return launch_decode_t<4, 2, 1, 4096, 1024, 512, 4>(p, G, smem, s);
    if (p.bits == 3) return launch_decode_t<3, 1, 1, 4096, 1024, 512, 4>(p, G, smem, s);
    return launch_decode_t<2, 1, 1, 4096, 1024, 512, 4>(p, G, smem, s);
  }
  if (p.hidden == 4096 && p.inter == 1024 && p.n_experts == 512 && p.k == 10 && !p.has_shared) {
    if (p.bits == 4) return launch_decode_t<4, 2, 1, 4096, 1024, 512, 10>(p, G, smem, s);
    if (p.bits == 3) return launch_decode_t<3, 1, 1, 4096, 1024, 512, 10>(p, G, smem, s);
    return launch_decode_t<2, 1, 1, 4096, 1024, 512, 10>(p, G, smem, s);
  }
#define FMOE_DEC(B, X, Y) \
  if (p.bits == B && cg == X && cd == Y) return launch_decode_t<B, X, Y, 0, 0, 0, 0>(p, G, smem, s);
  FMOE_DEC(4, 1, 1) FMOE_DEC(4, 2, 1) FMOE_DEC(4, 4, 1) FMOE_DEC(4, 1, 2) FMOE_DEC(4, 2, 2) FMOE_DEC(4, 4, 2)
  FMOE_DEC(4, 1, 4) FMOE_DEC(4, 2, 4) FMOE_DEC(4, 4, 4)
  FMOE_DEC(2, 1, 1) FMOE_DEC(2, 2, 1) FMOE_DEC(2, 4, 1) FMOE_DEC(2, 1, 2) FMOE_DEC(2, 2, 2) FMOE_DEC(2, 4, 2)
  FMOE_DEC(2, 1, 4) FMOE_DEC(2, 2, 4) FMOE_DEC(2, 4, 4)
  FMOE_DEC(3, 1, 1) FMOE_DEC(3, 2, 1) FMOE_DEC(3, 1, 2) FMOE_DEC(3, 2, 2)  // 3 bits: hidden, inter <= 8192
#undef FMOE_DEC
  return FMOE_ERR_SHAPE;
}

}  // namespace fmoe

#ifdef FMOE_TRACE
// Measurement builds only: where the decode kernels launched after this call on stream s
// write their phase stamps (null = off). Set by a one-thread kernel on the stream, so that
// traced launches can follow each other without a host synchronisation.
namespace fmoe {
__global__ void trace_set_kernel(uint64_t* stamps) { trace_stamps = stamps; }
}  // namespace fmoe
extern "C" int fmoe_trace_set(uint64_t* stamps, hipStream_t s) {
  hipLaunchKernelGGL(fmoe::trace_set_kernel, dim3(1), dim3(1), 0, s, stamps);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
#endif
