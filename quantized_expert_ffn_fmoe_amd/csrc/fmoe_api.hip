// fmoe_api.hip -- the C-ABI entry points: argument validation, workspace carving and
// dispatch to the kernels. Every check runs before anything is enqueued.
#include <string.h>

#include <mutex>

#include "fmoe_batched.h"
#include "fmoe_decode.h"
#include "fmoe_internal.h"

using namespace fmoe;

namespace {


bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

int check_device() {
  static thread_local int cached_dev = -1;
  static thread_local int cached_ok = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FMOE_ERR_HIP;
  if (dev != cached_dev) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FMOE_ERR_HIP;
    cached_ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    cached_dev = dev;
  }
  return cached_ok ? FMOE_OK : FMOE_ERR_DEVICE;
}

bool bits_ok(int bits) { return bits == 2 || bits == 3 || bits == 4; }

int check_qmat(const fmoe_qmat* W) {
  if (!W || !W->codes || !W->sb) return FMOE_ERR_NULL;
  if (!bits_ok(W->bits)) return FMOE_ERR_BITS;
  if (W->group != 64) return FMOE_ERR_GROUP;
  if (W->rows < 1 || W->cols < 64 || W->cols % 64 != 0) return FMOE_ERR_SHAPE;
  if (W->cols > (W->bits == 4 ? 8192 : 16384)) return FMOE_ERR_SHAPE;
  if (!aligned(W->codes, 16) || !aligned(W->sb, 16)) return FMOE_ERR_ALIGN;
  return FMOE_OK;
}

size_t up256(size_t n) { return (n + 255) & ~(size_t)255; }

// Layout of an FMOE_OP_MOE_LAYER workspace. Every offset is a constant, independent of the
// shape of a call, so one workspace serves calls of any shape in any order:
//   [kWsFlags, +32 KB)  the decode kernel's epoch slots [kRep][kMaxGrid] (uint32)
//   kWsErr              the error word (non-zero after a device-side wait gave up)
//   kWsDone             the multi-token sort's arrival counter (0 between calls)
//   [kWsLogits, kWsDecodeEnd)  the decode kernel's tagged exchange words, sized for the
//                       largest accepted shape (4096 + 1 router rows, hidden 8192, 16 slots
//                       of inter 8192), so they never overlap anything else
//   [kWsDecodeEnd, ...) the multi-token path's scratch (n_tokens > 1 only)
// The tagged words hold only values written by the decode kernel with epochs below the
// current one, whatever shapes earlier calls had.
constexpr size_t kWsFlags = 0;
constexpr size_t kWsErr = (size_t)kRep * kMaxGrid * 4;
constexpr size_t kWsDone = kWsErr + 256;
constexpr size_t kWsCtrlEnd = 65536;
constexpr size_t kWsLogits = kWsCtrlEnd;
constexpr size_t kWsH = kWsLogits + ((size_t)kRep * (4096 + 1) * 8 + 255) / 256 * 256;
constexpr size_t kWsA = kWsH + (size_t)kRep * 8192 * 8;
constexpr size_t kWsDecodeEnd = kWsA + (size_t)kRep * 16 * 8192 * 8;
static_assert(kWsDone + 4 <= kWsCtrlEnd, "control block");

struct DecodeWs {
  uint32_t* flags;
  uint64_t* logits;
  uint64_t* h;
  uint64_t* a;
  uint32_t* err;
};

DecodeWs carve_decode(void* ws) {
  char* b = static_cast<char*>(ws);
  DecodeWs d;
  d.flags = reinterpret_cast<uint32_t*>(b + kWsFlags);
  d.err = reinterpret_cast<uint32_t*>(b + kWsErr);
  d.logits = reinterpret_cast<uint64_t*>(b + kWsLogits);
  d.h = reinterpret_cast<uint64_t*>(b + kWsH);
  d.a = reinterpret_cast<uint64_t*>(b + kWsA);
  return d;
}

int moe_layer_impl(const fmoe_layer* layers, int n_layers, const float* x_in, float* h_out, int n_tokens, int k,
                   float eps, unsigned flags, int32_t* idx_out, float* w_out, void* ws, size_t ws_bytes,
                   hipStream_t s, bool zero_sync_region);

__global__ void zero_fill_kernel(uint4* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// Zero `bytes` (a multiple of 16) at a 16-byte aligned device address, on stream s (a
// kernel rather than a memset node, so that it replays correctly when captured).
int zero_fill(void* p, size_t bytes, hipStream_t s) {
  const size_t n = bytes / 16;
  hipLaunchKernelGGL(zero_fill_kernel, dim3(1024), dim3(256), 0, s, static_cast<uint4*>(p), n);
  return hipGetLastError() == hipSuccess ? FMOE_OK : FMOE_ERR_HIP;
}

// ---- the allocation-free variant's scratch
// The library's own workspace for fmoe_moe_layer_noalloc: one file-scope device array,
// of which every GPU the library runs on holds its own copy (zero at load) until the
// process ends. Host code never passes the array's name to a kernel (on the host it only
// stands for the symbol): the device address of each GPU's copy is looked up once per
// device with hipGetSymbolAddress and kept below.
constexpr size_t kScratchBytes = (size_t)32 << 20;
static_assert(kWsDecodeEnd <= kScratchBytes, "the scratch holds at least the single-token workspace");
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on device d (null until looked up)
bool g_scratch_zeroed[kMaxDevices];  // a zero-fill of its synchronization region was enqueued

// The current device's scratch address (looked up on the device's first call, with the
// device current), the device, and whether its synchronization region was zero-filled by
// a call already.
int scratch_of_current_device(void** out, int* dev_out, bool* zeroed) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FMOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return FMOE_ERR_DEVICE;
  int rc = check_device();
  if (rc) return rc;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FMOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  *dev_out = dev;
  *zeroed = g_scratch_zeroed[dev];
  return FMOE_OK;
}

void scratch_zero_enqueued(int dev) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  g_scratch_zeroed[dev] = true;
}

}  // namespace

extern "C" {

const char* fmoe_status_string(int status) {
  switch (status) {
    case FMOE_OK: return "ok";
    case FMOE_ERR_NULL: return "a required pointer is NULL";
    case FMOE_ERR_SHAPE: return "sizes out of range, not a multiple of 64, or inconsistent";
    case FMOE_ERR_BITS: return "bits must be 2, 3 or 4";
    case FMOE_ERR_GROUP: return "group must be 64";
    case FMOE_ERR_K: return "k must be in 1..min(16, n_experts)";
    case FMOE_ERR_ALIGN: return "pointer not 16-byte aligned (workspace, expert stride: 256-byte)";
    case FMOE_ERR_WORKSPACE: return "workspace missing or smaller than fmoe_workspace_bytes()";
    case FMOE_ERR_HIP: return "HIP call or kernel launch failed";
    case FMOE_ERR_INTERNAL: return "internal error";
    case FMOE_ERR_DEVICE: return "current device is not gfx950";
    case FMOE_ERR_OVERLAP: return "an output buffer overlaps an input buffer";
    case FMOE_ERR_SCRATCH: return "the call needs more than the library's static scratch (fmoe_moe_layer_noalloc)";
    default: return "unknown status";
  }
}

const char* fmoe_version(void) { return "fmoe 0.1 gfx950"; }

size_t fmoe_codes_bytes(int rows, int cols, int bits) {
  if (rows < 1 || cols < 64 || cols % 64 || !bits_ok(bits)) return 0;
  return (size_t)rows * cols * bits / 8;
}

size_t fmoe_sb_bytes(int rows, int cols, int group) {
  if (rows < 1 || cols < 64 || group != 64 || cols % group) return 0;
  return (size_t)rows * (cols / group) * 4;
}

size_t fmoe_expert_bytes(int hidden, int inter, int bits, int group) {
  size_t cb = fmoe_codes_bytes(inter, hidden, bits);
  size_t sb = fmoe_sb_bytes(inter, hidden, group);
  if (!cb || !sb || fmoe_codes_bytes(hidden, inter, bits) == 0) return 0;
  return 3 * (cb + sb);
}

int fmoe_expert_view(const void* blob, int hidden, int inter, int bits, int group, fmoe_expert* out) {
  if (!blob || !out) return FMOE_ERR_NULL;
  if (!bits_ok(bits)) return FMOE_ERR_BITS;
  if (group != 64) return FMOE_ERR_GROUP;
  if (fmoe_expert_bytes(hidden, inter, bits, group) == 0) return FMOE_ERR_SHAPE;
  const char* b = static_cast<const char*>(blob);
  size_t cb = fmoe_codes_bytes(inter, hidden, bits), sb = fmoe_sb_bytes(inter, hidden, group);
  out->gate = fmoe_qmat{b, reinterpret_cast<const uint32_t*>(b + 3 * cb), inter, hidden, bits, group};
  out->up = fmoe_qmat{b + cb, reinterpret_cast<const uint32_t*>(b + 3 * cb + sb), inter, hidden, bits, group};
  out->down = fmoe_qmat{b + 2 * cb, reinterpret_cast<const uint32_t*>(b + 3 * cb + 2 * sb), hidden, inter, bits, group};
  return FMOE_OK;
}

int fmoe_pack(const uint8_t* codes_canon, const uint16_t* scale, const uint16_t* bias, int rows, int cols, int bits,
              int group, void* codes_out, uint32_t* sb_out, fmoe_stream_t stream) {
  if (!codes_canon || !scale || !bias || !codes_out || !sb_out) return FMOE_ERR_NULL;
  if (!bits_ok(bits)) return FMOE_ERR_BITS;
  if (group != 64) return FMOE_ERR_GROUP;
  if (rows < 1 || cols < 64 || cols % 64) return FMOE_ERR_SHAPE;
  if (!aligned(codes_canon, 16) || !aligned(codes_out, 16) || !aligned(sb_out, 16) || !aligned(scale, 2) ||
      !aligned(bias, 2))
    return FMOE_ERR_ALIGN;
  size_t cb = fmoe_codes_bytes(rows, cols, bits), nsb = fmoe_sb_bytes(rows, cols, group);
  if (overlaps(codes_out, cb, codes_canon, cb)) return FMOE_ERR_OVERLAP;  // the layout permutes 16-byte chunks
  if (overlaps(sb_out, nsb, scale, nsb / 2) || overlaps(sb_out, nsb, bias, nsb / 2)) return FMOE_ERR_OVERLAP;
  int rc = check_device();
  if (rc) return rc;
  return launch_pack(codes_canon, scale, bias, rows, cols, bits, codes_out, sb_out, (hipStream_t)stream);
}

size_t fmoe_workspace_bytes(int op, int n_tokens, int hidden, int inter, int n_experts, int k) {
  if (n_tokens < 1 || hidden < 64 || inter < 64 || n_experts < 1 || k < 1 || k > 16) return 0;
  if (op == FMOE_OP_EXPERT_FFN) return up256((size_t)inter * 4);
  if (op == FMOE_OP_MOE_LAYER) {
    // the fixed control block and decode region first (every offset independent of the
    // shape), the multi-token scratch after them
    size_t bt = n_tokens > 1 ? batched_workspace_bytes(n_tokens, hidden, inter, n_experts, k) : 0;
    return kWsDecodeEnd + bt;
  }
  return 0;
}

int fmoe_dequant_matvec(const fmoe_qmat* W, const float* x, float* y, int n_vec, fmoe_stream_t stream) {
  int rc = check_qmat(W);
  if (rc) return rc;
  if (!x || !y) return FMOE_ERR_NULL;
  if (n_vec < 1 || n_vec > 64) return FMOE_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(y, 16)) return FMOE_ERR_ALIGN;
  if (overlaps(y, (size_t)n_vec * W->rows * 4, x, (size_t)n_vec * W->cols * 4)) return FMOE_ERR_OVERLAP;
  rc = check_device();
  if (rc) return rc;
  return launch_matvec(*W, x, y, n_vec, (hipStream_t)stream);
}

int fmoe_dequant_matvec_multi(const fmoe_qmat* W, int n_mats, const float* x, float* const* y, int n_vec,
                              fmoe_stream_t stream) {
  if (!W || !x || !y) return FMOE_ERR_NULL;
  if (n_mats < 1 || n_mats > kMaxMulti) return FMOE_ERR_SHAPE;
  int rc;
  for (int m = 0; m < n_mats; ++m)
    if ((rc = check_qmat(&W[m]))) return rc;
  for (int m = 1; m < n_mats; ++m)
    if (W[m].cols != W[0].cols || W[m].bits != W[0].bits) return FMOE_ERR_SHAPE;
  if (n_vec < 1 || n_vec > 64) return FMOE_ERR_SHAPE;
  if (!aligned(x, 16)) return FMOE_ERR_ALIGN;
  const size_t nx = (size_t)n_vec * W[0].cols * 4;
  for (int m = 0; m < n_mats; ++m) {
    if (!y[m]) return FMOE_ERR_NULL;
    if (!aligned(y[m], 16)) return FMOE_ERR_ALIGN;
    const size_t ny = (size_t)n_vec * W[m].rows * 4;
    if (overlaps(y[m], ny, x, nx)) return FMOE_ERR_OVERLAP;
    for (int m2 = 0; m2 < m; ++m2)
      if (overlaps(y[m], ny, y[m2], (size_t)n_vec * W[m2].rows * 4)) return FMOE_ERR_OVERLAP;
  }
  rc = check_device();
  if (rc) return rc;
  return launch_matvec_multi(W, n_mats, x, y, n_vec, (hipStream_t)stream);
}

int fmoe_route_topk(const float* router, const float* x, int n_tokens, int n_experts, int hidden, int k,
                    int32_t* idx, float* w, float* logits, fmoe_stream_t stream) {
  if (!router || !x || !idx || !w || !logits) return FMOE_ERR_NULL;
  if (n_tokens < 1 || n_tokens > 65535 || n_experts < 1 || n_experts > 4096) return FMOE_ERR_SHAPE;
  if (hidden < 64 || hidden % 64 || hidden > 16384) return FMOE_ERR_SHAPE;
  if (k < 1 || k > 16 || k > n_experts) return FMOE_ERR_K;
  if (!aligned(router, 16) || !aligned(x, 16) || !aligned(idx, 4) || !aligned(w, 4) || !aligned(logits, 4))
    return FMOE_ERR_ALIGN;
  size_t nl = (size_t)n_tokens * n_experts * 4, nk = (size_t)n_tokens * k * 4;
  size_t nr = (size_t)n_experts * hidden * 4, nx = (size_t)n_tokens * hidden * 4;
  if (overlaps(logits, nl, router, nr) || overlaps(logits, nl, x, nx) || overlaps(idx, nk, logits, nl) ||
      overlaps(w, nk, logits, nl) || overlaps(idx, nk, w, nk) || overlaps(idx, nk, x, nx) || overlaps(w, nk, x, nx))
    return FMOE_ERR_OVERLAP;
  int rc = check_device();
  if (rc) return rc;
  return launch_route(router, x, n_tokens, n_experts, hidden, k, idx, w, logits, (hipStream_t)stream);
}

int fmoe_expert_ffn(const fmoe_expert* e, const float* x, float* y, void* ws, size_t ws_bytes, fmoe_stream_t stream) {
  if (!e || !x || !y) return FMOE_ERR_NULL;
  int rc;
  if ((rc = check_qmat(&e->gate)) || (rc = check_qmat(&e->up)) || (rc = check_qmat(&e->down))) return rc;
  const int inter = e->gate.rows, hidden = e->gate.cols;
  if (e->up.rows != inter || e->up.cols != hidden || e->down.rows != hidden || e->down.cols != inter)
    return FMOE_ERR_SHAPE;
  if (e->up.bits != e->gate.bits || e->down.bits != e->gate.bits) return FMOE_ERR_BITS;
  if (!ws) return FMOE_ERR_WORKSPACE;
  if (ws_bytes < fmoe_workspace_bytes(FMOE_OP_EXPERT_FFN, 1, hidden, inter, 1, 1)) return FMOE_ERR_WORKSPACE;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(ws, 16)) return FMOE_ERR_ALIGN;
  if (overlaps(y, (size_t)hidden * 4, x, (size_t)hidden * 4) || overlaps(ws, ws_bytes, x, (size_t)hidden * 4) ||
      overlaps(ws, ws_bytes, y, (size_t)hidden * 4))
    return FMOE_ERR_OVERLAP;
  rc = check_device();
  if (rc) return rc;
  return launch_expert_ffn(*e, x, y, static_cast<float*>(ws), (hipStream_t)stream);
}

int fmoe_moe_layer(const fmoe_layer* layers, int n_layers, const float* x_in, float* h_out, int n_tokens, int k,
                   float eps, unsigned flags, int32_t* idx_out, float* w_out, void* ws, size_t ws_bytes,
                   fmoe_stream_t stream) {
  return moe_layer_impl(layers, n_layers, x_in, h_out, n_tokens, k, eps, flags, idx_out, w_out, ws, ws_bytes,
                        (hipStream_t)stream, false);
}

int fmoe_moe_layer_noalloc(const fmoe_layer* layers, int n_layers, const float* x_in, float* h_out, int n_tokens,
                           int k, float eps, unsigned flags, int32_t* idx_out, float* w_out, fmoe_stream_t stream) {
  if (!layers) return FMOE_ERR_NULL;
  const size_t need = fmoe_workspace_bytes(FMOE_OP_MOE_LAYER, n_tokens, layers[0].hidden, layers[0].inter,
                                           layers[0].n_experts, k);
  if (need > kScratchBytes) return FMOE_ERR_SCRATCH;  // (need == 0: the shape error is reported below)
  void* ptr = nullptr;
  int dev = 0;
  bool zeroed = false;
  int rc = scratch_of_current_device(&ptr, &dev, &zeroed);
  if (rc) return rc;
  const bool fill = !zeroed || (flags & FMOE_RESET_SCRATCH);
  rc = moe_layer_impl(layers, n_layers, x_in, h_out, n_tokens, k, eps, flags, idx_out, w_out, ptr, kScratchBytes,
                      (hipStream_t)stream, fill);
  if (rc == FMOE_OK && fill) scratch_zero_enqueued(dev);
  return rc;
}

}  // extern "C"

namespace {

int moe_layer_impl(const fmoe_layer* layers, int n_layers, const float* x_in, float* h_out, int n_tokens, int k,
                   float eps, unsigned flags, int32_t* idx_out, float* w_out, void* ws, size_t ws_bytes,
                   hipStream_t s, bool zero_sync_region) {
  if (!layers || !x_in || !h_out) return FMOE_ERR_NULL;
  if (n_layers < 1 || n_layers > 4096 || n_tokens < 1 || n_tokens > 4096) return FMOE_ERR_SHAPE;
  const fmoe_layer& L0 = layers[0];
  const int H = L0.hidden, I = L0.inter, E = L0.n_experts, bits = L0.bits;
  if (!bits_ok(bits)) return FMOE_ERR_BITS;
  if (L0.group != 64) return FMOE_ERR_GROUP;
  if (H < 64 || H % 64 || I < 64 || I % 64 || H > 8192 || I > 8192) return FMOE_ERR_SHAPE;
  if (E < 1 || E > 4096) return FMOE_ERR_SHAPE;
  if (k < 1 || k > 16 || k > E) return FMOE_ERR_K;
  const int hs = L0.shared_gate != nullptr;  // the layers have a shared expert
  if (hs && k + 1 > 16) return FMOE_ERR_K;
  if (hs && E + 1 > 4096) return FMOE_ERR_SHAPE;
  const size_t eb = fmoe_expert_bytes(H, I, bits, 64);
  for (int l = 0; l < n_layers; ++l) {
    const fmoe_layer& L = layers[l];
    if (!L.router || !L.experts) return FMOE_ERR_NULL;
    if (L.hidden != H || L.inter != I || L.n_experts != E) return FMOE_ERR_SHAPE;
    if (L.bits != bits) return FMOE_ERR_BITS;
    if (L.group != 64) return FMOE_ERR_GROUP;
    if (L.expert_stride < eb || L.expert_stride != L0.expert_stride) return FMOE_ERR_SHAPE;
    if (L.expert_stride % 256 || !aligned(L.experts, 256) || !aligned(L.router, 16)) return FMOE_ERR_ALIGN;
    if ((L.shared_gate != nullptr) != (hs != 0)) return FMOE_ERR_SHAPE;
    if (hs && !aligned(L.shared_gate, 16)) return FMOE_ERR_ALIGN;
  }
  if (!(eps >= 0.f) || !(eps < 1e30f)) return FMOE_ERR_SHAPE;
  if (!ws) return FMOE_ERR_WORKSPACE;
  if (ws_bytes < fmoe_workspace_bytes(FMOE_OP_MOE_LAYER, n_tokens, H, I, E, k)) return FMOE_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return FMOE_ERR_ALIGN;
  if (!aligned(x_in, 16) || !aligned(h_out, 16) || !aligned(idx_out, 4) || !aligned(w_out, 4)) return FMOE_ERR_ALIGN;
  const size_t nx = (size_t)n_tokens * H * 4, nk = (size_t)n_tokens * n_layers * k * 4;
  if (overlaps(h_out, nx, x_in, nx) || overlaps(ws, ws_bytes, x_in, nx) || overlaps(ws, ws_bytes, h_out, nx))
    return FMOE_ERR_OVERLAP;
  if (idx_out && (overlaps(idx_out, nk, x_in, nx) || overlaps(idx_out, nk, h_out, nx) ||
                  overlaps(idx_out, nk, ws, ws_bytes)))
    return FMOE_ERR_OVERLAP;
  if (w_out && (overlaps(w_out, nk, x_in, nx) || overlaps(w_out, nk, h_out, nx) || overlaps(w_out, nk, ws, ws_bytes) ||
                (idx_out && overlaps(w_out, nk, idx_out, nk))))
    return FMOE_ERR_OVERLAP;
  if (n_tokens > 1 && !batched_shape_ok(H, I)) return FMOE_ERR_SHAPE;
  if (n_tokens > 1 && !batched_bits_ok(bits)) return FMOE_ERR_BITS;
  int rc = check_device();
  if (rc) return rc;
  // every check has passed: from here on work is enqueued
  if (zero_sync_region && (rc = zero_fill(ws, kWsDecodeEnd, s))) return rc;

  if (n_tokens > 1) {
    char* b = static_cast<char*>(ws);
    return launch_batched(layers, n_layers, x_in, h_out, n_tokens, k, eps, flags, idx_out, w_out, b + kWsDecodeEnd,
                          ws_bytes - kWsDecodeEnd, reinterpret_cast<uint32_t*>(b + kWsDone), s);
  }

  // single-token decode: one persistent kernel per block of up to 64 layers
  int lpr_g, cpl_g, lpr_d, cpl_d;
  if ((rc = decode_geometry(H, I, bits, &lpr_g, &cpl_g, &lpr_d, &cpl_d))) return rc;
  int G = 0;
  if ((rc = decode_grid(&G))) return rc;
  if (G > kMaxGrid) G = kMaxGrid;
  const int rows_per_wg = (H + G - 1) / G;
  if (decode_smem_bytes(H, I, E + hs, k + hs, G, rows_per_wg, bits) > kDecodeMaxLds) return FMOE_ERR_SHAPE;
  DecodeWs d = carve_decode(ws);
  DecodeParams p;
  memset(&p, 0, sizeof(p));
  p.n_experts = E;
  p.hidden = H;
  p.inter = I;
  p.k = k;
  p.has_shared = hs;
  p.bits = bits;
  p.lpr_g = lpr_g;
  p.cpl_g = cpl_g;
  p.lpr_d = lpr_d;
  p.cpl_d = cpl_d;
  p.rows_per_wg = rows_per_wg;
  p.router_items = ((E + hs + G - 1) / G) * ((H + 1023) / 1024);
  p.eps = eps;
  p.flags = flags;
  p.x_in = x_in;
  p.h_out = h_out;
  p.idx_out = idx_out;
  p.w_out = w_out;
  p.h = d.h;
  p.a = d.a;
  p.logits = d.logits;
  p.flags_arr = d.flags;
  p.err = d.err;
  p.expert_stride = L0.expert_stride;
  for (int l0 = 0; l0 < n_layers; l0 += kMaxLayersPerLaunch) {
    const int nl = (n_layers - l0) < kMaxLayersPerLaunch ? (n_layers - l0) : kMaxLayersPerLaunch;
    for (int l = 0; l < nl; ++l) {
      p.router[l] = layers[l0 + l].router;
      p.shared_gate[l] = layers[l0 + l].shared_gate;
      p.experts[l] = static_cast<const uint8_t*>(layers[l0 + l].experts);
    }
    p.layer0 = l0;
    p.n_layers = nl;
    p.is_final = (l0 + nl == n_layers);
    if ((rc = launch_decode(p, G, s))) return rc;
  }
  return FMOE_OK;
}

}  // namespace

extern "C" {

int fmoe_workspace_error(const void* ws, size_t ws_bytes, uint32_t* err_out, fmoe_stream_t stream) {
  if (!ws || !err_out) return FMOE_ERR_NULL;
  if (ws_bytes < kWsDecodeEnd) return FMOE_ERR_WORKSPACE;
  if (!aligned(ws, 256) || !aligned(err_out, 4)) return FMOE_ERR_ALIGN;
  if (overlaps(err_out, 4, ws, ws_bytes)) return FMOE_ERR_OVERLAP;
  int rc = check_device();
  if (rc) return rc;
  const char* b = static_cast<const char*>(ws);
  return hipMemcpyAsync(err_out, b + kWsErr, 4, hipMemcpyDeviceToDevice, (hipStream_t)stream) == hipSuccess
             ? FMOE_OK
             : FMOE_ERR_HIP;
}

int fmoe_batched_a16(const void* ws, size_t ws_bytes, int n_tokens, int hidden, int inter, int n_experts, int k,
                     int bits, uint16_t* a16_out, fmoe_stream_t stream) {
  if (!ws || !a16_out) return FMOE_ERR_NULL;
  if (!bits_ok(bits) || !batched_bits_ok(bits)) return FMOE_ERR_BITS;
  if (n_tokens < 2 || n_tokens > 4096 || n_experts < 1 || n_experts > 4096) return FMOE_ERR_SHAPE;
  if (hidden < 256 || hidden > 8192 || inter < 128 || inter > 8192 || !batched_shape_ok(hidden, inter))
    return FMOE_ERR_SHAPE;
  if (k < 1 || k > 16 || k > n_experts) return FMOE_ERR_K;
  // k: the slots of the inspected call (its k, or k + 1 with a shared expert)
  if (ws_bytes < kWsDecodeEnd + batched_region_bytes(n_tokens, hidden, inter, n_experts, k)) return FMOE_ERR_WORKSPACE;
  if (!aligned(ws, 256) || !aligned(a16_out, 2)) return FMOE_ERR_ALIGN;
  if (overlaps(a16_out, (size_t)n_tokens * k * inter * 2, ws, ws_bytes)) return FMOE_ERR_OVERLAP;
  int rc = check_device();
  if (rc) return rc;
  return launch_batched_a16(static_cast<const char*>(ws) + kWsDecodeEnd, n_tokens, hidden, inter, n_experts, k, bits, a16_out,
                            (hipStream_t)stream);
}

}  // extern "C"
