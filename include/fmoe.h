/*
 * fmoe.h -- C-ABI of the MI355X (gfx950) quantized MoE expert-block library.
 *
 * The library computes the per-token Mixture-of-Experts expert block described on the
 * Flash-MoE pages:
 *   [aibit]  aibit.im, "397B MoE sur MacBook : 4,4 t/s Moteur Flash-MoE"
 *   [hada]   tr.news.hada.io topic 27758, "Flash-MoE - Dizustunde 397 milyar parametreli
 *            modeli calistirma"
 *   [radar]  openclawradar.com, "Autoresearch pousse Qwen3.5-397B a 20,34 tok/s sur M5 Max
 *            via le streaming SSD"
 * i.e. an fp32 router over the experts, top-k selection with softmax weights, affine
 * group-quantized (4-bit, 3-bit or 2-bit codes with a bf16 scale and bias per group of 64
 * weights) gate/up matvecs with a fused SwiGLU, the down matvec, and the weighted
 * combine plus residual, with an RMS norm between layers.
 *
 * Conventions shared by every entry point
 *  - Every data pointer is a DEVICE pointer owned by the caller (e.g. a torch tensor's
 *    data_ptr()). Descriptor structs (fmoe_qmat, fmoe_expert, fmoe_layer) live in host
 *    memory and are read only during the call. The library never allocates or frees
 *    caller memory; scratch memory comes from a caller workspace sized by
 *    fmoe_workspace_bytes().
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; 0 = the null stream).
 *    Buffers must stay alive until the stream reaches that point.
 *  - Every entry point returns FMOE_OK (0) or a negative fmoe_status. All arguments are
 *    validated before anything is enqueued: on an error nothing was enqueued. A failed
 *    launch returns FMOE_ERR_HIP. No C++ exception crosses this interface.
 *  - Entry points keep no mutable global state and may be called from several threads;
 *    two calls that share a workspace must not overlap on the device.
 *  - Alignment: codes, sb, activation and output pointers must be 16-byte aligned.
 *
 * Quantized matrix layout (the library's packed layout, produced by fmoe_pack)
 *  - canonical codes (fmoe_pack's input): row-major, rows x (cols*bits/8) bytes; a row is
 *    a little-endian bit stream with column c in bits bits*c .. bits*c + bits - 1. 4-bit:
 *    byte j of a row holds column 2j in bits 0-3 and column 2j+1 in bits 4-7. 2-bit: byte
 *    j holds column 4j+t in bits 2t..2t+1. 3-bit ([radar] "Optimisations efficaces": 3-bit
 *    experts): bytes 3j..3j+2, read as a little-endian 24-bit word, hold column 8j+t in
 *    bits 3t..3t+2.
 *  - packed 4-bit and 2-bit codes: the same rows * cols*bits/8 bytes, regrouped in blocks of 32
 *    consecutive rows. Each row is cut into pieces of 4 groups of 64 columns (128 bytes at
 *    4 bits, 64 at 2 bits); piece p of a block's rows is stored contiguously in row order,
 *    at block start + p * rows_in_block * piece bytes (a final block may hold fewer than
 *    32 rows); inside its piece, row r's 16-byte chunk k sits at position
 *    (k + rot) mod (chunks in the piece), rot = r mod 8 (4-bit) or (r mod 16) / 4 (2-bit);
 *    a row that ends in a shorter piece stores it the same way with its own size. 16-byte
 *    chunks keep their canonical contents.
 *  - packed 3-bit codes: two planes in the same rows * cols * 3 / 8 bytes. The low plane
 *    (rows * cols / 4 bytes) holds the low 2 bits of every code exactly as the packed codes
 *    of a 2-bit matrix of the same shape; the high plane follows it with the third bits,
 *    one uint32 per 32 columns (two per group), blocked like sb (below) with two words per
 *    group; in the word of columns 32h..32h+31 of a group, column 32h + c (c < 32) is bit
 *    4 * ((c % 16) / 2) + 2 * (c / 16) + c % 2.
 *  - sb: one uint32 per (row, group); bits 0-15 = bf16 scale s, bits 16-31 = bf16 bias b
 *    of the group; blocked like the codes: blocks of 32 rows, each row's words cut into
 *    pieces of 4 groups, piece p of a block's rows stored together in row order (short
 *    last pieces and blocks keep their own sizes). fmoe_pack's scale and bias inputs are
 *    row-major [rows][cols/group]. Weight (r, c) is q*s + b with s, b of group floor(c/group)
 *    ([aibit] "Techniques de rupture" item 2 and [hada] "FMA optimize dequant cekirdegi":
 *    the affine nibble*scale+bias form).
 *  - group must be 64 and cols a multiple of 64.
 *
 * Expert blob (one expert, fixed size fmoe_expert_bytes()):
 *    [gate codes][up codes][down codes][gate sb][up sb][down sb]
 *  gate/up are inter x hidden, down is hidden x inter. At hidden 4096, inter 1024 a
 *  4-bit blob is 7,077,888 bytes (the pages' "about 6.75 MB per expert", [aibit]
 *  "Techniques de rupture" item 1 and [hada] "SSD Expert Streaming"); 3-bit: 5,505,024
 *  (22% less); 2-bit: 3,932,160.
 */
#ifndef FMOE_H
#define FMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* fmoe_stream_t; /* same type as hipStream_t */

enum fmoe_status {
  FMOE_OK = 0,
  FMOE_ERR_NULL = -1,      /* a required pointer is NULL */
  FMOE_ERR_SHAPE = -2,     /* sizes out of range, not a multiple of 64, or inconsistent */
  FMOE_ERR_BITS = -3,      /* bits not in {2, 3, 4} */
  FMOE_ERR_GROUP = -4,     /* group != 64 */
  FMOE_ERR_K = -5,         /* k not in 1..min(16, n_experts) */
  FMOE_ERR_ALIGN = -6,     /* a pointer or stride is not 16-byte (stride: 256-byte) aligned */
  FMOE_ERR_WORKSPACE = -7, /* workspace NULL or smaller than fmoe_workspace_bytes() */
  FMOE_ERR_HIP = -8,       /* a HIP call or kernel launch failed */
  FMOE_ERR_INTERNAL = -9,  /* unexpected internal condition */
  FMOE_ERR_DEVICE = -10,   /* the current device is not gfx950 */
  FMOE_ERR_OVERLAP = -11,  /* an output buffer overlaps an input buffer */
  FMOE_ERR_SCRATCH = -12   /* fmoe_moe_layer_noalloc: the call needs more than the static scratch */
};

/* Flags of fmoe_moe_layer. */
#define FMOE_PRENORM 1u /* v = rmsnorm(h) feeds router and experts (between layers) */
#define FMOE_RESET_SCRATCH 2u /* fmoe_moe_layer_noalloc: zero the scratch's synchronization state first */

/* Operation ids of fmoe_workspace_bytes. */
enum fmoe_op { FMOE_OP_EXPERT_FFN = 1, FMOE_OP_MOE_LAYER = 2 };

typedef struct fmoe_qmat {
  const void* codes;  /* packed codes, see layout above */
  const uint32_t* sb; /* packed (scale, bias) pairs */
  int rows, cols, bits, group;
} fmoe_qmat;

typedef struct fmoe_expert {
  fmoe_qmat gate, up, down; /* gate/up: inter x hidden; down: hidden x inter */
} fmoe_expert;

typedef struct fmoe_layer {
  const float* router;  /* fp32 [n_experts][hidden], row-major */
  const void* experts;  /* n_experts expert blobs, blob e at experts + e * expert_stride */
  size_t expert_stride; /* bytes; >= fmoe_expert_bytes(), multiple of 256 */
  int n_experts, hidden, inter, bits, group;
  /* NULL, or the layer's shared expert ([hada] "Model mimarisi": one shared expert per
   * layer; "Metal Compute Shaders": a gate in the combine): an fp32 [hidden] gate vector
   * (16-byte aligned), and the expert set then holds n_experts + 1 blobs, the last (index
   * n_experts) being the shared expert, which every token runs with weight
   * 1 / (1 + exp(-gate . v)). All layers of a call have one or none; k + 1 <= 16 and
   * n_experts + 1 <= 4096. */
  const float* shared_gate;
} fmoe_layer;

/* Human-readable text of a status code (static storage). */
const char* fmoe_status_string(int status);

/* Library version string, e.g. "fmoe 0.1 gfx950". */
const char* fmoe_version(void);

/* Bytes of a packed matrix's codes and of its sb array; 0 if the shape is invalid. */
size_t fmoe_codes_bytes(int rows, int cols, int bits);
size_t fmoe_sb_bytes(int rows, int cols, int group);

/* Bytes of one expert blob (layout above); 0 if the shape is invalid. */
size_t fmoe_expert_bytes(int hidden, int inter, int bits, int group);

/* Views of the three matrices of the expert blob at `blob` (no device access). */
int fmoe_expert_view(const void* blob, int hidden, int inter, int bits, int group, fmoe_expert* out);

/* Canonical -> packed. codes_canon: uint8 [rows][cols*bits/8] (canonical layout);
 * scale, bias: bf16 bit patterns [rows][cols/group]. Writes codes_out (packed layout,
 * fmoe_codes_bytes bytes; it must not overlap codes_canon, FMOE_ERR_OVERLAP) and sb_out.
 * Device pointers. */
int fmoe_pack(const uint8_t* codes_canon, const uint16_t* scale, const uint16_t* bias, int rows, int cols,
              int bits, int group, void* codes_out, uint32_t* sb_out, fmoe_stream_t stream);

/* Workspace bytes needed by an operation (0 when none is needed). For FMOE_OP_MOE_LAYER
 * pass the largest n_tokens, hidden, inter, n_experts and k that the calls will use.
 * A FMOE_OP_MOE_LAYER workspace must be zero-filled before its first use; each call
 * leaves it ready for the next one (it holds the synchronization state of the decode
 * kernel), whatever the shapes of the calls: its control words and the decode kernel's
 * exchange region sit at fixed offsets (about 8.9 MB, the size for n_tokens == 1), the
 * multi-token scratch after them. After a call whose device-side wait gave up (see
 * fmoe_workspace_error), zero it again. Epochs are 32-bit: a workspace used by calls of
 * several shapes is best zeroed again after 2^32 / 3 layer passes (24 M tokens of 60
 * layers). */
size_t fmoe_workspace_bytes(int op, int n_tokens, int hidden, int inter, int n_experts, int k);

/* Enqueue on `stream` a copy of the workspace's error word into err_out (a device
 * uint32): 0 when every device-side wait of the decode path on this workspace completed,
 * non-zero once one gave up (its call wrote NaN to the rows of h_out it could not finish,
 * and later calls on the workspace give up too until it is zero-filled again). A wait
 * gives up when the persistent decode kernel's workgroups could not all run at once
 * (for example when other work held compute units for seconds). ws, ws_bytes: as
 * passed to fmoe_moe_layer (ws_bytes >= the single-token workspace size). */
int fmoe_workspace_error(const void* ws, size_t ws_bytes, uint32_t* err_out, fmoe_stream_t stream);

/*
 * y[v][r] = sum_c (q[r][c] * s[r][c/64] + b[r][c/64]) * x[v][c]  for v < n_vec.
 * The dequantized matvec of [aibit] "Techniques de rupture" item 4 (4-bit and 2-bit
 * dequant matvec; 3-bit as in [radar] "Optimisations efficaces"), computed per group as
 * s * sum(q*x) + b * sum(x) in fp32.
 * x: fp32 [n_vec][cols]; y: fp32 [n_vec][rows]; 1 <= n_vec <= 64; cols <= 8192 (4-bit)
 * or 16384 (3-bit, 2-bit). y must not overlap x.
 */
int fmoe_dequant_matvec(const fmoe_qmat* W, const float* x, float* y, int n_vec, fmoe_stream_t stream);

/*
 * Several dequantized matvecs over one input, in one launch ([radar] "Optimisations
 * efficaces": a fused Q/K/V projection kernel reads the input vector once instead of
 * once per matrix):  y[m][v][r] = sum_c W_m[r][c] * x[v][c]  for m < n_mats, each as
 * fmoe_dequant_matvec. Each wave of the kernel reads its part of x into registers once
 * and reuses it for the rows of every matrix.
 * W: host array of n_mats descriptors (1 <= n_mats <= 8) with equal cols and bits (rows
 * may differ); x: fp32 [n_vec][cols]; y: host array of n_mats device pointers, y[m] fp32
 * [n_vec][W[m].rows]. No output may overlap x or another output (FMOE_ERR_OVERLAP);
 * other limits and errors as fmoe_dequant_matvec.
 */
int fmoe_dequant_matvec_multi(const fmoe_qmat* W, int n_mats, const float* x, float* const* y, int n_vec,
                              fmoe_stream_t stream);

/*
 * Router + top-k for n_tokens tokens ([aibit] "Techniques de rupture" items 1 and 3,
 * [hada] "Model mimarisi": k of n_experts experts per token; the pages route on the
 * CPU, here it runs on the device):
 *   logits[t][e] = sum_i router[e][i] * x[t][i]                  (fp32)
 *   idx[t][0..k) = the k largest logits, descending; equal logits -> lower index first;
 *                  NaN ranks last
 *   w[t][j]      = exp(l_j - l_0) / sum_{j'<k} exp(l_j' - l_0)    (softmax over the k)
 * router: fp32 [n_experts][hidden]; x: fp32 [n_tokens][hidden]; idx: int32
 * [n_tokens][k]; w: fp32 [n_tokens][k]; logits: fp32 [n_tokens][n_experts] (required:
 * it is the scratch between the two steps).
 * Limits: 1 <= n_experts <= 4096, hidden multiple of 64 and <= 16384, 1 <= k <= 16.
 */
int fmoe_route_topk(const float* router, const float* x, int n_tokens, int n_experts, int hidden, int k,
                    int32_t* idx, float* w, float* logits, fmoe_stream_t stream);

/*
 * One expert's SwiGLU FFN for one token ([aibit] "Techniques de rupture" item 4: fused
 * SwiGLU, dequant matvecs):  y = Wd (silu(Wg x) * (Wu x)),  silu(z) = z / (1 + e^-z).
 * x: fp32 [hidden]; y: fp32 [hidden]; ws: >= fmoe_workspace_bytes(FMOE_OP_EXPERT_FFN,
 * 1, hidden, inter, 1, 1) bytes. All three matrices share bits and group; hidden <=
 * 8192, inter <= 8192 (4-bit limits of fmoe_dequant_matvec).
 */
int fmoe_expert_ffn(const fmoe_expert* e, const float* x, float* y, void* ws, size_t ws_bytes,
                    fmoe_stream_t stream);

/*
 * MoE layers. For each layer l in order ([aibit] "Techniques de rupture" item 3 and
 * [hada] "Deferred GPU Expert Compute": route, run the selected experts, then combine
 * with the residual and normalize for the next layer):
 *   v   = (flags & FMOE_PRENORM) ? h / sqrt(mean(h^2) + eps) : h
 *   idx, w = route(router_l, v, k)                  (as fmoe_route_topk)
 *   h   = h + sum_j w_j * FFN_{idx_j}(v)            (as fmoe_expert_ffn)
 *             [+ sigmoid(shared_gate . v) * FFN_shared(v) when the layers have one]
 * with h = x_in at the start; h_out receives the final h.
 * x_in, h_out: fp32 [n_tokens][hidden], must not overlap. idx_out (nullable): int32
 * [n_tokens][n_layers][k]; w_out (nullable): fp32 [n_tokens][n_layers][k].
 * n_tokens == 1 runs the single-token decode path (one persistent kernel for all
 * layers). n_tokens > 1 runs the batched path: tokens are grouped by expert and each
 * expert's gate/up/down run as bf16 matrix-core products with fp32 accumulation. The
 * codes enter the matrix cores exactly and each group's scale and bias are applied to
 * its fp32 partial sums, so no weight is rounded; the activations v (the input of
 * gate/up) and a = silu(g) * u (the input of down) are rounded to bf16. Routing, the
 * norm and the combine stay fp32.
 * All layers must share n_experts, hidden, inter, bits, group and expert_stride.
 * Limits: 64 <= hidden, inter <= 8192 (multiples of 64), 1 <= n_experts <= 4096,
 * 1 <= k <= min(16, n_experts), n_tokens <= 4096, n_layers <= 4096; the batched path
 * (n_tokens > 1) also needs hidden % 256 == 0 and inter % 128 == 0; the decode path
 * needs its per-workgroup state (the staged vectors, the logits and the selection)
 * within 160 KB of LDS (FMOE_ERR_SHAPE otherwise); at hidden 4096, inter 1024 that holds
 * k 4 with up to 4096 experts and, with 512 experts, k up to 14 (4-bit) or 15 (2-bit).
 * Pointers: x_in, h_out 16-byte aligned; experts 256-byte aligned; ws 256-byte aligned.
 */
int fmoe_moe_layer(const fmoe_layer* layers, int n_layers, const float* x_in, float* h_out, int n_tokens, int k,
                   float eps, unsigned flags, int32_t* idx_out, float* w_out, void* ws, size_t ws_bytes,
                   fmoe_stream_t stream);

/*
 * fmoe_moe_layer without a caller workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).
 * Same operation, arguments, limits and errors as fmoe_moe_layer; the workspace is the
 * library's own static scratch of 32 MiB per GPU (a file-scope device array that each GPU
 * the library runs on holds until the process ends). Nothing is allocated or freed.
 *  - A call whose fmoe_workspace_bytes(FMOE_OP_MOE_LAYER, n_tokens, hidden, inter,
 *    n_experts, k) exceeds 32 MiB returns FMOE_ERR_SCRATCH before enqueuing anything (the
 *    single-token path always fits; at hidden 4096, inter 1024, 512 experts, top-4 the
 *    multi-token path fits up to 150 tokens).
 *  - Every call on a GPU shares that GPU's scratch, which keeps the state of the last call:
 *    the first call on a GPU, and any call with FMOE_RESET_SCRATCH in flags, first
 *    zero-fills its synchronization state on `stream` (needed again after a call whose
 *    device-side wait gave up, visible as NaN rows of h_out). Calls that overlap on one GPU
 *    (other streams, other threads) race on the scratch and give undefined results.
 */
int fmoe_moe_layer_noalloc(const fmoe_layer* layers, int n_layers, const float* x_in, float* h_out, int n_tokens,
                           int k, float eps, unsigned flags, int32_t* idx_out, float* w_out, fmoe_stream_t stream);

/*
 * Inspection of the batched path's SwiGLU stage (for verifying it stage by stage). After
 * an fmoe_moe_layer call with n_tokens > 1 that used workspace `ws` (same n_tokens,
 * hidden, inter, n_experts and bits; k = the call's slots per token: its k, or k + 1 when
 * its layers have a shared expert), enqueue on `stream` a copy of the last layer's bf16
 * SwiGLU outputs: a16_out[t][j][c] = bf16(silu(g) * u) for token t, slot j (the j-th
 * selected expert; slot k of a call with a shared expert is the shared expert), row c, as
 * bf16 bit patterns [n_tokens][slots][inter] (device memory).
 */
int fmoe_batched_a16(const void* ws, size_t ws_bytes, int n_tokens, int hidden, int inter, int n_experts, int k,
                     int bits, uint16_t* a16_out, fmoe_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif
