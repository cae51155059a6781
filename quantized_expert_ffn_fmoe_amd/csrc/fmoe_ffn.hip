// fmoe_ffn.hip -- one expert's SwiGLU FFN for one token (standalone entry point).
//
// Gate and up rows i are read by the same lanes and combined at once into
// a[i] = silu(g_i) * u_i (the fused SwiGLU of aibit.im "Techniques de rupture" item 4);
// the down matvec then reuses the standalone dequantized matvec kernel.
#include "fmoe_device.h"
#include "fmoe_internal.h"
#include "fmoe_layout.h"

namespace fmoe {

template <int BITS, int CPL>
__global__ void __launch_bounds__(256) gate_up_kernel(const uint8_t* __restrict__ gcodes,
                                                      const uint32_t* __restrict__ gsb,
                                                      const uint8_t* __restrict__ ucodes,
                                                      const uint32_t* __restrict__ usb, const float* __restrict__ x,
                                                      float* __restrict__ a, int rows, int cols, int lpr) {
  using C = Chunk<BITS>;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rpw = kWave / lpr;
  const int sub = lane & (lpr - 1);
  const int rsel = lane / lpr;
  const int n_chunks = cols / C::kCodes;
  const int ngroups = cols / 64;

  XChunk<BITS> xc[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    int c = sub + lpr * j;
    if (c < n_chunks) load_xchunk<BITS>(xc[j], x + (size_t)c * C::kCodes);
  }
  const int waves_total = gridDim.x * (blockDim.x >> 6);
  for (int rb = (blockIdx.x * (blockDim.x >> 6) + wave) * rpw; rb < rows; rb += waves_total * rpw) {
    const int r = rb + rsel;
    float g = 0.f, u = 0.f;
    if (r < rows) {
      CChunk<BITS> wg[CPL], wu[CPL];
      uint32_t sg[CPL], su[CPL];
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        int c = sub + lpr * j;
        if (c < n_chunks) {
          load_cchunk<BITS>(wg[j], gcodes, rows, cols, r, c);
          load_cchunk<BITS>(wu[j], ucodes, rows, cols, r, c);
          const size_t so = sb_offset(rows, ngroups, r, c / C::kPerGroup);
          sg[j] = gsb[so];
          su[j] = usb[so];
        }
      }
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        int c = sub + lpr * j;
        if (c < n_chunks) {
          g += chunk_dot<BITS>(wg[j], sg[j], xc[j]);
          u += chunk_dot<BITS>(wu[j], su[j], xc[j]);
        }
      }
    }
    g = group_sum(g, lpr);
    u = group_sum(u, lpr);
    if (r < rows && sub == 0) a[r] = swiglu(g, u);
  }
}

int launch_expert_ffn(const fmoe_expert& e, const float* x, float* y, float* a_ws, hipStream_t s) {
  const int rows = e.gate.rows, cols = e.gate.cols, bits = e.gate.bits;
  const int n_chunks = cols / (bits == 4 ? 32 : 64);
  int lpr = 1;
  while (lpr < n_chunks && lpr < 64) lpr <<= 1;
  const int cpl = (n_chunks + lpr - 1) / lpr;
  const int rpw = 64 / lpr;
  int blocks = ((rows + rpw - 1) / rpw + 3) / 4;
  if (blocks > 2048) blocks = 2048;
  const uint8_t* gc = static_cast<const uint8_t*>(e.gate.codes);
  const uint8_t* uc = static_cast<const uint8_t*>(e.up.codes);
#define FMOE_GU(B, C)                                                                                         \
  hipLaunchKernelGGL((gate_up_kernel<B, C>), dim3(blocks), dim3(256), 0, s, gc, e.gate.sb, uc, e.up.sb, x, a_ws, \
                     rows, cols, lpr)
  if (bits == 4) {
    if (cpl == 1) FMOE_GU(4, 1);
    else if (cpl == 2) FMOE_GU(4, 2);
    else if (cpl <= 4) FMOE_GU(4, 4);
    else return FMOE_ERR_SHAPE;
  } else if (bits == 3) {
    if (cpl == 1) FMOE_GU(3, 1);
    else if (cpl == 2) FMOE_GU(3, 2);
    else if (cpl <= 4) FMOE_GU(3, 4);
    else return FMOE_ERR_SHAPE;
  } else {
    if (cpl == 1) FMOE_GU(2, 1);
    else if (cpl == 2) FMOE_GU(2, 2);
    else if (cpl <= 4) FMOE_GU(2, 4);
    else return FMOE_ERR_SHAPE;
  }
#undef FMOE_GU
  if (hipGetLastError() != hipSuccess) return FMOE_ERR_HIP;
  return launch_matvec(e.down, a_ws, y, 1, s);
}

}  // namespace fmoe
