// fmoe_internal.h -- host-side declarations shared by the fmoe translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fmoe.h"

namespace fmoe {

using QMat = fmoe_qmat;

int launch_matvec(const QMat& W, const float* x, float* y, int n_vec, hipStream_t s);
constexpr int kMaxMulti = 8;  // matrices of one fused multi-output matvec
struct MultiMat {
  const uint8_t* codes[kMaxMulti];
  const uint32_t* sb[kMaxMulti];
  float* y[kMaxMulti];
  int rows[kMaxMulti];
  int prow[kMaxMulti + 1];  // first row of each matrix in the padded row space
  int n_mats;
};
int launch_matvec_multi(const QMat* W, int n_mats, const float* x, float* const* y, int n_vec, hipStream_t s);
int launch_pack(const uint8_t* codes_in, const uint16_t* scale, const uint16_t* bias, int rows, int cols, int bits,
                void* codes_out, uint32_t* sb_out, hipStream_t s);
int launch_route(const float* R, const float* x, int n_tokens, int n_experts, int hidden, int k, int32_t* idx,
                 float* w, float* logits, hipStream_t s);
int launch_expert_ffn(const fmoe_expert& e, const float* x, float* y, float* a_ws, hipStream_t s);

}  // namespace fmoe
