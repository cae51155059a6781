// fmoe_decode.h -- parameters of the persistent single-token decode kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fmoe {

constexpr int kMaxLayersPerLaunch = 64;
constexpr int kMaxGrid = 1024;  // workgroups of the persistent kernel (>= compute units)
constexpr int kRep = 8;         // replicas of every exchanged item (logits, h, a)
constexpr size_t kDecodeMaxLds = 160 * 1024;  // a gfx950 workgroup's LDS (beyond 64 KB by opt-in)

struct DecodeParams {
  const float* router[kMaxLayersPerLaunch];
  const float* shared_gate[kMaxLayersPerLaunch];  // fp32 [hidden] gates when has_shared
  const uint8_t* experts[kMaxLayersPerLaunch];
  size_t expert_stride;
  int n_layers;   // layers in this launch
  int layer0;     // global index of the first of them
  int is_final;   // this launch ends with the last layer of the call
  int n_experts, hidden, inter, k, bits;
  int has_shared;  // 1: every layer also runs its shared expert (blob index n_experts)
  int lpr_g, cpl_g, lpr_d, cpl_d;
  int rows_per_wg, router_items;
  float eps;
  unsigned flags;
  const float* x_in;
  float* h_out;
  int32_t* idx_out;  // [n_layers_total][k] or null (single token)
  float* w_out;
  // workspace
  uint64_t* h;         // [kRep][hidden], tagged (value | epoch << 32)
  uint64_t* a;         // [kRep][k + has_shared][inter], tagged
  uint64_t* logits;    // [kRep][n_experts + has_shared], tagged
  uint32_t* flags_arr; // [kRep][kMaxGrid] epoch slots, zero-filled before the first call on a workspace
  uint32_t* err;       // [1]
};

int decode_geometry(int hidden, int inter, int bits, int* lpr_g, int* cpl_g, int* lpr_d, int* cpl_d);
size_t decode_smem_bytes(int hidden, int inter, int n_experts, int k, int G, int rows_per_wg, int bits);
int decode_grid(int* G_out);
int launch_decode(const DecodeParams& p, int G, hipStream_t s);

}  // namespace fmoe
