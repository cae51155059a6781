// fmoe_batched.h -- the multi-token (batched) path of fmoe_moe_layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "fmoe.h"

namespace fmoe {

bool batched_shape_ok(int hidden, int inter);
bool batched_bits_ok(int bits);
// ws: the multi-token scratch; done: the sort's arrival counter, a word of the workspace's
// fixed control block (0 between calls, whatever the shapes of earlier calls)
size_t batched_workspace_bytes(int n_tokens, int hidden, int inter, int n_experts, int k);
// bytes of the multi-token scratch as a call with k_slots slots per token lays it out
size_t batched_region_bytes(int n_tokens, int hidden, int inter, int n_experts, int k_slots);
int launch_batched_a16(const void* ws, int n_tokens, int hidden, int inter, int n_experts, int k, int bits,
                       uint16_t* out, hipStream_t s);
int launch_batched(const fmoe_layer* layers, int n_layers, const float* x_in, float* h_out, int n_tokens, int k,
                   float eps, unsigned flags, int32_t* idx_out, float* w_out, void* ws, size_t ws_bytes,
                   uint32_t* done, hipStream_t s);

}  // namespace fmoe
