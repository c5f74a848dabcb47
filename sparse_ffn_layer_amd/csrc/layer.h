// The whole layer behind the two entry points that run it:
// moe_layer_forward (caller's workspace) and moe_layer_forward_noalloc (the
// library's own scratch array).  Host code only.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace sfl {

// Pointer arguments of the layer, as in moe_layer_forward.
struct LayerArgs {
  const void* x;
  const void* W_r;
  const float* router_bias;
  const float* select_bias;
  const void* W1;
  const void* b1;
  const void* W2;
  const void* b2;
  const float* w1_scale;
  const float* w2_scale;
  void* y;
  int32_t* topk_idx_out;
  float* topk_gate_out;
  float* logits_out;
  int32_t* expert_counts_out;
};

// Validates the problem and the pointers on the host.  On MOE_OK, *need is
// the workspace the layer uses (0 when S == 0: then there is nothing to run).
int32_t layer_validate(const moe_problem* mp, const LayerArgs& a, size_t* need);

// Launches the layer on `ws` (at least *need bytes from layer_validate,
// 256-byte aligned); the arguments must have passed layer_validate.
int32_t layer_run(const moe_problem* mp, const LayerArgs& a, void* ws, hipStream_t st);

}  // namespace sfl
