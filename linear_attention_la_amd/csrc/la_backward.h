// Internal pieces of the backward pass (not part of the public ABI): its
// chains side by side in one launch of the one-workgroup-per-chain prefill
// kernel (d = 128), and an in-place state transpose for the segmented
// backward.
#pragma once

#include "la_internal.h"

namespace la {

// One of the three chains: queries, keys and values of the forward kernel,
// the gradient it writes as its output, its direction in time, and how its
// state enters and leaves: kv_init[s, h] (read transposed if
// init_transposed) times lambda^init_pow, or zeros if kv_init is nullptr;
// lambda^final_pow times the final state to kv_final[s, h] unless nullptr.
struct BackwardPass {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  const float* kv_init;
  float* kv_final;
  int32_t reverse;
  int32_t init_transposed;
  float init_pow;
  float final_pow;
};

// num_passes (2 or 3) passes of every chain; item i runs pass
// i % num_passes of chain i / num_passes, and the passes of a chain go to
// one XCD.
struct BackwardPasses {
  BackwardPass pass[3];
  int32_t num_passes;
};

// a.num_items = num_passes * S * H; a carries the decays, the sequence order
// and the slot map of the initial states.
hipError_t launch_backward_wide(const PrefillArgs& a, const BackwardPasses& bp,
                                la_dtype grad_dtype, hipStream_t stream);

// x[i] <- scale[h] * x[i]^T in place for num_states fp32 d x d states
// (state i belongs to head i % num_heads); scale: host [H].
hipError_t launch_state_transpose_inplace(float* x, int32_t num_states, int32_t num_heads,
                                          int32_t head_dim, const float* scale,
                                          hipStream_t stream);

}  // namespace la
