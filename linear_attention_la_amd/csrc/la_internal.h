// Internal interface between the host dispatch (la_host.cpp) and the kernel
// translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "la.h"

namespace la {

// Arguments of one prefill launch.  log2_decay[h] = log2(lambda_h), computed
// on the host in double precision and rounded to float; lambda = 1 gives
// exactly 0, so every decay power of a no-decay head is exactly 1.
struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* cu_seqlens;  // device [S+1]
  const float* kv_init;       // device [S,H,d,d] or nullptr
  void* o;                    // device [T,H,d]
  float* kv_final;            // device [S,H,d,d] or nullptr
  int32_t num_seqs;
  int32_t num_heads;
  int32_t num_items;          // S * H * (d / value-columns per workgroup)
  float log2_decay[LA_MAX_HEADS];
};

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  float* kv;
  void* o;
  int32_t batch;
  int32_t num_heads;
  float decay[LA_MAX_HEADS];
};

// Each returns hipSuccess or the launch error.  The caller has validated
// every argument.
hipError_t launch_prefill_bf16(const PrefillArgs& a, int head_dim, la_dtype out_dtype,
                               hipStream_t stream);
hipError_t launch_prefill_f32(const PrefillArgs& a, int head_dim, la_dtype out_dtype,
                              hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, int head_dim, la_dtype in_dtype,
                         hipStream_t stream);

// Value columns of the state handled by one workgroup in each prefill
// kernel (the d x d state is split by columns over d / cols workgroups).
constexpr int kBf16Cols = 32;
constexpr int kF32Cols = 32;

}  // namespace la
