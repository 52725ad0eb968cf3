// Internal interface between the host dispatch (la_host.cpp) and the kernel
// translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "la.h"

namespace la {

// Largest batch whose sequences the prefill dispatches in a chosen order
// (the order travels in the kernel arguments, 2 bytes per sequence).
constexpr int kMaxOrder = 512;

// Arguments of one prefill launch.  log2_decay[h] = log2(lambda_h), computed
// on the host in double precision and rounded to float; lambda = 1 gives
// exactly 0, so every decay power of a no-decay head is exactly 1.
struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* cu_seqlens;  // device [S+1]
  const float* kv_init;       // device [*,H,d,d] or nullptr
  void* o;                    // device [T,H,d] (unused by a state-only pass)
  float* kv_final;            // device [*,H,d,d] or nullptr
  // Optional device [S] maps from sequence to state slot of kv_init /
  // kv_final (nullptr: slot s for sequence s).  Only the bf16 kernel reads
  // them; the segmented prefill uses them to address its state workspace.
  const int32_t* init_slot;
  const int32_t* final_slot;
  int32_t num_seqs;
  int32_t num_heads;
  int32_t num_items;          // S * H * (d / value-columns per workgroup)
  float log2_decay[LA_MAX_HEADS];
  // Dispatch order of the sequences: with `ordered` set, the i-th sequence
  // taken up by the grid is seq_order[i] (longest first, so the longest
  // chains start in the first wave of workgroups); else sequence i.
  int32_t ordered;
  uint16_t seq_order[kMaxOrder];
  // Output normalisation (kernels launched with it only): per-(head, feature)
  // weight [H, d] fp32, the epsilon added to each row's mean square, and an
  // optional gate [T, H, d] bf16 whose sigmoid multiplies the output.
  const float* norm_weight;
  const void* gate;
  float norm_eps;
};

// Sequence index of the idx-th sequence in dispatch order.
__device__ __forceinline__ int seq_of(const PrefillArgs& a, int idx) {
  return a.ordered ? (int)a.seq_order[idx] : idx;
}

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  float* kv;
  // Optional device [B]: sequence b uses state kv[slots[b]] (nullptr: kv[b]).
  const int32_t* slots;
  void* o;
  int32_t batch;
  int32_t num_heads;
  // Workgroup i handles sequence (i / H * b_step) % batch (b_step coprime to
  // batch; 1 = in order): a stride through the batch spreads the states that
  // are streamed at the same time over memory.
  int32_t b_step;
  float decay[LA_MAX_HEADS];
  // Output normalisation (norm_weight non-null): per-(head, feature) weight
  // [H, d] fp32, the epsilon added to the row's mean square, and an
  // optional gate [B, H, d] of the input dtype whose sigmoid multiplies o.
  const float* norm_weight;
  const void* gate;
  float norm_eps;
};

// Chained-scan prefill (la_prefill_wide.hip, d = 128, bf16): one launch over
// the segments of a segment plan (see launch_segment_plan), a.cu_seqlens
// being the plan's cu_seg and a.num_items = segments * H.  Workgroup items
// (segment, head) compute their segment's local state, take the state
// entering the segment from the item of the previous segment (a chained
// exchange through `ring`, two slots of d x d fp32 per (sequence, head)),
// publish the state entering the next one, then write their outputs.
struct ScanArgs {
  const int32_t* init_slot;  // plan: init_slot[g] = g + (sequence of g)
  const int32_t* seq_first;  // plan: first segment of each sequence, [S+1]
  const float* kv_init;      // [S, H, d, d] or nullptr (zeros)
  float* kv_final;           // [S, H, d, d] or nullptr
  int32_t* ctrl;             // ticket, error word, 2 flags per chain; zero on entry
  float* ring;               // [S * H * 2][d * d]
  int32_t spin_limit;        // polls before a wait gives up (sets the error word)
};

// Control words of a scan launch: the ticket, the error word and 2 flags per
// (sequence, head) chain.
inline int64_t scan_ctrl_words(int64_t chains) { return 2 + 2 * chains; }

// Each returns hipSuccess or the launch error.  The caller has validated
// every argument.
// state_only: compute and write only the final states (no O): K and V are
// read, Q is not.  reverse: every sequence is processed backwards in time
// (token i of the chain is row end-1-i of q, k, v and o).
hipError_t launch_prefill_bf16(const PrefillArgs& a, int head_dim, la_dtype out_dtype,
                               bool state_only, bool reverse, hipStream_t stream);

// Wide decomposition (la_prefill_wide.hip): one workgroup per (sequence,
// head) chain for d = 128 with bf16 inputs; a.num_items = S * H.  Same
// semantics as launch_prefill_bf16 (state_only runs forward only).
hipError_t launch_prefill_wide(const PrefillArgs& a, la_dtype out_dtype, bool state_only,
                               bool reverse, hipStream_t stream);

hipError_t launch_prefill_scan(const PrefillArgs& a, const ScanArgs& sa, la_dtype out_dtype,
                               bool norm, hipStream_t stream);

// The one-workgroup-per-chain prefill (forwards, d = 128) with the output
// normalisation of a.norm_weight / a.norm_eps / a.gate fused into its
// output write.
hipError_t launch_prefill_wide_normed(const PrefillArgs& a, la_dtype out_dtype,
                                      hipStream_t stream);

// out[s,h] = scale[h] * (transpose ? in[s,h]^T : in[s,h]) for num_states x H
// fp32 d x d states (la_state.hip); out may be in only without transpose.
hipError_t launch_state_transform(const float* in, float* out, int32_t num_states,
                                  int32_t num_heads, int32_t head_dim, bool transpose,
                                  const float* scale, hipStream_t stream);

// Segmented prefill helpers (la_segment.hip).  Plan: from cu_seqlens [S+1]
// and segment_len, write cu_seg [n_seg+1], init_slot/final_slot [n_seg] and
// seq_first [S+1] (first segment of each sequence) for a state workspace
// holding n_seg + S slots: sequence s owns slots seq_first[s] + s ..
// seq_first[s] + s + n_s.
// The plan also zeroes ctrl[0 .. ctrl_words) (the control words of a scan
// launch; ctrl may be nullptr).
hipError_t launch_segment_plan(const int32_t* cu_seqlens, int32_t num_seqs, int32_t segment_len,
                               int32_t* cu_seg, int32_t* init_slot, int32_t* final_slot,
                               int32_t* seq_first, int32_t* ctrl, int64_t ctrl_words,
                               hipStream_t stream);
// Prefix over segments: slot 0 of each sequence <- kv_init (or 0); slot i+1
// <- lambda^len_i * slot i + slot i+1 (which holds segment i's local
// state); the last slot is also written to kv_final (if not null).  With
// `reverse` (a chain backwards in time) the same from the last slot down:
// slot n <- kv_init, slot i <- lambda^len_i * slot i+1 + slot i, and slot 0
// goes to kv_final.  log2_decay: host [H] (passed by value to the kernel).
hipError_t launch_segment_prefix(const int32_t* cu_seg, const int32_t* seq_first, int32_t num_seqs,
                                 int32_t num_heads, int32_t head_dim, const float* log2_decay,
                                 const float* kv_init, float* states, float* kv_final,
                                 bool reverse, hipStream_t stream);
hipError_t launch_prefill_f32(const PrefillArgs& a, int head_dim, la_dtype out_dtype,
                              hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, int head_dim, la_dtype in_dtype,
                         hipStream_t stream);

// Value columns of the state handled by one workgroup in each prefill
// kernel (the d x d state is split by columns over d / cols workgroups).
constexpr int kBf16Cols = 32;
constexpr int kF32Cols = 32;

}  // namespace la
