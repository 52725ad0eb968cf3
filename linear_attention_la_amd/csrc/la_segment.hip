// Segmented prefill: planning and the prefix over segment states.
//
// A long sequence is cut into segments that are processed as independent
// chains, which multiplies the number of workgroups when few (sequence,
// head) pairs exist.  Segment i of a sequence needs the state reached at its
// start; it is obtained from the local decayed state of every earlier
// segment, Shat_i = sum_{j in i} lambda^(len_i - 1 - j) k_j^T v_j (computed
// by a state-only pass of the prefill kernel), chained in order:
//   S_0 = S_init,   S_(i+1) = lambda^(len_i) S_i + Shat_i.
// A chain that runs backwards in time (the backward pass) takes the
// segments from the last to the first: with E_i the state entering segment
// i and L_i its local state, E_(n-1) = S_init and E_(i-1) = lambda^(len_i)
// E_i + L_i, the state after segment 0 being the final one.
// This is the one-exchange sequence split of LASP+ (mizuki blog "MiniMax-01：
// 4M 上下文破局", 五: local prefix sums, then an all-gather) carried out on
// one device; it is exact: expanding the chain gives the same sum of decayed
// k_j^T v_j terms as the token recurrence.

#include "la_internal.h"

namespace la {
namespace {

constexpr int kPlanThreads = 1024;

__device__ __forceinline__ int segments_of(int32_t len, int32_t segment_len) {
  return len <= 0 ? 1 : (int)((len + (int64_t)segment_len - 1) / segment_len);
}

constexpr int kPlanWaves = kPlanThreads / 64;

// Inclusive prefix sum over the 64 lanes of a wave (six shuffle steps).
__device__ __forceinline__ int32_t wave_inclusive_scan(int32_t x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

// One workgroup.  Thread t owns a contiguous range of sequences; a prefix
// sum of the per-thread segment counts (within each wave, then over the
// wave totals) gives each thread its first segment.
__global__ __launch_bounds__(kPlanThreads) void segment_plan_kernel(
    const int32_t* __restrict__ cu, int32_t num_seqs, int32_t segment_len, int32_t* cu_seg,
    int32_t* init_slot, int32_t* final_slot, int32_t* seq_first, int32_t* ctrl,
    int64_t ctrl_words) {
  __shared__ int32_t wave_total[kPlanWaves];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  if (ctrl)
    for (int64_t x = t; x < ctrl_words; x += kPlanThreads) ctrl[x] = 0;
  const int per = (num_seqs + kPlanThreads - 1) / kPlanThreads;
  const int s0 = min(num_seqs, t * per);
  const int s1 = min(num_seqs, s0 + per);
  int32_t count = 0;
  for (int s = s0; s < s1; ++s) count += segments_of(cu[s + 1] - cu[s], segment_len);
  const int32_t incl = wave_inclusive_scan(count, lane);
  if (lane == 63) wave_total[wave] = incl;
  __syncthreads();
  int32_t before = 0, run = 0;  // segments of earlier waves; of all waves
#pragma unroll
  for (int i = 0; i < kPlanWaves; ++i) {
    const int32_t c = wave_total[i];
    before += i < wave ? c : 0;
    run += c;
  }
  if (t == 0) {
    seq_first[num_seqs] = run;
    cu_seg[run] = cu[num_seqs];
  }
  int32_t g = before + incl - count;  // exclusive prefix of thread t
  for (int s = s0; s < s1; ++s) {
    seq_first[s] = g;
    const int32_t start = cu[s];
    const int32_t len = cu[s + 1] - start;
    const int n = segments_of(len, segment_len);
    for (int i = 0; i < n; ++i, ++g) {
      const int64_t off = (int64_t)i * segment_len;
      cu_seg[g] = start + (int32_t)(off < len ? off : len);
      init_slot[g] = g + s;       // slot of the state at the segment start
      final_slot[g] = g + s + 1;  // slot receiving its local state
    }
  }
}

struct PrefixArgs {
  const int32_t* cu_seg;
  const int32_t* seq_first;
  const float* kv_init;
  float* states;
  float* kv_final;
  int32_t num_heads;
  int32_t chunks;  // float4 chunks of 256 threads per d x d state
  int32_t reverse;
  float log2_decay[LA_MAX_HEADS];
};

// Workgroup (s, h, chunk): each thread carries 4 consecutive state elements
// through the segments of sequence s.  Sequence s owns slots first + s ..
// first + s + n of `states` (n segments from segment index first): forwards,
// slot first + s + i holds the state entering segment i and slot
// first + s + i + 1 arrives holding its local state; backwards, slot
// first + s + i + 1 holds the state entering segment i and slot first + s + i
// arrives holding its local state.  Each local state is replaced in place by
// the state the chain reaches after its segment.
__global__ __launch_bounds__(256) void segment_prefix_kernel(PrefixArgs a, int64_t dd) {
  const int chunk = blockIdx.x % a.chunks;
  const int sh = blockIdx.x / a.chunks;
  const int h = sh % a.num_heads;
  const int s = sh / a.num_heads;
  const int64_t e = ((int64_t)chunk * 256 + threadIdx.x) * 4;
  const int64_t head_off = (int64_t)h * dd + e;
  const int64_t slot_stride = (int64_t)a.num_heads * dd;
  float4 x = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  if (a.kv_init) x = *reinterpret_cast<const float4*>(a.kv_init + (int64_t)s * slot_stride + head_off);
  const int32_t first = a.seq_first[s];
  const int32_t n = a.seq_first[s + 1] - first;
  float* base = a.states + (int64_t)(first + s) * slot_stride + head_off;
  const float l2 = a.log2_decay[h];
  auto step = [&](int i, float* local) {
    const int32_t len = a.cu_seg[first + i + 1] - a.cu_seg[first + i];
    const float f = exp2f((float)len * l2);  // lambda^len
    const float4 loc = *reinterpret_cast<const float4*>(local);
    x = make_float4(fmaf(f, x.x, loc.x), fmaf(f, x.y, loc.y), fmaf(f, x.z, loc.z),
                    fmaf(f, x.w, loc.w));
    *reinterpret_cast<float4*>(local) = x;
  };
  if (!a.reverse) {
    *reinterpret_cast<float4*>(base) = x;
    for (int i = 0; i < n; ++i) step(i, base + (int64_t)(i + 1) * slot_stride);
  } else {
    *reinterpret_cast<float4*>(base + (int64_t)n * slot_stride) = x;
    for (int i = n - 1; i >= 0; --i) step(i, base + (int64_t)i * slot_stride);
  }
  if (a.kv_final) *reinterpret_cast<float4*>(a.kv_final + (int64_t)s * slot_stride + head_off) = x;
}

}  // namespace

hipError_t launch_segment_plan(const int32_t* cu_seqlens, int32_t num_seqs, int32_t segment_len,
                               int32_t* cu_seg, int32_t* init_slot, int32_t* final_slot,
                               int32_t* seq_first, int32_t* ctrl, int64_t ctrl_words,
                               hipStream_t stream) {
  hipLaunchKernelGGL(segment_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, cu_seqlens,
                     num_seqs, segment_len, cu_seg, init_slot, final_slot, seq_first, ctrl,
                     ctrl_words);
  return hipGetLastError();
}

hipError_t launch_segment_prefix(const int32_t* cu_seg, const int32_t* seq_first, int32_t num_seqs,
                                 int32_t num_heads, int32_t head_dim, const float* log2_decay,
                                 const float* kv_init, float* states, float* kv_final,
                                 bool reverse, hipStream_t stream) {
  PrefixArgs a;
  a.cu_seg = cu_seg;
  a.seq_first = seq_first;
  a.kv_init = kv_init;
  a.states = states;
  a.kv_final = kv_final;
  a.num_heads = num_heads;
  a.reverse = reverse ? 1 : 0;
  const int64_t dd = (int64_t)head_dim * head_dim;
  a.chunks = (int32_t)(dd / 1024);  // d = 64: 4, d = 128: 16
  for (int h = 0; h < num_heads; ++h) a.log2_decay[h] = log2_decay[h];
  const int64_t blocks = (int64_t)num_seqs * num_heads * a.chunks;
  hipLaunchKernelGGL(segment_prefix_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a, dd);
  return hipGetLastError();
}

}  // namespace la
