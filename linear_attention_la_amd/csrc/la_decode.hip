// Decode kernel: one token per sequence, fp32 state updated in place.
//
// The length-1 step that serving keeps in its own kernel, apart from the
// length > 1 prefill, so the two can run on separate streams (jvyan.cn news
// article on MiniMax-01, 二、计算优化; CSDN "【AI论文】MiniMax-01:利用闪电注意力
// 机制扩展基础模型" §3.2).  For each (b, h):
//   S <- lambda S + k^T v        (update first)
//   o <- q S                     (read out the updated state)
// Decay, update and read-out are fused into one pass over the state, so each
// 64 KiB fp32 state (d = 128) is read once and written once: the kernel is a
// pure HBM stream (0.5 flop per byte).
//
// A state pool is supported: with a slot map, sequence b reads and writes
// state slots[b] of the pool instead of state b (serving keeps the states of
// all live sequences in one pool and decodes any subset of them).
//
// With kNorm the output row is normalised before it is written: the
// normalisation of NormAttention (CSDN §2.1), read as an RMS normalisation
// over the d features with a per-(head, feature) weight, times
// sigmoid(gate) when a gate is given -- the memory-bound epilogue fused into
// the kernel that produces o (jvyan.cn 二、计算优化).
//
// Layout: one workgroup per (b, h).  Thread t owns the column quad
// 4*(t % (d/4)) and rows r = t / (d/4) + RP*n; each row of the state is read
// with float4 loads by d/4 consecutive lanes (coalesced 512 B rows for
// d = 128).  Row partial sums of o are combined through LDS.

#include "la_device.h"
#include "la_internal.h"

namespace la {
namespace {

constexpr int kThreads = 256;

template <typename InT>
__device__ __forceinline__ float load_in(const InT* p, int64_t i);
template <>
__device__ __forceinline__ float load_in<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_in<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_bits_to_f32(p[i]);
}

template <typename InT>
__device__ __forceinline__ void store_o(InT* p, int64_t i, floatx4 x);
template <>
__device__ __forceinline__ void store_o<float>(float* p, int64_t i, floatx4 x) {
  *reinterpret_cast<float4*>(p + i) = make_float4(x[0], x[1], x[2], x[3]);
}
template <>
__device__ __forceinline__ void store_o<uint16_t>(uint16_t* p, int64_t i, floatx4 x) {
  *reinterpret_cast<uint2*>(p + i) = make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
}

template <int D, typename InT, bool kNorm>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
  constexpr int CQ = D / 4;         // column quads per row
  constexpr int RP = kThreads / CQ;  // rows handled concurrently
  constexpr int NR = D / RP;         // rows per thread
  __shared__ float qs[D], ks[D];
  __shared__ floatx4 red[RP][CQ];

  const int h = blockIdx.x % a.num_heads;
  const int b = (int)((int64_t)(blockIdx.x / a.num_heads) * a.b_step % a.batch);
  const int64_t slot = a.slots ? a.slots[b] : b;  // validated on the host
  const int t = threadIdx.x;
  const int cq = t % CQ;
  const int rp = t / CQ;
  const int64_t vec_off = ((int64_t)b * a.num_heads + h) * D;
  const InT* __restrict__ q = static_cast<const InT*>(a.q);
  const InT* __restrict__ k = static_cast<const InT*>(a.k);
  const InT* __restrict__ v = static_cast<const InT*>(a.v);
  floatx4* __restrict__ S = reinterpret_cast<floatx4*>(a.kv + (slot * a.num_heads + h) * D * D);

  // Issue the whole state stream first (NR independent 16 B loads/thread).
  floatx4 sv[NR];
#pragma unroll
  for (int n = 0; n < NR; ++n)
    sv[n] = __builtin_nontemporal_load(&S[(rp + RP * n) * CQ + cq]);

  if (t < D) {
    qs[t] = load_in(q, vec_off + t);
    ks[t] = load_in(k, vec_off + t);
  }
  floatx4 vv;
#pragma unroll
  for (int m = 0; m < 4; ++m) vv[m] = load_in(v, vec_off + 4 * cq + m);
  const float lam = a.decay[h];
  __syncthreads();

  floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int n = 0; n < NR; ++n) {
    const int r = rp + RP * n;
    const float kr = ks[r], qr = qs[r];
    floatx4 s;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      s[m] = fmaf(lam, sv[n][m], kr * vv[m]);
      acc[m] = fmaf(qr, s[m], acc[m]);
    }
    __builtin_nontemporal_store(s, &S[r * CQ + cq]);
  }
  red[rp][cq] = acc;
  __syncthreads();
  if (t < 64) {  // wave 0: lane t < CQ completes columns 4t .. 4t + 3
    floatx4 o = {0.0f, 0.0f, 0.0f, 0.0f};
    if (t < CQ) {
      o = red[0][t];
#pragma unroll
      for (int p = 1; p < RP; ++p) o += red[p][t];
    }
    if constexpr (kNorm) {
      float ss = o[0] * o[0] + o[1] * o[1] + o[2] * o[2] + o[3] * o[3];  // 0 past the row
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
      const float inv = rsqrtf(ss * (1.0f / D) + a.norm_eps);
      if (t < CQ) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          float f = inv * a.norm_weight[h * D + 4 * t + m];
          if (a.gate)
            f *= __builtin_amdgcn_rcpf(
                1.0f + __builtin_amdgcn_exp2f(
                           -1.4426950408889634f *
                           load_in(static_cast<const InT*>(a.gate), vec_off + 4 * t + m)));
          o[m] *= f;
        }
      }
    }
    if (t < CQ) store_o(static_cast<InT*>(a.o), vec_off + 4 * t, o);
  }
}

template <int D, bool kNorm>
hipError_t launch_d(const DecodeArgs& a, la_dtype in_dtype, hipStream_t stream) {
  const dim3 grid((unsigned)a.batch * (unsigned)a.num_heads), block(kThreads);
  if (in_dtype == LA_FP32)
    hipLaunchKernelGGL((decode_kernel<D, float, kNorm>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((decode_kernel<D, uint16_t, kNorm>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int head_dim, la_dtype in_dtype,
                         hipStream_t stream) {
  const bool norm = a.norm_weight != nullptr;
  if (head_dim == 64)
    return norm ? launch_d<64, true>(a, in_dtype, stream) : launch_d<64, false>(a, in_dtype, stream);
  return norm ? launch_d<128, true>(a, in_dtype, stream) : launch_d<128, false>(a, in_dtype, stream);
}

}  // namespace la
