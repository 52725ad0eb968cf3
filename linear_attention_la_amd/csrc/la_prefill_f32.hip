// fp32 prefill kernel: blockwise causal linear attention with per-head decay,
// all arithmetic in fp32 FMA (no reduced-precision products).
//
// This is the path for fp32 inputs, whose results must stay within ~1e-5
// relative of the exact value; it favours plain, exact-order fp32 over speed.
// The bf16 path (la_prefill_bf16.hip) is the fast one.
//
// Method: per (sequence, head) the tokens are cut into blocks of BETA; inside
// a block the masked, decayed left product (Q K^T .* M) V is formed, and the
// carried d x d state contributes Q S (right product) before being advanced
// by K^T V (emonzhong.com "MiniMax-01: Scaling Foundation Models with
// Lightning Attention" 方法要点; mizuki blog "MiniMax-01：4M 上下文破局"
// 关键概念清单).  One workgroup owns one (sequence, head, 32-column slice of
// the state) chain and walks its blocks in order.

#include "la_device.h"
#include "la_internal.h"

namespace la {
namespace {

constexpr int kBeta = 32;
constexpr int kThreads = 256;

template <typename OutT>
__device__ __forceinline__ void store_out(OutT* p, float x);
template <>
__device__ __forceinline__ void store_out<float>(float* p, float x) { *p = x; }
template <>
__device__ __forceinline__ void store_out<uint16_t>(uint16_t* p, float x) {
  *p = f32_to_bf16_bits(x);
}

template <int D, typename OutT>
__global__ __launch_bounds__(kThreads) void prefill_f32_kernel(PrefillArgs a) {
  constexpr int DV = kF32Cols;
  constexpr int NDV = D / DV;
  __shared__ float Qs[kBeta][D + 1];
  __shared__ float Ks[kBeta][D + 1];
  __shared__ float Vs[kBeta][DV + 1];
  __shared__ float Ps[kBeta][kBeta + 1];
  __shared__ float St[D][DV + 1];
  __shared__ float pw[kBeta + 1];  // lambda^n, n = 0..kBeta

  const int item = xcd_remap(blockIdx.x, a.num_items, NDV);
  const int cs = item % NDV;
  const int sh = item / NDV;
  const int h = sh % a.num_heads;
  const int s = seq_of(a, sh / a.num_heads);
  const int t = threadIdx.x;
  const int H = a.num_heads;
  const int c0 = cs * DV;
  const int64_t start = a.cu_seqlens[s];
  const int64_t end = a.cu_seqlens[s + 1];
  const float* __restrict__ q = static_cast<const float*>(a.q);
  const float* __restrict__ k = static_cast<const float*>(a.k);
  const float* __restrict__ v = static_cast<const float*>(a.v);
  OutT* __restrict__ o = static_cast<OutT*>(a.o);
  const int64_t state_off = ((int64_t)s * H + h) * D * D;

  if (t <= kBeta) pw[t] = exp2f((float)t * a.log2_decay[h]);
  for (int idx = t; idx < D * DV; idx += kThreads) {
    const int r = idx / DV, c = idx % DV;
    St[r][c] = a.kv_init ? a.kv_init[state_off + (int64_t)r * D + c0 + c] : 0.0f;
  }
  __syncthreads();

  for (int64_t b0 = start; b0 < end; b0 += kBeta) {
    const int ell = (int)((end - b0) < kBeta ? (end - b0) : kBeta);
    // Stage the block (rows past the end of the sequence are zero).
    for (int idx = t; idx < kBeta * D; idx += kThreads) {
      const int row = idx / D, col = idx % D;
      float qv = 0.0f, kv = 0.0f;
      if (row < ell) {
        const int64_t off = ((b0 + row) * H + h) * (int64_t)D + col;
        qv = q[off];
        kv = k[off];
      }
      Qs[row][col] = qv;
      Ks[row][col] = kv;
    }
    for (int idx = t; idx < kBeta * DV; idx += kThreads) {
      const int row = idx / DV, col = idx % DV;
      Vs[row][col] = row < ell ? v[((b0 + row) * H + h) * (int64_t)D + c0 + col] : 0.0f;
    }
    __syncthreads();

    // Intra-block scores with the causal decay mask.
    for (int idx = t; idx < kBeta * kBeta; idx += kThreads) {
      const int i = idx / kBeta, j = idx % kBeta;
      float p = 0.0f;
      if (j <= i) {
        float acc = 0.0f;
#pragma unroll 8
        for (int r = 0; r < D; ++r) acc = fmaf(Qs[i][r], Ks[j][r], acc);
        p = acc * pw[i - j];
      }
      Ps[i][j] = p;
    }
    __syncthreads();

    // Output: intra (P V) + lambda^(i+1) * inter (Q S).
    for (int idx = t; idx < kBeta * DV; idx += kThreads) {
      const int i = idx / DV, c = idx % DV;
      if (i < ell) {
        float intra = 0.0f;
        for (int j = 0; j <= i; ++j) intra = fmaf(Ps[i][j], Vs[j][c], intra);
        float inter = 0.0f;
#pragma unroll 8
        for (int r = 0; r < D; ++r) inter = fmaf(Qs[i][r], St[r][c], inter);
        store_out(o + ((b0 + i) * H + h) * (int64_t)D + c0 + c, fmaf(pw[i + 1], inter, intra));
      }
    }
    __syncthreads();

    // State: S <- lambda^ell S + (diag(lambda^(ell-1-j)) K)^T V.
    const float fl = pw[ell];
    for (int idx = t; idx < D * DV; idx += kThreads) {
      const int r = idx / DV, c = idx % DV;
      float acc = 0.0f;
      for (int j = 0; j < ell; ++j) acc = fmaf(Ks[j][r] * pw[ell - 1 - j], Vs[j][c], acc);
      St[r][c] = fmaf(fl, St[r][c], acc);
    }
    __syncthreads();
  }

  if (a.kv_final) {
    for (int idx = t; idx < D * DV; idx += kThreads) {
      const int r = idx / DV, c = idx % DV;
      a.kv_final[state_off + (int64_t)r * D + c0 + c] = St[r][c];
    }
  }
}

template <int D>
hipError_t launch_d(const PrefillArgs& a, la_dtype out_dtype, hipStream_t stream) {
  const dim3 grid(a.num_items), block(kThreads);
  if (out_dtype == LA_FP32)
    hipLaunchKernelGGL((prefill_f32_kernel<D, float>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((prefill_f32_kernel<D, uint16_t>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs& a, int head_dim, la_dtype out_dtype,
                              hipStream_t stream) {
  if (head_dim == 64) return launch_d<64>(a, out_dtype, stream);
  return launch_d<128>(a, out_dtype, stream);
}

}  // namespace la
