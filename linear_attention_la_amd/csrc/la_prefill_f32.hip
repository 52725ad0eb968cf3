// fp32 prefill kernel: blockwise causal linear attention with per-head decay,
// every product and sum in fp32 (no reduced-precision operands).
//
// This is the path for fp32 inputs, whose results must stay within ~1e-5
// relative of the exact value.  Its contractions run on the fp32 matrix
// cores (v_mfma_f32_16x16x4_f32: fp32 operands, fp32 accumulation), which
// keep fp32 precision at twice the rate of unpacked fp32 FMA.  The bf16 path
// (la_prefill_bf16.hip) is the fast one.
//
// Method: per (sequence, head) the tokens are cut into blocks of BETA; inside
// a block the masked, decayed left product (Q K^T .* M) V is formed, and the
// carried d x d state contributes Q S (right product) before being advanced
// by K^T V (emonzhong.com "MiniMax-01: Scaling Foundation Models with
// Lightning Attention" 方法要点; mizuki blog "MiniMax-01：4M 上下文破局"
// 关键概念清单).  One workgroup of four waves owns one (sequence, head,
// 32-column slice of the state) chain and walks its blocks in order; the
// next block's rows load into registers while the current block computes.
//
// MFMA operand layout (16 x 16 x 4, wave64): lane l supplies A[l % 16][l / 16]
// and B[l / 16][l % 16] and receives D[4 (l / 16) + r][l % 16], r = 0..3.

#include <type_traits>

#include "la_device.h"
#include "la_internal.h"

namespace la {
namespace {

constexpr int kBeta = 32;
constexpr int kThreads = 256;  // four waves
constexpr int kPad = 4;        // LDS row padding (floats); keeps rows 16 B aligned

__device__ __forceinline__ floatx4 mfma4(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

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
  constexpr int QF = kBeta * D / 4 / kThreads;   // float4 of Q (and of K) per thread
  constexpr int VF = kBeta * DV / 4 / kThreads;  // float4 of V per thread
  static_assert(QF >= 1 && VF == 1 && DV == 32 && kBeta == 32, "tile shapes");
  // Q and K rows as loaded; V and the state slice transposed (row = value
  // column), so that every MFMA operand is a 16-byte read along the
  // reduction index.  Reductions take their index in the order
  // 16 c + 4 (l / 16) + e for element e of lane l's 16-byte piece of chunk c:
  // a permutation of the index, the same for A and B, so each product sum
  // is unchanged.
  __shared__ __attribute__((aligned(16))) float Qs[kBeta][D + kPad];
  __shared__ __attribute__((aligned(16))) float Ks[kBeta][D + kPad];
  __shared__ __attribute__((aligned(16))) float Vt[DV][kBeta + kPad];
  __shared__ __attribute__((aligned(16))) float Ps[kBeta][kBeta + kPad];
  __shared__ __attribute__((aligned(16))) float St[DV][D + kPad];  // S^T slice
  __shared__ float pw[kBeta + 1];  // lambda^n, n = 0..kBeta

  const int item = xcd_remap(blockIdx.x, a.num_items, NDV);
  const int cs = item % NDV;
  const int sh = item / NDV;
  const int h = sh % a.num_heads;
  const int s = seq_of(a, sh / a.num_heads);
  const int t = threadIdx.x;
  const int wave = t >> 6;
  const int lr = t & 15;         // operand row (A) / column (B, D) within a tile
  const int lk = (t >> 4) & 3;   // operand reduction lane group; D rows 4 lk .. 4 lk + 3
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
    St[c][r] = a.kv_init ? a.kv_init[state_off + (int64_t)r * D + c0 + c] : 0.0f;
  }

  // Rows of one block in registers: thread t holds float4 number t + n kThreads
  // of the block's Q and K rows (row-major, D / 4 per row) and float4 t of its
  // V slice (8 per row).  Rows past the sequence end are zero.
  float4 rq[QF], rk[QF], rv;
  auto load = [&](int64_t b0) {
    const int ell = (int)((end - b0) < kBeta ? (end - b0) : kBeta);
#pragma unroll
    for (int n = 0; n < QF; ++n) {
      const int f = t + n * kThreads, row = f / (D / 4), c4 = f % (D / 4);
      const int64_t off = ((b0 + row) * H + h) * (int64_t)D + 4 * c4;
      rq[n] = row < ell ? *reinterpret_cast<const float4*>(q + off) : make_float4(0, 0, 0, 0);
      rk[n] = row < ell ? *reinterpret_cast<const float4*>(k + off) : make_float4(0, 0, 0, 0);
    }
    const int row = t / (DV / 4), c4 = t % (DV / 4);
    const int64_t off = ((b0 + row) * H + h) * (int64_t)D + c0 + 4 * c4;
    rv = row < ell ? *reinterpret_cast<const float4*>(v + off) : make_float4(0, 0, 0, 0);
  };
  if (start < end) load(start);

  // The state update of a block, S <- lambda^ell S + (diag(lambda^(ell-1-j))
  // K)^T V, is accumulated in registers while the block's scores and
  // outputs are formed (wave 3, idle for the scores, takes the first four
  // 16 x 16 tiles of the D x 32 slice then; every wave takes NB more with
  // the outputs), and written back to LDS with the next block's rows, so a
  // block needs three barriers.
  constexpr int NT = (D / 16) * 2;  // state tiles of the slice
  constexpr int NB = (NT - 4) / 4;  // tiles per wave with the outputs
  floatx4 accA[4], accB[NB];
  float fl = 1.0f;
  bool pending = false;
  // Accumulate the updates of N tiles (tile -> key-row tile tr = tile / 2,
  // value-column tile tc = tile % 2) together, so that consecutive MFMAs
  // are independent.
  auto state_tiles = [&](auto n_tiles, int first, floatx4* acc, const float* wj) {
    constexpr int N = decltype(n_tiles)::value;
#pragma unroll
    for (int n = 0; n < N; ++n) acc[n] = floatx4{0, 0, 0, 0};
#pragma unroll
    for (int jc = 0; jc < kBeta; jc += 16) {
      float4 y[2];
      y[0] = *reinterpret_cast<const float4*>(&Vt[lr][jc + 4 * lk]);
      y[1] = *reinterpret_cast<const float4*>(&Vt[16 + lr][jc + 4 * lk]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float* kr = &Ks[jc + 4 * lk + e][0];
#pragma unroll
        for (int n = 0; n < N; ++n) {
          const int tile = first + n, tr = tile >> 1, tc = tile & 1;
          const float ye = e == 0 ? y[tc].x : e == 1 ? y[tc].y : e == 2 ? y[tc].z : y[tc].w;
          acc[n] = mfma4(kr[16 * tr + lr] * wj[jc / 4 + e], ye, acc[n]);
        }
      }
    }
  };
  auto write_tile = [&](int tile, const floatx4& acc) {
    const int tr = tile >> 1, tc = tile & 1;
    float4* p = reinterpret_cast<float4*>(&St[16 * tc + lr][16 * tr + 4 * lk]);
    float4 x = *p;
    x.x = fmaf(fl, x.x, acc[0]);
    x.y = fmaf(fl, x.y, acc[1]);
    x.z = fmaf(fl, x.z, acc[2]);
    x.w = fmaf(fl, x.w, acc[3]);
    *p = x;
  };
  auto write_state = [&]() {
    if (wave == 3) {
#pragma unroll
      for (int n = 0; n < 4; ++n) write_tile(n, accA[n]);
    }
#pragma unroll
    for (int n = 0; n < NB; ++n) write_tile(4 + wave * NB + n, accB[n]);
  };

  for (int64_t b0 = start; b0 < end; b0 += kBeta) {
    const int ell = (int)((end - b0) < kBeta ? (end - b0) : kBeta);
    if (pending) write_state();  // the previous block's update
#pragma unroll
    for (int n = 0; n < QF; ++n) {
      const int f = t + n * kThreads, row = f / (D / 4), c4 = f % (D / 4);
      *reinterpret_cast<float4*>(&Qs[row][4 * c4]) = rq[n];
      *reinterpret_cast<float4*>(&Ks[row][4 * c4]) = rk[n];
    }
    {
      const int row = t / (DV / 4), c4 = t % (DV / 4);
      Vt[4 * c4 + 0][row] = rv.x;
      Vt[4 * c4 + 1][row] = rv.y;
      Vt[4 * c4 + 2][row] = rv.z;
      Vt[4 * c4 + 3][row] = rv.w;
    }
    __syncthreads();
    if (b0 + kBeta < end) load(b0 + kBeta);

    // This lane's weights lambda^(ell-1-j) for its eight reduction indices j
    // of the state update (rows j >= ell of K are zero, so their weight only
    // has to be finite).
    float wj[kBeta / 4];
#pragma unroll
    for (int n = 0; n < kBeta / 4; ++n)
      wj[n] = pw[max(ell - 1 - (16 * (n / 4) + 4 * lk + n % 4), 0)];

    // Intra-block scores with the causal decay mask, one 16 x 16 tile per
    // wave for the three tiles on or below the diagonal (the tile above it
    // is never read); wave 3 meanwhile accumulates four state tiles.
    if (wave < 3) {
      const int ti = wave == 0 ? 0 : 1, tj = wave == 2 ? 1 : 0;
      floatx4 a0 = {0, 0, 0, 0}, a1 = a0, a2 = a0, a3 = a0;
#pragma unroll
      for (int kc = 0; kc < D; kc += 16) {
        const float4 x = *reinterpret_cast<const float4*>(&Qs[16 * ti + lr][kc + 4 * lk]);
        const float4 y = *reinterpret_cast<const float4*>(&Ks[16 * tj + lr][kc + 4 * lk]);
        a0 = mfma4(x.x, y.x, a0);
        a1 = mfma4(x.y, y.y, a1);
        a2 = mfma4(x.z, y.z, a2);
        a3 = mfma4(x.w, y.w, a3);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * ti + 4 * lk + r, j = 16 * tj + lr;
        const float f = pw[max(i - j, 0)];
        Ps[i][j] = j <= i ? ((a0[r] + a1[r]) + (a2[r] + a3[r])) * f : 0.0f;
      }
    } else {
      state_tiles(std::integral_constant<int, 4>(), 0, accA, wj);
    }
    __syncthreads();

    // Output: intra (P V) + lambda^(i+1) * inter (Q S), one 16 x 16 tile of
    // (query rows, value columns) per wave; then this wave's NB state tiles.
    {
      const int ti = wave >> 1, tc = wave & 1;
      const floatx4 z = {0, 0, 0, 0};
      floatx4 oi[4] = {z, z, z, z}, oe[4] = {z, z, z, z};
#pragma unroll
      for (int jc = 0; jc < 32; jc += 16) {
        if (jc > 16 * ti) break;
        const float4 x = *reinterpret_cast<const float4*>(&Ps[16 * ti + lr][jc + 4 * lk]);
        const float4 y = *reinterpret_cast<const float4*>(&Vt[16 * tc + lr][jc + 4 * lk]);
        oi[0] = mfma4(x.x, y.x, oi[0]);
        oi[1] = mfma4(x.y, y.y, oi[1]);
        oi[2] = mfma4(x.z, y.z, oi[2]);
        oi[3] = mfma4(x.w, y.w, oi[3]);
      }
#pragma unroll
      for (int kc = 0; kc < D; kc += 16) {
        const float4 x = *reinterpret_cast<const float4*>(&Qs[16 * ti + lr][kc + 4 * lk]);
        const float4 y = *reinterpret_cast<const float4*>(&St[16 * tc + lr][kc + 4 * lk]);
        oe[0] = mfma4(x.x, y.x, oe[0]);
        oe[1] = mfma4(x.y, y.y, oe[1]);
        oe[2] = mfma4(x.z, y.z, oe[2]);
        oe[3] = mfma4(x.w, y.w, oe[3]);
      }
      state_tiles(std::integral_constant<int, NB>(), 4 + wave * NB, accB, wj);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * ti + 4 * lk + r;
        if (i < ell)
          store_out(o + ((b0 + i) * H + h) * (int64_t)D + c0 + 16 * tc + lr,
                    fmaf(pw[i + 1], (oe[0][r] + oe[1][r]) + (oe[2][r] + oe[3][r]),
                         (oi[0][r] + oi[1][r]) + (oi[2][r] + oi[3][r])));
      }
    }
    fl = pw[ell];
    pending = true;
    __syncthreads();
  }
  if (pending) {
    write_state();
    __syncthreads();
  }

  if (a.kv_final) {
    for (int idx = t; idx < D * DV; idx += kThreads) {
      const int r = idx / DV, c = idx % DV;
      a.kv_final[state_off + (int64_t)r * D + c0 + c] = St[c][r];
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
