// bf16 prefill kernel for gfx950: blockwise causal linear attention with
// per-head decay on bf16 MFMA (v_mfma_f32_16x16x32_bf16), fp32 accumulation
// and an fp32 state carried in registers along each chain.
//
// Method (emonzhong.com "MiniMax-01: Scaling Foundation Models with Lightning
// Attention" 方法要点; CSDN "【AI论文】MiniMax-01:利用闪电注意力机制扩展基础模型"
// §2.1; mizuki blog "MiniMax-01：4M 上下文破局" 关键概念清单): the tokens of
// one (sequence, head) are cut into blocks of BETA = 64.  For block b with
// ell valid rows and local indices i, j:
//   P      = (Q_b K_b^T) .* M,  M[i][j] = lambda^(i-j) for i >= j, else 0
//   O_b    = P V_b + diag(lambda^(i+1)) Q_b S_b          (left + right product)
//   S_b+1  = lambda^ell S_b + (diag(lambda^(ell-1-j)) K_b)^T V_b
// The per-token cumsum is replaced by this per-block state chain.
//
// Decomposition: one workgroup (4 waves) owns one (sequence, head, 32-column
// slice of the value dimension) chain; the d x d state is split by value
// columns over d/32 workgroups, each of which recomputes Q K^T for its block
// (cheap next to the HBM stream) so that no cross-workgroup exchange exists.
//
// Rounding: P, the state as the MFMA operand of Q S, and the decayed K rows
// are rounded to bf16 (round to nearest even); all sums are fp32; the state
// itself stays fp32 and is written out in fp32.
//
// LDS tiles (bf16 bits):
//   Qs, Ks [64][d+8]   row-major, padded rows (conflict-free 16 B reads)
//   KTs    [d][64]     decayed K^T; 4-element chunks XOR-swizzled per row
//   VTs    [32][64]    V^T of the slice; same swizzle
//   Ps     [64][72]    masked, decayed scores
//   STs    [2][32][d+8]  state^T (bf16) for the Q S product, double-buffered
// MFMA operand layout (16x16x32 bf16): lane l supplies row (l % 16) of A and
// column (l % 16) of B, with 8 consecutive k at k = 8 * (l / 16); the 4
// results of lane l sit at rows 4 * (l / 16) + m, column l % 16.

#include "la_device.h"
#include "la_internal.h"

namespace la {
namespace {

constexpr int kBeta = 64;
constexpr int kThreads = 256;
constexpr int kDV = kBf16Cols;  // 32 value columns per workgroup
constexpr int kPS = kBeta + 8;  // Ps row stride

// Lower-triangular 16x16 tiles (ti >= tj) of the 64x64 score block.
__constant__ int8_t kTileI[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
__constant__ int8_t kTileJ[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};

__device__ __forceinline__ int swz(int row) { return (row + (row >> 3)) & 15; }

// Offset (in elements) of 4-element chunk `jc` of row `row` in a [rows][64]
// swizzled transposed tile.
__device__ __forceinline__ int tpos(int row, int jc) { return row * kBeta + ((jc ^ swz(row)) << 2); }

__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// 8 consecutive elements j = 8*jc2 .. 8*jc2+7 of a row of a swizzled tile.
__device__ __forceinline__ bf16x8 ld8_t(const uint16_t* base, int row, int jc2) {
  const uint2 lo = *reinterpret_cast<const uint2*>(base + tpos(row, 2 * jc2));
  const uint2 hi = *reinterpret_cast<const uint2*>(base + tpos(row, 2 * jc2 + 1));
  const uint4 w = {lo.x, lo.y, hi.x, hi.y};
  return __builtin_bit_cast(bf16x8, w);
}

__device__ __forceinline__ uint32_t word_of(const uint4& w, int i) {
  return i == 0 ? w.x : i == 1 ? w.y : i == 2 ? w.z : w.w;
}

// Element e (0..7) of 8 packed bf16 as float.
__device__ __forceinline__ float elem(const uint4& w, int e) {
  const uint32_t x = word_of(w, e >> 1);
  return (e & 1) ? bf16_hi(x) : bf16_lo(x);
}

__device__ __forceinline__ floatx4 mfma(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int D, bool kOutF32>
__global__ __launch_bounds__(kThreads) void prefill_bf16_kernel(PrefillArgs a) {
  constexpr int NDV = D / kDV;
  constexpr int QS = D + 8;      // Qs/Ks row stride
  constexpr int SS = D + 8;      // STs row stride
  constexpr int CH = D / 8;      // 16 B chunks per Q/K row
  constexpr int KSTAGE = CH * 16;  // threads staging Q/K (4 rows each)
  constexpr int NST = D / 32;    // state tiles per wave (and k-steps over d)

  __shared__ __attribute__((aligned(16))) uint16_t Qs[kBeta * QS];
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kBeta * QS];
  __shared__ __attribute__((aligned(16))) uint16_t KTs[D * kBeta];
  __shared__ __attribute__((aligned(16))) uint16_t VTs[kDV * kBeta];
  __shared__ __attribute__((aligned(16))) uint16_t Ps[kBeta * kPS];
  __shared__ __attribute__((aligned(16))) uint16_t STs[2][kDV * SS];
  __shared__ float pw[kBeta + 1];

  const int H = a.num_heads;
  const int item = xcd_remap(blockIdx.x, a.num_items, NDV);
  const int cs = item % NDV;
  const int sh = item / NDV;
  const int h = sh % H;
  const int s = sh / H;
  const int c0 = cs * kDV;
  const int t = threadIdx.x;
  const int w = t >> 6;
  const int l = t & 63;
  const int li = l & 15;
  const int g = l >> 4;
  const int tc = w & 1;  // value-column tile (of 2) this wave owns

  const int64_t start = a.cu_seqlens[s];
  const int64_t end = a.cu_seqlens[s + 1];
  const uint16_t* __restrict__ q = static_cast<const uint16_t*>(a.q);
  const uint16_t* __restrict__ k = static_cast<const uint16_t*>(a.k);
  const uint16_t* __restrict__ v = static_cast<const uint16_t*>(a.v);
  const int64_t state_off = ((int64_t)s * H + h) * D * D;
  const int64_t row_stride = (int64_t)H * D;  // elements between tokens

  if (t <= kBeta) pw[t] = exp2f((float)t * a.log2_decay[h]);
  // Strictly-upper tiles (0,1) and (2,3) are read by the P V product but never
  // produced; they stay zero.
  for (int idx = t; idx < 2 * 16 * 16; idx += kThreads) {
    const int tile = idx >> 8, e = idx & 255;
    const int i = (tile ? 32 : 0) + (e >> 4), j = (tile ? 48 : 16) + (e & 15);
    Ps[i * kPS + j] = 0;
  }

  // fp32 state in registers: tile n covers rows 16*tr.., tr = (w>>1) + 2n,
  // columns 16*tc..; lane holds rows 16tr+4g+m, column 16tc+li.
  floatx4 st[NST];
#pragma unroll
  for (int n = 0; n < NST; ++n) {
    const int tr = (w >> 1) + 2 * n;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int r = 16 * tr + 4 * g + m;
      st[n][m] = a.kv_init ? a.kv_init[state_off + (int64_t)r * D + c0 + 16 * tc + li] : 0.0f;
    }
  }
  __syncthreads();  // pw ready
  // bf16 copy of the initial state (transposed) for the first Q S product.
#pragma unroll
  for (int n = 0; n < NST; ++n) {
    const int tr = (w >> 1) + 2 * n;
    uint2 pk = {pack_bf16x2(st[n][0], st[n][1]), pack_bf16x2(st[n][2], st[n][3])};
    *reinterpret_cast<uint2*>(&STs[0][(16 * tc + li) * SS + 16 * tr + 4 * g]) = pk;
  }

  // Staging roles.  Q/K: thread t < KSTAGE loads rows 4*krg..4*krg+3, 16 B
  // chunk kch.  V: thread t < 64 loads rows 4*vrg..+3, chunk vch of the slice.
  const int kch = t % CH;
  const int krg = t / CH;
  const int vch = t & 3;
  const int vrg = t >> 2;
  uint4 qreg[4], kreg[4], vreg[4];

  auto load_block = [&](int64_t b0, int ell) {
    if (t < KSTAGE) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int row = 4 * krg + p;
        if (row < ell) {
          const int64_t off = (b0 + row) * row_stride + (int64_t)h * D + 8 * kch;
          qreg[p] = *reinterpret_cast<const uint4*>(q + off);
          kreg[p] = *reinterpret_cast<const uint4*>(k + off);
        } else {
          qreg[p] = make_uint4(0, 0, 0, 0);
          kreg[p] = make_uint4(0, 0, 0, 0);
        }
      }
    }
    if (t < 64) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int row = 4 * vrg + p;
        vreg[p] = row < ell ? *reinterpret_cast<const uint4*>(
                                  v + (b0 + row) * row_stride + (int64_t)h * D + c0 + 8 * vch)
                            : make_uint4(0, 0, 0, 0);
      }
    }
  };

  int64_t b0 = start;
  int ell = (int)((end - b0) < kBeta ? (end - b0) : kBeta);
  if (b0 < end) load_block(b0, ell);

  for (int bi = 0; b0 < end; ++bi) {
    const int cur = bi & 1;
    __syncthreads();  // previous block finished reading the staged tiles

    // ---- stage block b0 into LDS ----
    if (t < KSTAGE) {
      float kd[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int row = 4 * krg + p;
        kd[p] = row < ell ? pw[row < ell ? ell - 1 - row : 0] : 0.0f;
        *reinterpret_cast<uint4*>(&Qs[row * QS + 8 * kch]) = qreg[p];
        *reinterpret_cast<uint4*>(&Ks[row * QS + 8 * kch]) = kreg[p];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = 8 * kch + e;
        uint2 pk = {pack_bf16x2(elem(kreg[0], e) * kd[0], elem(kreg[1], e) * kd[1]),
                    pack_bf16x2(elem(kreg[2], e) * kd[2], elem(kreg[3], e) * kd[3])};
        *reinterpret_cast<uint2*>(&KTs[tpos(r, krg)]) = pk;
      }
    }
    if (t < 64) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = 8 * vch + e;
        const uint32_t e0 = (word_of(vreg[0], e >> 1) >> ((e & 1) * 16)) & 0xFFFFu;
        const uint32_t e1 = (word_of(vreg[1], e >> 1) >> ((e & 1) * 16)) & 0xFFFFu;
        const uint32_t e2 = (word_of(vreg[2], e >> 1) >> ((e & 1) * 16)) & 0xFFFFu;
        const uint32_t e3 = (word_of(vreg[3], e >> 1) >> ((e & 1) * 16)) & 0xFFFFu;
        *reinterpret_cast<uint2*>(&VTs[tpos(c, vrg)]) = make_uint2(e0 | (e1 << 16), e2 | (e3 << 16));
      }
    }

    // ---- prefetch the next block into registers ----
    const int64_t nb0 = b0 + kBeta;
    const int nell = nb0 < end ? (int)((end - nb0) < kBeta ? (end - nb0) : kBeta) : 0;
    if (nb0 < end) load_block(nb0, nell);
    __syncthreads();

    // ---- scores: S^T tiles -> masked, decayed P (bf16) ----
    for (int n = 0; n < 3; ++n) {
      const int idx = w + 4 * n;
      if (idx >= 10) break;
      const int ti = kTileI[idx], tj = kTileJ[idx];
      floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk)
        acc = mfma(ld8(&Ks[(16 * tj + li) * QS + 32 * kk + 8 * g]),
                   ld8(&Qs[(16 * ti + li) * QS + 32 * kk + 8 * g]), acc);
      const int i = 16 * ti + li;
      float p[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int j = 16 * tj + 4 * g + m;
        p[m] = j <= i ? acc[m] * pw[i >= j ? i - j : 0] : 0.0f;
      }
      *reinterpret_cast<uint2*>(&Ps[i * kPS + 16 * tj + 4 * g]) =
          make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]));
    }
    __syncthreads();

    // ---- output tiles: O^T = V^T P^T + diag-scaled S^T Q^T ----
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int ti = n == 0 ? (w >> 1) : 3 - (w >> 1);
      floatx4 acc_a = {0.0f, 0.0f, 0.0f, 0.0f};
      floatx4 acc_b = {0.0f, 0.0f, 0.0f, 0.0f};
      const int nk = ti >= 2 ? 2 : 1;
      for (int kk = 0; kk < nk; ++kk)
        acc_a = mfma(ld8_t(VTs, 16 * tc + li, 4 * kk + g),
                     ld8(&Ps[(16 * ti + li) * kPS + 32 * kk + 8 * g]), acc_a);
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk)
        acc_b = mfma(ld8(&STs[cur][(16 * tc + li) * SS + 32 * kk + 8 * g]),
                     ld8(&Qs[(16 * ti + li) * QS + 32 * kk + 8 * g]), acc_b);
      const int i = 16 * ti + li;
      if (i < ell) {
        const float f = pw[i + 1];
        float out[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) out[m] = fmaf(f, acc_b[m], acc_a[m]);
        const int64_t off = (b0 + i) * row_stride + (int64_t)h * D + c0 + 16 * tc + 4 * g;
        if constexpr (kOutF32) {
          *reinterpret_cast<float4*>(static_cast<float*>(a.o) + off) =
              make_float4(out[0], out[1], out[2], out[3]);
        } else {
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.o) + off) =
              make_uint2(pack_bf16x2(out[0], out[1]), pack_bf16x2(out[2], out[3]));
        }
      }
    }

    // ---- state: S <- lambda^ell S + Kd^T V, then its bf16 copy ----
    const float fl = pw[ell];
#pragma unroll
    for (int n = 0; n < NST; ++n) {
      const int tr = (w >> 1) + 2 * n;
      floatx4 acc = st[n] * fl;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        acc = mfma(ld8_t(KTs, 16 * tr + li, 4 * kk + g), ld8_t(VTs, 16 * tc + li, 4 * kk + g),
                   acc);
      st[n] = acc;
      *reinterpret_cast<uint2*>(&STs[cur ^ 1][(16 * tc + li) * SS + 16 * tr + 4 * g]) =
          make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
    }

    b0 = nb0;
    ell = nell;
  }

  if (a.kv_final) {
#pragma unroll
    for (int n = 0; n < NST; ++n) {
      const int tr = (w >> 1) + 2 * n;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int r = 16 * tr + 4 * g + m;
        a.kv_final[state_off + (int64_t)r * D + c0 + 16 * tc + li] = st[n][m];
      }
    }
  }
}

template <int D>
hipError_t launch_d(const PrefillArgs& a, la_dtype out_dtype, hipStream_t stream) {
  const dim3 grid(a.num_items), block(kThreads);
  if (out_dtype == LA_FP32)
    hipLaunchKernelGGL((prefill_bf16_kernel<D, true>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((prefill_bf16_kernel<D, false>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, int head_dim, la_dtype out_dtype,
                               hipStream_t stream) {
  if (head_dim == 64) return launch_d<64>(a, out_dtype, stream);
  return launch_d<128>(a, out_dtype, stream);
}

}  // namespace la
