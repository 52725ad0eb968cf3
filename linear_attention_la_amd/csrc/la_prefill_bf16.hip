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
//   S_b+1  = lambda^ell S_b + K_b^T diag(lambda^(ell-1-j)) V_b
// The per-token cumsum is replaced by this per-block state chain.
//
// Decomposition.  One workgroup (4 waves) owns one (sequence, head, 32-column
// slice of the value dimension) chain; the d x d state is split by value
// columns over d/32 workgroups, each of which recomputes Q K^T for its block
// so that no cross-workgroup exchange exists.  Inside a block, wave w owns
// the query strip i in [16w, 16w+16): it forms its strip of scores
// S^T = K Q^T, applies the mask and decay in registers, and feeds them
// straight back into the MFMA as the B operand of O^T = V^T P^T (the score
// tile's accumulator layout -- 4 consecutive keys per lane -- is a valid
// operand layout when the value operand uses the same key order), then adds
// diag(lambda^(i+1)) (S^T Q^T).  The state's 16x16 tiles are spread over the
// four waves (more tiles to the waves with shorter causal strips) and stay in
// fp32 accumulators for the whole chain.
//
// Precision.  The three intermediate operands that are not inputs -- P, the
// state as the operand of Q S, and the decayed V rows -- are each carried as
// a pair of bf16 values (hi = bf16(x), lo = bf16(x - hi)) and contracted with
// two MFMAs, so they enter the products with ~16 significant bits; inputs
// are bf16 already and every sum is fp32.  The state is stored in fp32.
//
// LDS (bf16 bits unless noted):
//   Qs, Ks  [64][d+16]   row-major; K is also read transposed by
//                        ds_read_b64_tr_b16 for the K^T operand
//   Vs      [64][32+16]  the slice of V (row-major, read transposed)
//   Vh, Vl  [64][32+16]  lambda^(ell-1-j)-scaled V rows, hi/lo
//   Sh, Sl  [2][32][d+8] state^T hi/lo for the Q S product, double-buffered
// MFMA operand layout (16x16x32 bf16): lane l supplies row (l % 16) of A and
// column (l % 16) of B, 8 k-values per lane in lane group g = l / 16; the 4
// results of lane l sit at rows 4g + m, column l % 16.  The order of the 8
// k-values is free as long as A and B agree.
// ds_read_b64_tr_b16: in each 16-lane group, lane 4r + a gives the address
// of 4 elements of row r; lane i receives element i of each of the 4 rows.

#include "la_device.h"
#include "la_internal.h"

namespace la {
namespace {

constexpr int kBeta = 64;
constexpr int kThreads = 256;
constexpr int kDV = kBf16Cols;  // 32 value columns per workgroup

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ floatx4 mfma(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// Transposed 4-element read (see the header comment); p must be 8 B aligned.
__device__ __forceinline__ v4i16 ld_tr(const uint16_t* p) {
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4i16*)(__attribute__((address_space(3))) uint16_t*)(p));
}

__device__ __forceinline__ bf16x8 cat(v4i16 a, v4i16 b) {
  v8i16 x = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, x);
}

// Two floats -> packed bf16 (hardware round to nearest even).
__device__ __forceinline__ uint32_t cvt2(float a, float b) {
  float2v f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

// hi/lo split of 4 floats: hi = bf16(x), lo = bf16(x - hi).
__device__ __forceinline__ void split4(const floatx4& x, uint2& hi, uint2& lo) {
  hi.x = cvt2(x[0], x[1]);
  hi.y = cvt2(x[2], x[3]);
  lo.x = cvt2(x[0] - bf16_lo(hi.x), x[1] - bf16_hi(hi.x));
  lo.y = cvt2(x[2] - bf16_lo(hi.y), x[3] - bf16_hi(hi.y));
}

__device__ __forceinline__ bf16x8 cat2(uint2 a, uint2 b) {
  const uint4 w = {a.x, a.y, b.x, b.y};
  return __builtin_bit_cast(bf16x8, w);
}

// State tiles (16x16, index n -> row tile n/2, column tile n%2) owned by each
// wave.  Waves with long causal strips get fewer tiles so the MFMA work per
// wave is even.
template <int D>
struct TileSplit;
template <>
struct TileSplit<128> {
  static constexpr int kMax = 6;
  __device__ static int begin(int w) { return w == 0 ? 0 : w == 1 ? 6 : w == 2 ? 11 : 14; }
  __device__ static int end(int w) { return w == 0 ? 6 : w == 1 ? 11 : w == 2 ? 14 : 16; }
};
template <>
struct TileSplit<64> {
  static constexpr int kMax = 3;
  __device__ static int begin(int w) { return w == 0 ? 0 : w == 1 ? 3 : w == 2 ? 6 : 7; }
  __device__ static int end(int w) { return w == 0 ? 3 : w == 1 ? 6 : w == 2 ? 7 : 8; }
};

template <int D, bool kOutF32>
__global__ __launch_bounds__(kThreads) void prefill_bf16_kernel(PrefillArgs a) {
  constexpr int NDV = D / kDV;
  constexpr int KS = D + 16;      // Qs/Ks row stride
  constexpr int VS = kDV + 16;    // V row stride
  constexpr int SS = D + 8;       // state^T row stride
  constexpr int NK = D / 32;      // k-steps over d
  constexpr int CH = D / 8;       // 16 B chunks per Q/K row
  constexpr int NQC = CH / 4;     // Q (and K) chunks staged per thread
  constexpr int MAXT = TileSplit<D>::kMax;

  __shared__ __attribute__((aligned(16))) uint16_t Qs[kBeta * KS];
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kBeta * KS];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[kBeta * VS];
  __shared__ __attribute__((aligned(16))) uint16_t Vh[kBeta * VS];
  __shared__ __attribute__((aligned(16))) uint16_t Vl[kBeta * VS];
  __shared__ __attribute__((aligned(16))) uint16_t Sh[2][kDV * SS];
  __shared__ __attribute__((aligned(16))) uint16_t Sl[2][kDV * SS];

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
  const int tr_r = li >> 2;  // row supplied to a transposed read
  const int tr_a = li & 3;   // 4-element chunk supplied to a transposed read

  const int64_t start = a.cu_seqlens[s];
  const int64_t end = a.cu_seqlens[s + 1];
  const uint16_t* __restrict__ q = static_cast<const uint16_t*>(a.q);
  const uint16_t* __restrict__ k = static_cast<const uint16_t*>(a.k);
  const uint16_t* __restrict__ v = static_cast<const uint16_t*>(a.v);
  const int64_t state_off = ((int64_t)s * H + h) * D * D;
  const int64_t row_stride = (int64_t)H * D;  // elements between tokens
  const float l2 = a.log2_decay[h];

  // Per-lane decay factors of the score strip.  Element (i, j) of tile
  // (ti = w, tj) has i - j = 16 (w - tj) + (li - 4g - m).
  //   diagonal tile:     lambda^(li-4g-m) if >= 0, else 0
  //   tile with w > tj:  lambda^(16 (w-tj-1)) * lambda^(16 + li - 4g - m)
  // (no negative exponents, so no overflow for small lambda).
  floatx4 fdiag, foff;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int x = li - 4 * g - m;
    fdiag[m] = x >= 0 ? exp2f((float)x * l2) : 0.0f;
    foff[m] = exp2f((float)(16 + x) * l2);
  }
  const float f16 = exp2f(16.0f * l2);
  const float qdecay = exp2f((float)(16 * w + li + 1) * l2);  // lambda^(i+1)

  // State tiles of this wave, fp32, in accumulator layout.
  const int tb = TileSplit<D>::begin(w);
  const int te = TileSplit<D>::end(w);
  floatx4 st[MAXT];
#pragma unroll
  for (int n = 0; n < MAXT; ++n) {
    const int tile = tb + n;
    const int tr = tile >> 1, tc = tile & 1;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int r = 16 * tr + 4 * g + m;
      st[n][m] = (tile < te && a.kv_init)
                     ? a.kv_init[state_off + (int64_t)r * D + c0 + 16 * tc + li]
                     : 0.0f;
    }
    if (tile < te) {
      uint2 hi, lo;
      split4(st[n], hi, lo);
      *reinterpret_cast<uint2*>(&Sh[0][(16 * tc + li) * SS + 16 * tr + 4 * g]) = hi;
      *reinterpret_cast<uint2*>(&Sl[0][(16 * tc + li) * SS + 16 * tr + 4 * g]) = lo;
    }
  }

  // Staging roles.  Q/K chunk p of thread t: id = t + 256 p, row id / CH,
  // 16 B chunk id % CH (a wave covers whole rows: coalesced).  V: row t / 4,
  // chunk t % 4 of the 32-column slice.
  const int vrow = t >> 2;
  const int vch = t & 3;
  uint4 qreg[NQC], kreg[NQC], vreg;

  auto load_block = [&](int64_t b0, int ell) {
#pragma unroll
    for (int p = 0; p < NQC; ++p) {
      const int id = t + kThreads * p;
      const int row = id / CH;
      if (row < ell) {
        const int64_t off = (b0 + row) * row_stride + (int64_t)h * D + 8 * (id % CH);
        qreg[p] = *reinterpret_cast<const uint4*>(q + off);
        kreg[p] = *reinterpret_cast<const uint4*>(k + off);
      } else {
        qreg[p] = make_uint4(0, 0, 0, 0);
        kreg[p] = make_uint4(0, 0, 0, 0);
      }
    }
    vreg = vrow < ell ? *reinterpret_cast<const uint4*>(v + (b0 + vrow) * row_stride +
                                                         (int64_t)h * D + c0 + 8 * vch)
                      : make_uint4(0, 0, 0, 0);
  };

  int64_t b0 = start;
  int ell = (int)((end - b0) < kBeta ? (end - b0) : kBeta);
  if (b0 < end) load_block(b0, ell);

  for (int bi = 0; b0 < end; ++bi) {
    const int cur = bi & 1;
    const bool full = ell == kBeta;
    __syncthreads();  // the previous block is done with every staged tile

    // ---- stage the block ----
#pragma unroll
    for (int p = 0; p < NQC; ++p) {
      const int id = t + kThreads * p;
      const int row = id / CH, col = 8 * (id % CH);
      *reinterpret_cast<uint4*>(&Qs[row * KS + col]) = qreg[p];
      *reinterpret_cast<uint4*>(&Ks[row * KS + col]) = kreg[p];
    }
    {
      *reinterpret_cast<uint4*>(&Vs[vrow * VS + 8 * vch]) = vreg;
      // V row scaled by lambda^(ell-1-j), split hi/lo.
      const float wv = vrow < ell ? exp2f((float)(ell - 1 - vrow) * l2) : 0.0f;
      const uint32_t wds[4] = {vreg.x, vreg.y, vreg.z, vreg.w};
      uint32_t hp[4], lp[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = bf16_lo(wds[e]) * wv, x1 = bf16_hi(wds[e]) * wv;
        const uint32_t hh = cvt2(x0, x1);
        hp[e] = hh;
        lp[e] = cvt2(x0 - bf16_lo(hh), x1 - bf16_hi(hh));
      }
      *reinterpret_cast<uint4*>(&Vh[vrow * VS + 8 * vch]) = make_uint4(hp[0], hp[1], hp[2], hp[3]);
      *reinterpret_cast<uint4*>(&Vl[vrow * VS + 8 * vch]) = make_uint4(lp[0], lp[1], lp[2], lp[3]);
    }

    // ---- prefetch the next block ----
    const int64_t nb0 = b0 + kBeta;
    const int nell = nb0 < end ? (int)((end - nb0) < kBeta ? (end - nb0) : kBeta) : 0;
    if (nb0 < end) load_block(nb0, nell);
    __syncthreads();

    // ---- query strip operands ----
    bf16x8 qb[NK];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) qb[kk] = ld8(&Qs[(16 * w + li) * KS + 32 * kk + 8 * g]);

    // ---- scores S^T = K Q^T for tiles tj <= w; mask, decay, hi/lo ----
    uint2 ph[4], pl[4];
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) {
      ph[tj] = make_uint2(0, 0);
      pl[tj] = make_uint2(0, 0);
      if (tj <= w) {
        floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < NK; ++kk)
          acc = mfma(ld8(&Ks[(16 * tj + li) * KS + 32 * kk + 8 * g]), qb[kk], acc);
        floatx4 f;
        if (tj == w) {
          f = fdiag;
        } else {
          const int dd = w - tj - 1;  // 0, 1, 2
          const float sc = dd == 0 ? 1.0f : dd == 1 ? f16 : f16 * f16;
          f = foff * sc;
        }
        split4(acc * f, ph[tj], pl[tj]);
      }
    }

    // ---- O^T = V^T P^T + lambda^(i+1) S^T Q^T, two value-column tiles ----
#pragma unroll
    for (int tc = 0; tc < 2; ++tc) {
      floatx4 oi = {0.0f, 0.0f, 0.0f, 0.0f};
      floatx4 oe = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk2 = 0; kk2 < 2; ++kk2) {
        if (2 * kk2 <= w) {
          const int j0 = 32 * kk2 + 4 * g;
          const bf16x8 va = cat(ld_tr(&Vs[(j0 + tr_r) * VS + 16 * tc + 4 * tr_a]),
                                ld_tr(&Vs[(j0 + 16 + tr_r) * VS + 16 * tc + 4 * tr_a]));
          oi = mfma(va, cat2(ph[2 * kk2], ph[2 * kk2 + 1]), oi);
          oi = mfma(va, cat2(pl[2 * kk2], pl[2 * kk2 + 1]), oi);
        }
      }
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const int off = (16 * tc + li) * SS + 32 * kk + 8 * g;
        oe = mfma(ld8(&Sh[cur][off]), qb[kk], oe);
        oe = mfma(ld8(&Sl[cur][off]), qb[kk], oe);
      }
      const int i = 16 * w + li;
      if (i < ell) {
        float out[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) out[m] = fmaf(qdecay, oe[m], oi[m]);
        const int64_t off = (b0 + i) * row_stride + (int64_t)h * D + c0 + 16 * tc + 4 * g;
        if constexpr (kOutF32) {
          *reinterpret_cast<float4*>(static_cast<float*>(a.o) + off) =
              make_float4(out[0], out[1], out[2], out[3]);
        } else {
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.o) + off) =
              make_uint2(cvt2(out[0], out[1]), cvt2(out[2], out[3]));
        }
      }
    }

    // ---- state: S <- lambda^ell S + K^T Vd, then its bf16 hi/lo copy ----
    const float fl = full ? exp2f(64.0f * l2) : exp2f((float)ell * l2);
#pragma unroll
    for (int n = 0; n < MAXT; ++n) {
      const int tile = tb + n;
      if (tile < te) {
        const int tr = tile >> 1, tc = tile & 1;
        floatx4 acc = st[n] * fl;
#pragma unroll
        for (int kk2 = 0; kk2 < 2; ++kk2) {
          const int j0 = 32 * kk2 + 8 * g;
          const int ko = 16 * tr + 4 * tr_a;
          const int vo = 16 * tc + 4 * tr_a;
          const bf16x8 ka = cat(ld_tr(&Ks[(j0 + tr_r) * KS + ko]),
                                ld_tr(&Ks[(j0 + 4 + tr_r) * KS + ko]));
          const bf16x8 vh = cat(ld_tr(&Vh[(j0 + tr_r) * VS + vo]),
                                ld_tr(&Vh[(j0 + 4 + tr_r) * VS + vo]));
          const bf16x8 vl = cat(ld_tr(&Vl[(j0 + tr_r) * VS + vo]),
                                ld_tr(&Vl[(j0 + 4 + tr_r) * VS + vo]));
          acc = mfma(ka, vh, acc);
          acc = mfma(ka, vl, acc);
        }
        st[n] = acc;
        uint2 hi, lo;
        split4(acc, hi, lo);
        *reinterpret_cast<uint2*>(&Sh[cur ^ 1][(16 * tc + li) * SS + 16 * tr + 4 * g]) = hi;
        *reinterpret_cast<uint2*>(&Sl[cur ^ 1][(16 * tc + li) * SS + 16 * tr + 4 * g]) = lo;
      }
    }

    b0 = nb0;
    ell = nell;
  }

  if (a.kv_final) {
#pragma unroll
    for (int n = 0; n < MAXT; ++n) {
      const int tile = tb + n;
      if (tile < te) {
        const int tr = tile >> 1, tc = tile & 1;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int r = 16 * tr + 4 * g + m;
          a.kv_final[state_off + (int64_t)r * D + c0 + 16 * tc + li] = st[n][m];
        }
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
