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
// Decomposition.  One workgroup (8 waves) owns one (sequence, head, 32-column
// slice of the value dimension) chain; the d x d state is split by value
// columns over d/32 workgroups, each of which recomputes Q K^T for its block
// so that no cross-workgroup exchange exists.  Within the workgroup:
//  * strip waves 0..3: wave k owns query rows i in [16k, 16k+16), whose Q rows
//    it loads from HBM straight into its MFMA operand registers.  It forms
//    its strip of scores S^T = K Q^T, applies mask and decay in registers and
//    feeds them straight back into the MFMA as the B operand of O^T = V^T P^T
//    (the score tile's accumulator layout -- 4 consecutive keys per lane -- is
//    a valid operand layout when the value operand uses the same key order),
//    adds diag(lambda^(i+1)) S^T Q^T and writes its rows of O;
//  * state waves 4..7: own 16-row tiles of the 32-column state slice in fp32
//    accumulators for the whole chain and advance them by K^T Vd.
// Strip waves stage K and state waves stage V (HBM -> LDS, two blocks ahead).
// Wave k and wave k+4 share a SIMD; each state wave owns a pair of 16-row
// state tiles (for d = 64 only state waves 0 and 1 have one, beside the two
// shortest query strips).
// LDS stages are double-buffered: block b+1 is loaded from HBM while block b
// is computed, so each block needs one workgroup barrier.  Only the state
// waves load and only the strip waves store, and the barrier waits for LDS
// traffic alone, so no wave ever waits for its own stores to reach HBM.
//
// Precision.  The three intermediate operands that are not inputs -- P, the
// state as the operand of Q S, and the decayed V rows -- are each carried as
// a pair of bf16 values (hi = bf16(x), lo = bf16(x - hi)) and contracted with
// two MFMAs, so they enter the products with ~16 significant bits; inputs
// are bf16 already and every sum is fp32.  The state is stored in fp32.
//
// LDS (bf16 bits).  The LDS of gfx950 serves 256 B per clock to reads (a
// 16 B read serves 16 lanes per clock, a transposed 8 B read 32 lanes) and
// 128 B per clock to writes (a 16 B write serves 8 consecutive lanes).  Each
// array is laid out so that every access pattern issued below is free of
// bank conflicts:
//   Ks      [2][64][d]    16 B chunk c of row r at chunk c ^ kswz(r)
//   Vs      [2][64][32]   the value slice; in rows j with bit 2 set the
//                         8-byte halves of each 16-byte chunk are swapped
//   Vh, Vl  [2][64][32]   its lambda^(ell-1-j)-scaled rows as hi/lo; chunk c
//                         of row j at c ^ ((j/2) % 4)
//   Sh, Sl  [2][32][d]    state^T hi/lo for the Q S product; chunk q of
//                         row c at q ^ key(c) (s_off)
// MFMA operand layout (16x16x32 bf16): lane l supplies row (l % 16) of A and
// column (l % 16) of B, 8 k-values per lane in lane group g = l / 16; the 4
// results of lane l sit at rows 4g + m, column l % 16.  The order of the 8
// k-values is free as long as A and B agree.
// ds_read_b64_tr_b16: in each 16-lane group, lane 4r + a gives the address
// of 4 elements of row r; lane i receives element i of each of the 4 rows.

#include "la_internal.h"
#include "la_mfma.h"

namespace la {
namespace {

constexpr int kBeta = 64;
constexpr int kThreads = 512;
constexpr int kDV = kBf16Cols;  // 32 value columns per workgroup

// Element offset of (row j, column col) of a value-slice array (64 B rows).
__device__ __forceinline__ int v_off(int j, int col) {
  return j * kDV + 8 * ((col >> 3) ^ ((j >> 1) & 3)) + (col & 7);
}

// Layout of the plain value slice Vs, which only the strip waves read: in
// rows with bit 2 set the two 8-byte halves of every 16-byte chunk trade
// places, so that the transposed reads of the interleaved column tiles
// (8 lanes of a row group take the 4 chunks of one half, lanes of row j and
// j + 4 arrive together) fall on distinct banks.
__device__ __forceinline__ int vs_off(int j, int col) {
  return j * kDV + 8 * (col >> 3) + 4 * (((col >> 2) & 1) ^ ((j >> 2) & 1)) + (col & 3);
}

// Element offset of state^T row c (a value column), key rows 8q .. 8q+7.
// The chunk swizzle keeps both access patterns free of bank conflicts: the
// writer's 8 consecutive lanes take c = 16 tc + 0..7 and the reader's 16
// lanes take c = sv_col(tc, 0..15) (bits 0, 1, 3, 4 of c vary, bit 2 fixed).
template <int D>
__device__ __forceinline__ int s_off(int c, int q) {
  const int key = (c & 3) | ((((c >> 2) ^ (c >> 3)) & 1) << 2) | (((c >> 4) & 1) << 3);
  // d = 64: two 128 B rows share a bank line, so row parity (bit 0) already
  // separates them and the key drops it
  return c * D + 8 * (q ^ (D == 128 ? key : key >> 1));
}

// Value column of row r of the strip waves' column tile tc: tile tc takes
// columns 8 (r / 4) + 4 tc + r % 4, so the two tiles' results in one lane
// are 8 consecutive columns (one 16 B store of bf16).
__device__ __forceinline__ int sv_col(int tc, int r) { return 8 * (r >> 2) + 4 * tc + (r & 3); }

// State row tiles [begin, end) owned by state wave k: the pair (2k, 2k+1).
// d = 128: 8 tiles, 2 per state wave.  d = 64: 4 tiles on state waves 0 and
// 1, which share their SIMDs with the two shortest query strips.
template <int D>
struct RowSplit {
  static constexpr int kTiles = D / 16;
  static constexpr int kMax = 2;
  __device__ static int begin(int k) { return 2 * k < kTiles ? 2 * k : kTiles; }
  __device__ static int end(int k) { return 2 * k + 2 < kTiles ? 2 * k + 2 : kTiles; }
};

template <int D, bool kOutF32, bool kStateOnly, bool kReverse>
__global__ __launch_bounds__(kThreads) void prefill_bf16_kernel(PrefillArgs a) {
  constexpr int NDV = D / kDV;
  constexpr int NK = D / 32;       // k-steps over d
  constexpr int CH = D / 8;        // 16 B chunks per K row
  constexpr int NKC = CH / 4;      // K chunks staged per strip thread
  constexpr int MAXR = RowSplit<D>::kMax;
  constexpr int KSZ = kBeta * D;
  constexpr int VSZ = kBeta * kDV;

  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][KSZ];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][VSZ];
  __shared__ __attribute__((aligned(16))) uint16_t Vh[2][VSZ];
  __shared__ __attribute__((aligned(16))) uint16_t Vl[2][VSZ];
  __shared__ __attribute__((aligned(16))) uint16_t Sh[2][kDV * D];
  __shared__ __attribute__((aligned(16))) uint16_t Sl[2][kDV * D];

  const int H = a.num_heads;
  const int item = xcd_remap(blockIdx.x, a.num_items, NDV);
  const int cs = item % NDV;
  const int sh = item / NDV;
  const int h = sh % H;
  const int s = seq_of(a, sh / H);
  const int c0 = cs * kDV;
  const int t = threadIdx.x;
  const int wid = uniform(t >> 6);
  const bool strip = wid < 4;
  const int k = wid & 3;      // strip index, or state-wave index
  const int l = t & 63;
  const int li = l & 15;
  const int g = l >> 4;
  const int tr_r = li >> 2;   // row supplied to a transposed read
  const int tr_a = li & 3;    // 4-element piece supplied to a transposed read

  const int64_t start = a.cu_seqlens[s];
  const int64_t end = a.cu_seqlens[s + 1];
  const int nblocks = (int)((end - start + kBeta - 1) / kBeta);
  const uint16_t* __restrict__ q = static_cast<const uint16_t*>(a.q);
  const uint16_t* __restrict__ kp = static_cast<const uint16_t*>(a.k);
  const uint16_t* __restrict__ v = static_cast<const uint16_t*>(a.v);
  // state slots of this sequence in kv_init / kv_final
  const int64_t init_off = ((int64_t)(a.init_slot ? a.init_slot[s] : s) * H + h) * D * D;
  const int64_t final_off = ((int64_t)(a.final_slot ? a.final_slot[s] : s) * H + h) * D * D;
  const int row_stride = H * D;  // elements between tokens (< 2^15)
  const float l2 = a.log2_decay[h];
  const float lam_beta = exp2f((float)kBeta * l2);

  // ---- per-lane decay factors (strip waves) ----
  // Element (i, j) of score tile (k, tj) has i - j = 16 (k - tj) + (li-4g-m):
  //   diagonal tile:     lambda^(li-4g-m) if >= 0, else 0
  //   tile with k > tj:  lambda^(16 (k-tj-1)) * lambda^(16 + li - 4g - m)
  // (no negative exponents, so no overflow for small lambda).
  floatx4 fdiag, foff[3];
  {
    const float f16 = exp2f(16.0f * l2);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int x = li - 4 * g - m;
      fdiag[m] = x >= 0 ? exp2f((float)x * l2) : 0.0f;
      foff[0][m] = exp2f((float)(16 + x) * l2);
      foff[1][m] = foff[0][m] * f16;
      foff[2][m] = foff[1][m] * f16;
    }
  }
  const float qdecay = exp2f((float)(16 * k + li + 1) * l2);  // lambda^(i+1)

  // ---- state row tiles (state waves), fp32 accumulator layout ----
  // st[n][tc]: key rows srow(rb + n, g) + m, column 16 tc + li of the slice.
  const int rb = RowSplit<D>::begin(k);
  const int re = strip ? rb : RowSplit<D>::end(k);
  // Writes state tiles (rb, rb+1) to state^T as hi/lo chunks in buffer buf.
  auto put_state = [&](const floatx4(&x)[MAXR][2], int buf) {
    const bool odd = g & 1;
#pragma unroll
    for (int tc = 0; tc < 2; ++tc) {
      uint2 h0, l0, h1, l1;
      split4(x[0][tc], h0, l0);
      split4(x[1][tc], h1, l1);
      const uint4 hv = odd ? make_uint4(h1.x, h1.y, h0.x, h0.y) : make_uint4(h0.x, h0.y, h1.x, h1.y);
      const uint4 lv = odd ? make_uint4(l1.x, l1.y, l0.x, l0.y) : make_uint4(l0.x, l0.y, l1.x, l1.y);
      const int so = s_off<D>(16 * tc + li, 4 * (rb >> 1) + g);
      *reinterpret_cast<uint4*>(&Sh[buf][so]) = hv;
      *reinterpret_cast<uint4*>(&Sl[buf][so]) = lv;
    }
  };
  floatx4 st[MAXR][2];
#pragma unroll
  for (int n = 0; n < MAXR; ++n) {
#pragma unroll
    for (int tc = 0; tc < 2; ++tc) {
      st[n][tc] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
      if (rb + n < re && a.kv_init) {
#pragma unroll
        for (int m = 0; m < 4; ++m)
          st[n][tc][m] =
              a.kv_init[init_off + (int64_t)(srow(rb + n, g) + m) * D + c0 + 16 * tc + li];
      }
    }
  }
  if (re > rb) put_state(st, 0);

  // Valid rows of block b (0 past the end of the sequence).
  auto block_len = [&](int b) -> int {
    const int64_t rem = end - (start + (int64_t)b * kBeta);
    return rem <= 0 ? 0 : rem < kBeta ? (int)rem : kBeta;
  };
  // Buffer resource over the valid rows (all heads) of block b of a [T, H, d]
  // tensor with elements of `esize` bytes.
  // With kReverse the chain runs backwards in time: logical token i of the
  // sequence is physical row end - 1 - i, so block b holds the physical rows
  // [end - 64b - ell, end - 64b) in decreasing order.  Rows are addressed
  // inside a block resource by prow(); logical rows past the end of the
  // sequence map outside the resource either way.
  auto block_rsrc = [&](const void* base, int b, int esize) {
    const int ell = block_len(b);
    const int64_t row0 = kReverse ? end - (int64_t)b * kBeta - ell : start + (int64_t)b * kBeta;
    const char* p = static_cast<const char*>(base) + row0 * row_stride * (int64_t)esize;
    return buf_rsrc(p, ell * row_stride * esize);
  };
  auto prow = [&](int r, int ell) { return kReverse ? ell - 1 - r : r; };

  // ---- strip waves: their 16 query rows go straight from HBM into the
  // MFMA operand registers (lane (li, g) holds Q[16k+li][32kk+8g..+7]) ----
  auto load_q = [&](bf16x8(&dst)[NK], int b) {
    const __amdgpu_buffer_rsrc_t r = block_rsrc(q, b, 2);
    const int off = 2 * (prow(16 * k + li, block_len(b)) * row_stride + h * D + 8 * g);
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
      dst[kk] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off + 64 * kk, 0, 0));
  };

  // ---- staging: K and V move HBM -> registers -> LDS two blocks ahead.
  // Strip thread t moves K chunks id = t + 256 p (row id / CH, chunk id % CH:
  // a wave reads whole rows, coalesced).  State thread u = t - 256 moves the
  // value slice: row u / 4, chunk u % 4, plus its lambda^(ell-1-j)-scaled
  // hi/lo copies. ----
  const int u = t - 256;
  const int vrow = u >> 2;
  const int vch = u & 3;
  struct KStage {
    uint4 k[NKC];
  };
  struct VStage {
    uint4 v;
  };

  auto load_k = [&](KStage& r, int b) {
    const __amdgpu_buffer_rsrc_t rk = block_rsrc(kp, b, 2);
    const int ell = block_len(b);
#pragma unroll
    for (int p = 0; p < NKC; ++p) {
      const int id = t + 256 * p;
      r.k[p] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(
                     rk, 2 * (prow(id / CH, ell) * row_stride + h * D + 8 * (id % CH)), 0, 0));
    }
  };
  auto store_k = [&](const KStage& r, int buf) {
#pragma unroll
    for (int p = 0; p < NKC; ++p) {
      const int id = t + 256 * p;
      *reinterpret_cast<uint4*>(&Ks[buf][qk_off<D>(id / CH, id % CH)]) = r.k[p];
    }
  };
  auto load_v = [&](VStage& r, int b) {
    const __amdgpu_buffer_rsrc_t rv = block_rsrc(v, b, 2);
    r.v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                        rv, 2 * (prow(vrow, block_len(b)) * row_stride + h * D + c0 + 8 * vch), 0, 0));
  };
  auto store_v = [&](const VStage& r, int buf, int b) {
    const int ell = block_len(b);
    const int o = v_off(vrow, 8 * vch);
    *reinterpret_cast<uint4*>(&Vs[buf][vrow * kDV + 8 * vch]) =
        vrow & 4 ? make_uint4(r.v.z, r.v.w, r.v.x, r.v.y) : r.v;  // vs_off layout
    // value row scaled by lambda^(ell-1-j), split hi/lo
    const float wv = vrow < ell ? exp2f((float)(ell - 1 - vrow) * l2) : 0.0f;
    const uint32_t wd[4] = {r.v.x, r.v.y, r.v.z, r.v.w};
    uint32_t hp[4], lp[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x0 = bf16_lo(wd[e]) * wv, x1 = bf16_hi(wd[e]) * wv;
      const uint32_t hh = cvt2(x0, x1);
      hp[e] = hh;
      lp[e] = cvt2(x0 - bf16_lo(hh), x1 - bf16_hi(hh));
    }
    *reinterpret_cast<uint4*>(&Vh[buf][o]) = make_uint4(hp[0], hp[1], hp[2], hp[3]);
    *reinterpret_cast<uint4*>(&Vl[buf][o]) = make_uint4(lp[0], lp[1], lp[2], lp[3]);
  };

  // ---- one block of a strip wave (strip index KS fixed at compile time) ----
  auto strip_body = [&](auto KS_, const bf16x8(&qb)[NK], int cur, int b) {
    constexpr int KS = decltype(KS_)::value;
    const uint16_t* Kc = Ks[cur];
    const uint16_t* Vc = Vs[cur];

    // scores S^T = K Q^T for tiles tj <= KS (independent chains interleaved)
    floatx4 sc[KS + 1];
#pragma unroll
    for (int tj = 0; tj <= KS; ++tj) sc[tj] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
#pragma unroll
      for (int tj = 0; tj <= KS; ++tj)
        sc[tj] = mfma(ld8(&Kc[qk_off<D>(16 * tj + li, 4 * kk + g)]), qb[kk], sc[tj]);
    // mask, decay, hi/lo
    uint2 ph[4], pl[4];
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) {
      if (tj <= KS) {
        const floatx4 f = tj == KS ? fdiag : foff[KS - tj - 1 < 0 ? 0 : KS - tj - 1];
        split4(sc[tj] * f, ph[tj], pl[tj]);
      } else {
        ph[tj] = make_uint2(0, 0);
        pl[tj] = make_uint2(0, 0);
      }
    }

    // O^T = V^T P^T + lambda^(i+1) S^T Q^T for the two value-column tiles
    constexpr int NJ = KS / 2 + 1;  // 32-key chunks with nonzero scores
    floatx4 oi[2], oe[2];
#pragma unroll
    for (int tc = 0; tc < 2; ++tc) {
      oi[tc] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
      oe[tc] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    }
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
#pragma unroll
      for (int tc = 0; tc < 2; ++tc) {
        const int so = s_off<D>(sv_col(tc, li), 4 * kk + g);
        oe[tc] = mfma(ld8(&Sh[cur][so]), qb[kk], oe[tc]);
        oe[tc] = mfma(ld8(&Sl[cur][so]), qb[kk], oe[tc]);
      }
    }
#pragma unroll
    for (int kk2 = 0; kk2 < NJ; ++kk2) {
      const int j0 = 32 * kk2 + 4 * g + tr_r;
      const bf16x8 p_h = cat2(ph[2 * kk2], ph[2 * kk2 + 1]);
      const bf16x8 p_l = cat2(pl[2 * kk2], pl[2 * kk2 + 1]);
#pragma unroll
      for (int tc = 0; tc < 2; ++tc) {
        const bf16x8 va = cat(ld_tr(&Vc[vs_off(j0, 8 * tr_a + 4 * tc)]),
                              ld_tr(&Vc[vs_off(j0 + 16, 8 * tr_a + 4 * tc)]));
        oi[tc] = mfma(va, p_h, oi[tc]);
        oi[tc] = mfma(va, p_l, oi[tc]);
      }
    }
    // rows past the end of the sequence fall outside the resource: dropped
    constexpr int ES = kOutF32 ? 4 : 2;
    const __amdgpu_buffer_rsrc_t ro = block_rsrc(a.o, b, ES);
    // lane (li, g) holds columns 8g .. 8g+7 of query row 16 KS + li
    const int off = ES * (prow(16 * KS + li, block_len(b)) * row_stride + h * D + c0 + 8 * g);
    float out[8];
#pragma unroll
    for (int tc = 0; tc < 2; ++tc)
#pragma unroll
      for (int m = 0; m < 4; ++m) out[4 * tc + m] = fmaf(qdecay, oe[tc][m], oi[tc][m]);
    if constexpr (kOutF32) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{__builtin_bit_cast(unsigned, out[4 * h2]),
                                                     __builtin_bit_cast(unsigned, out[4 * h2 + 1]),
                                                     __builtin_bit_cast(unsigned, out[4 * h2 + 2]),
                                                     __builtin_bit_cast(unsigned, out[4 * h2 + 3])},
                                               ro, off + 16 * h2, 0, 0);
    } else {
      __builtin_amdgcn_raw_buffer_store_b128(
          u32x4{cvt2(out[0], out[1]), cvt2(out[2], out[3]), cvt2(out[4], out[5]), cvt2(out[6], out[7])},
          ro, off, 0, 0);
    }
  };

  // ---- one block of a state wave (its pair of row tiles) ----
  auto state_body = [&](int cur, int ell) {
    constexpr int NR = MAXR;
    const uint16_t* Kc = Ks[cur];
    const uint16_t* Hc = Vh[cur];
    const uint16_t* Lc = Vl[cur];
    const float fl = ell == kBeta ? lam_beta : exp2f((float)ell * l2);
    // decayed-V operands of both column tiles and both key halves
    bf16x8 vh[2][2], vl[2][2];
#pragma unroll
    for (int kk2 = 0; kk2 < 2; ++kk2) {
#pragma unroll
      for (int tc = 0; tc < 2; ++tc) {
        const int j0 = 32 * kk2 + 4 * g + tr_r;
        const int vo = 16 * tc + 4 * tr_a;
        vh[kk2][tc] = cat(ld_tr(&Hc[v_off(j0, vo)]), ld_tr(&Hc[v_off(j0 + 16, vo)]));
        vl[kk2][tc] = cat(ld_tr(&Lc[v_off(j0, vo)]), ld_tr(&Lc[v_off(j0 + 16, vo)]));
      }
    }
    bf16x8 ka[NR][2];
#pragma unroll
    for (int n = 0; n < NR; ++n) {
      const int tr = rb + n;
#pragma unroll
      for (int kk2 = 0; kk2 < 2; ++kk2) {
        const int j0 = 32 * kk2 + 4 * g + tr_r;
        const int e = srow(tr, tr_a);  // A rows 4 tr_a .. 4 tr_a + 3 of tile tr
        ka[n][kk2] = cat(ld_tr(&Kc[qk_off<D>(j0, e >> 3) + (e & 7)]),
                         ld_tr(&Kc[qk_off<D>(j0 + 16, e >> 3) + (e & 7)]));
      }
    }
    floatx4 acc[NR][2];
#pragma unroll
    for (int n = 0; n < NR; ++n)
#pragma unroll
      for (int tc = 0; tc < 2; ++tc) acc[n][tc] = st[n][tc] * fl;
#pragma unroll
    for (int kk2 = 0; kk2 < 2; ++kk2) {
#pragma unroll
      for (int n = 0; n < NR; ++n)
#pragma unroll
        for (int tc = 0; tc < 2; ++tc) acc[n][tc] = mfma(ka[n][kk2], vh[kk2][tc], acc[n][tc]);
#pragma unroll
      for (int n = 0; n < NR; ++n)
#pragma unroll
        for (int tc = 0; tc < 2; ++tc) acc[n][tc] = mfma(ka[n][kk2], vl[kk2][tc], acc[n][tc]);
    }
#pragma unroll
    for (int n = 0; n < NR; ++n)
#pragma unroll
      for (int tc = 0; tc < 2; ++tc) st[n][tc] = acc[n][tc];
    put_state(st, cur ^ 1);
  };

  // ---- pipeline ----
  // Strip waves hold Q of block b in one register set and load block b+1
  // into the other; both roles keep two register stages of their share of
  // K / V: at block b, the stage that held block b (already in LDS) receives
  // block b+2 from HBM, and the stage holding block b+1 is written to LDS
  // after block b's arithmetic.  One barrier per block publishes the LDS
  // writes.  The two roles run separate loops with the same number of
  // barriers, so the registers of one role are not kept live in the other.
  if (strip && kStateOnly) {
    // state-only pass: the strip waves only stage K
    KStage k0, k1;
    load_k(k0, 0);
    load_k(k1, 1);
    store_k(k0, 0);
    lds_barrier();
    auto kstep = [&](int b, KStage& kfree, KStage& kfull) {
      load_k(kfree, b + 2);  // empty range past the last block
      if (b + 1 < nblocks) store_k(kfull, (b & 1) ^ 1);
      lds_barrier();
    };
    for (int b = 0; b < nblocks; b += 2) {
      kstep(b, k0, k1);
      if (b + 1 < nblocks) kstep(b + 1, k1, k0);
    }
  } else if (strip) {
    bf16x8 qa[NK], qb2[NK];
    KStage k0, k1;
    load_q(qa, 0);
    load_k(k0, 0);
    load_k(k1, 1);
    store_k(k0, 0);
    lds_barrier();
    auto sstep = [&](int b, bf16x8(&qc)[NK], bf16x8(&qn)[NK], KStage& kfree, KStage& kfull) {
      load_q(qn, b + 1);     // empty range past the last block
      load_k(kfree, b + 2);  // likewise
      switch (k) {
        case 0: strip_body(IC<0>{}, qc, b & 1, b); break;
        case 1: strip_body(IC<1>{}, qc, b & 1, b); break;
        case 2: strip_body(IC<2>{}, qc, b & 1, b); break;
        default: strip_body(IC<3>{}, qc, b & 1, b); break;
      }
      if (b + 1 < nblocks) store_k(kfull, (b & 1) ^ 1);
      lds_barrier();
    };
    for (int b = 0; b < nblocks; b += 2) {
      sstep(b, qa, qb2, k0, k1);
      if (b + 1 < nblocks) sstep(b + 1, qb2, qa, k1, k0);
    }
  } else {
    VStage r0, r1;
    load_v(r0, 0);
    load_v(r1, 1);
    store_v(r0, 0, 0);
    lds_barrier();
    auto tstep = [&](int b, VStage& rfree, VStage& rfull) {
      const int cur = b & 1;
      load_v(rfree, b + 2);  // empty range past the last block
      const int ell = block_len(b);
      if (re > rb) state_body(cur, ell);
      if (b + 1 < nblocks) store_v(rfull, cur ^ 1, b + 1);
      lds_barrier();
    };
    for (int b = 0; b < nblocks; b += 2) {
      tstep(b, r0, r1);
      if (b + 1 < nblocks) tstep(b + 1, r1, r0);
    }

    if (a.kv_final) {
#pragma unroll
      for (int n = 0; n < MAXR; ++n) {
        const int tr = rb + n;
        if (tr < re) {
#pragma unroll
          for (int tc = 0; tc < 2; ++tc)
#pragma unroll
            for (int m = 0; m < 4; ++m)
              a.kv_final[final_off + (int64_t)(srow(tr, g) + m) * D + c0 + 16 * tc + li] =
                  st[n][tc][m];
        }
      }
    }
  }
}

template <int D>
hipError_t launch_d(const PrefillArgs& a, la_dtype out_dtype, bool state_only, bool reverse,
                    hipStream_t stream) {
  const dim3 grid(a.num_items), block(kThreads);
  if (state_only && reverse)
    hipLaunchKernelGGL((prefill_bf16_kernel<D, false, true, true>), grid, block, 0, stream, a);
  else if (state_only)
    hipLaunchKernelGGL((prefill_bf16_kernel<D, false, true, false>), grid, block, 0, stream, a);
  else if (reverse && out_dtype == LA_FP32)
    hipLaunchKernelGGL((prefill_bf16_kernel<D, true, false, true>), grid, block, 0, stream, a);
  else if (reverse)
    hipLaunchKernelGGL((prefill_bf16_kernel<D, false, false, true>), grid, block, 0, stream, a);
  else if (out_dtype == LA_FP32)
    hipLaunchKernelGGL((prefill_bf16_kernel<D, true, false, false>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((prefill_bf16_kernel<D, false, false, false>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, int head_dim, la_dtype out_dtype,
                               bool state_only, bool reverse, hipStream_t stream) {
  if (head_dim == 64) return launch_d<64>(a, out_dtype, state_only, reverse, stream);
  return launch_d<128>(a, out_dtype, state_only, reverse, stream);
}

}  // namespace la
