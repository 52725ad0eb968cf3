// bf16 prefill for gfx950, wide decomposition (d = 128): one workgroup per
// (sequence, head) chain.
//
// Method (emonzhong.com "MiniMax-01: Scaling Foundation Models with Lightning
// Attention" 方法要点; CSDN "【AI论文】MiniMax-01:利用闪电注意力机制扩展基础模型"
// §2.1; mizuki blog "MiniMax-01：4M 上下文破局" 关键概念清单): blocks of
// BETA = 64 tokens, ell valid rows, local indices i (query) and j (key):
//   P      = (Q_b K_b^T) .* M,  M[i][j] = lambda^(i-j) for i >= j, else 0
//   O_b    = P V_b + diag(lambda^(i+1)) Q_b S_b          (left + right product)
//   S_b+1  = lambda^ell S_b + K_b^T diag(lambda^(ell-1-j)) V_b
//
// Decomposition.  The 32-column kernel (la_prefill_bf16.hip) splits the state
// over four workgroups per chain, each of which reads all Q and K rows and
// forms Q K^T again.  Here one workgroup of 8 waves owns the whole chain, so
// every input row crosses into the CU once and Q K^T is formed once; it is
// the faster of the two when there are more chains than half the CUs (many
// sequences, or a long sequence cut into segments).  Wave w owns value
// columns [16w, 16w+16) of the fp32 d x d state -- all 128 key rows, eight
// 16 x 16 accumulator tiles -- for the whole chain.  Per block:
//   phase 1  waves 0..5 each form one 16-query x 32-key unit of P (scores,
//            mask, decay, hi/lo split) and write it to LDS; every wave forms
//            S^T Q^T for its 16 columns with its state registers as the A
//            operand (the accumulator layout of a pair of key tiles is the
//            operand layout of one 32-key step);
//   phase 2  every wave completes O^T = V^T P^T + diag(lambda^(i+1)) S^T Q^T
//            for its columns and stores them, then advances its state by
//            K^T (diag(lambda^(ell-1-j)) V) -- the decayed values are formed in
//            registers from the V^T operand it already holds.
// Two barriers per block: one publishes the staged Q, K, V rows, one the
// scores.  Q, K and V of block b+1 are loaded during block b and written to
// the other LDS buffer at its end.
//
// Precision as in the 32-column kernel: P, the state operand of Q S and the
// decayed V rows enter the MFMAs as bf16 hi/lo pairs; every sum is fp32 and
// the state stays fp32.
//
// LDS (bf16 bits), every access pattern below free of bank conflicts on
// gfx950 (reads 256 B/clk, writes 128 B/clk):
//   Qs, Ks [2][64][128]  16 B chunk c of row r at chunk c ^ kswz(r); in Qs
//                        the two 8 B halves of odd chunks are swapped
//   Vs     [2][64][128]  chunk c of row r at chunk c ^ (2r mod 16)
//   Ph, Pl [64][64]      query row i; 16 B unit u = 4 kk2 + g holds keys
//                        32 kk2 + 4g + (0..3) and 32 kk2 + 16 + 4g + (0..3),
//                        stored at unit u ^ (i mod 8)

#include "la_backward.h"
#include "la_internal.h"
#include "la_mfma.h"

namespace la {
namespace {

constexpr int kD = 128;
constexpr int kBeta = 64;
constexpr int kThreads = 512;
constexpr int kTok = kBeta * kD;  // elements of one staged block

__device__ __forceinline__ int v_woff(int r, int col) {
  return r * kD + 8 * ((col >> 3) ^ ((2 * r) & 15)) + (col & 7);
}
__device__ __forceinline__ int p_off(int i, int u) { return i * kBeta + 8 * (u ^ (i & 7)); }

// Score units: (query tile, 32-key step) pairs on or below the diagonal.
__device__ __forceinline__ int unit_qt(int u) { return (0x332120 >> (4 * u)) & 15; }
__device__ __forceinline__ int unit_kk2(int u) { return (0x22 >> u) & 1; }

// Element e of a bf16x8 as float.  The whole vector is reinterpreted before
// indexing: a bit cast applied to one element of a vector value is lowered by
// this compiler to a splat of element 0.
__device__ __forceinline__ float bf16_at(const bf16x8& x, int e) {
  const v8i16 xi = __builtin_bit_cast(v8i16, x);
  return __builtin_bit_cast(float, (uint32_t)(uint16_t)xi[e] << 16);
}

// The packed bf16 pair (-1, 0) (low half -1), produced in a scalar register:
// left as a constant, the compiler encodes it as the inline constant -1.0,
// whose fp32 bit pattern v_dot2 reads as the pair (0, -1).
__device__ __forceinline__ uint32_t neg_lo_pair() {
  uint32_t c;
  asm("s_mov_b32 %0, 0xbf80" : "=s"(c));
  return c;
}

// hi/lo split of 4 floats, hi = bf16(x), lo = bf16(x - hi), for a temporary
// x: each difference is one v_dot2 of the packed hi pair with (-1, 0) or
// (0, -1) accumulated onto x (exact in fp32, since hi is x rounded to bf16).
// The dot product accumulates in place, so for an x that stays live (the
// state) the plain split4 is cheaper.  nlo must be neg_lo_pair().
__device__ __forceinline__ void split4t(floatx4 x, uint2& hi, uint2& lo, uint32_t nlo) {
  const bf16x2 n_lo = __builtin_bit_cast(bf16x2, nlo);
  const bf16x2 n_hi = __builtin_bit_cast(bf16x2, 0xBF800000u);
  hi.x = cvt2(x[0], x[1]);
  hi.y = cvt2(x[2], x[3]);
  const bf16x2 h0 = __builtin_bit_cast(bf16x2, hi.x), h1 = __builtin_bit_cast(bf16x2, hi.y);
  lo.x = cvt2(__builtin_amdgcn_fdot2_f32_bf16(h0, n_lo, x[0], false),
              __builtin_amdgcn_fdot2_f32_bf16(h0, n_hi, x[1], false));
  lo.y = cvt2(__builtin_amdgcn_fdot2_f32_bf16(h1, n_lo, x[2], false),
              __builtin_amdgcn_fdot2_f32_bf16(h1, n_hi, x[3], false));
}

// One chain: its sequence and head, the tensors it reads and writes, its
// direction in time and how its states enter and leave.  The state
// starts from kv_init[s, h] (transposed if asked) times lambda^init_pow,
// or from zeros; lambda^final_pow times the final state goes to
// kv_final[s, h].  The prefill sets both powers to 0.
struct Chain {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  const float* kv_init;
  float* kv_final;
  int s, h;
  bool reverse, init_transposed;
  float init_pow, final_pow;
};

// The LDS arrays of one chain (declared by each kernel, so that two passes
// of one kernel can share them); a state-only pass uses Ks and Vs alone.
struct Lds {
  uint16_t* Qs;  // [2][64][128]
  uint16_t* Ks;  // [2][64][128]
  uint16_t* Vs;  // [2][64][128]
  uint16_t* Ph;  // [64][64]
  uint16_t* Pl;  // [64][64]
  float* Ob;     // [64][128] fp32: a block's output rows (normed output only)
};

// Thread t's place in the state: wave w owns value columns [16w, 16w+16) and
// tile n of its eight 16 x 16 accumulator tiles holds key rows srow(n, g) + m
// (m = 0..3) of column 16w + li, with li = lane % 16 and g = lane / 16.
struct StatePos {
  int c0, li, g;
  __device__ explicit StatePos(int t) : c0(16 * uniform(t >> 6)), li(t & 15), g((t & 63) >> 4) {}
  __device__ int row(int n, int m) const { return srow(n, g) + m; }
  __device__ int col() const { return c0 + li; }
};

// Runs the blocks of chain c with the state st (fp32, held in registers;
// updated in place): with kStateOnly only the state advances (K and V are
// read, Q is not, O is not written).  With kNorm each output row is
// normalised before it is written (see the output epilogue below).  Starts
// with an LDS write, so a caller that used the LDS arrays before must have
// passed a workgroup barrier.
template <bool kOutF32, bool kStateOnly, bool kNorm = false>
__device__ __forceinline__ void wide_blocks(const PrefillArgs& a, const Chain& c, const Lds& sm,
                                            floatx4 (&st)[8]) {
  uint16_t* const Qs = sm.Qs;
  uint16_t* const Ks = sm.Ks;
  uint16_t* const Vs = sm.Vs;
  uint16_t* const Ph = sm.Ph;
  uint16_t* const Pl = sm.Pl;
  float* const Ob = sm.Ob;

  const int H = a.num_heads;
  const int h = c.h;
  const int s = c.s;
  const int t = threadIdx.x;
  const int w = uniform(t >> 6);  // value-column tile of this wave
  const int c0 = 16 * w;
  const int l = t & 63;
  const int li = l & 15;
  const int g = l >> 4;
  const int tr_r = li >> 2;
  const int tr_a = li & 3;
  const uint32_t nlo = neg_lo_pair();

  const int64_t start = a.cu_seqlens[s];
  const int64_t end = a.cu_seqlens[s + 1];
  const int nblocks = (int)((end - start + kBeta - 1) / kBeta);
  const int row_stride = H * kD;
  const float l2 = a.log2_decay[h];
  const float lam_beta = exp2f((float)kBeta * l2);

  auto block_len = [&](int b) -> int {
    const int64_t rem = end - (start + (int64_t)b * kBeta);
    return rem <= 0 ? 0 : rem < kBeta ? (int)rem : kBeta;
  };
  // Buffer resource over the valid rows (all heads) of block b: loads past
  // the end of the sequence return zero and stores there are dropped.
  // A reverse chain runs backwards in time: logical token i of the
  // sequence is physical row end - 1 - i, so block b holds the physical rows
  // [end - 64b - ell, end - 64b) in decreasing order.  Rows are addressed
  // inside a block resource by prow(); logical rows past the end of the
  // sequence map outside the resource either way.
  auto block_rsrc = [&](const void* base, int b, int esize) {
    const int ell = block_len(b);
    const int64_t row0 = c.reverse ? end - (int64_t)b * kBeta - ell : start + (int64_t)b * kBeta;
    const char* p = static_cast<const char*>(base) + row0 * row_stride * (int64_t)esize;
    return buf_rsrc(p, ell * row_stride * esize);
  };
  auto prow = [&](int r, int ell) { return c.reverse ? ell - 1 - r : r; };

  // ---- per-lane decay factors ----
  // Score unit of this wave (waves 0..5): query tile qt, keys 32 kk2 .. +31
  // as key tiles kt = 2 kk2 and 2 kk2 + 1.  Element (key 16 kt + 4g + m,
  // query 16 qt + li) has i - j = 16 (qt - kt) + li - 4g - m.
  const int su = w < 6 ? w : 0;
  const int sqt = unit_qt(su);
  const int skk2 = unit_kk2(su);
  floatx4 fs[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int kt = 2 * skk2 + e;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int x = 16 * (sqt - kt) + li - 4 * g - m;
      fs[e][m] = x >= 0 ? exp2f((float)x * l2) : 0.0f;
    }
  }
  float qdec[4];  // lambda^(i+1) of query 16 qt + li
#pragma unroll
  for (int qt = 0; qt < 4; ++qt) qdec[qt] = exp2f((float)(16 * qt + li + 1) * l2);
  // lambda^(ell-1-j) for the 16 tokens of this lane's V^T operands (key step
  // kk2, element e: token 32 kk2 + 16 (e / 4) + 4g + e % 4); 0 past ell.
  auto vweights = [&](float (&wv)[2][8], int ell) {
#pragma unroll
    for (int kk2 = 0; kk2 < 2; ++kk2)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = 32 * kk2 + 16 * (e >> 2) + 4 * g + (e & 3);
        wv[kk2][e] = j < ell ? exp2f((float)(ell - 1 - j) * l2) : 0.0f;
      }
  };
  float wfull[2][8];
  vweights(wfull, kBeta);

  // ---- output epilogue (kNorm): the normalisation of NormAttention (CSDN
  // §2.1), read as an RMS normalisation of each head's output row over its
  // d features with a per-(head, feature) weight, times sigmoid(gate) when a
  // gate is given.  Phase 2 writes the block's fp32 output to Ob instead of
  // storing it; after the block's closing barrier, wave w takes rows
  // 8w .. 8w+7 whole: lane l holds row 8w + l / 8, columns 8j .. 8j+7 and
  // 64 + 8j .. 64 + 8j+7 (j = l % 8: each of its two 16-byte accesses of a
  // row then covers, with the other 7 lanes of the row, 128 contiguous
  // bytes), so a row's sum of squares is a reduction over 8 consecutive lanes (three
  // DPP steps within the VALU), and its gate values are loaded and its
  // outputs stored as whole 256-byte rows.  Ob chunk q (16 B) of row r sits
  // at chunk q ^ (r % 16), which keeps the tile writes (16 rows, one chunk)
  // free of bank conflicts.  The head's weights are staged in LDS once; the
  // gate rows of a block are loaded at the top of its step.
  auto ob_off = [](int r, int q) { return r * kD + 4 * (q ^ (r & 15)); };
  const int er = 8 * w + (l >> 3);  // epilogue row of this lane
  const int ec = 8 * (l & 7);       // its first column (and ec + 64)
  // sum over the 8 consecutive lanes of x's group: quad xor 1, quad xor 2,
  // then each lane with lane 7 - l of its half row
  auto sum8 = [](float x) {
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
    return x;
  };
  if constexpr (kNorm) {
    if (t < kD) Ob[kBeta * kD + t] = a.norm_weight[h * kD + t];  // weights after the rows
    // (published by the first block's barriers before the first epilogue)
  }
  auto load_gate = [&](uint4 (&gt)[2], int b) {
    if constexpr (kNorm) {
      if (a.gate) {
        const __amdgpu_buffer_rsrc_t rg = block_rsrc(a.gate, b, 2);
        const int off = 2 * (prow(er, block_len(b)) * row_stride + h * kD + ec);
        gt[0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rg, off, 0, 0));
        gt[1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rg, off + 128, 0, 0));
      }
    }
  };
  auto epilogue = [&](int b, const uint4 (&gt)[2]) {
    constexpr int ES = kOutF32 ? 4 : 2;
    const __amdgpu_buffer_rsrc_t ro = block_rsrc(c.o, b, ES);
    floatx4 x[4];
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = *reinterpret_cast<const floatx4*>(&Ob[ob_off(er, (ec >> 2) + (i & 1) + 16 * (i >> 1))]);
      ss += x[i][0] * x[i][0] + x[i][1] * x[i][1] + x[i][2] * x[i][2] + x[i][3] * x[i][3];
    }
    ss = sum8(ss);
    const float inv = rsqrtf(ss * (1.0f / kD) + a.norm_eps);
    const float* wb = &Ob[kBeta * kD + ec];
    const uint32_t* gw = reinterpret_cast<const uint32_t*>(&gt[0]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      floatx4 f = *reinterpret_cast<const floatx4*>(wb + 4 * (i & 1) + 64 * (i >> 1)) * inv;
      if (a.gate) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const uint32_t pw = gw[2 * i + (m >> 1)];
          const float gv = (m & 1) ? bf16_hi(pw) : bf16_lo(pw);
          // sigmoid(gv) = 1 / (1 + 2^(-gv log2 e)), hardware exp2 and reciprocal
          f[m] *= __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * gv));
        }
      }
      x[i] *= f;
    }
    const int off = ES * (prow(er, block_len(b)) * row_stride + h * kD + ec);
    if constexpr (kOutF32) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x[i]), ro,
                                               off + 16 * (i & 1) + 256 * (i >> 1), 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i)
        __builtin_amdgcn_raw_buffer_store_b128(
            u32x4{cvt2(x[2 * i][0], x[2 * i][1]), cvt2(x[2 * i][2], x[2 * i][3]),
                  cvt2(x[2 * i + 1][0], x[2 * i + 1][1]), cvt2(x[2 * i + 1][2], x[2 * i + 1][3])},
            ro, off + 128 * i, 0, 0);
    }
  };

  // ---- staging: thread t moves 16 B chunks t and t + 512 of each block
  // (row id / 16, chunk id % 16) of Q, K and V ----
  struct Stage {
    uint4 q[2], k[2], v[2];
  };
  auto load_stage = [&](Stage& r, int b) {
    const __amdgpu_buffer_rsrc_t rq = block_rsrc(c.q, b, 2);
    const __amdgpu_buffer_rsrc_t rk = block_rsrc(c.k, b, 2);
    const __amdgpu_buffer_rsrc_t rv = block_rsrc(c.v, b, 2);
    const int ell = block_len(b);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int id = t + kThreads * p;
      const int off = 2 * (prow(id >> 4, ell) * row_stride + h * kD + 8 * (id & 15));
      if (!kStateOnly)
        r.q[p] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
      r.k[p] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0));
      r.v[p] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0));
    }
  };
  auto store_stage = [&](const Stage& r, int buf) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int id = t + kThreads * p;
      const int row = id >> 4, ch = id & 15;
      if (!kStateOnly) {
        // odd chunks of Q rows are stored with their two 8 B halves swapped
        const uint4 x = r.q[p];
        *reinterpret_cast<uint4*>(&Qs[buf * kTok + qk_off<kD>(row, ch)]) =
            (ch & 1) ? make_uint4(x.z, x.w, x.x, x.y) : x;
      }
      *reinterpret_cast<uint4*>(&Ks[buf * kTok + qk_off<kD>(row, ch)]) = r.k[p];
      *reinterpret_cast<uint4*>(&Vs[buf * kTok + v_woff(row, 8 * ch)]) = r.v[p];
    }
  };

  // ---- phase 1: one unit of P (waves 0..5) and S^T Q^T (all waves) ----
  floatx4 oe[4];
  const int hsw = 4 * (g & 1);  // element offset of a lane group's first Q half
  auto phase1 = [&](auto cur_) {
    constexpr int cur = decltype(cur_)::value;
    const uint16_t* Qc = Qs + cur * kTok;
    const uint16_t* Kc = Ks + cur * kTok;
    if (w < 6) {
      floatx4 sc[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) sc[e] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
      // One loop per case of the (wave-uniform) test, so that each is a
      // single basic block whose LDS reads the compiler can issue ahead of
      // the MFMAs.
      auto scores = [&](auto both_) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int qo = qk_off<kD>(16 * sqt + li, 4 * kk + g);
          const bf16x8 qb = cat(*reinterpret_cast<const v4i16*>(&Qc[qo + hsw]),
                                *reinterpret_cast<const v4i16*>(&Qc[qo + 4 - hsw]));
          sc[0] = mfma(ld8(&Kc[qk_off<kD>(32 * skk2 + li, 4 * kk + g)]), qb, sc[0]);
          if (decltype(both_)::value)
            sc[1] = mfma(ld8(&Kc[qk_off<kD>(32 * skk2 + 16 + li, 4 * kk + g)]), qb, sc[1]);
        }
      };
      if (2 * skk2 + 1 > sqt)  // second key tile above the diagonal: stays zero
        scores(std::false_type{});
      else
        scores(std::true_type{});
      uint2 h0, l0, h1, l1;
      split4t(sc[0] * fs[0], h0, l0, nlo);
      split4t(sc[1] * fs[1], h1, l1, nlo);
      const int po = p_off(16 * sqt + li, 4 * skk2 + g);
      *reinterpret_cast<uint4*>(&Ph[po]) = make_uint4(h0.x, h0.y, h1.x, h1.y);
      *reinterpret_cast<uint4*>(&Pl[po]) = make_uint4(l0.x, l0.y, l1.x, l1.y);
    }
    // S^T Q^T: the A operand of key step kk is the pair of state tiles
    // (2kk, 2kk+1), whose lane group g holds keys 32kk + 8g + (0..7) -- in
    // the order (4..7, 0..3) for odd g (see srow), which is the order in
    // which Q chunk 4kk + g is stored.
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) oe[qt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      uint2 ah0, al0, ah1, al1;
      split4(st[2 * kk], ah0, al0);
      split4(st[2 * kk + 1], ah1, al1);
      const bf16x8 ahi = cat2(ah0, ah1);
      const bf16x8 alo = cat2(al0, al1);
      // the hi products of the four query tiles, then the lo products: no
      // MFMA waits for the one just before it
      bf16x8 qb[4];
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) {
        qb[qt] = ld8(&Qc[qk_off<kD>(16 * qt + li, 4 * kk + g)]);
        oe[qt] = mfma(ahi, qb[qt], oe[qt]);
      }
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) oe[qt] = mfma(alo, qb[qt], oe[qt]);
    }
  };

  // ---- phase 2: P V, output, state update ----
  auto phase2 = [&](auto cur_, int b) {
    constexpr int cur = decltype(cur_)::value;
    const uint16_t* Kc = Ks + cur * kTok;
    const uint16_t* Vc = Vs + cur * kTok;
    const int ell = block_len(b);
    // V^T operands of this wave's columns: lane (li, g) holds column c0 + li
    // of tokens 32 kk2 + 4g + (0..3) and 32 kk2 + 16 + 4g + (0..3)
    bf16x8 va[2];
#pragma unroll
    for (int kk2 = 0; kk2 < 2; ++kk2) {
      const int j0 = 32 * kk2 + 4 * g + tr_r;
      va[kk2] = cat(ld_tr(&Vc[v_woff(j0, c0 + 4 * tr_a)]), ld_tr(&Vc[v_woff(j0 + 16, c0 + 4 * tr_a)]));
    }
    if (!kStateOnly) {
      constexpr int ES = kOutF32 ? 4 : 2;
      const __amdgpu_buffer_rsrc_t ro = block_rsrc(c.o, b, ES);
      floatx4 acc[4];
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) acc[qt] = oe[qt] * qdec[qt];
      // hi products of every (query tile, key step), then the lo products
#pragma unroll
      for (int hl = 0; hl < 2; ++hl)
#pragma unroll
        for (int kk2 = 0; kk2 < 2; ++kk2)
#pragma unroll
          for (int qt = 2 * kk2; qt < 4; ++qt)
            acc[qt] = mfma(va[kk2], ld8(&(hl ? Pl : Ph)[p_off(16 * qt + li, 4 * kk2 + g)]), acc[qt]);
      if constexpr (kNorm) {  // to Ob; the epilogue stores the normalised rows
#pragma unroll
        for (int qt = 0; qt < 4; ++qt)
          *reinterpret_cast<floatx4*>(&Ob[ob_off(16 * qt + li, 4 * w + g)]) = acc[qt];
      } else {
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) {
        // lane (li, g): query 16 qt + li, value columns c0 + 4g + (0..3)
        const int off = ES * (prow(16 * qt + li, ell) * row_stride + h * kD + c0 + 4 * g);
        if constexpr (kOutF32) {
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[qt]), ro, off, 0, 0);
        } else {
          __builtin_amdgcn_raw_buffer_store_b64(
              u32x2{cvt2(acc[qt][0], acc[qt][1]), cvt2(acc[qt][2], acc[qt][3])}, ro, off, 0, 0);
        }
      }
      }
    }
    // decayed values lambda^(ell-1-j) V as hi/lo operands; only the last
    // block of a chain can be partial, so its weights replace the full ones
    if (ell != kBeta) vweights(wfull, ell);
    bf16x8 vdh[2], vdl[2];
#pragma unroll
    for (int kk2 = 0; kk2 < 2; ++kk2) {
      floatx4 x0, x1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x0[e] = bf16_at(va[kk2], e) * wfull[kk2][e];
        x1[e] = bf16_at(va[kk2], e + 4) * wfull[kk2][e + 4];
      }
      uint2 h0, l0, h1, l1;
      split4t(x0, h0, l0, nlo);
      split4t(x1, h1, l1, nlo);
      vdh[kk2] = cat2(h0, h1);
      vdl[kk2] = cat2(l0, l1);
    }
    const float fl = ell == kBeta ? lam_beta : exp2f((float)ell * l2);
#pragma unroll
    for (int n = 0; n < 8; ++n) st[n] = st[n] * fl;
    // Four groups (key step kk2, key tiles n0 .. n0+3): the K^T operands of
    // group grp+1 are read before the MFMAs of group grp issue, so the LDS
    // latency is covered; within a group the hi products of its four tiles
    // go first, then the lo products.
    auto kload = [&](bf16x8(&dst)[4], int grp) {
      const int j0 = 32 * (grp >> 1) + 4 * g + tr_r;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = srow(4 * (grp & 1) + i, tr_a);  // A rows 4 tr_a .. +3 of the key tile
        dst[i] = cat(ld_tr(&Kc[qk_off<kD>(j0, e >> 3) + (e & 7)]),
                     ld_tr(&Kc[qk_off<kD>(j0 + 16, e >> 3) + (e & 7)]));
      }
    };
    bf16x8 ka[2][4];
    kload(ka[0], 0);
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      if (grp < 3) kload(ka[(grp + 1) & 1], grp + 1);
      const int kk2 = grp >> 1, n0 = 4 * (grp & 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) st[n0 + i] = mfma(ka[grp & 1][i], vdh[kk2], st[n0 + i]);
#pragma unroll
      for (int i = 0; i < 4; ++i) st[n0 + i] = mfma(ka[grp & 1][i], vdl[kk2], st[n0 + i]);
    }
  };

  // ---- pipeline ----
  // Block b uses LDS buffer b % 2; the loops are unrolled by two so that
  // every LDS address is a per-lane base plus a constant.  An empty
  // asm volatile("" ::: "memory") after each block's loads is a compiler-only
  // fence: it keeps the loads at the top of the block, instead of being sunk
  // next to their use (which would expose their latency); it emits no
  // instruction and waits for nothing.
  if constexpr (kStateOnly) {
    // Little arithmetic per block: the loads run two blocks ahead, through
    // two register stages (the stage that held block b, already in LDS,
    // receives block b+2; the one holding block b+1 goes to LDS at the end).
    Stage s0, s1;
    load_stage(s0, 0);
    load_stage(s1, 1);
    store_stage(s0, 0);
    lds_barrier();
    auto step = [&](int b, auto cur_, Stage& sfree, Stage& snext) {
      constexpr int cur = decltype(cur_)::value;
      load_stage(sfree, b + 2);  // empty range past the last block
      asm volatile("" ::: "memory");
      phase2(cur_, b);
      if (b + 1 < nblocks) store_stage(snext, cur ^ 1);
      lds_barrier();
    };
    for (int b = 0; b < nblocks; b += 2) {
      step(b, IC<0>{}, s0, s1);
      if (b + 1 < nblocks) step(b + 1, IC<1>{}, s1, s0);
    }
  } else {
    {
      Stage r;
      load_stage(r, 0);
      store_stage(r, 0);
    }
    lds_barrier();
    auto step = [&](int b, auto cur_) {
      constexpr int cur = decltype(cur_)::value;
      Stage r;
      load_stage(r, b + 1);  // empty range past the last block
      uint4 gt[2] = {};
      load_gate(gt, b);
      asm volatile("" ::: "memory");
      phase1(cur_);
      lds_barrier();
      phase2(cur_, b);
      if (b + 1 < nblocks) store_stage(r, cur ^ 1);
      lds_barrier();
      if constexpr (kNorm) epilogue(b, gt);
    };
    for (int b = 0; b < nblocks; b += 2) {
      step(b, IC<0>{});
      if (b + 1 < nblocks) step(b + 1, IC<1>{});
    }
  }

}

// One whole chain: the state from kv_init[s, h] (slot map, transposition
// and scale as the chain asks) or zeros, the blocks, then the final state to
// kv_final[s, h].
template <bool kOutF32, bool kStateOnly, bool kNorm = false>
__device__ __forceinline__ void wide_chain(const PrefillArgs& a, const Chain& c, const Lds& sm) {
  const int H = a.num_heads;
  const int h = c.h;
  const int s = c.s;
  const StatePos sp(threadIdx.x);
  const float l2 = a.log2_decay[h];
  const int64_t init_off = ((int64_t)(a.init_slot ? a.init_slot[s] : s) * H + h) * kD * kD;
  const int64_t final_off = ((int64_t)(a.final_slot ? a.final_slot[s] : s) * H + h) * kD * kD;

  floatx4 st[8];
  const float init_scale = c.init_pow == 0.0f ? 1.0f : exp2f(c.init_pow * l2);
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    st[n] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    if (c.kv_init) {
#pragma unroll
      for (int m = 0; m < 4; ++m)
        st[n][m] = init_scale * (c.init_transposed
                                     ? c.kv_init[init_off + (int64_t)sp.col() * kD + sp.row(n, m)]
                                     : c.kv_init[init_off + (int64_t)sp.row(n, m) * kD + sp.col()]);
    }
  }

  wide_blocks<kOutF32, kStateOnly, kNorm>(a, c, sm, st);

  if (c.kv_final) {
    const float final_scale = c.final_pow == 0.0f ? 1.0f : exp2f(c.final_pow * l2);
#pragma unroll
    for (int n = 0; n < 8; ++n)
#pragma unroll
      for (int m = 0; m < 4; ++m)
        c.kv_final[final_off + (int64_t)sp.row(n, m) * kD + sp.col()] = final_scale * st[n][m];
  }
}

// LDS of a full chain (kStateOnly: of a state-only chain; kNorm: with the
// output rows of a block for the normalisation).
#define LA_WIDE_LDS(kStateOnly, kNorm)                                                \
  __shared__ __attribute__((aligned(16))) uint16_t Qs_[(kStateOnly) ? 8 : 2 * kTok];  \
  __shared__ __attribute__((aligned(16))) uint16_t Ks_[2 * kTok];                     \
  __shared__ __attribute__((aligned(16))) uint16_t Vs_[2 * kTok];                     \
  __shared__ __attribute__((aligned(16))) uint16_t Ph_[(kStateOnly) ? 8 : kBeta * kBeta]; \
  __shared__ __attribute__((aligned(16))) uint16_t Pl_[(kStateOnly) ? 8 : kBeta * kBeta]; \
  __shared__ __attribute__((aligned(16))) float Ob_[(kNorm) ? kBeta * kD + kD : 4];   \
  const Lds sm{Qs_, Ks_, Vs_, Ph_, Pl_, Ob_}

// Prefill: workgroup i runs the chain of head i % H of the (i / H)-th
// sequence in dispatch order, forwards in time (or backwards, kReverse);
// kNorm: with the output normalisation (forwards, full chains only).
template <bool kOutF32, bool kStateOnly, bool kReverse, bool kNorm = false>
__global__ __launch_bounds__(kThreads) void prefill_wide_kernel(PrefillArgs a) {
  Chain c;
  c.q = a.q;
  c.k = a.k;
  c.v = a.v;
  c.o = a.o;
  c.kv_init = a.kv_init;
  c.kv_final = a.kv_final;
  c.h = blockIdx.x % a.num_heads;
  c.s = seq_of(a, blockIdx.x / a.num_heads);
  c.reverse = kReverse;
  c.init_transposed = false;
  c.init_pow = 0.0f;
  c.final_pow = 0.0f;
  LA_WIDE_LDS(kStateOnly, kNorm);
  wide_chain<kOutF32, kStateOnly, kNorm>(a, c, sm);
}

// The chains of the backward pass in one launch: item i runs pass i % np
// of chain i / np (head chain % H of the (chain / H)-th sequence in dispatch
// order), np = bp.num_passes: all three chains, or the two reverse-time
// output passes of the segmented backward.  The passes of a chain go to one
// XCD, where the two reverse-time passes read the same Q and dO rows at the
// same time.
template <bool kOutF32>
__global__ __launch_bounds__(kThreads) void backward_wide_kernel(PrefillArgs a, BackwardPasses bp) {
  const int np = bp.num_passes;
  const int item = xcd_remap(blockIdx.x, a.num_items, np);
  const int chain = item / np;
  const BackwardPass& p = bp.pass[item - chain * np];
  Chain c;
  c.q = p.q;
  c.k = p.k;
  c.v = p.v;
  c.o = p.o;
  c.kv_init = p.kv_init;
  c.kv_final = p.kv_final;
  c.h = chain % a.num_heads;
  c.s = seq_of(a, chain / a.num_heads);
  c.reverse = p.reverse != 0;
  c.init_transposed = p.init_transposed != 0;
  c.init_pow = p.init_pow;
  c.final_pow = p.final_pow;
  LA_WIDE_LDS(false, false);
  wide_chain<kOutF32, false>(a, c, sm);
}

// ---- the chained scan over segments (one launch) ----
//
// A sequence cut into segments runs as independent (segment, head) items,
// so that few long sequences still fill the GPU.  Item (segment i of a
// sequence, head h), one workgroup:
//   A  the local decayed state of the segment, Shat_i = sum_j
//      lambda^(len_i - 1 - j) k_j^T v_j, by a state-only pass from zero
//      (skipped for the last segment, whose state no later segment needs);
//   B  the state entering the segment, E_i: kv_init (or zero) for i = 0, else
//      read from item i - 1, which publishes E_(i-1) ... as
//      P_(i-1) = lambda^(len_(i-1)) E_(i-1) + Shat_(i-1) = E_i; the item then
//      publishes its own P_i;
//   C  the full blocks of the segment from E_i (O written), and for the last
//      segment the final state.
// This is the local-prefix-sum exchange of the LASP+ sequence split (mizuki
// blog "MiniMax-01：4M 上下文破局", 五) chained inside one launch: only the
// small step B is serial, and an item waits in it only for its predecessor.
//
// Progress.  Items are handed out in the order in which workgroups start (a
// ticket counter), item (g, h) of global segment g being ticket g H + h, and
// an item waits only for the item of the previous segment of its sequence,
// ticket g H + h - H: a workgroup that has already started, whose own wait
// is for a smaller ticket again.  So every wait ends whatever order the
// hardware starts workgroups in and however many of them are resident.  A
// wait is also bounded (spin_limit polls); a wait that runs out sets the
// error word, after which every wait ends at once (results are then
// invalid).
//
// Exchange.  P_i goes to one of two ring slots of its chain (sequence, head),
// slot i % 2, in register order; the flag of the slot then receives i + 1.
// Item i + 1 polls that flag for i + 1, then reads the slot.  Every access to
// the ring and the flags is a device-scope access (sc1 buffer loads and
// stores, agent-scope atomics for the flags: they read from and write to the
// device's coherence point, past the per-XCD L2), and the flag store is
// issued only after every wave's
// ring stores have completed (a wait for the wave's stores, then a workgroup
// barrier).  No cache-wide maintenance is needed: an agent-scope release or
// acquire fence would write back or invalidate a whole L2 per wave, which on
// 32 workgroups of one XCD publishing at once serialises into tens of
// microseconds.  Two slots suffice: item i writes slot i % 2 only after
// reading P_(i-1), which item i - 1 published only after it had read
// P_(i-2) from the slot being overwritten.  The plan kernel zeroes the
// ticket, the error word and the flags before each launch.

// Cache policy of a buffer access at device scope (sc1): it reads from and
// writes to the device's coherence point rather than one XCD's L2.
constexpr int kCpolSc1 = 16;

// Control words of the scan workspace.
constexpr int kCtrlTicket = 0;
constexpr int kCtrlError = 1;
constexpr int kCtrlFlags = 2;  // then 2 flags per (sequence, head) chain

template <bool kOutF32, bool kNorm>
__global__ __launch_bounds__(kThreads) void prefill_scan_kernel(PrefillArgs a, ScanArgs sa) {
  LA_WIDE_LDS(false, kNorm);
  __shared__ int32_t ticket_s;
  const int t = threadIdx.x;
  if (t == 0)
    ticket_s = __hip_atomic_fetch_add(sa.ctrl + kCtrlTicket, 1, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int item = uniform(ticket_s);
  const int H = a.num_heads;
  const int g = item / H;                 // global segment
  const int h = item - g * H;
  const int s = sa.init_slot[g] - g;      // its sequence (the plan's slot of g is g + s)
  const int i = g - sa.seq_first[s];      // its index in the sequence
  const bool last = g + 1 == sa.seq_first[s + 1];
  const int chain = s * H + h;
  const float l2 = a.log2_decay[h];
  const StatePos sp(t);

  Chain c;
  c.q = a.q;
  c.k = a.k;
  c.v = a.v;
  c.o = a.o;
  c.kv_init = nullptr;
  c.kv_final = nullptr;
  c.s = g;  // rows of segment g: a.cu_seqlens is the plan's cu_seg
  c.h = h;
  c.reverse = false;
  c.init_transposed = false;
  c.init_pow = 0.0f;
  c.final_pow = 0.0f;

  // A: the segment's local state
  floatx4 loc[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) loc[n] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  if (!last) wide_blocks<false, true>(a, c, sm, loc);

  // B: the state entering the segment
  floatx4 st[8];
  // ring slot x of this chain (d x d fp32, thread t's tile n at float4
  // n * 512 + t), accessed at device scope
  auto slot_rsrc = [&](int x) {
    return buf_rsrc(sa.ring + ((int64_t)chain * 2 + x) * (kD * kD), kD * kD * 4);
  };
  if (i == 0) {
    const int64_t off = (int64_t)chain * kD * kD;
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      st[n] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
      if (sa.kv_init) {
#pragma unroll
        for (int m = 0; m < 4; ++m) st[n][m] = sa.kv_init[off + (int64_t)sp.row(n, m) * kD + sp.col()];
      }
    }
  } else {
    int32_t* flag = sa.ctrl + kCtrlFlags + 2 * chain + ((i - 1) & 1);
    if (t == 0) {
      for (int polls = 0;; ++polls) {
        if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == i) break;
        if ((polls & 255) == 255 &&
            (polls > sa.spin_limit ||
             __hip_atomic_load(sa.ctrl + kCtrlError, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))) {
          __hip_atomic_store(sa.ctrl + kCtrlError, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    // the ring is read only after the flag was seen (a workgroup-scope
    // acquire keeps the loads below the barrier)
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    const __amdgpu_buffer_rsrc_t src = slot_rsrc((i - 1) & 1);
#pragma unroll
    for (int n = 0; n < 8; ++n)
      st[n] = __builtin_bit_cast(
          floatx4, __builtin_amdgcn_raw_buffer_load_b128(src, 16 * (n * kThreads + t), 0, kCpolSc1));
  }
  if (!last) {
    const int len = a.cu_seqlens[g + 1] - a.cu_seqlens[g];
    const float f = exp2f((float)len * l2);  // lambda^len
    const __amdgpu_buffer_rsrc_t dst = slot_rsrc(i & 1);
#pragma unroll
    for (int n = 0; n < 8; ++n)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, st[n] * f + loc[n]), dst,
                                             16 * (n * kThreads + t), 0, kCpolSc1);
    // every wave waits for its ring stores to complete (a workgroup-scope
    // release does not wait for them on this target), then one flag store
    // for the workgroup
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (t == 0)
      __hip_atomic_store(sa.ctrl + kCtrlFlags + 2 * chain + (i & 1), i + 1, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();

  // C: the segment's outputs from its start state
  wide_blocks<kOutF32, false, kNorm>(a, c, sm, st);
  if (last && sa.kv_final) {
    const int64_t off = (int64_t)chain * kD * kD;
#pragma unroll
    for (int n = 0; n < 8; ++n)
#pragma unroll
      for (int m = 0; m < 4; ++m) sa.kv_final[off + (int64_t)sp.row(n, m) * kD + sp.col()] = st[n][m];
  }
}

}  // namespace

hipError_t launch_prefill_wide(const PrefillArgs& a, la_dtype out_dtype, bool state_only,
                               bool reverse, hipStream_t stream) {
  const dim3 grid(a.num_items), block(kThreads);
  const bool f32 = out_dtype == LA_FP32;
  if (state_only && reverse)
    hipLaunchKernelGGL((prefill_wide_kernel<false, true, true>), grid, block, 0, stream, a);
  else if (state_only)
    hipLaunchKernelGGL((prefill_wide_kernel<false, true, false>), grid, block, 0, stream, a);
  else if (reverse && f32)
    hipLaunchKernelGGL((prefill_wide_kernel<true, false, true>), grid, block, 0, stream, a);
  else if (reverse)
    hipLaunchKernelGGL((prefill_wide_kernel<false, false, true>), grid, block, 0, stream, a);
  else if (f32)
    hipLaunchKernelGGL((prefill_wide_kernel<true, false, false>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((prefill_wide_kernel<false, false, false>), grid, block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_backward_wide(const PrefillArgs& a, const BackwardPasses& bp,
                                la_dtype grad_dtype, hipStream_t stream) {
  const dim3 grid(a.num_items), block(kThreads);
  if (grad_dtype == LA_FP32)
    hipLaunchKernelGGL(backward_wide_kernel<true>, grid, block, 0, stream, a, bp);
  else
    hipLaunchKernelGGL(backward_wide_kernel<false>, grid, block, 0, stream, a, bp);
  return hipGetLastError();
}

hipError_t launch_prefill_scan(const PrefillArgs& a, const ScanArgs& sa, la_dtype out_dtype,
                               bool norm, hipStream_t stream) {
  const dim3 grid(a.num_items), block(kThreads);
  const bool f32 = out_dtype == LA_FP32;
  if (norm && f32)
    hipLaunchKernelGGL((prefill_scan_kernel<true, true>), grid, block, 0, stream, a, sa);
  else if (norm)
    hipLaunchKernelGGL((prefill_scan_kernel<false, true>), grid, block, 0, stream, a, sa);
  else if (f32)
    hipLaunchKernelGGL((prefill_scan_kernel<true, false>), grid, block, 0, stream, a, sa);
  else
    hipLaunchKernelGGL((prefill_scan_kernel<false, false>), grid, block, 0, stream, a, sa);
  return hipGetLastError();
}

hipError_t launch_prefill_wide_normed(const PrefillArgs& a, la_dtype out_dtype,
                                      hipStream_t stream) {
  const dim3 grid(a.num_items), block(kThreads);
  if (out_dtype == LA_FP32)
    hipLaunchKernelGGL((prefill_wide_kernel<true, false, false, true>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((prefill_wide_kernel<false, false, false, true>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace la
