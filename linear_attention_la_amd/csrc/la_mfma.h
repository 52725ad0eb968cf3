// Device helpers shared by the bf16 prefill kernels for gfx950: MFMA and LDS
// access wrappers, the hi/lo bf16 split, raw buffer resources and the LDS
// swizzles that both kernels use for K and Q rows.
#pragma once

#include <type_traits>

#include "la_device.h"

namespace la {

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

// Transposed 4-element read (ds_read_b64_tr_b16); p must be 8 B aligned.  In
// each 16-lane group, lane 4r + a gives the address of 4 consecutive elements
// (piece a) of row r; lane i then receives element i of the 16 elements that
// the four pieces form, from each of the 4 rows.
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

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Raw buffer resource over [base, base + bytes).  Buffer loads outside the
// range return zero and stores outside it are dropped, so every memory
// instruction of a block is issued unconditionally: rows past the end of a
// sequence need no branch, and the number of outstanding vector-memory
// operations is the same on every path, which lets each wait count only
// the operations it needs (a data-dependent count forces waiting for all).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// Swizzle of the 16 B chunks of a K row: a permutation of the bits of the
// row index, chosen so that three patterns are free of bank conflicts:
//  * one chunk of 16 consecutive rows (MFMA operand reads, 16 B per lane),
//  * four chunks of 8 consecutive rows (transposed reads, 8 B per lane, with
//    the row pieces that srow() below assigns), and
//  * whole rows (staging writes).
template <int D>
__device__ __forceinline__ int kswz(int r);
template <>
__device__ __forceinline__ int kswz<128>(int r) {
  return (r & 1) | ((r & 6) << 1) | ((r & 8) >> 2);
}
template <>
__device__ __forceinline__ int kswz<64>(int r) {
  return ((r & 2) >> 1) | (r & 4) | ((r & 8) >> 2);
}
// Element offset of 16 B chunk c of K row r.
template <int D>
__device__ __forceinline__ int qk_off(int r, int c) {
  return r * D + 8 * (c ^ kswz<D>(r));
}


// First of the 4 consecutive key rows of state tile n held by lane group g
// (accumulator rows 4g .. 4g+3).  Tiles 2p and 2p+1 together give group g
// the 8 rows 32p + 8g .. 32p + 8g + 7, so that a lane writes its state^T
// values as one 16 B chunk; tile 2p takes the lower half for even g and the
// upper half for odd g, which spreads the transposed K reads of a tile over
// both 8 B halves of every chunk.
__device__ __forceinline__ int srow(int n, int g) {
  return 32 * (n >> 1) + 8 * g + 4 * ((n & 1) ^ (g & 1));
}

// Workgroup barrier for LDS traffic only.  __syncthreads() also waits for
// every outstanding global store and load of the wave (vmcnt(0)); here the
// waves that store O never need to wait for those stores, and the waves that
// prefetch the next block wait for their loads only where they use them.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int N>
using IC = std::integral_constant<int, N>;

}  // namespace la
