// Device-side helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// fp32 -> bf16 bits, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, static_cast<uint32_t>(b) << 16);
}

// Two floats -> one dword of two bf16 (lo = a, hi = b), RNE.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return static_cast<uint32_t>(f32_to_bf16_bits(a)) |
         (static_cast<uint32_t>(f32_to_bf16_bits(b)) << 16);
}

// Low / high bf16 of a dword as float.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) {
  return __builtin_bit_cast(float, w & 0xFFFF0000u);
}

// Workgroup index remap so that consecutive work items land on one XCD.
// The hardware deals workgroups round-robin over the 8 XCDs (workgroup x goes
// to XCD x % 8).  Items are grouped in runs of `run` (the column slices of one
// (sequence, head) chain read the same Q and K rows); a run is placed on one
// XCD so its slices share that XCD's L2.  Bijective on [0, n); the tail that
// does not fill a whole 8 * run group keeps the identity map.
__device__ __forceinline__ int xcd_remap(int x, int n, int run) {
  const int group = 8 * run;
  const int full = (n / group) * group;
  if (x >= full) return x;
  const int a = x / group;
  const int rem = x - a * group;
  const int slice = rem / 8;
  const int xcd = rem - slice * 8;
  return (a * 8 + xcd) * run + slice;
}

}  // namespace la
