// MFMA issue peak of the GPU, measured (libla_peak.so; not part of la.h and
// not used by the library): a loop of bf16 MFMAs with no memory traffic,
// for the benchmark's measured-peak line.  Each wave keeps eight
// independent 16 x 16 fp32 accumulators and issues, per iteration, one
// v_mfma_f32_16x16x32_bf16 on each, with its own pair of operand vectors,
// so consecutive instructions take different inputs (the operand data
// decides how much the matrix cores switch, and with it how much power the
// loop draws and how fast the board's power limit lets it clock).  Each wave
// also records its shader-clock and constant-clock (100 MHz) counts over the
// loop, from which the clock it ran at follows.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// 16 waves a workgroup (4 per SIMD), at most 128 VGPRs each: with that
// budget the accumulators stay in VGPRs and the loop is eight MFMAs (with
// the larger budget of a smaller workgroup the compiler moves them through
// accumulation registers every iteration).
constexpr int kThreads = 1024;
constexpr int kAcc = 8;

// ops: per thread 2 * kAcc operand vectors (8 bf16 each: A then B operands),
// thread g at ops[16 g .. 16 g + 15]; sums: one float per thread; clocks:
// per wave (shader-clock count, constant-clock count) over the loop.
__global__ __launch_bounds__(kThreads) void mfma_loop_kernel(const bf16x8* __restrict__ ops,
                                                             float* __restrict__ sums,
                                                             int64_t* __restrict__ clocks,
                                                             int iters) {
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  bf16x8 a[kAcc], b[kAcc];
#pragma unroll
  for (int j = 0; j < kAcc; ++j) {
    a[j] = ops[2 * kAcc * gid + j];
    b[j] = ops[2 * kAcc * gid + kAcc + j];
  }
  floatx4 acc[kAcc];
#pragma unroll
  for (int j = 0; j < kAcc; ++j) acc[j] = floatx4{(float)j, 0.0f, 0.0f, 0.0f};
  const int64_t t0 = __builtin_amdgcn_s_memtime();
  const int64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < kAcc; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], b[j], acc[j], 0, 0, 0);
  }
  const int64_t t1 = __builtin_amdgcn_s_memtime();
  const int64_t r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < kAcc; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  sums[gid] = s;
  if ((threadIdx.x & 63) == 0) {
    const int64_t wave = gid >> 6;
    clocks[2 * wave] = t1 - t0;
    clocks[2 * wave + 1] = r1 - r0;
  }
}

// The same loop on v_mfma_f32_16x16x4_f32 (fp32 operands and accumulation):
// ops holds 2 * kAcc floats per thread (A then B operands), thread g at
// ops[16 g .. 16 g + 15].
__global__ __launch_bounds__(kThreads) void mfma_loop_f32_kernel(const float* __restrict__ ops,
                                                                 float* __restrict__ sums,
                                                                 int64_t* __restrict__ clocks,
                                                                 int iters) {
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  float a[kAcc], b[kAcc];
#pragma unroll
  for (int j = 0; j < kAcc; ++j) {
    a[j] = ops[2 * kAcc * gid + j];
    b[j] = ops[2 * kAcc * gid + kAcc + j];
  }
  floatx4 acc[kAcc];
#pragma unroll
  for (int j = 0; j < kAcc; ++j) acc[j] = floatx4{(float)j, 0.0f, 0.0f, 0.0f};
  const int64_t t0 = __builtin_amdgcn_s_memtime();
  const int64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < kAcc; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], acc[j], 0, 0, 0);
  }
  const int64_t t1 = __builtin_amdgcn_s_memtime();
  const int64_t r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < kAcc; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  sums[gid] = s;
  if ((threadIdx.x & 63) == 0) {
    const int64_t wave = gid >> 6;
    clocks[2 * wave] = t1 - t0;
    clocks[2 * wave + 1] = r1 - r0;
  }
}

}  // namespace

extern "C" {

// Enqueues one launch of `workgroups` workgroups of 1024 threads on
// `stream` (a hipStream_t; NULL: the default stream).  ops: device bf16
// [workgroups * 1024 * 128] (16-byte aligned); sums: device fp32
// [workgroups * 1024]; clocks: device int64 [workgroups * 16 * 2].  Each
// wave issues iters * 8 MFMAs of 16 * 16 * 32 * 2 flops.  Returns the HIP error
// code of the launch (0 = success); nothing is checked beyond iters >= 0
// and workgroups > 0.
__attribute__((visibility("default"))) int la_peak_mfma_bf16(const void* ops, float* sums,
                                                               int64_t* clocks, int workgroups,
                                                               int iters, void* stream) {
  if (workgroups <= 0 || iters < 0 || !ops || !sums || !clocks)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(workgroups), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const bf16x8*>(ops), sums,
                     clocks, iters);
  return (int)hipGetLastError();
}

// As la_peak_mfma_bf16 for the fp32 loop: ops device fp32
// [workgroups * 1024 * 16]; each wave issues iters * 8 MFMAs of 16 * 16 * 4 * 2
// flops.
__attribute__((visibility("default"))) int la_peak_mfma_f32(const void* ops, float* sums,
                                                              int64_t* clocks, int workgroups,
                                                              int iters, void* stream) {
  if (workgroups <= 0 || iters < 0 || !ops || !sums || !clocks)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_loop_f32_kernel, dim3(workgroups), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const float*>(ops), sums,
                     clocks, iters);
  return (int)hipGetLastError();
}

}  // extern "C"
