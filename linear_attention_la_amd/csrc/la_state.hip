// Per-head scaled copy, optionally transposed, of fp32 d x d states.  The
// backward pass feeds the forward kernel with transformed states: S0^T for
// dQ, dS_L^T / lambda and dS_L / lambda for dK and dV, and scales the last
// state by lambda to obtain dS0.

#include "la_internal.h"

namespace la {
namespace {

constexpr int kTile = 32;

struct StateArgs {
  const float* in;
  float* out;
  int32_t num_heads;
  int32_t tiles;  // tiles per row of a state (d / 32)
  float scale[LA_MAX_HEADS];
};

// Workgroup (state, tile row, tile column), 32 x 8 threads; each thread
// moves 4 elements of a 32 x 32 tile.  The transposed path goes through a
// padded LDS tile so that reads and writes stay row-contiguous.
template <bool kTranspose>
__global__ __launch_bounds__(256) void state_transform_kernel(StateArgs a, int d) {
  __shared__ float tile[kTile][kTile + 1];
  const int per_state = a.tiles * a.tiles;
  const int sh = blockIdx.x / per_state;
  const int tr = (blockIdx.x % per_state) / a.tiles;
  const int tc = blockIdx.x % a.tiles;
  const int h = sh % a.num_heads;
  const int64_t base = (int64_t)sh * d * d;
  const float f = a.scale[h];
  const int x = threadIdx.x % kTile, y = threadIdx.x / kTile;  // y in [0, 8)
  if (!kTranspose) {
#pragma unroll
    for (int i = 0; i < kTile; i += 8) {
      const int64_t idx = base + (int64_t)(tr * kTile + y + i) * d + tc * kTile + x;
      a.out[idx] = f * a.in[idx];
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < kTile; i += 8)
    tile[y + i][x] = a.in[base + (int64_t)(tr * kTile + y + i) * d + tc * kTile + x];
  __syncthreads();
  // out[c][r] = in[r][c]: tile (tr, tc) of the input lands at tile (tc, tr)
#pragma unroll
  for (int i = 0; i < kTile; i += 8)
    a.out[base + (int64_t)(tc * kTile + y + i) * d + tr * kTile + x] = f * tile[x][y + i];
}

}  // namespace

hipError_t launch_state_transform(const float* in, float* out, int32_t num_states,
                                  int32_t num_heads, int32_t head_dim, bool transpose,
                                  const float* scale, hipStream_t stream) {
  StateArgs a;
  a.in = in;
  a.out = out;
  a.num_heads = num_heads;
  a.tiles = head_dim / kTile;
  for (int h = 0; h < num_heads; ++h) a.scale[h] = scale[h];
  const int64_t blocks = (int64_t)num_states * num_heads * a.tiles * a.tiles;
  if (transpose)
    hipLaunchKernelGGL(state_transform_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       a, head_dim);
  else
    hipLaunchKernelGGL(state_transform_kernel<false>, dim3((unsigned)blocks), dim3(256), 0,
                       stream, a, head_dim);
  return hipGetLastError();
}

}  // namespace la
