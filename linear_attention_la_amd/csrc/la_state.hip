// Per-head scaled copy, optionally transposed, of fp32 d x d states.  The
// d = 64 backward feeds the forward kernel with transformed states: S0^T for
// dQ, dS_L^T / lambda and dS_L / lambda for dK and dV, and scales the last
// state by lambda to obtain dS0.  (For d = 128 the backward kernel reads and
// writes the states in these forms itself.)

#include "la_backward.h"
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

// Workgroup (state, tile row, tile column), 256 threads, one 32 x 32 tile:
// thread t moves the 4 consecutive elements (4 (t % 8) .. + 3) of tile row
// t / 8 with one 16-byte load and one 16-byte store.  The transposed path
// goes through a padded LDS tile: a thread writes its input quad into 4 LDS
// rows (one per column) and reads back 4 consecutive elements of one output
// row.
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
  const int row = threadIdx.x / 8, q4 = 4 * (threadIdx.x % 8);  // row in [0, 32), quad start
  const float4 x =
      *reinterpret_cast<const float4*>(a.in + base + (int64_t)(tr * kTile + row) * d + tc * kTile + q4);
  if (!kTranspose) {
    *reinterpret_cast<float4*>(a.out + base + (int64_t)(tr * kTile + row) * d + tc * kTile + q4) =
        make_float4(f * x.x, f * x.y, f * x.z, f * x.w);
    return;
  }
  tile[q4][row] = x.x;
  tile[q4 + 1][row] = x.y;
  tile[q4 + 2][row] = x.z;
  tile[q4 + 3][row] = x.w;
  __syncthreads();
  // out[c][r] = in[r][c]: tile (tr, tc) of the input lands at tile (tc, tr);
  // LDS row c of the tile now holds input column c
  *reinterpret_cast<float4*>(a.out + base + (int64_t)(tc * kTile + row) * d + tr * kTile + q4) =
      make_float4(f * tile[row][q4], f * tile[row][q4 + 1], f * tile[row][q4 + 2],
                  f * tile[row][q4 + 3]);
}

// In-place transpose with a per-head scale: workgroup (state, tile pair)
// with tile row tr <= tile column tc loads tiles (tr, tc) and (tc, tr) into
// LDS before writing either, then writes each, transposed, over the other
// (a diagonal tile over itself).  Different workgroups touch disjoint tiles.
__global__ __launch_bounds__(256) void state_transpose_inplace_kernel(StateArgs a, int d) {
  __shared__ float tile[2][kTile][kTile + 1];
  const int pairs = a.tiles * (a.tiles + 1) / 2;
  const int sh = blockIdx.x / pairs;
  int p = blockIdx.x % pairs, tr = 0;
  while (p >= a.tiles - tr) {  // pairs of tile row tr: tc = tr .. tiles - 1
    p -= a.tiles - tr;
    ++tr;
  }
  const int tc = tr + p;
  const int h = sh % a.num_heads;
  float* x = a.out + (int64_t)sh * d * d;
  const float f = a.scale[h];
  const int row = threadIdx.x / 8, q4 = 4 * (threadIdx.x % 8);
  const int nt = tr == tc ? 1 : 2;
  for (int i = 0; i < nt; ++i) {  // tile 0 = (tr, tc), tile 1 = (tc, tr)
    const int r0 = i ? tc : tr, c0 = i ? tr : tc;
    const float4 v = *reinterpret_cast<const float4*>(x + (int64_t)(r0 * kTile + row) * d + c0 * kTile + q4);
    tile[i][q4][row] = v.x;
    tile[i][q4 + 1][row] = v.y;
    tile[i][q4 + 2][row] = v.z;
    tile[i][q4 + 3][row] = v.w;
  }
  __syncthreads();
  for (int i = 0; i < nt; ++i) {  // the transpose of tile (r0, c0) goes to (c0, r0)
    const int r0 = i ? tc : tr, c0 = i ? tr : tc;
    *reinterpret_cast<float4*>(x + (int64_t)(c0 * kTile + row) * d + r0 * kTile + q4) =
        make_float4(f * tile[i][row][q4], f * tile[i][row][q4 + 1], f * tile[i][row][q4 + 2],
                    f * tile[i][row][q4 + 3]);
  }
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

hipError_t launch_state_transpose_inplace(float* x, int32_t num_states, int32_t num_heads,
                                          int32_t head_dim, const float* scale,
                                          hipStream_t stream) {
  StateArgs a;
  a.in = x;
  a.out = x;
  a.num_heads = num_heads;
  a.tiles = head_dim / kTile;
  for (int h = 0; h < num_heads; ++h) a.scale[h] = scale[h];
  const int64_t blocks = (int64_t)num_states * (a.tiles * (a.tiles + 1) / 2);
  hipLaunchKernelGGL(state_transpose_inplace_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     a, head_dim);
  return hipGetLastError();
}

}  // namespace la
