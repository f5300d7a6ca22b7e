// Row-wise L2 normalisation (QK-norm), forward and backward, gfx950.
//
// "Training GEM at LLM scale" (Meta engineering post), section "Generalized
// Dot-Product Attention (GDPA)", item on the ALU-only activation: the
// polynomial GELU relies on the bounded scores that QK-norm (query/key
// normalisation) enforces.  Every row of D elements (one token of one head)
// becomes  y = x r,  r = 1 / max(||x||_2, eps);  the backward is
// dx = r (dy - y (y . dy)), the projection term only where ||x|| > eps.
//
// HBM-bound streaming kernels: a group of D/8 lanes owns a row, each lane 8
// consecutive elements (one 16-byte load in bf16, two in fp32); the row sums
// are reduced inside the group with lane exchanges, and a grid-stride loop
// covers every row.  A group's lanes read their whole row before any of them
// writes, so the output may alias the input when the element types match.
#include "common.hpp"
#include "kernels.hpp"

namespace jattn {
namespace {

constexpr float kL2Eps = 1e-12f;

__device__ __forceinline__ void load8(const bf16* p, float* v) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] = __uint_as_float(w[j] << 16);
    v[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float* v) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[j] = a[j];
    v[4 + j] = b[j];
  }
}
__device__ __forceinline__ void store8(bf16* p, const float* v) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (bf16)v[j];
  *reinterpret_cast<bf16x8*>(p) = r;
}
__device__ __forceinline__ void store8(float* p, const float* v) {
  *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
  *reinterpret_cast<f32x4*>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
}

// sum over the G lanes of an aligned lane group
template <int G>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int m = G / 2; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

template <typename TX, typename TY, int D>
__global__ __launch_bounds__(256) void l2norm_fwd_kernel(const TX* __restrict__ x, TY* y, float* rnorm,
                                                         int64_t rows) {
  constexpr int G = D / 8;        // lanes per row
  constexpr int RPB = 256 / G;    // rows per workgroup pass
  const int gl = threadIdx.x % G;
  for (int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / G; row < rows; row += (int64_t)gridDim.x * RPB) {
    float v[8];
    load8(x + row * D + gl * 8, v);
    float ss = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) ss = fmaf(v[j], v[j], ss);
    ss = group_sum<G>(ss);
    const float r = 1.0f / fmaxf(sqrtf(ss), kL2Eps);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] *= r;
    store8(y + row * D + gl * 8, v);
    if (rnorm != nullptr && gl == 0) rnorm[row] = r;
  }
}

template <typename TX, typename TG, typename TD, int D>
__global__ __launch_bounds__(256) void l2norm_bwd_kernel(const TX* __restrict__ x, const TG* dy, TD* dx,
                                                         int64_t rows) {
  constexpr int G = D / 8;
  constexpr int RPB = 256 / G;
  const int gl = threadIdx.x % G;
  for (int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / G; row < rows; row += (int64_t)gridDim.x * RPB) {
    float v[8], g[8];
    load8(x + row * D + gl * 8, v);
    load8(dy + row * D + gl * 8, g);
    float ss = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) ss = fmaf(v[j], v[j], ss);
    ss = group_sum<G>(ss);
    const float n = sqrtf(ss);
    const float r = 1.0f / fmaxf(n, kL2Eps);
    float dot = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) dot = fmaf(v[j] * r, g[j], dot);
    dot = group_sum<G>(dot);
    if (!(n > kL2Eps)) dot = 0.0f;  // y = x / eps is linear there
#pragma unroll
    for (int j = 0; j < 8; ++j) g[j] = r * (g[j] - v[j] * r * dot);
    store8(dx + row * D + gl * 8, g);
  }
}

int grid_for(int64_t rows, int D) {
  const int64_t rpb = 256 / (D / 8);
  const int64_t need = (rows + rpb - 1) / rpb;
  return (int)(need < 8192 ? (need > 0 ? need : 1) : 8192);
}

template <int D>
hipError_t fwd_d(const void* x, void* y, float* rnorm, int64_t rows, bool x_f32, bool y_f32, hipStream_t st) {
  const int grid = grid_for(rows, D);
  if (x_f32 && y_f32)
    hipLaunchKernelGGL((l2norm_fwd_kernel<float, float, D>), dim3(grid), dim3(256), 0, st, (const float*)x, (float*)y, rnorm, rows);
  else if (x_f32)
    hipLaunchKernelGGL((l2norm_fwd_kernel<float, bf16, D>), dim3(grid), dim3(256), 0, st, (const float*)x, (bf16*)y, rnorm, rows);
  else if (y_f32)
    hipLaunchKernelGGL((l2norm_fwd_kernel<bf16, float, D>), dim3(grid), dim3(256), 0, st, (const bf16*)x, (float*)y, rnorm, rows);
  else
    hipLaunchKernelGGL((l2norm_fwd_kernel<bf16, bf16, D>), dim3(grid), dim3(256), 0, st, (const bf16*)x, (bf16*)y, rnorm, rows);
  return hipGetLastError();
}

template <typename TX, typename TG, int D>
hipError_t bwd_dx(const void* x, const void* dy, void* dx, int64_t rows, bool dx_f32, hipStream_t st) {
  const int grid = grid_for(rows, D);
  if (dx_f32)
    hipLaunchKernelGGL((l2norm_bwd_kernel<TX, TG, float, D>), dim3(grid), dim3(256), 0, st, (const TX*)x, (const TG*)dy, (float*)dx, rows);
  else
    hipLaunchKernelGGL((l2norm_bwd_kernel<TX, TG, bf16, D>), dim3(grid), dim3(256), 0, st, (const TX*)x, (const TG*)dy, (bf16*)dx, rows);
  return hipGetLastError();
}

template <int D>
hipError_t bwd_d(const void* x, const void* dy, void* dx, int64_t rows, bool x_f32, bool dy_f32, bool dx_f32,
                 hipStream_t st) {
  if (x_f32) return dy_f32 ? bwd_dx<float, float, D>(x, dy, dx, rows, dx_f32, st) : bwd_dx<float, bf16, D>(x, dy, dx, rows, dx_f32, st);
  return dy_f32 ? bwd_dx<bf16, float, D>(x, dy, dx, rows, dx_f32, st) : bwd_dx<bf16, bf16, D>(x, dy, dx, rows, dx_f32, st);
}

}  // namespace

hipError_t launch_l2norm_fwd(const void* x, void* y, float* rnorm, int64_t rows, int D, bool x_f32, bool y_f32,
                             hipStream_t st) {
  if (D == 128) return fwd_d<128>(x, y, rnorm, rows, x_f32, y_f32, st);
  if (D == 64) return fwd_d<64>(x, y, rnorm, rows, x_f32, y_f32, st);
  return fwd_d<32>(x, y, rnorm, rows, x_f32, y_f32, st);
}

hipError_t launch_l2norm_bwd(const void* x, const void* dy, void* dx, int64_t rows, int D, bool x_f32, bool dy_f32,
                             bool dx_f32, hipStream_t st) {
  if (D == 128) return bwd_d<128>(x, dy, dx, rows, x_f32, dy_f32, dx_f32, st);
  if (D == 64) return bwd_d<64>(x, dy, dx, rows, x_f32, dy_f32, dx_f32, st);
  return bwd_d<32>(x, dy, dx, rows, x_f32, dy_f32, dx_f32, st);
}

}  // namespace jattn
