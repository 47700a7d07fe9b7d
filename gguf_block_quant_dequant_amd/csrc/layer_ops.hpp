// The steps either side of the decode GEMVs as standalone kernels ("GGUF
// Inferencer in R", section 5.2): RMSN(v) = norm * v / sqrt(mean(v^2) + eps),
// the gated activation SiLU(G) * U with SiLU(x) = x / (1 + exp(-x)), the
// residual add, and the input half of a fused RMSN (v * norm and the partial
// sums of v^2 per 64 elements, the form the GEMV epilogue consumes). The
// partial sums use the same 64-lane butterfly as the GEMV epilogue, so both
// paths give the same bits.
#pragma once

#include "device_common.hpp"

namespace gqk {

__device__ __forceinline__ float wave_sum64(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

// x * x rounded on its own (kept out of a following add, which could take it
// unrounded as an fma), as the GEMV epilogue squares its outputs.
__device__ __forceinline__ float square_rounded(float x) {
  float sq = x * x;
  asm volatile("" : "+v"(sq));
  return sq;
}

// vw = v * norm_w; ss[j] = sum of v^2 over elements 64 j .. 64 j + 63.
// One wave per 64 elements.
__global__ __launch_bounds__(256) void rmsnorm_prep_kernel(const float* __restrict__ v,
                                                           const float* __restrict__ w,
                                                           float* __restrict__ vw,
                                                           float* __restrict__ ss, int64_t n) {
  const int lane = threadIdx.x & 63;
  const int64_t j = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t i = j * 64 + lane;
  if (j * 64 >= n) return;
  const bool live = i < n;
  const float x = live ? v[i] : 0.f;
  if (live) vw[i] = x * w[i];
  const float s = wave_sum64(square_rounded(x));
  if (lane == 0) ss[j] = s;
}

// out = norm_w * v / sqrt(mean(v^2) + eps) for one vector, one block of 16
// waves: each wave sums the squares of its 64-element groups (as above) into
// LDS, thread 0 adds the group sums in order (up to kNormGroups per pass).
constexpr int kNormGroups = 1024;
__global__ __launch_bounds__(1024) void rmsnorm_kernel(const float* __restrict__ v,
                                                       const float* __restrict__ w, float eps,
                                                       float* __restrict__ out, int64_t n) {
  __shared__ float part[kNormGroups];
  __shared__ float scale;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t ngroups = (n + 63) / 64;
  float total = 0.f;   // thread 0's running sum
  for (int64_t g0 = 0; g0 < ngroups; g0 += kNormGroups) {
    const int gn = (int)((ngroups - g0) < kNormGroups ? (ngroups - g0) : kNormGroups);
    for (int j = wave; j < gn; j += 16) {
      const int64_t i = (g0 + j) * 64 + lane;
      const float s = wave_sum64(square_rounded(i < n ? v[i] : 0.f));
      if (lane == 0) part[j] = s;
    }
    __syncthreads();
    if (threadIdx.x == 0)
      for (int j = 0; j < gn; ++j) total += part[j];
    __syncthreads();
  }
  if (threadIdx.x == 0) scale = 1.0f / sqrtf(total * (1.0f / (float)n) + eps);
  __syncthreads();
  const float sc = scale;
  for (int64_t i = threadIdx.x; i < n; i += 1024) out[i] = v[i] * w[i] * sc;
}

__global__ __launch_bounds__(256) void swiglu_kernel(const float* __restrict__ g,
                                                     const float* __restrict__ u,
                                                     float* __restrict__ out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const float gv = g[i];
  out[i] = gv / (1.0f + expf(-gv)) * u[i];
}

__global__ __launch_bounds__(256) void add_kernel(const float* __restrict__ a,
                                                  const float* __restrict__ b,
                                                  float* __restrict__ out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = a[i] + b[i];
}

}  // namespace gqk
