// Streaming-read probe: the achievable HBM read bandwidth of this device for
// a pure read stream with the same 16-byte vector loads the GEMV kernels use.
#pragma once

#include "device_common.hpp"

namespace gqk {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 4;

__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const u32x4* __restrict__ p,
                                                                   int64_t n16,
                                                                   uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // Never true for the probe's zero-filled buffers; keeps the loads alive.
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

// Latency probe: one wave; lane l starts at entry l and follows the chain
// i = next[i] & mask `steps` times, each load waiting for the one before (the
// lanes' loads of a step go out together). The mask keeps every index inside
// the buffer whatever it holds. out[0]: elapsed ticks of the constant 100 MHz
// clock; out[1]: lane 0's last index (keeps the chain alive).
__global__ __launch_bounds__(64) void probe_chase_kernel(const uint32_t* __restrict__ next, uint32_t mask,
                                                         int64_t steps, uint64_t* __restrict__ out) {
  uint32_t i = threadIdx.x & mask;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (int64_t s = 0; s < steps; ++s) i = next[i] & mask;
  asm volatile("" : "+v"(i));   // the last load is complete before the second stamp
  const uint64_t t1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    out[0] = t1 - t0;
    out[1] = i;
  }
}

}  // namespace gqk
