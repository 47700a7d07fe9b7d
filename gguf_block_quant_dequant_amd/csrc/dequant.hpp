// Standalone dequantization kernels: blocks -> fp32 (or bf16) row-major.
// One thread produces 4 consecutive weights, so every thread issues one
// 16-byte (fp32) or 8-byte (bf16) store and a wave writes a contiguous 1 KiB
// (512 B) span: the kernel is bound by the output stream.
#pragma once

#include "device_common.hpp"

namespace gqk {

// Q8_0: weight = int8 q * fp16 d; the product is exact in fp32.
__global__ __launch_bounds__(256) void dequant_q8_0_kernel(const uint8_t* __restrict__ W,
                                                           float4* __restrict__ out,
                                                           int64_t n_quads) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n_quads) return;
  const int64_t blk = t >> 3;               // 8 quads per 32-weight block
  const int i0 = (int)(t & 7) * 4;          // first weight of this quad in the block
  const uint8_t* b = W + blk * kQ80BlockBytes;
  const uint16_t* b16 = reinterpret_cast<const uint16_t*>(b);   // blocks are 2-byte aligned
  const float d = half_lo(b16[0]);
  const uint32_t q = (uint32_t)b16[1 + i0 / 2] | ((uint32_t)b16[2 + i0 / 2] << 16);
  out[t] = make_float4(sbyte0(q) * d, sbyte1(q) * d, sbyte2(q) * d, sbyte3(q) * d);
}

// Q4_K: weight i of super-block s, sub-block j = i / 32:
//   w = d*sc[j]*q - dmin*m[j], with d*sc[j] and dmin*m[j] exact in fp32;
// the fused multiply-add rounds the exact difference once.
template <bool kBf16>
__device__ __forceinline__ void q4k_quad(const uint8_t* __restrict__ W, int64_t t, float (&w)[4]) {
  const int64_t sb = t >> 6;                 // 64 quads per super-block
  const int qi = (int)(t & 63);
  const int i0 = qi * 4;                     // first weight in the super-block
  const int j = i0 >> 5;                     // sub-block
  const int g = j >> 1, hi = j & 1, l0 = i0 & 31;
  const uint32_t* h = reinterpret_cast<const uint32_t*>(W + sb * kQ4KBlockBytes);
  float dsc[8], dmm[8];
  q4k_scales(h[0], h[1], h[2], h[3], dsc, dmm);
  const uint32_t qb = h[4 + (32 * g + l0) / 4];
  const uint32_t q = opaque(hi ? ((qb >> 4) & 0x0F0F0F0Fu) : (qb & 0x0F0F0F0Fu));
  w[0] = fmaf(dsc[j], ubyte0(q), -dmm[j]);
  w[1] = fmaf(dsc[j], ubyte1(q), -dmm[j]);
  w[2] = fmaf(dsc[j], ubyte2(q), -dmm[j]);
  w[3] = fmaf(dsc[j], ubyte3(q), -dmm[j]);
}

__global__ __launch_bounds__(256) void dequant_q4_k_kernel(const uint8_t* __restrict__ W,
                                                           float4* __restrict__ out,
                                                           int64_t n_quads) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n_quads) return;
  float w[4];
  q4k_quad<false>(W, t, w);
  out[t] = make_float4(w[0], w[1], w[2], w[3]);
}

__global__ __launch_bounds__(256) void dequant_q4_k_bf16_kernel(const uint8_t* __restrict__ W,
                                                                uint2* __restrict__ out,
                                                                int64_t n_quads) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n_quads) return;
  float w[4];
  q4k_quad<true>(W, t, w);
  out[t] = make_uint2(pack_bf16x2(w[0], w[1]), pack_bf16x2(w[2], w[3]));
}

}  // namespace gqk
