// Prefill: Y[n, r] = sum_k X[n, k] W[r, k], X and Y bf16, W Q4_K, on the
// gfx950 matrix cores (v_mfma_f32_32x32x16_bf16, fp32 accumulation).
//
// Block tile: 128 tokens x 128 weight rows, K consumed 64 at a time (one
// sub-block pair of a super-block). Per step every thread stages 32 bf16 of X
// and decodes 32 weights of W (fp32 dequant rounded to nearest-even bf16) into
// LDS; the four waves then each multiply a 64x64 sub-tile as 2x2 MFMA tiles.
// LDS rows are padded to 144 bytes (36 dwords, 4 modulo 32 banks) so the
// 16-byte operand reads of 32 consecutive rows are conflict-free.
//
// MFMA operand layout used (32x32x16): lane l supplies A[i = l % 32][8 k] and
// B[8 k][j = l % 32] from k-group l / 32; because A and B are fed with the
// same (k-group, element) labels the product is independent of how the
// hardware orders k inside a group. Accumulator element e of lane l is
// D[8 (e / 4) + 4 (l / 32) + e % 4][l % 32].
#pragma once

#include "device_common.hpp"

namespace gqk {

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr int kGemmBM = 128;
constexpr int kGemmBN = 128;
constexpr int kGemmBK = 64;
constexpr int kGemmLdsRow = kGemmBK * 2 + 16;   // 144 bytes

__global__ __launch_bounds__(256) void gemm_q4_k_kernel(const uint8_t* __restrict__ W,
                                                        const uint16_t* __restrict__ X,
                                                        uint16_t* __restrict__ Y, int64_t n_tokens,
                                                        int64_t rows, int nsb) {
  __shared__ __attribute__((aligned(16))) uint8_t xs[kGemmBM * kGemmLdsRow];
  __shared__ __attribute__((aligned(16))) uint8_t ws[kGemmBN * kGemmLdsRow];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wi = wave >> 1, wj = wave & 1;
  const int64_t n0 = (int64_t)blockIdx.y * kGemmBM;
  const int64_t r0 = (int64_t)blockIdx.x * kGemmBN;
  const int64_t K = (int64_t)nsb * kQ4KBlockWeights;
  const int64_t row_bytes = (int64_t)nsb * kQ4KBlockBytes;

  const int ld_row = tid >> 1, ld_half = tid & 1;
  const int64_t xr = (n0 + ld_row) < n_tokens ? (n0 + ld_row) : (n_tokens - 1);
  const int64_t wr = (r0 + ld_row) < rows ? (r0 + ld_row) : (rows - 1);
  const uint16_t* xrow = X + xr * K + 32 * ld_half;
  const uint8_t* wrow = W + wr * row_bytes;

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;

  for (int64_t k0 = 0; k0 < K; k0 += kGemmBK) {
    const int64_t s = k0 >> 8;
    const int g = (int)((k0 >> 6) & 3);
    const uint4* xp = reinterpret_cast<const uint4*>(xrow + k0);
    const uint4 xv0 = xp[0], xv1 = xp[1], xv2 = xp[2], xv3 = xp[3];
    const uint8_t* sb = wrow + s * kQ4KBlockBytes;
    const uint4 hdr = *reinterpret_cast<const uint4*>(sb);
    const uint4 qv = *reinterpret_cast<const uint4*>(sb + 16 + 32 * g + 16 * ld_half);
    float dsc[8], dmm[8];
    q4k_scales(hdr.x, hdr.y, hdr.z, hdr.w, dsc, dmm);
    const float dl = dsc[2 * g], ml = dmm[2 * g], dh = dsc[2 * g + 1], mh = dmm[2 * g + 1];
    const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
    uint32_t lo_bf[8], hi_bf[8];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t lo = opaque(qw[t] & 0x0F0F0F0Fu);
      const uint32_t hi = opaque((qw[t] >> 4) & 0x0F0F0F0Fu);
      lo_bf[2 * t] = pack_bf16x2(fmaf(dl, ubyte0(lo), -ml), fmaf(dl, ubyte1(lo), -ml));
      lo_bf[2 * t + 1] = pack_bf16x2(fmaf(dl, ubyte2(lo), -ml), fmaf(dl, ubyte3(lo), -ml));
      hi_bf[2 * t] = pack_bf16x2(fmaf(dh, ubyte0(hi), -mh), fmaf(dh, ubyte1(hi), -mh));
      hi_bf[2 * t + 1] = pack_bf16x2(fmaf(dh, ubyte2(hi), -mh), fmaf(dh, ubyte3(hi), -mh));
    }
    __syncthreads();   // the previous step's operand reads are done
    uint4* xd = reinterpret_cast<uint4*>(xs + ld_row * kGemmLdsRow + 64 * ld_half);
    xd[0] = xv0; xd[1] = xv1; xd[2] = xv2; xd[3] = xv3;
    // low nibbles: k = 16 ld_half + 0..15 of this 64-k step; high: 32 + 16 ld_half + 0..15
    uint4* wl = reinterpret_cast<uint4*>(ws + ld_row * kGemmLdsRow + 32 * ld_half);
    uint4* wh = reinterpret_cast<uint4*>(ws + ld_row * kGemmLdsRow + 64 + 32 * ld_half);
    wl[0] = make_uint4(lo_bf[0], lo_bf[1], lo_bf[2], lo_bf[3]);
    wl[1] = make_uint4(lo_bf[4], lo_bf[5], lo_bf[6], lo_bf[7]);
    wh[0] = make_uint4(hi_bf[0], hi_bf[1], hi_bf[2], hi_bf[3]);
    wh[1] = make_uint4(hi_bf[4], hi_bf[5], hi_bf[6], hi_bf[7]);
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kGemmBK; kk += 16) {
      const int kb = (kk + 8 * (lane >> 5)) * 2;
      bf16x8 a[2], b[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        a[t] = *reinterpret_cast<const bf16x8*>(xs + (wi * 64 + t * 32 + (lane & 31)) * kGemmLdsRow + kb);
        b[t] = *reinterpret_cast<const bf16x8*>(ws + (wj * 64 + t * 32 + (lane & 31)) * kGemmLdsRow + kb);
      }
#pragma unroll
      for (int it = 0; it < 2; ++it)
#pragma unroll
        for (int jt = 0; jt < 2; ++jt)
          acc[it][jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[it], b[jt], acc[it][jt], 0, 0, 0);
    }
  }

#pragma unroll
  for (int it = 0; it < 2; ++it)
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
      const int64_t r = r0 + wj * 64 + jt * 32 + (lane & 31);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t n = n0 + wi * 64 + it * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        if (n < n_tokens && r < rows) Y[n * rows + r] = to_bf16(acc[it][jt][e]);
      }
    }
}

}  // namespace gqk
