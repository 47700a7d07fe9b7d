// Q4_0 and Q6_K: standalone dequantization and the batch-1 GEMV
// y[r] = sum_k w[r,k] x[k] (the other block types of GGUF files).
//
// Formats (GGUF's on-disk layout; the block sizes are the pages'):
//   Q4_0  18-byte blocks of 32 weights: fp16 d, then 16 bytes; byte j holds the
//         code of weight j in its low nibble and of weight j + 16 in its high
//         nibble; w = (code - 8) d.
//   Q6_K  210-byte super-blocks of 256 weights: ql[128] low 4 bits of the 6-bit
//         codes, qh[64] high 2 bits, sc[16] int8 scales of 16 weights each,
//         fp16 d at byte 208. For half n and l = 0..31 (L = ql + 64 n,
//         H = qh + 32 n), weight 128 n + 32 k + l has low bits
//         (k even: L[l], k odd: L[l + 32]) >> (k < 2 ? 0 : 4) and high bits
//         (H[l] >> 2 k) & 3; w = d sc[i / 16] (code - 32).
// Both dequantized values are exact in fp32 (at most 4 + 11 and 7 + 5 + 11
// significant bits), so the dequant is bit-exact.
//
// Alignment. Q4_0 blocks and Q6_K super-blocks start at even byte offsets
// (18 and 210 are even, W is 16-byte aligned) but not always at multiples of
// 4. A lane reads the 4-byte words around what it needs (4-byte loads at
// 4-byte boundaries, 2-byte loads at 2-byte boundaries) and re-aligns them
// with v_alignbyte. A window may start up to 2 bytes before its block (which
// then is not the matrix's first, whose start is 16-byte aligned) but never
// ends past its block, so every load stays inside the matrix.
//
// GEMV: a wave owns kOtherRows rows and walks K in steps of 64 units, lane =
// unit (Q4_0: one block of 32 weights; Q6_K: one "quad", 4 consecutive l of
// one half of a super-block = 16 weights). Its x values are loaded once per
// step and reused for the wave's rows; each row's 64 lane partials are added
// by a butterfly at the end (fixed order: deterministic).
#pragma once

#include "device_common.hpp"
#include "gemv_types.hpp"

namespace gqk {

constexpr int kOtherRows = 4;      // rows per wave
constexpr int kOtherWaves = 4;     // waves per block

__device__ __forceinline__ uint32_t ld_u32(const uint8_t* p) {
  return *reinterpret_cast<const uint32_t*>(p);
}
__device__ __forceinline__ uint32_t ld_u16(const uint8_t* p) {
  return *reinterpret_cast<const uint16_t*>(p);
}

// The 4 bytes at p (p even): two aligned words re-aligned when p % 4 == 2.
// Reads bytes [p & ~3, (p & ~3) + 8): the caller guarantees they end inside
// the block.
__device__ __forceinline__ uint32_t ld4_even(const uint8_t* p) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  const uint8_t* q = reinterpret_cast<const uint8_t*>(a & ~uintptr_t(3));
  return __builtin_amdgcn_alignbyte(ld_u32(q + 4), ld_u32(q), (uint32_t)(a & 3u));
}

// Q4_0 block at p (p even): fp16 d and the 16 code bytes as 4 words. Loads:
// 4 words at p & ~3 (bytes up to p + 15 at most), the 2 bytes at (p & ~3) + 16
// and the 2 bytes at p + 16; together they cover [p, p + 18) and end inside it.
__device__ __forceinline__ void q40_block(const uint8_t* p, uint32_t& dbits, uint32_t (&qb)[4]) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  const uint8_t* q = reinterpret_cast<const uint8_t*>(a & ~uintptr_t(3));
  const uint32_t s = (uint32_t)(a & 2u);   // 0 or 2
  const uint32_t w0 = ld_u32(q), w1 = ld_u32(q + 4), w2 = ld_u32(q + 8), w3 = ld_u32(q + 12);
  const uint32_t w4 = ld_u16(q + 16) | (ld_u16(p + 16) << 16);
  // window [q, q + 20): d at offset s, codes at offset s + 2
  dbits = (s ? (w0 >> 16) : w0) & 0xFFFFu;
  qb[0] = s ? w1 : __builtin_amdgcn_alignbyte(w1, w0, 2);
  qb[1] = s ? w2 : __builtin_amdgcn_alignbyte(w2, w1, 2);
  qb[2] = s ? w3 : __builtin_amdgcn_alignbyte(w3, w2, 2);
  // s == 2: w4 holds bytes p + 14 .. p + 17; s == 0: bytes p + 16, p + 17 twice
  qb[3] = s ? w4 : __builtin_amdgcn_alignbyte(w4, w3, 2);
}

// Q6_K quad u (0..15) of the super-block at p: half n = u / 8, l0 = 4 (u % 8).
// Returns the 16 codes as 4 words (word k: codes of weights 128 n + 32 k + l0
// .. + 3, one per byte), the 4 scales (k = 0..3) and d.
__device__ __forceinline__ void q6k_quad(const uint8_t* p, int u, uint32_t (&code)[4],
                                         float (&sc)[4], float& d) {
  const int n = u >> 3, l0 = 4 * (u & 7);
  const uint32_t lo0 = ld4_even(p + 64 * n + l0);        // L[l0..l0+3]
  const uint32_t lo1 = ld4_even(p + 64 * n + 32 + l0);   // L[l0+32..]
  const uint32_t hi = ld4_even(p + 128 + 32 * n + l0);   // H[l0..l0+3]
  code[0] = (lo0 & 0x0F0F0F0Fu) | ((hi << 4) & 0x30303030u);
  code[1] = (lo1 & 0x0F0F0F0Fu) | ((hi << 2) & 0x30303030u);
  code[2] = ((lo0 >> 4) & 0x0F0F0F0Fu) | (hi & 0x30303030u);
  code[3] = ((lo1 >> 4) & 0x0F0F0F0Fu) | ((hi >> 2) & 0x30303030u);
  // scales sc[8 n + 2 k + l0 / 16], k = 0..3: bytes 192 + 8 n + (l0 >= 16) + 2 k
  // (2-byte loads: the half's 8 scale bytes exactly; the upper half's end at
  // byte 208, and a 4-byte window there could reach past the super-block)
  const uint8_t* sp = p + 192 + 8 * n;
  const uint32_t s0 = ld_u16(sp) | (ld_u16(sp + 2) << 16);       // bytes 0..3 of the half's scales
  const uint32_t s1 = ld_u16(sp + 4) | (ld_u16(sp + 6) << 16);   // bytes 4..7
  const int h = l0 >> 4;                                  // 0 or 1
  const uint32_t ev = h ? ((s0 >> 8) & 0xFFu) | ((s0 >> 16) & 0xFF00u) | ((s1 << 8) & 0xFF0000u) |
                              (s1 & 0xFF000000u)
                        : (s0 & 0xFFu) | ((s0 >> 8) & 0xFF00u) | ((s1 << 16) & 0xFF0000u) |
                              ((s1 << 8) & 0xFF000000u);
  sc[0] = sbyte0(ev);
  sc[1] = sbyte1(ev);
  sc[2] = sbyte2(ev);
  sc[3] = sbyte3(ev);
  d = half_lo(ld_u16(p + 208));
}

// ------------------------------------------------------------------ dequant

// Thread = one Q4_0 block (32 fp32 outputs).
__global__ __launch_bounds__(256) void dequant_q4_0_kernel(const uint8_t* __restrict__ W,
                                                           float* __restrict__ out, int64_t nblocks) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  uint32_t dbits, qb[4];
  q40_block(W + b * kQ40BlockBytes, dbits, qb);
  const float d = half_lo(dbits);
  float4* o = reinterpret_cast<float4*>(out + b * kQ40BlockWeights);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = qb[i] & 0x0F0F0F0Fu, hi = (qb[i] >> 4) & 0x0F0F0F0Fu;
    o[i] = make_float4((ubyte0(lo) - 8.f) * d, (ubyte1(lo) - 8.f) * d, (ubyte2(lo) - 8.f) * d,
                       (ubyte3(lo) - 8.f) * d);
    o[4 + i] = make_float4((ubyte0(hi) - 8.f) * d, (ubyte1(hi) - 8.f) * d, (ubyte2(hi) - 8.f) * d,
                           (ubyte3(hi) - 8.f) * d);
  }
}

// Thread = one Q6_K quad (16 fp32 outputs, 4 runs of 4).
__global__ __launch_bounds__(256) void dequant_q6_k_kernel(const uint8_t* __restrict__ W,
                                                           float* __restrict__ out, int64_t nquads) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= nquads) return;
  const int64_t sb = t >> 4;
  const int u = (int)(t & 15);
  uint32_t code[4];
  float sc[4], d;
  q6k_quad(W + sb * kQ6KBlockBytes, u, code, sc, d);
  const int n = u >> 3, l0 = 4 * (u & 7);
  float* o = out + sb * kQ6KBlockWeights + 128 * n + l0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float ds = d * sc[k];   // exact: 11 + 8 bits
    *reinterpret_cast<float4*>(o + 32 * k) =
        make_float4(ds * (ubyte0(code[k]) - 32.f), ds * (ubyte1(code[k]) - 32.f),
                    ds * (ubyte2(code[k]) - 32.f), ds * (ubyte3(code[k]) - 32.f));
  }
}

// --------------------------------------------------------------------- GEMV
//
// Each step's loads (x and the raw words of every row) are issued one step
// ahead, so that they are in flight while the previous step computes; the
// words are re-aligned and decoded when their step computes.

typedef float gqk_f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

// Raw words of one Q4_0 block (see q40_block): w[0..3] at p & ~3, then the two
// 2-byte loads; s = p & 2.
struct Q40Raw {
  uint32_t w[6];
  uint32_t s;
};

__device__ __forceinline__ void q40_fetch(const uint8_t* p, Q40Raw& r) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  const uint8_t* q = reinterpret_cast<const uint8_t*>(a & ~uintptr_t(3));
  r.s = (uint32_t)(a & 2u);
  r.w[0] = ld_u32(q);
  r.w[1] = ld_u32(q + 4);
  r.w[2] = ld_u32(q + 8);
  r.w[3] = ld_u32(q + 12);
  r.w[4] = ld_u16(q + 16);
  r.w[5] = ld_u16(p + 16);
}

__device__ __forceinline__ void q40_assemble(const Q40Raw& r, uint32_t& dbits, uint32_t (&qb)[4]) {
  const uint32_t w4 = r.w[4] | (r.w[5] << 16);
  dbits = (r.s ? (r.w[0] >> 16) : r.w[0]) & 0xFFFFu;
  qb[0] = r.s ? r.w[1] : __builtin_amdgcn_alignbyte(r.w[1], r.w[0], 2);
  qb[1] = r.s ? r.w[2] : __builtin_amdgcn_alignbyte(r.w[2], r.w[1], 2);
  qb[2] = r.s ? r.w[3] : __builtin_amdgcn_alignbyte(r.w[3], r.w[2], 2);
  qb[3] = r.s ? w4 : __builtin_amdgcn_alignbyte(w4, r.w[3], 2);
}

struct Q40Step {
  gqk_f32x4 x[8];
  Q40Raw w[kOtherRows];
};

__device__ __forceinline__ void q40_step_fetch(Q40Step& f, const uint8_t* W, const float* x,
                                               int64_t row0, int64_t rows, int64_t row_bytes,
                                               int64_t b, int64_t nb) {
  if (b >= nb) return;
  const gqk_f32x4* xv = reinterpret_cast<const gqk_f32x4*>(x + b * kQ40BlockWeights);
#pragma unroll
  for (int i = 0; i < 8; ++i) f.x[i] = xv[i];
#pragma unroll
  for (int r = 0; r < kOtherRows; ++r) {
    const int64_t row = (row0 + r) < rows ? (row0 + r) : (rows - 1);
    q40_fetch(W + row * row_bytes + b * kQ40BlockBytes, f.w[r]);
  }
}

__device__ __forceinline__ void q40_step_compute(const Q40Step& f, float (&acc)[kOtherRows]) {
  float xsum = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) xsum += (f.x[i].x + f.x[i].y) + (f.x[i].z + f.x[i].w);
#pragma unroll
  for (int r = 0; r < kOtherRows; ++r) {
    uint32_t dbits, qb[4];
    q40_assemble(f.w[r], dbits, qb);
    // sum (code - 8) d x = 512 d sum (code / 512) x - 8 d sum x
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float lo[4], hi[4];
      nibbles_div512(qb[i] & 0x0F0F0F0Fu, lo);
      nibbles_div512((qb[i] >> 4) & 0x0F0F0F0Fu, hi);
      const gqk_f32x4 xl = f.x[i], xh = f.x[4 + i];
      a0 = fmaf(lo[0], xl.x, a0);
      a0 = fmaf(lo[1], xl.y, a0);
      a0 = fmaf(lo[2], xl.z, a0);
      a0 = fmaf(lo[3], xl.w, a0);
      a1 = fmaf(hi[0], xh.x, a1);
      a1 = fmaf(hi[1], xh.y, a1);
      a1 = fmaf(hi[2], xh.z, a1);
      a1 = fmaf(hi[3], xh.w, a1);
    }
    const float d = half_lo(dbits);
    acc[r] = fmaf(d * 512.f, a0 + a1, acc[r]);
    acc[r] = fmaf(-8.f * d, xsum, acc[r]);
  }
}

// grid: ceil(rows / (kOtherRows * kOtherWaves)) blocks of kOtherWaves waves.
__global__ __launch_bounds__(kOtherWaves * 64) void gemv_q4_0_kernel(
    const uint8_t* __restrict__ W, const float* __restrict__ x, float* __restrict__ y,
    int64_t rows, int64_t nb) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row0 = ((int64_t)blockIdx.x * kOtherWaves + wave) * kOtherRows;
  if (row0 >= rows) return;
  const int64_t row_bytes = nb * kQ40BlockBytes;
  float acc[kOtherRows];
#pragma unroll
  for (int r = 0; r < kOtherRows; ++r) acc[r] = 0.f;
  Q40Step cur, nxt;
  q40_step_fetch(cur, W, x, row0, rows, row_bytes, lane, nb);
  for (int64_t b0 = 0; b0 < nb; b0 += 64) {
    if (b0 + 64 < nb) q40_step_fetch(nxt, W, x, row0, rows, row_bytes, b0 + 64 + lane, nb);
    if (b0 + lane < nb) q40_step_compute(cur, acc);
    cur = nxt;
  }
#pragma unroll
  for (int r = 0; r < kOtherRows; ++r) {
    const float v = wave_sum(acc[r]);
    if (lane == 0 && row0 + r < rows) y[row0 + r] = v;
  }
}

// Raw words of one Q6_K quad (see q6k_quad): three aligned pairs, the 4
// scale 2-byte loads and d.
struct Q6KRaw {
  uint32_t lo0[2], lo1[2], hi[2], sc[4], d;
  uint32_t s;   // p & 2 (the super-block's offset from a 4-byte boundary)
};

__device__ __forceinline__ void q6k_fetch(const uint8_t* p, int u, Q6KRaw& r) {
  const int n = u >> 3, l0 = 4 * (u & 7);
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  r.s = (uint32_t)(a & 2u);
  const uint8_t* q0 = reinterpret_cast<const uint8_t*>((a + 64 * n + l0) & ~uintptr_t(3));
  const uint8_t* q1 = reinterpret_cast<const uint8_t*>((a + 64 * n + 32 + l0) & ~uintptr_t(3));
  const uint8_t* q2 = reinterpret_cast<const uint8_t*>((a + 128 + 32 * n + l0) & ~uintptr_t(3));
  r.lo0[0] = ld_u32(q0);
  r.lo0[1] = ld_u32(q0 + 4);
  r.lo1[0] = ld_u32(q1);
  r.lo1[1] = ld_u32(q1 + 4);
  r.hi[0] = ld_u32(q2);
  r.hi[1] = ld_u32(q2 + 4);
  const uint8_t* sp = p + 192 + 8 * n;
  r.sc[0] = ld_u16(sp);
  r.sc[1] = ld_u16(sp + 2);
  r.sc[2] = ld_u16(sp + 4);
  r.sc[3] = ld_u16(sp + 6);
  r.d = ld_u16(p + 208);
}

__device__ __forceinline__ void q6k_assemble(const Q6KRaw& r, int u, uint32_t (&code)[4],
                                             float (&sc)[4], float& d) {
  // the three 4-byte fields sit at offsets that are multiples of 4 from p
  const uint32_t lo0 = __builtin_amdgcn_alignbyte(r.lo0[1], r.lo0[0], r.s);
  const uint32_t lo1 = __builtin_amdgcn_alignbyte(r.lo1[1], r.lo1[0], r.s);
  const uint32_t hi = __builtin_amdgcn_alignbyte(r.hi[1], r.hi[0], r.s);
  code[0] = (lo0 & 0x0F0F0F0Fu) | ((hi << 4) & 0x30303030u);
  code[1] = (lo1 & 0x0F0F0F0Fu) | ((hi << 2) & 0x30303030u);
  code[2] = ((lo0 >> 4) & 0x0F0F0F0Fu) | (hi & 0x30303030u);
  code[3] = ((lo1 >> 4) & 0x0F0F0F0Fu) | ((hi >> 2) & 0x30303030u);
  const uint32_t s0 = r.sc[0] | (r.sc[1] << 16), s1 = r.sc[2] | (r.sc[3] << 16);
  const int h = (u & 7) >> 2;   // l0 >= 16
  const uint32_t ev = h ? ((s0 >> 8) & 0xFFu) | ((s0 >> 16) & 0xFF00u) | ((s1 << 8) & 0xFF0000u) |
                              (s1 & 0xFF000000u)
                        : (s0 & 0xFFu) | ((s0 >> 8) & 0xFF00u) | ((s1 << 16) & 0xFF0000u) |
                              ((s1 << 8) & 0xFF000000u);
  sc[0] = sbyte0(ev);
  sc[1] = sbyte1(ev);
  sc[2] = sbyte2(ev);
  sc[3] = sbyte3(ev);
  d = half_lo(r.d);
}

struct Q6KStep {
  gqk_f32x4 x[4];
  Q6KRaw w[kOtherRows];
};

__device__ __forceinline__ void q6k_step_fetch(Q6KStep& f, const uint8_t* W, const float* x,
                                               int64_t row0, int64_t rows, int64_t row_bytes,
                                               int64_t sb, int64_t nsb, int u) {
  if (sb >= nsb) return;
  const int n = u >> 3, l0 = 4 * (u & 7);
  const float* xb = x + sb * kQ6KBlockWeights + 128 * n + l0;
#pragma unroll
  for (int k = 0; k < 4; ++k) f.x[k] = *reinterpret_cast<const gqk_f32x4*>(xb + 32 * k);
#pragma unroll
  for (int r = 0; r < kOtherRows; ++r) {
    const int64_t row = (row0 + r) < rows ? (row0 + r) : (rows - 1);
    q6k_fetch(W + row * row_bytes + sb * kQ6KBlockBytes, u, f.w[r]);
  }
}

__device__ __forceinline__ void q6k_step_compute(const Q6KStep& f, int u, float (&acc)[kOtherRows]) {
  float xsum[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) xsum[k] = (f.x[k].x + f.x[k].y) + (f.x[k].z + f.x[k].w);
#pragma unroll
  for (int r = 0; r < kOtherRows; ++r) {
    uint32_t code[4];
    float sc[4], d;
    q6k_assemble(f.w[r], u, code, sc, d);
    // sum_k d sc_k (sum_i code_i x_i - 32 sum_i x_i)
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float a = ubyte0(code[k]) * f.x[k].x;
      a = fmaf(ubyte1(code[k]), f.x[k].y, a);
      a = fmaf(ubyte2(code[k]), f.x[k].z, a);
      a = fmaf(ubyte3(code[k]), f.x[k].w, a);
      a = fmaf(-32.f, xsum[k], a);
      t = fmaf(sc[k], a, t);
    }
    acc[r] = fmaf(d, t, acc[r]);
  }
}

__global__ __launch_bounds__(kOtherWaves * 64) void gemv_q6_k_kernel(
    const uint8_t* __restrict__ W, const float* __restrict__ x, float* __restrict__ y,
    int64_t rows, int64_t nsb) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row0 = ((int64_t)blockIdx.x * kOtherWaves + wave) * kOtherRows;
  if (row0 >= rows) return;
  const int64_t row_bytes = nsb * kQ6KBlockBytes;
  const int u = lane & 15;
  const int sl = lane >> 4;   // this lane's super-block within a step of 4
  float acc[kOtherRows];
#pragma unroll
  for (int r = 0; r < kOtherRows; ++r) acc[r] = 0.f;
  Q6KStep cur, nxt;
  q6k_step_fetch(cur, W, x, row0, rows, row_bytes, sl, nsb, u);
  for (int64_t s0 = 0; s0 < nsb; s0 += 4) {
    if (s0 + 4 < nsb) q6k_step_fetch(nxt, W, x, row0, rows, row_bytes, s0 + 4 + sl, nsb, u);
    if (s0 + sl < nsb) q6k_step_compute(cur, u, acc);
    cur = nxt;
  }
#pragma unroll
  for (int r = 0; r < kOtherRows; ++r) {
    const float v = wave_sum(acc[r]);
    if (lane == 0 && row0 + r < rows) y[row0 + r] = v;
  }
}

}  // namespace gqk
