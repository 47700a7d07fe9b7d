// Device-side helpers shared by the gfx950 kernels of libgguf_qk.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqk {

constexpr int kQ80BlockBytes = 34;     // fp16 scale + 32 int8
constexpr int kQ80BlockWeights = 32;
constexpr int kQ4KBlockBytes = 144;    // fp16 d, fp16 dmin, 12 B scales, 128 B quants
constexpr int kQ4KBlockWeights = 256;
constexpr int kQ6KBlockBytes = 210;    // 128 B low 4 bits, 64 B high 2 bits, 16 int8 scales, fp16 d
constexpr int kQ6KBlockWeights = 256;
constexpr int kWave = 64;

typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;

#define GQK_LDS(p) ((__attribute__((address_space(3))) void*)(p))
#define GQK_GLOBAL __attribute__((address_space(1)))

// fp16 bit pattern (low 16 bits) -> fp32. v_cvt_f32_f16 is exact for every
// finite half, subnormals included (fp16 denormals are enabled in the kernel
// mode register), and maps inf/NaN to inf/NaN.
__device__ __forceinline__ float half_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float half_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// fp32 -> bf16 bit pattern, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
// Both halves in one v_cvt_pk_bf16_f32 (the per-element form took two
// conversions, a shift and an or); nearest-even, as to_bf16.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// Hide a value from the optimizer so that byte-wise conversions of a masked
// word stay v_cvt_f32_ubyteN (one instruction) instead of being re-folded into
// a bit-field extract followed by a conversion (two instructions).
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  asm("" : "+v"(v));
  return v;
}

__device__ __forceinline__ float ubyte0(uint32_t v) { return (float)(v & 0xFFu); }
__device__ __forceinline__ float ubyte1(uint32_t v) { return (float)((v >> 8) & 0xFFu); }
__device__ __forceinline__ float ubyte2(uint32_t v) { return (float)((v >> 16) & 0xFFu); }
__device__ __forceinline__ float ubyte3(uint32_t v) { return (float)(v >> 24); }

// Four bytes holding values 0..15 converted to fp32 as value / 512, two per
// instruction: read as OCP E4M3 fp8, a byte b < 16 is b x 2^-9 exactly
// (b < 8: subnormal m x 2^-9; 8 <= b < 16: exponent 1, (8 + m) x 2^-9).
typedef float gqk_f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void nibbles_div512(uint32_t v, float (&q)[4]) {
  const gqk_f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)v, false);
  const gqk_f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)v, true);
  q[0] = lo.x;
  q[1] = lo.y;
  q[2] = hi.x;
  q[3] = hi.y;
}
__device__ __forceinline__ float sbyte0(uint32_t v) { return (float)(int)(int8_t)(v & 0xFFu); }
__device__ __forceinline__ float sbyte1(uint32_t v) { return (float)(int)(int8_t)((v >> 8) & 0xFFu); }
__device__ __forceinline__ float sbyte2(uint32_t v) { return (float)(int)(int8_t)((v >> 16) & 0xFFu); }
__device__ __forceinline__ float sbyte3(uint32_t v) { return (float)(int)(int8_t)(v >> 24); }

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4] left at 7, lgkmcnt [11:8] at 15).
#define GQK_WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

// Direct global -> LDS 16-byte load: lane i writes bytes [16 i, 16 i + 16) of
// the wave's 1 KiB window starting at `lds_window`.
__device__ __forceinline__ void dma16(const void* g, void* lds_window) {
  __builtin_amdgcn_global_load_lds(g, GQK_LDS(lds_window), 16, 0, 0);
}

// Reads of LDS filled by direct loads are issued as inline assembly so that
// the compiler, which cannot tell which LDS bytes an in-flight direct load
// writes, does not insert a wait for ALL outstanding vector loads before them;
// the caller has already waited (GQK_WAIT_VMCNT) for the loads that filled
// these bytes. Each block ends with lgkmcnt(0), so results are ready on exit.
// Outputs are early-clobber: a read may return before the block's later reads
// have issued, so no destination may share registers with the address.
__device__ __forceinline__ void lds_read_9x16(uint32_t addr, uint32_t (&o)[36]) {
  i32x4 v0, v1, v2, v3, v4, v5, v6, v7, v8;
  asm volatile(
      "ds_read_b128 %0, %9\n"
      "ds_read_b128 %1, %9 offset:16\n"
      "ds_read_b128 %2, %9 offset:32\n"
      "ds_read_b128 %3, %9 offset:48\n"
      "ds_read_b128 %4, %9 offset:64\n"
      "ds_read_b128 %5, %9 offset:80\n"
      "ds_read_b128 %6, %9 offset:96\n"
      "ds_read_b128 %7, %9 offset:112\n"
      "ds_read_b128 %8, %9 offset:128\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v0), "=&v"(v1), "=&v"(v2), "=&v"(v3), "=&v"(v4), "=&v"(v5), "=&v"(v6), "=&v"(v7), "=&v"(v8)
      : "v"(addr)
      : "memory");
  const i32x4 v[9] = {v0, v1, v2, v3, v4, v5, v6, v7, v8};
#pragma unroll
  for (int j = 0; j < 9; ++j) {
#pragma unroll
    for (int e = 0; e < 4; ++e) o[4 * j + e] = (uint32_t)v[j][e];
  }
}

__device__ __forceinline__ void lds_read_17x16(uint32_t addr, uint32_t (&o)[68]) {
  i32x4 v0, v1, v2, v3, v4, v5, v6, v7, v8, v9, v10, v11, v12, v13, v14, v15, v16;
  asm volatile(
      "ds_read_b128 %0, %17\n"
      "ds_read_b128 %1, %17 offset:16\n"
      "ds_read_b128 %2, %17 offset:32\n"
      "ds_read_b128 %3, %17 offset:48\n"
      "ds_read_b128 %4, %17 offset:64\n"
      "ds_read_b128 %5, %17 offset:80\n"
      "ds_read_b128 %6, %17 offset:96\n"
      "ds_read_b128 %7, %17 offset:112\n"
      "ds_read_b128 %8, %17 offset:128\n"
      "ds_read_b128 %9, %17 offset:144\n"
      "ds_read_b128 %10, %17 offset:160\n"
      "ds_read_b128 %11, %17 offset:176\n"
      "ds_read_b128 %12, %17 offset:192\n"
      "ds_read_b128 %13, %17 offset:208\n"
      "ds_read_b128 %14, %17 offset:224\n"
      "ds_read_b128 %15, %17 offset:240\n"
      "ds_read_b128 %16, %17 offset:256\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v0), "=&v"(v1), "=&v"(v2), "=&v"(v3), "=&v"(v4), "=&v"(v5), "=&v"(v6), "=&v"(v7), "=&v"(v8),
        "=&v"(v9), "=&v"(v10), "=&v"(v11), "=&v"(v12), "=&v"(v13), "=&v"(v14), "=&v"(v15), "=&v"(v16)
      : "v"(addr)
      : "memory");
  const i32x4 v[17] = {v0, v1, v2, v3, v4, v5, v6, v7, v8, v9, v10, v11, v12, v13, v14, v15, v16};
#pragma unroll
  for (int j = 0; j < 17; ++j) {
#pragma unroll
    for (int e = 0; e < 4; ++e) o[4 * j + e] = (uint32_t)v[j][e];
  }
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)GQK_LDS(p);
}

// Q4_K super-block header: word 0 = d | dmin << 16, words 1..3 = scale bytes
// S[0..11]. Produces d*sc[j] and dmin*m[j] for the 8 sub-blocks; both
// products are exact in fp32 (11-bit significand times a 6-bit integer).
//   j < 4 : sc = S[j] & 63,  m = S[j+4] & 63
//   j >= 4: sc = (S[j+4] & 15) | ((S[j-4] >> 6) << 4)
//           m  = (S[j+4] >> 4) | ((S[j]   >> 6) << 4)
__device__ __forceinline__ void q4k_scales(uint32_t h0, uint32_t h1, uint32_t h2, uint32_t h3,
                                           float (&dsc)[8], float (&dmm)[8]) {
  const float d = half_lo(h0);
  const float dmin = half_hi(h0);
  const uint32_t sc_lo = opaque(h1 & 0x3F3F3F3Fu);                               // sc[0..3]
  const uint32_t m_lo = opaque(h2 & 0x3F3F3F3Fu);                                // m[0..3]
  const uint32_t sc_hi = opaque((h3 & 0x0F0F0F0Fu) | ((h1 >> 2) & 0x30303030u)); // sc[4..7]
  const uint32_t m_hi = opaque(((h3 >> 4) & 0x0F0F0F0Fu) | ((h2 >> 2) & 0x30303030u));
  dsc[0] = d * ubyte0(sc_lo); dsc[1] = d * ubyte1(sc_lo);
  dsc[2] = d * ubyte2(sc_lo); dsc[3] = d * ubyte3(sc_lo);
  dsc[4] = d * ubyte0(sc_hi); dsc[5] = d * ubyte1(sc_hi);
  dsc[6] = d * ubyte2(sc_hi); dsc[7] = d * ubyte3(sc_hi);
  dmm[0] = dmin * ubyte0(m_lo); dmm[1] = dmin * ubyte1(m_lo);
  dmm[2] = dmin * ubyte2(m_lo); dmm[3] = dmin * ubyte3(m_lo);
  dmm[4] = dmin * ubyte0(m_hi); dmm[5] = dmin * ubyte1(m_hi);
  dmm[6] = dmin * ubyte2(m_hi); dmm[7] = dmin * ubyte3(m_hi);
}

}  // namespace gqk
