// Prefill: Y[n, r] = sum_k X[n, k] W[r, k], X and Y bf16, W Q4_K, on the
// gfx950 matrix cores (v_mfma_f32_32x32x16_bf16, fp32 accumulation).
//
// Block tile: 128 tokens x 128 weight rows, 4 waves, each wave a 64 x 64
// sub-tile held as 2 x 2 MFMA accumulators. K is consumed 128 at a time (half
// a super-block). Each thread stages, in registers, the next step's 64 bf16
// of X (16 bytes from each of 8 token rows) and 32 bytes of nibbles (+ the
// 16-byte super-block header) of one weight row, loaded while the current
// step's MFMAs run; at its step the thread decodes the 64 weights (fp32
// dequant rounded to nearest-even bf16, as the bf16 dequant entry point) and
// stores both operands to LDS. (A second
// staged step does not fit the register file beside the accumulators and
// the unrolled operand reads without spilling.)
//
// Split K: a launch may cut K into S ranges of whole super-blocks (grid z).
// With S > 1 each block stores its fp32 tile to scratch with agent-scope
// stores, waits for them, and bumps the tile's counter; the block that
// arrives last adds the S partial tiles in range order 0..S-1 (the result
// does not depend on arrival order), writes Y in bf16 and resets the counter.
//
// LDS rows are 272 bytes (68 dwords, 4 modulo 32 banks): the 16-byte operand
// reads of 8 consecutive rows by 8 lanes cover all 32 banks once.
//
// MFMA operand layout used (32x32x16): lane l supplies A[i = l % 32][8 k] and
// B[8 k][j = l % 32] from k-group l / 32; A and B are fed with the same
// (k-group, element) labels, so the product does not depend on how the
// hardware orders k inside a group. Accumulator element e of lane l is
// D[8 (e / 4) + 4 (l / 32) + e % 4][l % 32].
#pragma once

#include "device_common.hpp"
#include "mfma_types.hpp"

namespace gqk {

constexpr int kGemmBM = 128;                     // tokens per block
constexpr int kGemmBN = 128;                     // weight rows per block
constexpr int kGemmBK = 128;                     // k per step (half a super-block)
constexpr int kGemmLdsRow = kGemmBK * 2 + 16;    // 272 bytes
constexpr int kGemmTileFloats = kGemmBM * kGemmBN;
constexpr int kGemmCounterStride = 32;           // ints: one 128-byte line per tile counter

// Loads step `step` into stage set S: 16 bytes of X from each of this
// thread's 8 token rows (16 consecutive lanes read one row's 256 bytes, so a
// wave's load touches 8 cache lines) and the header and 32 nibble bytes of
// its weight row.
#define GQK_GEMM_LOAD(S, step)                                                                 \
  do {                                                                                         \
    const int64_t ko_ = (int64_t)(step) * kGemmBK + 8 * xc;                                    \
    x##S##0 = *reinterpret_cast<const uint4*>(X + xoff0 + ko_);                                \
    x##S##1 = *reinterpret_cast<const uint4*>(X + xoff1 + ko_);                                \
    x##S##2 = *reinterpret_cast<const uint4*>(X + xoff2 + ko_);                                \
    x##S##3 = *reinterpret_cast<const uint4*>(X + xoff3 + ko_);                                \
    x##S##4 = *reinterpret_cast<const uint4*>(X + xoff4 + ko_);                                \
    x##S##5 = *reinterpret_cast<const uint4*>(X + xoff5 + ko_);                                \
    x##S##6 = *reinterpret_cast<const uint4*>(X + xoff6 + ko_);                                \
    x##S##7 = *reinterpret_cast<const uint4*>(X + xoff7 + ko_);                                \
    const uint8_t* sb_ = wrow + (int64_t)((step) >> 1) * kQ4KBlockBytes;                       \
    h##S = *reinterpret_cast<const uint4*>(sb_);                                               \
    const uint4* q_ = reinterpret_cast<const uint4*>(sb_ + 16 + 32 * (2 * ((step) & 1) + half)); \
    qa##S = q_[0];                                                                             \
    qb##S = q_[1];                                                                             \
  } while (0)

// Decodes stage set S (step `step`), stores it to LDS, refills S with step
// `next` (if inside this block's range) and runs the step's MFMAs.
#define GQK_GEMM_STEP(S, step, next)                                                           \
  do {                                                                                         \
    const int hs_ = (step) & 1;                                                                \
    const float d_ = half_lo(h##S.x), dmin_ = half_hi(h##S.x);                                 \
    const uint32_t scw_ = hs_ ? ((h##S.w & 0x0F0F0F0Fu) | ((h##S.y >> 2) & 0x30303030u))       \
                              : (h##S.y & 0x3F3F3F3Fu);                                        \
    const uint32_t mw_ = hs_ ? (((h##S.w >> 4) & 0x0F0F0F0Fu) | ((h##S.z >> 2) & 0x30303030u)) \
                             : (h##S.z & 0x3F3F3F3Fu);                                         \
    const uint32_t scp_ = opaque(scw_ >> (16 * half)), mp_ = opaque(mw_ >> (16 * half));      \
    const float dl_ = d_ * ubyte0(scp_), dh_ = d_ * ubyte1(scp_);                              \
    const float ml_ = dmin_ * ubyte0(mp_), mh_ = dmin_ * ubyte1(mp_);                          \
    const uint32_t qw_[8] = {qa##S.x, qa##S.y, qa##S.z, qa##S.w,                               \
                             qb##S.x, qb##S.y, qb##S.z, qb##S.w};                              \
    uint32_t lo_[16], hi_[16];                                                                 \
    _Pragma("unroll") for (int t_ = 0; t_ < 8; ++t_) {                                         \
      const uint32_t l4_ = opaque(qw_[t_] & 0x0F0F0F0Fu);                                      \
      const uint32_t h4_ = opaque((qw_[t_] >> 4) & 0x0F0F0F0Fu);                               \
      lo_[2 * t_] = pack_bf16x2(fmaf(dl_, ubyte0(l4_), -ml_), fmaf(dl_, ubyte1(l4_), -ml_));    \
      lo_[2 * t_ + 1] = pack_bf16x2(fmaf(dl_, ubyte2(l4_), -ml_), fmaf(dl_, ubyte3(l4_), -ml_)); \
      hi_[2 * t_] = pack_bf16x2(fmaf(dh_, ubyte0(h4_), -mh_), fmaf(dh_, ubyte1(h4_), -mh_));    \
      hi_[2 * t_ + 1] = pack_bf16x2(fmaf(dh_, ubyte2(h4_), -mh_), fmaf(dh_, ubyte3(h4_), -mh_)); \
    }                                                                                          \
    __syncthreads(); /* the previous step's operand reads are done */                          \
    uint8_t* xd_ = xs + xr0 * kGemmLdsRow + 16 * xc;                                           \
    *reinterpret_cast<uint4*>(xd_ + 0 * 16 * kGemmLdsRow) = x##S##0;                           \
    *reinterpret_cast<uint4*>(xd_ + 1 * 16 * kGemmLdsRow) = x##S##1;                           \
    *reinterpret_cast<uint4*>(xd_ + 2 * 16 * kGemmLdsRow) = x##S##2;                           \
    *reinterpret_cast<uint4*>(xd_ + 3 * 16 * kGemmLdsRow) = x##S##3;                           \
    *reinterpret_cast<uint4*>(xd_ + 4 * 16 * kGemmLdsRow) = x##S##4;                           \
    *reinterpret_cast<uint4*>(xd_ + 5 * 16 * kGemmLdsRow) = x##S##5;                           \
    *reinterpret_cast<uint4*>(xd_ + 6 * 16 * kGemmLdsRow) = x##S##6;                           \
    *reinterpret_cast<uint4*>(xd_ + 7 * 16 * kGemmLdsRow) = x##S##7;                           \
    uint4* wd_ = reinterpret_cast<uint4*>(ws + ld_row * kGemmLdsRow + 128 * half);             \
    wd_[0] = make_uint4(lo_[0], lo_[1], lo_[2], lo_[3]);                                       \
    wd_[1] = make_uint4(lo_[4], lo_[5], lo_[6], lo_[7]);                                       \
    wd_[2] = make_uint4(lo_[8], lo_[9], lo_[10], lo_[11]);                                     \
    wd_[3] = make_uint4(lo_[12], lo_[13], lo_[14], lo_[15]);                                   \
    wd_[4] = make_uint4(hi_[0], hi_[1], hi_[2], hi_[3]);                                       \
    wd_[5] = make_uint4(hi_[4], hi_[5], hi_[6], hi_[7]);                                       \
    wd_[6] = make_uint4(hi_[8], hi_[9], hi_[10], hi_[11]);                                     \
    wd_[7] = make_uint4(hi_[12], hi_[13], hi_[14], hi_[15]);                                   \
    __syncthreads();                                                                           \
    if ((next) < step_end) GQK_GEMM_LOAD(S, (next));                                           \
    _Pragma("unroll") for (int kk_ = 0; kk_ < kGemmBK; kk_ += 16) {                            \
      const int kb_ = (kk_ + 8 * (lane >> 5)) * 2;                                             \
      const bf16x8 a0_ = *reinterpret_cast<const bf16x8*>(                                     \
          xs + (wi * 64 + (lane & 31)) * kGemmLdsRow + kb_);                                   \
      const bf16x8 a1_ = *reinterpret_cast<const bf16x8*>(                                     \
          xs + (wi * 64 + 32 + (lane & 31)) * kGemmLdsRow + kb_);                              \
      const bf16x8 b0_ = *reinterpret_cast<const bf16x8*>(                                     \
          ws + (wj * 64 + (lane & 31)) * kGemmLdsRow + kb_);                                   \
      const bf16x8 b1_ = *reinterpret_cast<const bf16x8*>(                                     \
          ws + (wj * 64 + 32 + (lane & 31)) * kGemmLdsRow + kb_);                              \
      acc00 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0_, b0_, acc00, 0, 0, 0);               \
      acc01 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0_, b1_, acc01, 0, 0, 0);               \
      acc10 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1_, b0_, acc10, 0, 0, 0);               \
      acc11 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1_, b1_, acc11, 0, 0, 0);               \
    }                                                                                          \
  } while (0)

// Writes accumulator `acc` (sub-tile it, jt of this wave) to Y as bf16.
__device__ __forceinline__ void gemm_store_bf16(const f32x16& acc, uint16_t* __restrict__ Y,
                                                int64_t n_tokens, int64_t rows, int64_t n0,
                                                int64_t r0, int wi, int wj, int it, int jt,
                                                int lane) {
  const int64_t r = r0 + wj * 64 + jt * 32 + (lane & 31);
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int64_t n = n0 + wi * 64 + it * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
    if (n < n_tokens && r < rows) Y[n * rows + r] = to_bf16(acc[e]);
  }
}

// Partial tile layout in scratch: [wave][it][jt][e][lane] floats, so each
// (wave, it, jt, e) is 64 consecutive floats written and read by one wave.
__device__ __forceinline__ float* gemm_partial_slot(float* tile, int wave, int it, int jt, int e,
                                                    int lane) {
  return tile + ((((wave * 2 + it) * 2 + jt) * 16 + e) * 64 + lane);
}

// The last block of a split tile: the S partial tiles summed in range order
// and stored as bf16. Two accumulator tiles at a time: a range's 32 values per
// lane are loaded together, so the sum costs 2 S memory round trips (4 S with
// one tile at a time; all four tiles together took the kernel past 256
// registers, one wave per SIMD).
__device__ __forceinline__ void gemm_sum_partials(const float* partials, int64_t ntiles, int64_t tile,
                                                  int64_t tile_floats, int S, int wave, int lane, uint16_t* Y,
                                                  int64_t n_tokens, int64_t rows, int64_t n0, int64_t r0, int wi,
                                                  int wj) {
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    f32x16 sum[2];
#pragma unroll
    for (int jt = 0; jt < 2; ++jt)
#pragma unroll
      for (int e = 0; e < 16; ++e) sum[jt][e] = 0.f;
    for (int sp = 0; sp < S; ++sp) {
      float* p = const_cast<float*>(partials) + ((int64_t)sp * ntiles + tile) * tile_floats;
      float v[2][16];
#pragma unroll
      for (int jt = 0; jt < 2; ++jt)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          v[jt][e] = __hip_atomic_load(gemm_partial_slot(p, wave, it, jt, e, lane), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
      for (int jt = 0; jt < 2; ++jt)
#pragma unroll
        for (int e = 0; e < 16; ++e) sum[jt][e] += v[jt][e];
    }
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) gemm_store_bf16(sum[jt], Y, n_tokens, rows, n0, r0, wi, wj, it, jt, lane);
  }
}

__global__ __launch_bounds__(256) void gemm_q4_k_kernel(const uint8_t* __restrict__ W,
                                                        const uint16_t* __restrict__ X,
                                                        uint16_t* __restrict__ Y, int64_t n_tokens,
                                                        int64_t rows, int nsb, float* partials,
                                                        int* counters) {
  __shared__ __attribute__((aligned(16))) uint8_t xs[kGemmBM * kGemmLdsRow];
  __shared__ __attribute__((aligned(16))) uint8_t ws[kGemmBN * kGemmLdsRow];
  __shared__ int last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wi = wave >> 1, wj = wave & 1;
  const int64_t n0 = (int64_t)blockIdx.y * kGemmBM;
  const int64_t r0 = (int64_t)blockIdx.x * kGemmBN;
  const int S = (int)gridDim.z, split = (int)blockIdx.z;
  const int64_t K = (int64_t)nsb * kQ4KBlockWeights;
  const int64_t row_bytes = (int64_t)nsb * kQ4KBlockBytes;
  // this block's steps: super-blocks [nsb * split / S, nsb * (split + 1) / S)
  const int step_begin = 2 * (int)((int64_t)nsb * split / S);
  const int step_end = 2 * (int)((int64_t)nsb * (split + 1) / S);

  // Staging roles. X: thread t stages 16 bytes (k 8 xc .. 8 xc + 7 of the
  // step, xc = t % 16) of token rows xr0 + 16 j, j = 0..7 (xr0 = t / 16).
  // W: thread = (row, half) decodes nibble group g = 2 h + half of the step's
  // half super-block h, i.e. Qb[32 g .. 32 g + 31]: low nibbles are local k
  // 64 half + 0..31, high nibbles local k 64 half + 32..63. Rows past the end
  // are clamped (read, never stored).
  const int xc = tid & 15, xr0 = tid >> 4;
  auto xrow_off = [&](int j) -> int64_t {
    const int64_t n = n0 + xr0 + 16 * j;
    return (n < n_tokens ? n : n_tokens - 1) * K;
  };
  const int64_t xoff0 = xrow_off(0), xoff1 = xrow_off(1), xoff2 = xrow_off(2), xoff3 = xrow_off(3);
  const int64_t xoff4 = xrow_off(4), xoff5 = xrow_off(5), xoff6 = xrow_off(6), xoff7 = xrow_off(7);
  const int ld_row = tid >> 1, half = tid & 1;
  const int64_t wr = (r0 + ld_row) < rows ? (r0 + ld_row) : (rows - 1);
  const uint8_t* wrow = W + wr * row_bytes;

  uint4 xA0, xA1, xA2, xA3, xA4, xA5, xA6, xA7, hA, qaA, qbA;
  f32x16 acc00, acc01, acc10, acc11;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc00[e] = acc01[e] = acc10[e] = acc11[e] = 0.f;

  GQK_GEMM_LOAD(A, step_begin);
  for (int step = step_begin; step < step_end; ++step) GQK_GEMM_STEP(A, step, step + 1);

  if (S == 1) {
    gemm_store_bf16(acc00, Y, n_tokens, rows, n0, r0, wi, wj, 0, 0, lane);
    gemm_store_bf16(acc01, Y, n_tokens, rows, n0, r0, wi, wj, 0, 1, lane);
    gemm_store_bf16(acc10, Y, n_tokens, rows, n0, r0, wi, wj, 1, 0, lane);
    gemm_store_bf16(acc11, Y, n_tokens, rows, n0, r0, wi, wj, 1, 1, lane);
    return;
  }

  const int64_t tile = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
  const int64_t ntiles = (int64_t)gridDim.x * gridDim.y;
  float* mine = partials + ((int64_t)split * ntiles + tile) * kGemmTileFloats;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    __hip_atomic_store(gemm_partial_slot(mine, wave, 0, 0, e, lane), acc00[e], __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(gemm_partial_slot(mine, wave, 0, 1, e, lane), acc01[e], __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(gemm_partial_slot(mine, wave, 1, 0, e, lane), acc10[e], __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(gemm_partial_slot(mine, wave, 1, 1, e, lane), acc11[e], __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
  // every wave's partial stores have completed before thread 0 signals
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  GQK_WAIT_VMCNT(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (tid == 0) {
    const int old = __hip_atomic_fetch_add(&counters[tile * kGemmCounterStride], 1,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = old == S - 1;
  }
  __syncthreads();
  if (!last) return;
  gemm_sum_partials(partials, ntiles, tile, kGemmTileFloats, S, wave, lane, Y, n_tokens, rows, n0, r0, wi, wj);
  if (tid == 0)
    __hip_atomic_store(&counters[tile * kGemmCounterStride], 0, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

#undef GQK_GEMM_LOAD
#undef GQK_GEMM_STEP


// ---------------------------------------------------------------------------
// The same product with the operand tiles double-buffered in LDS, in two
// block shapes: kWi = 2 (4 waves, 128 tokens x 128 weight rows) or kWi = 4
// (8 waves, 256 tokens x 128 rows). Either way a wave computes a 64 x 64
// sub-tile (wave w: tokens 64 (w / 2), rows 64 (w % 2)) with the MFMA layout
// above. Steps of 64 k (one 32-byte nibble group: sub-blocks 2 g and 2 g + 1
// of a super-block); each thread holds the raw bytes of the next steps in
// registers (X: 16 bytes of 4 token rows; W: the super-block header and 32
// (kWi = 2) or 16 (kWi = 4) nibble bytes of one weight row, of which it
// decodes one nibble half: 32 or 16 weights), and while a wave's MFMAs read
// step s from one LDS buffer it decodes step s + 1 into the other: one
// barrier per step, and the decode's VALU work and LDS stores sit between the
// MFMAs instead of before them. A weight is decoded once per block, so the
// 256-token block spends half the decode work per MFMA of the 128-token one.
// The tile values are the same bits as the kernel above (fma(d sc, q, -dmin m)
// in fp32, rounded to nearest-even bf16). Split K and the partial-tile
// epilogue are those of the kernel above (a partial tile is the block's 128
// kWi x 64 fp32 values); the partial tiles and counters are indexed by the
// grid tile, so the matrices of a group share them.
// ---------------------------------------------------------------------------
// Load step `step` (clamped to the block's last: every slot issues the same
// loads, so the in-order wait counts stay exact; re-read steps are never
// decoded): X into register set S (2 sets), W into set G = step mod 4 (4
// sets: the weights come from HBM and get three steps of lead, X from L2 one).
#define GQK_GDB_STEP_CLAMP(step) ((step) < step_end ? (step) : step_end - 1)
#define GQK_GDB_LOAD_X(S, step)                                                                 \
  do {                                                                                          \
    const uint32_t ko_ = (uint32_t)GQK_GDB_STEP_CLAMP(step) * (kGdbBK * 2);                     \
    x##S##0 = *reinterpret_cast<const uint4*>(xbase + (xoff[0] + ko_));                        \
    x##S##1 = *reinterpret_cast<const uint4*>(xbase + (xoff[1] + ko_));                        \
    x##S##2 = *reinterpret_cast<const uint4*>(xbase + (xoff[2] + ko_));                        \
    x##S##3 = *reinterpret_cast<const uint4*>(xbase + (xoff[3] + ko_));                        \
  } while (0)
#define GQK_GDB_LOAD_W(G, step)                                                                 \
  do {                                                                                          \
    const int st_ = GQK_GDB_STEP_CLAMP(step);                                                   \
    const uint8_t* sb_ = wrow + (int64_t)(st_ >> 2) * kQ4KBlockBytes;                           \
    h##G = *reinterpret_cast<const uint4*>(sb_);                                                \
    const uint4* q_ = reinterpret_cast<const uint4*>(sb_ + 16 + 32 * (st_ & 3) + qpart);        \
    qa##G = q_[0];                                                                              \
    if constexpr (kWi == 2) qb##G = q_[1];                                                      \
  } while (0)

// Decodes X register set S and W register set G, a step of nibble group G (a
// constant 0..3), into LDS buffer BUF. Sub-block 2 G + half: 6-bit scale and min (sub-blocks 0..3:
// bytes j and j + 4 of the 12; 4..7: low / high nibble of byte j + 4 and the
// top two bits of bytes j - 4 / j). G is a constant and half only moves
// shifts, so the decode is straight-line code the scheduler can place
// between the MFMAs.
#define GQK_GDB_DECODE(S, G, BUF)                                                               \
  do {                                                                                          \
    uint8_t* xs_ = lds + (BUF) * kStage;                                                        \
    uint8_t* ws_ = xs_ + kBM * kGdbRow;                                                         \
    *reinterpret_cast<uint4*>(xs_ + (xr + 0 * kXRows) * kGdbRow + 16 * xc) = x##S##0;           \
    *reinterpret_cast<uint4*>(xs_ + (xr + 1 * kXRows) * kGdbRow + 16 * xc) = x##S##1;           \
    *reinterpret_cast<uint4*>(xs_ + (xr + 2 * kXRows) * kGdbRow + 16 * xc) = x##S##2;           \
    *reinterpret_cast<uint4*>(xs_ + (xr + 3 * kXRows) * kGdbRow + 16 * xc) = x##S##3;           \
    const uint32_t b_ = 8u * (2u * (uint32_t)((G) & 1) + (uint32_t)half);                       \
    const uint32_t s0_ = (h##G.y >> b_) & 0xFFu, s4_ = (h##G.z >> b_) & 0xFFu;                  \
    const uint32_t s8_ = (h##G.w >> b_) & 0xFFu;                                                \
    const uint32_t sc_ = (G) >= 2 ? ((s8_ & 15u) | ((s0_ >> 6) << 4)) : (s0_ & 63u);            \
    const uint32_t mm_ = (G) >= 2 ? ((s8_ >> 4) | ((s4_ >> 6) << 4)) : (s4_ & 63u);             \
    const float dl_ = half_lo(h##G.x) * (float)sc_;                                             \
    const float ml_ = half_hi(h##G.x) * (float)mm_;                                             \
    uint32_t qw_[kQWords];                                                                      \
    qw_[0] = qa##G.x;                                                                           \
    qw_[1] = qa##G.y;                                                                           \
    qw_[2] = qa##G.z;                                                                           \
    qw_[3] = qa##G.w;                                                                           \
    if constexpr (kWi == 2) {                                                                   \
      qw_[4 % kQWords] = qb##G.x;                                                               \
      qw_[5 % kQWords] = qb##G.y;                                                               \
      qw_[6 % kQWords] = qb##G.z;                                                               \
      qw_[7 % kQWords] = qb##G.w;                                                               \
    }                                                                                           \
    uint32_t o_[2 * kQWords];                                                                   \
    _Pragma("unroll") for (int t_ = 0; t_ < kQWords; ++t_) {                                    \
      const uint32_t n4_ = opaque((qw_[t_] >> nsh) & 0x0F0F0F0Fu);                              \
      o_[2 * t_] = pack_bf16x2(fmaf(dl_, ubyte0(n4_), -ml_), fmaf(dl_, ubyte1(n4_), -ml_));      \
      o_[2 * t_ + 1] = pack_bf16x2(fmaf(dl_, ubyte2(n4_), -ml_), fmaf(dl_, ubyte3(n4_), -ml_));  \
    }                                                                                           \
    uint4* wd_ = reinterpret_cast<uint4*>(ws_ + ld_row * kGdbRow + 64 * half + 2 * qpart);      \
    _Pragma("unroll") for (int t_ = 0; t_ < kQWords / 2; ++t_)                                  \
      wd_[t_] = make_uint4(o_[4 * t_], o_[4 * t_ + 1], o_[4 * t_ + 2], o_[4 * t_ + 3]);          \
  } while (0)

// Up to four Q4_K matrices of one X (q, k, v; gate, up) in one launch: their
// row tiles are laid end to end along grid x.
constexpr int kGemmMaxGroup = 4;
struct GemmGroup {
  const uint8_t* W[kGemmMaxGroup];
  uint16_t* Y[kGemmMaxGroup];
  int64_t rows[kGemmMaxGroup];
  int tile_begin[kGemmMaxGroup];   // first grid-x index of each matrix
  int n;
};

constexpr int kGdbBK = 64;                                   // k per step
constexpr int kGdbRow = kGdbBK * 2 + 16;                     // 144-byte LDS rows (36 dwords)
// tokens per block and fp32 values per partial tile of the kWi shape
constexpr int gdb_bm(int wi) { return 64 * wi; }
constexpr int64_t gdb_tile_floats(int wi) { return (int64_t)gdb_bm(wi) * kGemmBN; }

// Grid: one dimension. Blocks [0, nfull) take grid tiles 0 .. nfull - 1 over
// all of K; the later tiles are split into nsplit K ranges, range-major:
// block nfull + j nt + i takes K range j of tile nfull + i (nt split tiles),
// so that the blocks of one range of neighbouring tiles run together (taking
// a tile's ranges together ran the 128-token down and output GEMMs 7 and 4 us
// slower). A grid tile is (row tile t % gx, token tile t / gx). The host
// splits only the tiles past the last whole round of blocks, so that they
// fill one short round instead of a mostly idle full one.
// (The 256-token instance is held to two waves per SIMD explicitly: with the
// hint the compiler allocates 193 registers instead of 229, and the gate/up
// launch ran 67.0 against 69.2 us in a trace, 70.4 against 71.7 alone; the
// 128-token instance, one wave per SIMD at 288 registers, spills under it.)
template <int kWi>
__global__ __launch_bounds__(128 * kWi, kWi == 4 ? 2 : 1) void gemm_q4_k_db_kernel(GemmGroup G, const uint16_t* __restrict__ X,
                                                                 int64_t n_tokens, int nsb, int gx, int nfull,
                                                                 int nsplit, float* partials, int* counters) {
  static_assert(kWi == 2 || kWi == 4, "128 or 256 tokens per block");
  constexpr int kBM = gdb_bm(kWi);                       // tokens per block
  constexpr int kThreads = 128 * kWi;
  constexpr int kStage = (kBM + kGemmBN) * kGdbRow;      // one buffer: X rows, then W rows
  constexpr int kXRows = kThreads / 8;                   // token rows per X copy round
  constexpr int kQWords = 16 / kWi;                      // nibble words a thread decodes per step
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kStage];
  __shared__ int last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wi = wave >> 1, wj = wave & 1;
  // this block's grid tile and K range
  const int b = (int)blockIdx.x;
  const bool whole = b < nfull;
  const int ntr = ((int)gridDim.x - nfull) / nsplit;
  const int nt = ntr > 0 ? ntr : 1;                   // split tiles (none: 1, unused)
  const int q = b - nfull;
  const int qs = whole ? 0 : q / nt;
  const int tile = whole ? b : nfull + (q - qs * nt);
  const int S = whole ? 1 : nsplit, split = qs;
  const int bx = tile % gx, by = tile / gx;
  // its matrix and row tile
  const int m = (G.n > 1 && bx >= G.tile_begin[1]) + (G.n > 2 && bx >= G.tile_begin[2]) +
                (G.n > 3 && bx >= G.tile_begin[3]);
  const uint8_t* const W = m == 0 ? G.W[0] : m == 1 ? G.W[1] : m == 2 ? G.W[2] : G.W[3];
  uint16_t* const Y = m == 0 ? G.Y[0] : m == 1 ? G.Y[1] : m == 2 ? G.Y[2] : G.Y[3];
  const int64_t rows = m == 0 ? G.rows[0] : m == 1 ? G.rows[1] : m == 2 ? G.rows[2] : G.rows[3];
  const int tb = m == 0 ? G.tile_begin[0] : m == 1 ? G.tile_begin[1] : m == 2 ? G.tile_begin[2] : G.tile_begin[3];
  const int64_t n0 = (int64_t)by * kBM;
  const int64_t r0 = (int64_t)(bx - tb) * kGemmBN;
  const int64_t K = (int64_t)nsb * kQ4KBlockWeights;
  const int64_t row_bytes = (int64_t)nsb * kQ4KBlockBytes;
  // this block's steps: super-blocks [nsb * split / S, nsb * (split + 1) / S), 4 steps each
  const int step_begin = 4 * (int)((int64_t)nsb * split / S);
  const int step_end = 4 * (int)((int64_t)nsb * (split + 1) / S);

  // X: thread t copies the 16 bytes at k 8 xc .. 8 xc + 7 of the step of
  // token rows xr + kXRows j, j = 0..3 (a wave reads 8 whole 128-byte row
  // slices). W: kWi threads per weight row ld_row; thread t decodes nibble
  // half `half` (sub-block 2 g + half) of the group's bytes [qpart, qpart +
  // 32 / (kWi / 2)). Rows past the end are clamped (read, never stored).
  const int xc = tid & 7, xr = tid >> 3;
  uint32_t xoff[4];   // byte offsets (the host keeps X below 4 GiB for this kernel)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t n = n0 + xr + kXRows * j;
    xoff[j] = (uint32_t)(((n < n_tokens ? n : n_tokens - 1) * K + 8 * xc) * 2);
  }
  const int ld_row = tid / kWi;
  const int half = (tid / (kWi / 2)) & 1;
  const int qpart = kWi == 2 ? 0 : 16 * (tid & 1);
  const int64_t wr = (r0 + ld_row) < rows ? (r0 + ld_row) : (rows - 1);
  const uint8_t* wrow = W + wr * row_bytes;
  const uint32_t nsh = 4u * (uint32_t)half;   // low (half 0) or high nibbles

  // Register sets of raw step bytes: X (16 bytes of token rows xr + kXRows j),
  // sets A and B; W (the super-block header and the thread's nibble bytes),
  // sets 0..3 by nibble group. Named variables (arrays captured by helpers
  // stayed in scratch memory).
  uint4 xA0, xA1, xA2, xA3, xB0, xB1, xB2, xB3;
  uint4 h0, qa0, qb0, h1, qa1, qb1, h2, qa2, qb2, h3, qa3, qb3;
  (void)qb0;
  (void)qb1;
  (void)qb2;
  (void)qb3;
  const uint8_t* const xbase = reinterpret_cast<const uint8_t*>(X);

  f32x16 acc00, acc01, acc10, acc11;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc00[e] = acc01[e] = acc10[e] = acc11[e] = 0.f;
  auto mfma_step = [&](int buf) {
    const uint8_t* xs = lds + buf * kStage;
    const uint8_t* ws = xs + kBM * kGdbRow;
#pragma unroll
    for (int kk = 0; kk < kGdbBK; kk += 16) {
      const int kb = (kk + 8 * (lane >> 5)) * 2;
      const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(xs + (wi * 64 + (lane & 31)) * kGdbRow + kb);
      const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(xs + (wi * 64 + 32 + (lane & 31)) * kGdbRow + kb);
      const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(ws + (wj * 64 + (lane & 31)) * kGdbRow + kb);
      const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(ws + (wj * 64 + 32 + (lane & 31)) * kGdbRow + kb);
      acc00 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, acc00, 0, 0, 0);
      acc01 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, acc01, 0, 0, 0);
      acc10 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, acc10, 0, 0, 0);
      acc11 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, acc11, 0, 0, 0);
    }
  };

  // Pipeline: step s computes from buffer (s - step_begin) & 1 while the
  // registers of step s + 1 are decoded into the other buffer and step s + 2
  // is loaded into the registers just freed. A block has 4 steps per
  // super-block and at least one super-block (the host never splits K finer),
  // so the loop runs whole super-blocks; its last decode writes the re-read
  // last step into the buffer that is not read again. The body is
  // straight-line code, so the decode can be scheduled between the MFMAs.
  GQK_GDB_LOAD_X(A, step_begin);
  GQK_GDB_LOAD_W(0, step_begin);
  GQK_GDB_LOAD_X(B, step_begin + 1);
  GQK_GDB_LOAD_W(1, step_begin + 1);
  GQK_GDB_LOAD_W(2, step_begin + 2);
  GQK_GDB_LOAD_W(3, step_begin + 3);
  GQK_GDB_DECODE(A, 0, 0);
  __syncthreads();
  // one super-block (4 steps, groups 0..3) per pass; step_begin is a
  // multiple of 4, so step s + j has group j & 3
  for (int s = step_begin; s < step_end; s += 4) {
    GQK_GDB_LOAD_X(A, s + 2);
    GQK_GDB_LOAD_W(0, s + 4);
    mfma_step(0);
    GQK_GDB_DECODE(B, 1, 1);
    __syncthreads();
    GQK_GDB_LOAD_X(B, s + 3);
    GQK_GDB_LOAD_W(1, s + 5);
    mfma_step(1);
    GQK_GDB_DECODE(A, 2, 0);
    __syncthreads();
    GQK_GDB_LOAD_X(A, s + 4);
    GQK_GDB_LOAD_W(2, s + 6);
    mfma_step(0);
    GQK_GDB_DECODE(B, 3, 1);
    __syncthreads();
    GQK_GDB_LOAD_X(B, s + 5);
    GQK_GDB_LOAD_W(3, s + 7);
    mfma_step(1);
    GQK_GDB_DECODE(A, 0, 0);
    __syncthreads();
  }

  if (S == 1) {
    gemm_store_bf16(acc00, Y, n_tokens, rows, n0, r0, wi, wj, 0, 0, lane);
    gemm_store_bf16(acc01, Y, n_tokens, rows, n0, r0, wi, wj, 0, 1, lane);
    gemm_store_bf16(acc10, Y, n_tokens, rows, n0, r0, wi, wj, 1, 0, lane);
    gemm_store_bf16(acc11, Y, n_tokens, rows, n0, r0, wi, wj, 1, 1, lane);
    return;
  }

  // partial tiles and counters of the split tiles only, indexed from nfull
  const int64_t st = tile - nfull;
  const int64_t ntiles = nt;
  float* mine = partials + ((int64_t)split * ntiles + st) * gdb_tile_floats(kWi);
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    __hip_atomic_store(gemm_partial_slot(mine, wave, 0, 0, e, lane), acc00[e], __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(gemm_partial_slot(mine, wave, 0, 1, e, lane), acc01[e], __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(gemm_partial_slot(mine, wave, 1, 0, e, lane), acc10[e], __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(gemm_partial_slot(mine, wave, 1, 1, e, lane), acc11[e], __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
  // every wave's partial stores have completed before thread 0 signals
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  GQK_WAIT_VMCNT(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (tid == 0) {
    const int old = __hip_atomic_fetch_add(&counters[st * kGemmCounterStride], 1,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = old == S - 1;
  }
  __syncthreads();
  if (!last) return;
  gemm_sum_partials(partials, ntiles, st, gdb_tile_floats(kWi), S, wave, lane, Y, n_tokens, rows, n0, r0, wi,
                    wj);
  if (tid == 0)
    __hip_atomic_store(&counters[st * kGemmCounterStride], 0, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

#undef GQK_GDB_STEP_CLAMP
#undef GQK_GDB_LOAD_X
#undef GQK_GDB_LOAD_W
#undef GQK_GDB_DECODE

}  // namespace gqk
