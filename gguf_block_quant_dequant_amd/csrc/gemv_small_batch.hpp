// Small batch: Y[n, r] = sum_k X[n, k] w[r, k] for a few fp32 activation
// vectors (tokens) at once, W Q8_0 or Q4_K, Y fp32, on the gfx950 matrix
// cores. It is the decode matvec applied to each token row of X.
//
// Precision. The weight operand of the matrix instruction is the block's
// integer quant q (Q4_K 0..15, taken as q / 512; Q8_0 -128..127), exact in
// bf16. Each activation is split x = hi + lo with hi = bf16(x) and
// lo = bf16(x - hi), both rounded to nearest even (x - hi is exact in fp32),
// so hi + lo equals x within 2^-16 |x|. One 16-wide k step runs two MFMAs
// (hi, then lo) into the fp32 accumulator C of its 32-weight group (a Q4_K
// sub-block or a Q8_0 block), and the group's scale is applied in fp32 once
// the group is complete:
//   Q8_0: y += d * C
//   Q4_K: y += (512 d sc_j) * C_j for each sub-block j, then, once per
//         super-block, y -= dmin * sum_j m_j Xs_j, where Xs_j is the fp32 sum
//         of x over sub-block j, split hi/lo like x. That sum over j is one
//         more MFMA pair whose k slots 0..7 carry (Xs_j, m_j) and 8..15 zeros.
//
// Block: 4 waves, 128 weight rows (32 per wave) x 32 tokens; K is consumed
// 256 at a time (one Q4_K super-block, eight Q8_0 blocks). Each thread loads
// the next step's raw weight bytes and X values into registers while the
// current step's MFMAs run, then, after a barrier, stores them to LDS: the
// weights as the raw row segments (144 or 272 bytes per row, 36 or 68 dwords:
// 4 modulo 32 banks, so 16-byte reads of consecutive rows do not conflict),
// X as rows of 528 bytes (256 bf16 + the 8 Q4_K sub-block sums), once for hi
// and once for lo.
//
// MFMA operands (32x32x16 bf16, D = A B): A = X (lane l: token l % 32),
// B = W (lane l: weight row l % 32), both from k-group c = l / 32; slot
// e = 0..7 of a group carries the same k on both sides:
//   Q4_K step (g, h, s), g = 0..3, h = 0..1, s = 0..1: the lane of group c
//   holds quant bytes 32 g + 16 c + 8 s + e; their low (h = 0) or high
//   (h = 1) nibbles are weights k = 64 g + 32 h + 16 c + 8 s + e of
//   sub-block 2 g + h.
//   Q8_0 step (b, s), b = 0..7: k = 32 b + 16 c + 8 s + e of block b.
// D element e of lane l is token 8 (e / 4) + 4 (l / 32) + e % 4, weight row
// l % 32.
//
// Split K: gridDim.z ranges of whole 256-k steps. With more than one, each
// block stores its fp32 partial tile with agent-scope stores and bumps the
// tile's counter; the block that arrives last adds the partial tiles in range
// order (the result does not depend on arrival order), writes Y and resets
// the counter.
#pragma once

#include "device_common.hpp"
#include "mfma_types.hpp"

namespace gqk {

constexpr int kSbRows = 128;                        // weight rows per block
constexpr int kSbTokens = 32;                       // tokens per block
constexpr int kSbK = 256;                           // k per step
constexpr int kSbXRow = 528;                        // LDS bytes per token row (hi or lo)
constexpr int kSbTileFloats = kSbRows * kSbTokens;  // one fp32 partial tile
constexpr int kSbCounterStride = 32;                // ints: one 128-byte line per tile counter

template <bool Q4K>
struct SbFormat {
  static constexpr int kStepBytes = Q4K ? kQ4KBlockBytes : 8 * kQ80BlockBytes;  // per row
  static constexpr int kPieces = kStepBytes / 16;                               // 9 or 17
  static constexpr int kBlockPieces = kSbRows * kPieces;
  static constexpr int kPiecesPerThread = (kBlockPieces + 255) / 256;           // 5 or 9
};

// bf16 pair (a, b) from the upper halves of two fp32 values that have at most
// 8 significant bits (exact: nothing is rounded).
__device__ __forceinline__ uint32_t upper_halves(float a, float b) {
  return (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xFFFF0000u);
}

// Four bytes holding 0..15 as bf16 q / 512, two per instruction: read as OCP
// E4M3 fp8, a byte b < 16 is b x 2^-9 exactly, and bf16 holds that exactly.
template <bool kUpper>
__device__ __forceinline__ uint32_t nib2_bf16(uint32_t n) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)n, 1.0f, kUpper));
}
__device__ __forceinline__ bf16x8 nib8_bf16(uint32_t n0, uint32_t n1) {
  const uint32_t w0 = nib2_bf16<false>(n0), w1 = nib2_bf16<true>(n0);
  const uint32_t w2 = nib2_bf16<false>(n1), w3 = nib2_bf16<true>(n1);
  return __builtin_bit_cast(bf16x8, make_uint4(w0, w1, w2, w3));
}

// Eight signed bytes (two words) as bf16, exact.
__device__ __forceinline__ bf16x8 int8x8_bf16(uint32_t v0, uint32_t v1) {
  const uint32_t w0 = upper_halves(sbyte0(v0), sbyte1(v0));
  const uint32_t w1 = upper_halves(sbyte2(v0), sbyte3(v0));
  const uint32_t w2 = upper_halves(sbyte0(v1), sbyte1(v1));
  const uint32_t w3 = upper_halves(sbyte2(v1), sbyte3(v1));
  return __builtin_bit_cast(bf16x8, make_uint4(w0, w1, w2, w3));
}

__device__ __forceinline__ f32x16 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 lds_bf16x8(const uint8_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// One Q4_K super-block of this wave's 32 rows against the 32 staged tokens.
__device__ __forceinline__ void sb_q4k_step(const uint8_t* ws, const uint8_t* xh,
                                            const uint8_t* xl, int wave, int lane, f32x16& acc) {
  const int c = lane >> 5, rl = lane & 31;
  const uint8_t* wr = ws + (wave * 32 + rl) * kQ4KBlockBytes;
  const uint4 hd = *reinterpret_cast<const uint4*>(wr);
  const float d512 = half_lo(hd.x) * 512.0f, dmin = half_hi(hd.x);
  const uint32_t sc_lo = opaque(hd.y & 0x3F3F3F3Fu);
  const uint32_t sc_hi = opaque((hd.w & 0x0F0F0F0Fu) | ((hd.y >> 2) & 0x30303030u));
  const uint32_t m_lo = opaque(hd.z & 0x3F3F3F3Fu);
  const uint32_t m_hi = opaque(((hd.w >> 4) & 0x0F0F0F0Fu) | ((hd.z >> 2) & 0x30303030u));
  const float dsc[8] = {d512 * ubyte0(sc_lo), d512 * ubyte1(sc_lo), d512 * ubyte2(sc_lo),
                        d512 * ubyte3(sc_lo), d512 * ubyte0(sc_hi), d512 * ubyte1(sc_hi),
                        d512 * ubyte2(sc_hi), d512 * ubyte3(sc_hi)};
  const uint8_t* ah = xh + rl * kSbXRow + 32 * c;
  const uint8_t* al = xl + rl * kSbXRow + 32 * c;
  f32x16 zero;
#pragma unroll
  for (int e = 0; e < 16; ++e) zero[e] = 0.f;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const uint4 qv = *reinterpret_cast<const uint4*>(wr + 16 + 32 * g + 16 * c);
    f32x16 c0 = zero, c1 = zero;   // sub-blocks 2g (low nibbles) and 2g+1 (high nibbles)
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const uint32_t v0 = s ? qv.z : qv.x, v1 = s ? qv.w : qv.y;
      const bf16x8 blo = nib8_bf16(v0 & 0x0F0F0F0Fu, v1 & 0x0F0F0F0Fu);
      const bf16x8 bhi = nib8_bf16((v0 >> 4) & 0x0F0F0F0Fu, (v1 >> 4) & 0x0F0F0F0Fu);
      const int ko = 128 * g + 16 * s;
      c0 = mfma_bf16(lds_bf16x8(ah + ko), blo, c0);
      c0 = mfma_bf16(lds_bf16x8(al + ko), blo, c0);
      c1 = mfma_bf16(lds_bf16x8(ah + ko + 64), bhi, c1);
      c1 = mfma_bf16(lds_bf16x8(al + ko + 64), bhi, c1);
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      acc[e] = fmaf(dsc[2 * g], c0[e], acc[e]);
      acc[e] = fmaf(dsc[2 * g + 1], c1[e], acc[e]);
    }
    // keep the scheduler from hoisting every group's operands at once
    __builtin_amdgcn_sched_barrier(0);
  }
  // min term: k slots 0..7 of group 0 carry (Xs_j, m_j); group 1 is zero
  uint4 mw = make_uint4(0u, 0u, 0u, 0u), xsh = mw, xsl = mw;
  if (c == 0) {
    mw = make_uint4(upper_halves(ubyte0(m_lo), ubyte1(m_lo)), upper_halves(ubyte2(m_lo), ubyte3(m_lo)),
                    upper_halves(ubyte0(m_hi), ubyte1(m_hi)), upper_halves(ubyte2(m_hi), ubyte3(m_hi)));
    xsh = *reinterpret_cast<const uint4*>(xh + rl * kSbXRow + 512);
    xsl = *reinterpret_cast<const uint4*>(xl + rl * kSbXRow + 512);
  }
  const bf16x8 mb = __builtin_bit_cast(bf16x8, mw);
  f32x16 mm = mfma_bf16(__builtin_bit_cast(bf16x8, xsh), mb, zero);
  mm = mfma_bf16(__builtin_bit_cast(bf16x8, xsl), mb, mm);
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = fmaf(-dmin, mm[e], acc[e]);
}

// Eight Q8_0 blocks (256 k) of this wave's 32 rows against the staged tokens.
__device__ __forceinline__ void sb_q80_step(const uint8_t* ws, const uint8_t* xh,
                                            const uint8_t* xl, int wave, int lane, f32x16& acc) {
  const int c = lane >> 5, rl = lane & 31;
  const uint8_t* wr = ws + (wave * 32 + rl) * (8 * kQ80BlockBytes);
  const uint8_t* ah = xh + rl * kSbXRow + 32 * c;
  const uint8_t* al = xl + rl * kSbXRow + 32 * c;
  f32x16 zero;
#pragma unroll
  for (int e = 0; e < 16; ++e) zero[e] = 0.f;
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const float d = half_lo(*reinterpret_cast<const uint16_t*>(wr + kQ80BlockBytes * b));
    // quant bytes [o, o + 16) of this lane, o = 34 b + 2 + 16 c: 4-byte aligned
    // for odd b, 2 past a 4-byte boundary for even b
    const int o = kQ80BlockBytes * b + 2 + 16 * c;
    const uint32_t* pw = reinterpret_cast<const uint32_t*>(wr + (o & ~3));
    uint32_t q[4];
    if (b & 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i) q[i] = pw[i];
    } else {
      uint32_t v[5];
#pragma unroll
      for (int i = 0; i < 5; ++i) v[i] = pw[i];
#pragma unroll
      for (int i = 0; i < 4; ++i) q[i] = __builtin_amdgcn_alignbyte(v[i + 1], v[i], 2);
    }
    f32x16 cb = zero;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const bf16x8 bq = int8x8_bf16(q[2 * s], q[2 * s + 1]);
      const int ko = 64 * b + 16 * s;
      cb = mfma_bf16(lds_bf16x8(ah + ko), bq, cb);
      cb = mfma_bf16(lds_bf16x8(al + ko), bq, cb);
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = fmaf(d, cb[e], acc[e]);
  }
}

// Loads one step's staged operands into registers: this thread's weight
// pieces (byte offsets woff from the step's base wb) and its X values (four
// per token row, at k0 of each row).
// (Plain vector types, not HIP's uint4 struct: a struct copy is a memcpy that
// would keep the staging array in private memory.)
// Only the wave's first nvx token rows (the valid tokens) are loaded.
template <int N>
__device__ __forceinline__ void sb_load(i32x4 (&wreg)[N], float4 (&xr)[8], const uint8_t* wb,
                                        const uint32_t (&woff)[N], const float* const (&xrow)[8],
                                        int64_t k0, int xlane, int nvx) {
#pragma unroll
  for (int i = 0; i < N; ++i) wreg[i] = *reinterpret_cast<const i32x4*>(wb + woff[i]);
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (i < nvx) xr[i] = *reinterpret_cast<const float4*>(xrow[i] + k0 + xlane);
}

// Partial tile layout in scratch: [wave][e][lane] floats.
__device__ __forceinline__ float* sb_partial_slot(float* tile, int wave, int e, int lane) {
  return tile + ((wave * 16 + e) * 64 + lane);
}

__device__ __forceinline__ void sb_store(const f32x16& acc, float* __restrict__ Y, int n_tokens,
                                         int64_t rows, int n0, int64_t r0, int wave, int lane) {
  const int64_t r = r0 + wave * 32 + (lane & 31);
  if (r >= rows) return;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int n = n0 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
    if (n < n_tokens) Y[(int64_t)n * rows + r] = acc[e];
  }
}

// Up to four matrices of one X (q, k, v; gate, up) in one launch: their row
// tiles are laid end to end along grid x.
constexpr int kSbMaxGroup = 4;
struct SbGroup {
  const uint8_t* W[kSbMaxGroup];
  float* Y[kSbMaxGroup];
  int64_t rows[kSbMaxGroup];
  int tile_begin[kSbMaxGroup];   // first grid-x index of each matrix
  int n;
};

// grid (row tiles of all matrices, ceil(n_tokens / 32), S), block 256.
// `steps` = K / 256. The partial tiles and counters are indexed by the grid
// tile, so the matrices of a group share them.
template <bool Q4K>
__global__ __launch_bounds__(256, 2) void gemv_small_batch_kernel(
    SbGroup G, const float* __restrict__ X, int n_tokens, int steps, float* partials, int* counters) {
  using F = SbFormat<Q4K>;
  __shared__ __attribute__((aligned(16))) uint8_t ws[F::kBlockPieces * 16];
  __shared__ __attribute__((aligned(16))) uint8_t xh[kSbTokens * kSbXRow];
  __shared__ __attribute__((aligned(16))) uint8_t xl[kSbTokens * kSbXRow];
  __shared__ int last;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bx = (int)blockIdx.x;
  const int m = (G.n > 1 && bx >= G.tile_begin[1]) + (G.n > 2 && bx >= G.tile_begin[2]) +
                (G.n > 3 && bx >= G.tile_begin[3]);
  const uint8_t* const W = m == 0 ? G.W[0] : m == 1 ? G.W[1] : m == 2 ? G.W[2] : G.W[3];
  float* const Y = m == 0 ? G.Y[0] : m == 1 ? G.Y[1] : m == 2 ? G.Y[2] : G.Y[3];
  const int64_t rows = m == 0 ? G.rows[0] : m == 1 ? G.rows[1] : m == 2 ? G.rows[2] : G.rows[3];
  const int tb = m == 0 ? G.tile_begin[0] : m == 1 ? G.tile_begin[1] : m == 2 ? G.tile_begin[2] : G.tile_begin[3];
  const int64_t r0 = (int64_t)(bx - tb) * kSbRows;
  const int n0 = (int)blockIdx.y * kSbTokens;
  const int S = (int)gridDim.z, split = (int)blockIdx.z;
  const int64_t K = (int64_t)steps * kSbK;
  const int64_t row_bytes = (int64_t)steps * F::kStepBytes;
  const int st_begin = (int)((int64_t)steps * split / S);
  const int st_end = (int)((int64_t)steps * (split + 1) / S);

  // Weight staging: piece p = tid + 256 i is bytes [16 p, 16 p + 16) of the
  // block's LDS image, i.e. bytes [16 (p % P), ...) of row p / P's step
  // segment (P = 9 or 17 pieces per row). Rows past the end are clamped
  // (read, never stored); pieces past the image are not stored.
  const uint8_t* Wb = W + r0 * row_bytes;
  uint32_t woff[F::kPiecesPerThread];
#pragma unroll
  for (int i = 0; i < F::kPiecesPerThread; ++i) {
    int p = tid + 256 * i;
    if (p >= F::kBlockPieces) p = F::kBlockPieces - 1;
    const int row = p / F::kPieces, col = p % F::kPieces;
    const int64_t rr = (r0 + row < rows) ? row : (rows - 1 - r0);
    woff[i] = (uint32_t)(rr * row_bytes + 16 * col);
  }
  // X staging: wave w, i = 0..7 stages token w + 4 i, lane l its values
  // k = 4 l .. 4 l + 3 of the step (one 1 KiB row per wave load). Only the
  // valid tokens (i < nvx) are loaded and staged: the LDS rows of tokens past
  // the end hold stale values, which reach only outputs that are never stored
  // (each output element belongs to one token).
  // (row bases are wave-uniform: scalar registers; the lane offset is common)
  const float* xrow[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int n = n0 + wave + 4 * i;
    if (n >= n_tokens) n = n_tokens - 1;
    xrow[i] = X + (int64_t)n * K;
  }
  const int xlane = 4 * lane;
  int nvx = (n_tokens - n0 - wave + 3) / 4;   // valid token rows of this wave
  nvx = nvx < 0 ? 0 : nvx > 8 ? 8 : nvx;
  // token groups of 8 holding a valid token: partial tiles carry only these
  const int ng = (n_tokens - n0 < kSbTokens ? n_tokens - n0 + 7 : kSbTokens) / 8;

  i32x4 wreg[F::kPiecesPerThread];
  float4 xr[8];
  f32x16 acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;

  sb_load(wreg, xr, Wb + (int64_t)st_begin * F::kStepBytes, woff, xrow, (int64_t)st_begin * kSbK, xlane, nvx);
  for (int st = st_begin; st < st_end; ++st) {
    __syncthreads();   // the previous step's LDS reads are done
#pragma unroll
    for (int i = 0; i < F::kPiecesPerThread - 1; ++i)
      *reinterpret_cast<i32x4*>(ws + 16 * (tid + 256 * i)) = wreg[i];
    if (tid + 256 * (F::kPiecesPerThread - 1) < F::kBlockPieces)
      *reinterpret_cast<i32x4*>(ws + 16 * (tid + 256 * (F::kPiecesPerThread - 1))) =
          wreg[F::kPiecesPerThread - 1];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i >= nvx) break;
      const int t = wave + 4 * i;
      const float4 v = xr[i];
      const uint32_t h01 = pack_bf16x2(v.x, v.y), h23 = pack_bf16x2(v.z, v.w);
      const float l0 = v.x - __uint_as_float(h01 << 16);
      const float l1 = v.y - __uint_as_float(h01 & 0xFFFF0000u);
      const float l2 = v.z - __uint_as_float(h23 << 16);
      const float l3 = v.w - __uint_as_float(h23 & 0xFFFF0000u);
      *reinterpret_cast<uint2*>(xh + t * kSbXRow + 8 * lane) = make_uint2(h01, h23);
      *reinterpret_cast<uint2*>(xl + t * kSbXRow + 8 * lane) =
          make_uint2(pack_bf16x2(l0, l1), pack_bf16x2(l2, l3));
      if (Q4K) {
        // sub-block j = lane / 8 covers the 8 lanes 8 j .. 8 j + 7
        float s = (v.x + v.y) + (v.z + v.w);
        s += __shfl_xor(s, 1);
        s += __shfl_xor(s, 2);
        s += __shfl_xor(s, 4);
        if ((lane & 7) == 0) {
          const uint16_t sh = to_bf16(s);
          const float sl = s - __uint_as_float((uint32_t)sh << 16);
          *reinterpret_cast<uint16_t*>(xh + t * kSbXRow + 512 + 2 * (lane >> 3)) = sh;
          *reinterpret_cast<uint16_t*>(xl + t * kSbXRow + 512 + 2 * (lane >> 3)) = to_bf16(sl);
        }
      }
    }
    __syncthreads();
    if (st + 1 < st_end)
      sb_load(wreg, xr, Wb + (int64_t)(st + 1) * F::kStepBytes, woff, xrow, (int64_t)(st + 1) * kSbK, xlane,
              nvx);
    if (Q4K)
      sb_q4k_step(ws, xh, xl, wave, lane, acc);
    else
      sb_q80_step(ws, xh, xl, wave, lane, acc);
  }

  if (S == 1) {
    sb_store(acc, Y, n_tokens, rows, n0, r0, wave, lane);
    return;
  }
  const int64_t tile = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
  const int64_t ntiles = (int64_t)gridDim.x * gridDim.y;
  float* mine = partials + ((int64_t)split * ntiles + tile) * kSbTileFloats;
  // element e holds token 8 (e / 4) + ...: only groups with a valid token
#pragma unroll
  for (int e = 0; e < 16; ++e)
    if ((e >> 2) < ng)
      __hip_atomic_store(sb_partial_slot(mine, wave, e, lane), acc[e], __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  // every wave's partial stores have completed before thread 0 signals
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  GQK_WAIT_VMCNT(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (tid == 0) {
    const int old = __hip_atomic_fetch_add(&counters[tile * kSbCounterStride], 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
    last = old == S - 1;
  }
  __syncthreads();
  if (!last) return;
  // The partial tiles are read four ranges at a time (one round trip per four,
  // indexes past the last range clamped and not added) and added in range
  // order. Every load is issued, whatever the valid token groups (a group
  // past them re-reads group 0's slot and is not added): loads under a
  // condition went out one at a time.
  f32x16 sum;
#pragma unroll
  for (int e = 0; e < 16; ++e) sum[e] = 0.f;
  for (int s0 = 0; s0 < S; s0 += 4) {
    float v[4][16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = s0 + i < S ? s0 + i : S - 1;
      float* p = partials + ((int64_t)s * ntiles + tile) * kSbTileFloats;
#pragma unroll
      for (int e = 0; e < 16; ++e)
        v[i][e] = __hip_atomic_load(sb_partial_slot(p, wave, (e >> 2) < ng ? e : (e & 3), lane), __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (s0 + i < S) {
#pragma unroll
        for (int e = 0; e < 16; ++e) sum[e] += (e >> 2) < ng ? v[i][e] : 0.f;
      }
  }
  sb_store(sum, Y, n_tokens, rows, n0, r0, wave, lane);
  if (tid == 0)
    __hip_atomic_store(&counters[tile * kSbCounterStride], 0, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace gqk
