// Small batch, Q4_K rows: Y[n, r] = sum_k X[n, k] w[r, k] for up to 16 fp32
// activation vectors (tokens) per block, Y fp32, on the gfx950 matrix cores.
// It is the decode matvec applied to each token row of X.
//
// Matrix instruction v_mfma_f32_16x16x32_bf16, D[i][j] = sum_k A[i][k] B[k][j]
// with A = X (row i = token slot), B = W (column j = weight row) and one
// 32-weight sub-block per instruction. Lane l holds A row / B column l % 16
// and k = 8 (l / 16) + e, e = 0..7; D lane l holds column l % 16 (one weight
// row) and rows 4 (l / 16) + i, i = 0..3 (four tokens).
//
// Precision. B is the sub-block's integer quant q as bf16 q / 512 (exact: a
// byte b < 16 read as OCP E4M3 is b 2^-9). Each activation is split
// x = hi + lo, hi = bf16(x), lo = bf16(x - hi) (both nearest even; x - hi is
// exact in fp32), so hi + lo equals x within 2^-16 |x|. One sub-block runs two
// MFMAs (hi, then lo) into an fp32 C, and the row's scale is applied in fp32:
// y += (512 d sc_j) C_j; once per super-block y -= dmin sum_j m_j Xs_j, where
// Xs_j is the fp32 sum of x over sub-block j (a fixed order: eight values per
// lane, then the four lanes of the token), split hi/lo like x: one more MFMA
// pair whose k slots 0..7 of the lanes with l / 16 = 0 carry (Xs_j, m_j) and
// every other slot zero.
//
// Block: RT row tiles of 16 rows of one matrix, the tokens of one grid-y
// chunk (at most 16), K range [sb0, sb1) of super-blocks (gridDim.z
// ranges); wave w takes super-block sb0 + w of the range. The block stages
// the range's activations once (whole 1 KiB rows per load, split into bf16
// hi and lo in the A layout in LDS) and each wave takes its super-block's
// operands into registers; it then streams the row tiles' weights through a
// register ring of kSbwDepth tiles (a header and four 8-byte quant pieces per
// lane and tile: bytes
// 32 g + 8 (l / 16) of group g, whose low nibbles are sub-block 2 g and high
// nibbles 2 g + 1), runs each tile's MFMAs from registers and leaves its
// sums in LDS. The waves' sums are then added in wave order. Weights are read
// once per launch for up to 16 tokens.
//
// Paired layout (at most eight tokens, kPair): token slots 0..7 and 8..15
// carry the same tokens, so one instruction can take two sub-blocks at
// once: lane l (row l % 16, group c = l / 16) loads 16 consecutive quant
// bytes 16 c .. 16 c + 15 (then 64 + 16 c ..) of its row, so the four lanes
// of a row read 64 consecutive bytes per load (three loads per tile: header
// and two quant halves; the layout above takes five narrower ones, each
// touching sixteen rows in 8-byte pieces). Lanes c = 0, 1 then hold quant
// group 2 q and lanes c = 2, 3 group 2 q + 1 (q the half). The A operand of
// slots 0..7 is zero in the k slots of lanes c >= 2, that of slots 8..15 zero
// in those of lanes c < 2, so D rows 0..7 sum one sub-block and rows 8..15
// the other: lanes c < 2 hold the first (tokens 4 c + i), lanes c >= 2 the
// second (tokens 4 (c - 2) + i), each scaled by its own sub-block's factor,
// and the two lanes of a (row, token) are added with the wave sums. Each
// instruction still covers 32 weights of one sub-block per D row: eighteen
// MFMAs per tile, as above.
//
// Split K: with more than one range, each block stores its fp32 sums (valid
// tokens only) with agent-scope stores and bumps its tile's counter; the
// block that arrives last adds the partial tiles in range order (the result
// does not depend on arrival order), writes Y and resets the counter.
#pragma once

#include "coherent.hpp"
#include "device_common.hpp"
#include "gemv_small_batch.hpp"
#include "timeline.hpp"

namespace gqk {

typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef uint32_t sbw_u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t sbw_u32x4 __attribute__((ext_vector_type(4)));

constexpr int kSbwMaxTokens = 16;   // tokens per block (grid y covers more)
constexpr int kSbwRouteTokens = 32; // token counts the small-batch calls send here
constexpr int kSbwMaxWaves = 8;     // super-blocks of one K range at most
constexpr int kSbwMaxTiles = 16;    // row tiles of 16 per block at most
// weight ring (row tiles in flight per wave): two measured faster than three
// or four (8 tokens: 1.33 / 1.34 / 1.36 ms per pass)
constexpr int kSbwDepth = 2;

// LDS bytes of a block: the staged activations of its (at most nw)
// super-blocks (token slots x 16 bytes x (64 A operand groups + 2 sums) each),
// and the waves' sums [row tile][wave][4 x 64 floats]: in the same area for
// the shared staging, one after the other for the paired layout's per-wave
// staging (eight token slots).
constexpr size_t sbw_lds_bytes(int rt, int nw, int slots, bool pair) {
  const size_t x = (size_t)nw * slots * 16 * 66, r = (size_t)rt * nw * 256 * 4;
  return pair ? x + r : x > r ? x : r;
}
constexpr int kSbwPairWaveBytes = 8 * 16 * 66;   // one wave's staged super-block, eight slots
constexpr size_t kSbwLdsLimit = 160 * 1024 - 256;   // dynamic LDS at most (the static part stays below 256 bytes)

// Launch arguments past the leading scalar ones (the first fourteen dwords,
// preloaded into scalar registers): the fourth matrix, the outputs and the
// split-K scratch.
struct SbwRest {
  const uint8_t* W3;
  float* Y[kSbMaxGroup];
  int rows3;
  float* partials;   // split K only
  int* counters;
};

// The packed launch shape: waves per block, row tiles per block, matrices,
// K ranges (at most 8, 16, 4 and 65535).
__host__ __device__ constexpr uint32_t sbw_shape(int nw, int rt, int n, int S) {
  return (uint32_t)nw | ((uint32_t)rt << 4) | ((uint32_t)n << 9) | ((uint32_t)S << 12);
}

// A DPP move of a float (bound_ctrl set: lanes without a source read 0).
template <int kCtrl>
__device__ __forceinline__ float sbw_dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, true));
}

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <bool kPair>
struct SbwUnit {
  sbw_u32x4 h;      // super-block header of the lane's row
  sbw_u32x2 q[4];   // quant bytes 32 g + 8 (l / 16) .. + 7, g = 0..3
};

template <>
struct SbwUnit<true> {
  sbw_u32x4 h;    // super-block header of the lane's row
  sbw_u32x4 qa;   // quant bytes 16 (l / 16) .. + 15
  sbw_u32x4 qb;   // quant bytes 64 + 16 (l / 16) .. + 15
};

// Eight fp32 values as bf16 hi and lo halves (x = hi + lo within 2^-16 |x|).
__device__ __forceinline__ void split8(const float4& a, const float4& b, bf16x8& hi, bf16x8& lo) {
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    const float l0 = v[2 * i] - __uint_as_float(h[i] << 16);
    const float l1 = v[2 * i + 1] - __uint_as_float(h[i] & 0xFFFF0000u);
    l[i] = pack_bf16x2(l0, l1);
  }
  hi = __builtin_bit_cast(bf16x8, make_uint4(h[0], h[1], h[2], h[3]));
  lo = __builtin_bit_cast(bf16x8, make_uint4(l[0], l[1], l[2], l[3]));
}

// grid (row-tile groups of all matrices, token chunks of 16, K ranges),
// block of 64 x (longest range) threads. Matrix m's weights and rows: W0..W2
// / R.W3, rows0..2 / R.rows3; its blocks follow the previous matrix's along
// grid x, ceil(ceil(rows / 16) / rt) of them; shape = sbw_shape(nw, rt, n, S).
// kPair: the paired layout (one token chunk of at most eight tokens).
template <bool kPair>
__global__ __launch_bounds__(64 * kSbwMaxWaves) void gemv_sbw_kernel(const uint8_t* W0, const uint8_t* W1,
                                                                   const uint8_t* W2, const float* __restrict__ X,
                                                                   int nsb, int n_tokens, uint32_t shape,
                                                                   int rows0, int rows1, int rows2, SbwRest R) {
  constexpr int kD = kSbwDepth;
  extern __shared__ __attribute__((aligned(16))) float lds_f[];
  __shared__ int last;
  TlStamps tl;
  tl.stamp(0);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nw = (int)(shape & 15u), RT = (int)((shape >> 4) & 31u), ng = (int)((shape >> 9) & 7u);
  const int S = (int)(shape >> 12);
  const int nthreads = 64 * nw;
  const int bx = (int)blockIdx.x;
  const int n0 = (int)blockIdx.y * kSbwMaxTokens;
  const int nb = n_tokens - n0 < kSbwMaxTokens ? n_tokens - n0 : kSbwMaxTokens;   // tokens of this block
  const int split = (int)blockIdx.z;
  // (nsb S < 2^23: 32-bit division)
  const int sb0 = (int)((uint32_t)(nsb * split) / (uint32_t)S);
  const int sb1 = (int)((uint32_t)(nsb * (split + 1)) / (uint32_t)S);
  const bool active = sb0 + wave < sb1;      // the longest range has nw super-blocks
  const int sb = active ? sb0 + wave : sb0;  // an idle wave re-reads the range's first one
  const int64_t K = (int64_t)nsb * 256;
  // Paired layout: the nb token rows of the wave's own super-block (rows past
  // nb re-read the last and are not staged), loaded before anything else,
  // from preloaded arguments only.
  float4 xp[8];
  if constexpr (kPair) {
    const float* const xsb = X + (int64_t)n0 * K + (int64_t)sb * 256 + 4 * lane;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = i < nb ? i : nb - 1;
      xp[i] = *reinterpret_cast<const float4*>(xsb + (int64_t)t * K);
    }
  }
  auto blocks_of = [&](int r) { return (int)((((uint32_t)r + 15u) / 16u + (uint32_t)RT - 1u) / (uint32_t)RT); };
  const int tb1 = blocks_of(rows0);
  const int tb2 = ng > 2 ? tb1 + blocks_of(rows1) : INT32_MAX;
  const int tb3 = ng > 3 ? tb2 + blocks_of(rows2) : INT32_MAX;
  const int m = (ng > 1 && bx >= tb1) + (bx >= tb2) + (bx >= tb3);
  const uint8_t* W = m == 0 ? W0 : m == 1 ? W1 : W2;
  int rows = m == 0 ? rows0 : m == 1 ? rows1 : rows2;
  if (m == 3) {
    // (kept as a branch: read on every path, these arguments would be waited
    // for before the first weight load of every launch)
    asm volatile("" ::: "memory");
    W = R.W3;
    rows = R.rows3;
  }
  const int tb = m == 0 ? 0 : m == 1 ? tb1 : m == 2 ? tb2 : tb3;
  const int r0 = (bx - tb) * 16 * RT;
  const int ntile = (rows - r0 + 15) / 16 < RT ? (rows - r0 + 15) / 16 : RT;   // >= 1
  const uint32_t row_bytes = (uint32_t)nsb * kQ4KBlockBytes;
  const int c4 = lane >> 4, col = lane & 15;

  // row tile u of the block (rows past the matrix re-read its last row, which
  // is never stored). A slot past the block's last tile loads the first 16
  // bytes of the wave's super-block column in every lane (one cache line); the
  // choice is made per lane, so every slot issues the same loads on every
  // path and the in-order load counter stays exact (a uniform branch around
  // the loads made the compiler wait for the whole ring before the
  // activations were staged).
  const GQK_GLOBAL uint8_t* const wb = (const GQK_GLOBAL uint8_t*)W + (uint32_t)sb * kQ4KBlockBytes;
  auto issue = [&](int u, SbwUnit<kPair>& L) {
    int on = u < ntile;
    asm volatile("" : "+v"(on));
    int r = r0 + 16 * (u < ntile ? u : ntile - 1) + col;
    r = r < rows ? r : rows - 1;
    const GQK_GLOBAL uint8_t* const b = wb + (int64_t)r * row_bytes;
    auto at = [&](uint32_t off) { return on ? b + off : wb; };
    L.h = *reinterpret_cast<const GQK_GLOBAL sbw_u32x4*>(at(0u));
    if constexpr (kPair) {
      L.qa = *reinterpret_cast<const GQK_GLOBAL sbw_u32x4*>(at(16u + 16u * c4));
      L.qb = *reinterpret_cast<const GQK_GLOBAL sbw_u32x4*>(at(80u + 16u * c4));
    } else {
#pragma unroll
      for (int g = 0; g < 4; ++g)
        L.q[g] = *reinterpret_cast<const GQK_GLOBAL sbw_u32x2*>(at(16u + 32u * g + 8u * c4));
    }
  };
  SbwUnit<kPair> ring[kD];
  // Activations: the block's waves load the (super-block, token) rows of the
  // range, one 1 KiB row per wave load (lane q: float4 q, k = 4 q: sub-block
  // j = q / 8, k group c = (q / 2) % 4, half q % 2), split them into bf16 hi
  // and lo in the A layout in LDS, with each sub-block's sum; then each wave
  // takes its super-block's operands into registers. The first eight rows of
  // a wave are loaded before the weight ring is issued (loads complete in
  // order), further ones (more than eight tokens) after.
  //   A at ((sbl 2 + p) 32 + j 4 + c) kSlots + token) 16 bytes (p 0 hi, 1 lo)
  //   sums at A end + ((sbl 2 + p) kSlots + token) 16 bytes (8 bf16: j)
  const int ns = sb1 - sb0;                            // super-blocks of the range
  const int slots = kPair ? 8 : nb <= 8 ? 8 : 16;      // token slots per sub-block
  // paired layout: wave w stages its own super-block at w kSbwPairWaveBytes
  // (the sums of the waves after all of them); else the block's range from 0
  // (the sums in the same area, once the operands are read)
  uint8_t* const xl = reinterpret_cast<uint8_t*>(lds_f) + (kPair ? wave * kSbwPairWaveBytes : 0);
  float* const red = kPair ? lds_f + nw * (kSbwPairWaveBytes / 4) : lds_f;
  const int a_bytes = (kPair ? 1 : ns) * 2 * 32 * slots * 16;
  const int npr = ns * nb;
  auto load_rows = [&](int pb, float4 (&xv)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int pr = pb + nw * i;
      pr = pr < npr ? pr : npr - 1;
      const int sl = pr / nb, t = pr - sl * nb;
      xv[i] = *reinterpret_cast<const float4*>(X + (int64_t)(n0 + t) * K + (int64_t)(sb0 + sl) * 256 + 4 * lane);
    }
  };
  // token t of super-block sl of the staged range: A operands and sums
  auto stage_one = [&](int sl, int t, const float4& v) {
      const uint32_t h01 = pack_bf16x2(v.x, v.y), h23 = pack_bf16x2(v.z, v.w);
      const float l0 = v.x - __uint_as_float(h01 << 16);
      const float l1 = v.y - __uint_as_float(h01 & 0xFFFF0000u);
      const float l2 = v.z - __uint_as_float(h23 << 16);
      const float l3 = v.w - __uint_as_float(h23 & 0xFFFF0000u);
      const int j = lane >> 3, c = (lane >> 1) & 3, half = lane & 1;
      uint8_t* ap = xl + (((sl * 2) * 32 + j * 4 + c) * slots + t) * 16 + 8 * half;
      *reinterpret_cast<uint2*>(ap) = make_uint2(h01, h23);
      *reinterpret_cast<uint2*>(ap + 32 * slots * 16) = make_uint2(pack_bf16x2(l0, l1), pack_bf16x2(l2, l3));
      // sub-block j covers lanes 8 j .. 8 j + 7 (a half row): every lane
      // gets their sum (pairs, quads, then the other quad of the half row)
      float sum = (v.x + v.y) + (v.z + v.w);
      sum += sbw_dpp<0xB1>(sum);   // quad_perm 1,0,3,2
      sum += sbw_dpp<0x4E>(sum);   // quad_perm 2,3,0,1
      sum += sbw_dpp<0x141>(sum);  // row_half_mirror
      if ((lane & 7) == 0) {
        const uint16_t shi = to_bf16(sum);
        const float slo = sum - __uint_as_float((uint32_t)shi << 16);
        uint8_t* sp = xl + a_bytes + ((sl * 2) * slots + t) * 16 + 2 * j;
        *reinterpret_cast<uint16_t*>(sp) = shi;
        *reinterpret_cast<uint16_t*>(sp + slots * 16) = to_bf16(slo);
      }
  };
  auto stage_rows = [&](int pb, const float4 (&xv)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int pr = pb + nw * i;
      if (pr >= npr) break;
      const int sl = pr / nb, t = pr - sl * nb;
      stage_one(sl, t, xv[i]);
    }
  };
  if constexpr (kPair) {
    // the weight ring, then the wave's rows into its own area and a
    // wave-level exchange: no block barrier
#pragma unroll
    for (int p = 0; p < kD; ++p) issue(p, ring[p]);
    tl.stamp(1);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i < nb) stage_one(0, i, xp[i]);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  } else {
    float4 xv[8];
    load_rows(wave, xv);
#pragma unroll
    for (int p = 0; p < kD; ++p) issue(p, ring[p]);
    tl.stamp(1);
    if (wave < npr) stage_rows(wave, xv);
    for (int pb = wave + 8 * nw; pb < npr; pb += 8 * nw) {
      load_rows(pb, xv);
      stage_rows(pb, xv);
    }
    __syncthreads();
  }
  bf16x8 z8;
#pragma unroll
  for (int e = 0; e < 8; ++e) z8[e] = 0;
  bf16x8 ah[8], al[8], zh, zl;
  {
    // token slot col (slots past the valid tokens hold stale values, which
    // reach only outputs that are never stored); an idle wave reads the
    // range's first super-block
    const int sl = kPair ? 0 : active ? wave : 0, ts = col & (slots - 1);
    if constexpr (kPair) {
      // operand q 4 + h 2 + e: sub-block 2 (2 q + c4 / 2) + h, k chunk
      // 2 (c4 % 2) + e; zero where the lane's group does not feed its slot
      const bool on = (col < 8) == (c4 < 2);
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int sbk = 2 * (2 * q + (c4 >> 1)) + h, ck = 2 * (c4 & 1) + e;
            const uint8_t* ap = xl + (((sl * 2) * 32 + sbk * 4 + ck) * slots + ts) * 16;
            // (only the lanes whose group feeds their slot read: half the
            // LDS traffic of reading in every lane and selecting)
            bf16x8 vh = z8, vl = z8;
            if (on) {
              vh = *reinterpret_cast<const bf16x8*>(ap);
              vl = *reinterpret_cast<const bf16x8*>(ap + 32 * slots * 16);
            }
            ah[q * 4 + h * 2 + e] = vh;
            al[q * 4 + h * 2 + e] = vl;
          }
    } else {
      const uint8_t* ap = xl + (((sl * 2) * 32 + c4) * slots + ts) * 16;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        ah[j] = *reinterpret_cast<const bf16x8*>(ap + j * 4 * slots * 16);
        al[j] = *reinterpret_cast<const bf16x8*>(ap + (32 + j * 4) * slots * 16);
      }
    }
    const uint8_t* sp = xl + a_bytes + ((sl * 2) * slots + ts) * 16;
    const bf16x8 sh = *reinterpret_cast<const bf16x8*>(sp), sl2 = *reinterpret_cast<const bf16x8*>(sp + slots * 16);
    // the minimum terms: slots 0..7 only in the paired layout
    const bool zon = c4 == 0 && (!kPair || col < 8);
    zh = zon ? sh : z8;
    zl = zon ? sl2 : z8;
  }
  // every wave has its operands: the area is reused for the sums
  if constexpr (!kPair) __syncthreads();
  tl.stamp(2);
  f32x4 zero4;
#pragma unroll
  for (int i = 0; i < 4; ++i) zero4[i] = 0.f;

  // row tile u: its sums (element i of this lane) to red[u][wave]
  auto tile = [&](int u, const SbwUnit<kPair>& L) {
    const uint32_t h0 = L.h.x, h1 = L.h.y, h2 = L.h.z, h3 = L.h.w;
    const float d512 = half_lo(h0) * 512.0f, dmin = half_hi(h0);
    const uint32_t sc_lo = opaque(h1 & 0x3F3F3F3Fu);
    const uint32_t sc_hi = opaque((h3 & 0x0F0F0F0Fu) | ((h1 >> 2) & 0x30303030u));
    const uint32_t m_lo = opaque(h2 & 0x3F3F3F3Fu);
    const uint32_t m_hi = opaque(((h3 >> 4) & 0x0F0F0F0Fu) | ((h2 >> 2) & 0x30303030u));
    f32x4 c = zero4;
    if constexpr (kPair) {
      // the lane's sub-blocks 4 q + 2 (c4 / 2) + h: bytes 2 (c4 / 2) + h of
      // sc_lo (q = 0) and sc_hi (q = 1)
      const uint32_t bsh = 16u * (uint32_t)(c4 >> 1);
      const float dq[2][2] = {{d512 * (float)((sc_lo >> bsh) & 0xFFu), d512 * (float)((sc_lo >> (bsh + 8u)) & 0xFFu)},
                              {d512 * (float)((sc_hi >> bsh) & 0xFFu), d512 * (float)((sc_hi >> (bsh + 8u)) & 0xFFu)}};
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const sbw_u32x4 Q = q == 0 ? L.qa : L.qb;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          f32x4 cc = zero4;
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const uint32_t v0 = Q[2 * e] >> (4 * h), v1 = Q[2 * e + 1] >> (4 * h);
            const bf16x8 bq = nib8_bf16(v0 & 0x0F0F0F0Fu, v1 & 0x0F0F0F0Fu);
            cc = mfma16(ah[q * 4 + h * 2 + e], bq, cc);
            cc = mfma16(al[q * 4 + h * 2 + e], bq, cc);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) c[i] = fmaf(dq[q][h], cc[i], c[i]);
        }
      }
    } else {
    const float dsc[8] = {d512 * ubyte0(sc_lo), d512 * ubyte1(sc_lo), d512 * ubyte2(sc_lo),
                          d512 * ubyte3(sc_lo), d512 * ubyte0(sc_hi), d512 * ubyte1(sc_hi),
                          d512 * ubyte2(sc_hi), d512 * ubyte3(sc_hi)};
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint32_t v0 = L.q[g].x, v1 = L.q[g].y;
      const bf16x8 blo = nib8_bf16(v0 & 0x0F0F0F0Fu, v1 & 0x0F0F0F0Fu);
      const bf16x8 bhi = nib8_bf16((v0 >> 4) & 0x0F0F0F0Fu, (v1 >> 4) & 0x0F0F0F0Fu);
      f32x4 c0 = mfma16(ah[2 * g], blo, zero4);
      c0 = mfma16(al[2 * g], blo, c0);
      f32x4 c1 = mfma16(ah[2 * g + 1], bhi, zero4);
      c1 = mfma16(al[2 * g + 1], bhi, c1);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c[i] = fmaf(dsc[2 * g], c0[i], c[i]);
        c[i] = fmaf(dsc[2 * g + 1], c1[i], c[i]);
      }
    }
    }
    const bf16x8 mb = __builtin_bit_cast(
        bf16x8, make_uint4(upper_halves(ubyte0(m_lo), ubyte1(m_lo)), upper_halves(ubyte2(m_lo), ubyte3(m_lo)),
                           upper_halves(ubyte0(m_hi), ubyte1(m_hi)), upper_halves(ubyte2(m_hi), ubyte3(m_hi))));
    f32x4 mm = mfma16(zh, mb, zero4);
    mm = mfma16(zl, mb, mm);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c[i] = fmaf(-dmin, mm[i], c[i]);
      red[(u * nw + wave) * 256 + i * 64 + lane] = active ? c[i] : 0.f;
    }
    if (u == 0) tl.stamp(3);
  };
  // groups of kD tiles: tile u0 + p uses ring[p] and refills it with the tile
  // kD ahead; the last ntile % kD tiles are computed without refills
  int u0 = 0;
  for (; u0 + kD <= ntile; u0 += kD) {
#pragma unroll
    for (int p = 0; p < kD; ++p) {
      tile(u0 + p, ring[p]);
      issue(u0 + p + kD, ring[p]);
    }
  }
#pragma unroll
  for (int p = 0; p < kD - 1; ++p)
    if (u0 + p < ntile) tile(u0 + p, ring[p]);
  tl.stamp(4);
  __syncthreads();

  float* const Y = m == 0 ? R.Y[0] : m == 1 ? R.Y[1] : m == 2 ? R.Y[2] : R.Y[3];
  float* const partials = R.partials;
  int* const counters = R.counters;
  // element e = u 256 + i 64 + l: row r0 + 16 u + l % 16, token
  // n0 + 4 (l / 16) + i; the waves' sums added in wave order. Paired:
  // e = u 128 + i 32 + l, l < 32, the sum of lanes l and l + 32 per wave.
  constexpr int kTileElems = kPair ? 128 : 256;
  const int ne = ntile * kTileElems;
  auto coords = [&](int e, int& r, int& t) {
    const int l = e & (kPair ? 31 : 63), i = (e >> (kPair ? 5 : 6)) & 3, u = e / kTileElems;
    r = r0 + 16 * u + (l & 15);
    t = 4 * (l >> 4) + i;
  };
  // (the nw values are read together, then added in wave order)
  auto wave_sum = [&](int e) {
    const int u = e / kTileElems;
    const int k = kPair ? ((e >> 5) & 3) * 64 + (e & 31) : e & 255;
    float v[kSbwMaxWaves];
#pragma unroll
    for (int w = 0; w < kSbwMaxWaves; ++w) {
      const float* rw = red + (u * nw + w) * 256 + k;
      v[w] = w < nw ? (kPair ? rw[0] + rw[32] : rw[0]) : 0.f;
    }
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < kSbwMaxWaves; ++w) sum += v[w];
    return sum;
  };
  if (S == 1) {
    for (int e = tid; e < ne; e += nthreads) {
      int r, t;
      coords(e, r, t);
      if (r < rows && t < nb) Y[(int64_t)(n0 + t) * rows + r] = wave_sum(e);
    }
    tl.stamp(5);
    tl_put(W0, tl);
    return;
  }
  const int64_t btile = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
  const int64_t ntiles = (int64_t)gridDim.x * gridDim.y;
  const int64_t tile_floats = (int64_t)RT * 256;
  float* mine = partials + ((int64_t)split * ntiles + btile) * tile_floats;
  for (int e = tid; e < ne; e += nthreads) {
    int r, t;
    coords(e, r, t);
    if (t < nb) __hip_atomic_store(mine + e, wave_sum(e), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // every thread's partial stores have completed before thread 0 signals
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  GQK_WAIT_VMCNT(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (tid == 0) {
    const int old = __hip_atomic_fetch_add(&counters[btile * kSbCounterStride], 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
    last = old == S - 1;
  }
  __syncthreads();
  if (!last) {
    tl.stamp(5);
    tl_put(W0, tl);
    return;
  }
  // the partial values of an element are read eight ranges at a time, all
  // eight in flight (indexes past the last range re-read it and are not
  // added), and added in range order
  for (int e = tid; e < ne; e += nthreads) {
    int r, t;
    coords(e, r, t);
    if (r >= rows || t >= nb) continue;
    float sum = 0.f;
    for (int s0 = 0; s0 < S; s0 += 8) {
      const float* pp[8];
#pragma unroll
      for (int sp = 0; sp < 8; ++sp) {
        const int spc = s0 + sp < S ? s0 + sp : S - 1;
        pp[sp] = partials + ((int64_t)spc * ntiles + btile) * tile_floats + e;
      }
      float v[8];
      coherent_load8(pp, v);
#pragma unroll
      for (int sp = 0; sp < 8; ++sp)
        if (s0 + sp < S) sum += v[sp];
    }
    Y[(int64_t)(n0 + t) * rows + r] = sum;
  }
  if (tid == 0)
    __hip_atomic_store(&counters[btile * kSbCounterStride], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  tl.stamp(5);
  tl_put(W0, tl);
}

}  // namespace gqk
