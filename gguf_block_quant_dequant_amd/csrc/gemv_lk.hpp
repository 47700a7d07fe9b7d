// Batch-1 Q4_K GEMV with lanes along K, for rows of at most 16 super-blocks
// (K = 256, 512, 1024, 2048 or 4096): the decode stages whose rows are short.
//
// Work mapping: a row is cut into U = K / 64 "quarters" (a quarter is 64
// weights: sub-blocks 2g and 2g + 1 of a super-block, whose quants share the
// 32-byte nibble group g). Lane l takes quarter l mod U of row l / U, so a wave
// covers 64 / U whole rows per step ("row step") and walks a contiguous range
// of row steps. A lane's quarter is the same in every step, so its 64
// activations and their two sub-block sums are formed once, held in VGPRs,
// and reused for every row the wave visits; the block stages x in LDS once
// (padded so that the lanes' 256-byte slices start on different banks), so x
// crosses the L1 once per block instead of once per lane. Weight bytes go straight
// from HBM to registers: per step a lane loads the super-block header (16 B)
// and its 32 bytes of quants with three 16-byte loads, and the loads of the
// next kLkDepth - 1 steps are in flight while a step computes. Consecutive
// lanes read consecutive bytes of a row, and a wave's rows are consecutive, so
// a wave streams one contiguous byte range. Each row's U lane sums are added
// by a fixed butterfly (DPP within 16 lanes, then lane shuffles), so results
// do not depend on timing, and no partial sum leaves the wave: there is no
// split-K hand-off and no scratch.
//
// Every block of the launch belongs to one GEMV of the group (its four waves
// share the GEMV's x); the host gives each GEMV blocks in proportion to its
// rows, each block an equal share of that GEMV's row steps, and each wave a
// quarter of its block's.
#pragma once

#include "device_common.hpp"
#include "gemv_types.hpp"
#include "timeline.hpp"

namespace gqk {

constexpr int kLkWaves = 4;   // waves per block (the default; kernels take 4 or 8)
constexpr int kLkMaxGroup = 4;

// One GEMV of a launch (64 bytes, read as one 16-dword scalar load). Its row
// steps are cut among its blocks by the host: block lb (counted from
// block_begin) takes q + (lb < r) consecutive steps starting at
// lb q + min(lb, r).
struct LkDesc {
  const uint8_t* W;
  const float* x;
  float* y;
  int rows;
  int block_begin;   // first block of this GEMV in the launch
  int q;             // row steps per block
  int r;             // blocks that take one step more
  int nsb;           // super-blocks per row
  int pad;
  const float* scale_ss;   // the epilogue's input RMSN partial sums (kEpScale), else null
  int scale_n;
  int ep_flags;            // the epilogue's flags (0: none)
};
static_assert(sizeof(LkDesc) == 64, "one 16-dword load per descriptor");

struct LkGroup {
  LkDesc d[kLkMaxGroup];
  int n;
  int total_blocks;
  GemvEpilogue ep[kLkMaxGroup];   // read by the kernel variants with epilogues only
};

// Host side: how a group is launched (rows of 256 nsb weights; long rows are
// those of more than 16 super-blocks) and the launch of one block type,
// instantiated per type in lk_typed.hip.
struct LkPlan {
  int nsb;
  bool longrow;
  int depth;     // load ring depth: 2 or 4
  int bw;        // waves per block: 4 or 8
  size_t lds;    // dynamic LDS bytes of the long-row kernel
};
template <int kType, bool kEp>
void launch_lk_typed(const LkGroup& grp, const LkPlan& p, hipStream_t stream);
struct LksGroup;
template <int kType>
void launch_lks_typed(const LksGroup& grp, const GemvEpilogue* ep, int nsb, int R, int nw, int rps, int depth,
                      int blocks, hipStream_t stream);

// The block's share of a launch: its GEMV (pointers, rows, super-blocks per
// row) and the wave's row steps [st0, st0 + n).
struct LkBlock {
  const GQK_GLOBAL uint8_t* W;
  const GQK_GLOBAL float* x;
  GQK_GLOBAL float* y;
  int64_t rows;
  int64_t st0;
  int n;
  int nsb;
  int bs0;           // the block's row steps [bs0, bs0 + bn)
  int bn;
  int g;             // which GEMV of the launch
  const GQK_GLOBAL uint8_t* W2;   // kEpPairInWave: the up matrix and its output
  GQK_GLOBAL float* y2;
  const GQK_GLOBAL float* scale_ss;
  int scale_n;
  int ep_flags;
};

// The kernel arguments sit in memory that is cold at every launch: all four
// descriptors and the count are read in one batch of scalar loads (the empty
// asm consumes every word, so no load can be deferred behind a branch on
// another), and the block's own descriptor is picked with selects. The
// pointers come through the asm, which hides that they are global ones: they
// are cast back, or every access would become a flat access (counted against
// the LDS counter too, so each LDS wait would also wait for the weight loads).
template <int kW>
__device__ __forceinline__ LkBlock lk_block(const LkGroup& grp, int b, int wave) {
  typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));
  u32x16 dw[kLkMaxGroup];
#pragma unroll
  for (int k = 0; k < kLkMaxGroup; ++k) dw[k] = *reinterpret_cast<const u32x16*>(&grp.d[k]);
  int ng = grp.n;
  asm volatile("" : "+s"(dw[0]), "+s"(dw[1]), "+s"(dw[2]), "+s"(dw[3]), "+s"(ng));
  LkDesc dd[kLkMaxGroup];
#pragma unroll
  for (int k = 0; k < kLkMaxGroup; ++k) dd[k] = __builtin_bit_cast(LkDesc, dw[k]);
  const int g = (ng > 1 && b >= dd[1].block_begin) + (ng > 2 && b >= dd[2].block_begin) +
                (ng > 3 && b >= dd[3].block_begin);
  auto pick = [g](auto a0, auto a1, auto a2, auto a3) {
    return g == 0 ? a0 : g == 1 ? a1 : g == 2 ? a2 : a3;
  };
  LkBlock o;
  o.W = (const GQK_GLOBAL uint8_t*)pick(dd[0].W, dd[1].W, dd[2].W, dd[3].W);
  o.x = (const GQK_GLOBAL float*)pick(dd[0].x, dd[1].x, dd[2].x, dd[3].x);
  o.y = (GQK_GLOBAL float*)pick(dd[0].y, dd[1].y, dd[2].y, dd[3].y);
  o.rows = pick(dd[0].rows, dd[1].rows, dd[2].rows, dd[3].rows);
  o.nsb = pick(dd[0].nsb, dd[1].nsb, dd[2].nsb, dd[3].nsb);
  o.g = g;
  o.scale_ss = (const GQK_GLOBAL float*)pick(dd[0].scale_ss, dd[1].scale_ss, dd[2].scale_ss, dd[3].scale_ss);
  o.scale_n = pick(dd[0].scale_n, dd[1].scale_n, dd[2].scale_n, dd[3].scale_n);
  o.ep_flags = pick(dd[0].ep_flags, dd[1].ep_flags, dd[2].ep_flags, dd[3].ep_flags);
  // the up half of an in-wave gate/up pair is the next descriptor
  o.W2 = (const GQK_GLOBAL uint8_t*)(g == 0 ? dd[1].W : g == 1 ? dd[2].W : dd[3].W);
  o.y2 = (GQK_GLOBAL float*)(g == 0 ? dd[1].y : g == 1 ? dd[2].y : dd[3].y);
  const int lb = b - pick(dd[0].block_begin, dd[1].block_begin, dd[2].block_begin, dd[3].block_begin);
  const int q = pick(dd[0].q, dd[1].q, dd[2].q, dd[3].q);
  const int r = pick(dd[0].r, dd[1].r, dd[2].r, dd[3].r);
  const int bn = q + (lb < r ? 1 : 0);
  const int bs0 = lb * q + (lb < r ? lb : r);
  o.st0 = bs0 + (wave * bn) / kW;
  o.n = ((wave + 1) * bn) / kW - (wave * bn) / kW;
  o.bs0 = bs0;
  o.bn = bn;
  return o;
}

// d * sc and dmin * m of the two sub-blocks 2 gq and 2 gq + 1 of a Q4_K
// super-block header (h0 = d | dmin << 16, h1..h3 = scale bytes S[0..11]);
// d * sc comes out multiplied by 512 to undo the q / 512 of the nibble
// conversion (exact: a power of two).
//   j < 4 : sc = S[j] & 63,  m = S[j+4] & 63
//   j >= 4: sc = (S[j+4] & 15) | ((S[j-4] >> 6) << 4)
//           m  = (S[j+4] >> 4) | ((S[j]   >> 6) << 4)
// Both sub-blocks of the pair have the same j / 4 and their bytes sit in the
// same half of each scale word (t0 = 2 (gq & 1)): sh = 16 (gq & 1), and
// hi_mask is all ones for gq >= 2 (j >= 4), else zero; both are per lane and
// the two forms are blended without a branch.
__device__ __forceinline__ void q4k_pair_scales(uint32_t h0, uint32_t h1, uint32_t h2, uint32_t h3,
                                                uint32_t sh, uint32_t hi_mask, float& dsc0,
                                                float& dsc1, float& dmm0, float& dmm1) {
  const float d512 = half_lo(h0) * 512.0f;
  const float dmin = half_hi(h0);
  const uint32_t a = (h1 >> sh) & 0xFFFFu;   // S[t0], S[t0 + 1]
  const uint32_t b = (h2 >> sh) & 0xFFFFu;   // S[t0 + 4], S[t0 + 5]
  const uint32_t c = (h3 >> sh) & 0xFFFFu;   // S[t0 + 8], S[t0 + 9]
  const uint32_t sc_hi = (c & 0x0F0Fu) | ((a >> 2) & 0x3030u);
  const uint32_t m_hi = ((c >> 4) & 0x0F0Fu) | ((b >> 2) & 0x3030u);
  const uint32_t sc = (sc_hi & hi_mask) | (a & 0x3F3Fu & ~hi_mask);
  const uint32_t m = (m_hi & hi_mask) | (b & 0x3F3Fu & ~hi_mask);
  dsc0 = d512 * ubyte0(sc);
  dsc1 = d512 * ubyte1(sc);
  dmm0 = dmin * ubyte0(m);
  dmm1 = dmin * ubyte1(m);
}

// A DPP move of a float (bound_ctrl set: lanes without a source read 0).
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float s) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s), kCtrl, 0xF, 0xF, true));
}

// Sum over each aligned segment of kU lanes (kU = 4 .. 64) in a fixed order.
// Lane kU - 1 of each segment ends with the segment's sum (for kU <= 16 every
// lane of the segment does). For kU >= 32 the 16-lane row sums are joined
// with row broadcasts: row_bcast:15 adds row 2k's sum into row 2k + 1, and
// row_bcast:31 adds lane 31 (rows 0 + 1) into rows 2 and 3.
template <int kU>
__device__ __forceinline__ float lk_segment_sum(float v) {
  v += dpp_f32<0xB1>(v);                 // quad_perm 1,0,3,2
  v += dpp_f32<0x4E>(v);                 // quad_perm 2,3,0,1
  if constexpr (kU == 8) v += dpp_f32<0x141>(v);   // row_half_mirror
  if constexpr (kU >= 16) {
    v += dpp_f32<0x124>(v);              // row_ror:4
    v += dpp_f32<0x128>(v);              // row_ror:8
  }
  if constexpr (kU >= 32)
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142, 0xA, 0xF, false));
  if constexpr (kU >= 64)
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x143, 0xC, 0xF, false));
  return v;
}

typedef uint32_t lk_u32x4 __attribute__((ext_vector_type(4)));
typedef float lk_f32x4 __attribute__((ext_vector_type(4)));

struct LkLoad {
  lk_u32x4 h, qa, qb;
};

// A Q8_0 quarter: two 34-byte blocks, 17 dwords.
struct LkLoad8 {
  lk_u32x4 a, b, c, d;
  uint32_t e;
};

// A Q6_K unit of 64 weights: within half n (0, 1) of a super-block, bytes
// 16h .. 16h + 15 (h = 0, 1) of its 64 low-bit bytes, the same 16 bytes 32
// further on, 16 bytes of its 32 high-bit bytes, its 8 scale bytes and d. The
// 210-byte super-blocks leave every field 2 bytes off a word boundary in
// every other super-block (mis = 2): each 16-byte field is read as the five
// aligned words around it and re-aligned, the scales as three words (the
// third re-reads the second when mis = 0, so no read leaves the super-block),
// d as a 2-byte load.
struct LkLoad6 {
  uint32_t a[5], b[5], h[5], s[3];
  uint32_t d;
  uint32_t mis;
};

template <int kType>
struct LkLoadOf {
  using type = LkLoad;
};
template <>
struct LkLoadOf<8> {
  using type = LkLoad8;
};
template <>
struct LkLoadOf<14> {
  using type = LkLoad6;
};

// Unit u of the Q6_K row at rowp: super-block u / 4, half (u / 2) % 2,
// h = u % 2. Lane slice order of its 64 weights: position 16 m + t is weight
// 128 n + 32 m + 16 h + t of the super-block (m = 0..3, t = 0..15).
__device__ __forceinline__ void q6k_unit_issue(const GQK_GLOBAL uint8_t* rowp, uint32_t u, LkLoad6& L) {
  const uint32_t sb = (u >> 2) * (uint32_t)kQ6KBlockBytes;
  const uint32_t n = (u >> 1) & 1u, h = u & 1u;
  const uint32_t mis = ((uint32_t)(uintptr_t)rowp + sb) & 2u;
  // (rowp + sb) - mis as pointer arithmetic: for the first super-block of a
  // row that starts 2 bytes off a word boundary the window starts 2 bytes
  // before the row (inside the previous row; row 0 is aligned), and sb - mis
  // in 32-bit unsigned arithmetic would wrap
  const GQK_GLOBAL uint32_t* w = reinterpret_cast<const GQK_GLOBAL uint32_t*>((rowp + sb) - mis);
  const uint32_t ia = 16u * n + 4u * h, ib = ia + 8u, ih = 32u + 8u * n + 4u * h, is = 48u + 2u * n;
#pragma unroll
  for (int k = 0; k < 5; ++k) {
    L.a[k] = w[ia + k];
    L.b[k] = w[ib + k];
    L.h[k] = w[ih + k];
  }
  L.s[0] = w[is];
  L.s[1] = w[is + 1];
  L.s[2] = w[is + 1 + (mis >> 1)];
  L.d = *reinterpret_cast<const GQK_GLOBAL uint16_t*>(rowp + sb + 208u);
  L.mis = mis;
}

// The unit's 64-weight dot product with its slice xv (xv[16 m + t], see
// above) and the slice's sums over each m (xs[m]):
//   d sum_m sc_m (sum_t code x - 32 sum_t x),   code = low 4 | high 2 << 4.
// Byte l of the low-bit fields holds weights l (low nibble of the first
// field), 32 + l (low nibble of the second), 64 + l and 96 + l (the high
// nibbles); bits 0-1, 2-3, 4-5, 6-7 of high-bit byte l are their top bits.
template <class XAt>
__device__ __forceinline__ float q6k_unit_dot(const LkLoad6& L, uint32_t h, XAt xat, const float (&xs)[4]) {
  const uint32_t mis = L.mis;
  uint32_t qa[4], qb[4], hh[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    qa[k] = __builtin_amdgcn_alignbyte(L.a[k + 1], L.a[k], mis);
    qb[k] = __builtin_amdgcn_alignbyte(L.b[k + 1], L.b[k], mis);
    hh[k] = __builtin_amdgcn_alignbyte(L.h[k + 1], L.h[k], mis);
  }
  // one run of 16 weights (one scale) at a time
  float S[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t c = m == 0   ? (qa[k] & 0x0F0F0F0Fu) | ((hh[k] & 0x03030303u) << 4)
                         : m == 1 ? (qb[k] & 0x0F0F0F0Fu) | ((hh[k] & 0x0C0C0C0Cu) << 2)
                         : m == 2 ? ((qa[k] >> 4) & 0x0F0F0F0Fu) | (hh[k] & 0x30303030u)
                                  : ((qb[k] >> 4) & 0x0F0F0F0Fu) | ((hh[k] >> 2) & 0x30303030u);
      acc = fmaf((float)(c & 0xFFu), xat(16 * m + 4 * k + 0), acc);
      acc = fmaf((float)((c >> 8) & 0xFFu), xat(16 * m + 4 * k + 1), acc);
      acc = fmaf((float)((c >> 16) & 0xFFu), xat(16 * m + 4 * k + 2), acc);
      acc = fmaf((float)(c >> 24), xat(16 * m + 4 * k + 3), acc);
    }
    S[m] = acc;
  }
  // scale of weights 128 n + 32 m + 16 h + t: byte 2 m + h of the 8 scale
  // bytes of half n
  const uint32_t s0 = __builtin_amdgcn_alignbyte(L.s[1], L.s[0], mis);
  const uint32_t s1 = __builtin_amdgcn_alignbyte(L.s[2], L.s[1], mis);
  const uint32_t sh = 8u * h;
  float r = 0.f;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const uint32_t word = m < 2 ? s0 : s1;
    const float sc = (float)(int)(int8_t)((word >> (16u * (m & 1) + sh)) & 0xFFu);
    r = fmaf(sc, fmaf(-32.0f, xs[m], S[m]), r);
  }
  return half_lo(L.d) * r;
}

// A lane's quarter (64 weights: sub-blocks 2 gq and 2 gq + 1 of one Q4_K
// super-block) against its 64 activations xv and their two sub-block sums:
// sum_j (d sc_j) sum_i q_i x_i - (dmin m_j) sum_i x_i over the two
// sub-blocks. L: the super-block header and the 32 quant bytes of the
// quarter; sh and hi_mask as q4k_pair_scales takes them for gq.
__device__ __forceinline__ float q4k_quarter_dot(const LkLoad& L, uint32_t sh, uint32_t hi_mask,
                                                 const float (&xv)[64], float xs0, float xs1) {
  float dsc0, dsc1, dmm0, dmm1;
  q4k_pair_scales(L.h.x, L.h.y, L.h.z, L.h.w, sh, hi_mask, dsc0, dsc1, dmm0, dmm1);
  const uint32_t qw[8] = {L.qa.x, L.qa.y, L.qa.z, L.qa.w, L.qb.x, L.qb.y, L.qb.z, L.qb.w};
  float la0 = 0.f, la1 = 0.f, ha0 = 0.f, ha1 = 0.f;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    // byte 4t + e: low nibble = weight 4t + e of sub-block 2 gq,
    // high nibble = weight 4t + e of sub-block 2 gq + 1
    float ql[4], qh[4];
    nibbles_div512(opaque(qw[t] & 0x0F0F0F0Fu), ql);
    nibbles_div512(opaque((qw[t] >> 4) & 0x0F0F0F0Fu), qh);
    float& la = (t & 1) ? la1 : la0;
    float& ha = (t & 1) ? ha1 : ha0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      la = fmaf(ql[e], xv[4 * t + e], la);
      ha = fmaf(qh[e], xv[32 + 4 * t + e], ha);
    }
  }
  float r = dsc0 * (la0 + la1);
  r = fmaf(dsc1, ha0 + ha1, r);
  r = fmaf(-dmm0, xs0, r);
  r = fmaf(-dmm1, xs1, r);
  return r;
}

// A lane's Q4_0 quarter (two 18-byte blocks read as nine aligned words: d0 |
// codes 0..1, codes 2..5, 6..9, 10..13, codes 14..15 | d1, then block 1's 16
// code bytes) against its 64 activations: w = (code - 8) d, so each block adds
// 512 d sum(code / 512 x) - 8 d sum(x); byte j of a block holds the code of
// weight j (low nibble) and of weight j + 16 (high nibble).
__device__ __forceinline__ float q40_quarter_dot(const LkLoad& L, const float (&xv)[64], float xs0,
                                                 float xs1) {
  const uint32_t w[9] = {L.h.x, L.h.y, L.h.z, L.h.w, L.qa.x, L.qa.y, L.qa.z, L.qa.w, L.qb.x};
  const float d0 = half_lo(w[0]), d1 = half_hi(w[4]);
  uint32_t c[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    c[k] = __builtin_amdgcn_alignbyte(w[k + 1], w[k], 2);   // block 0, codes 4k .. 4k + 3
    c[4 + k] = w[5 + k];                                     // block 1
  }
  float s0a = 0.f, s0b = 0.f, s1a = 0.f, s1b = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float l0[4], h0[4], l1[4], h1[4];
    nibbles_div512(opaque(c[k] & 0x0F0F0F0Fu), l0);
    nibbles_div512(opaque((c[k] >> 4) & 0x0F0F0F0Fu), h0);
    nibbles_div512(opaque(c[4 + k] & 0x0F0F0F0Fu), l1);
    nibbles_div512(opaque((c[4 + k] >> 4) & 0x0F0F0F0Fu), h1);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s0a = fmaf(l0[e], xv[4 * k + e], s0a);
      s0b = fmaf(h0[e], xv[16 + 4 * k + e], s0b);
      s1a = fmaf(l1[e], xv[32 + 4 * k + e], s1a);
      s1b = fmaf(h1[e], xv[48 + 4 * k + e], s1b);
    }
  }
  float r = (d0 * 512.0f) * (s0a + s0b);
  r = fmaf(d1 * 512.0f, s1a + s1b, r);
  r = fmaf(-8.0f * d0, xs0, r);
  r = fmaf(-8.0f * d1, xs1, r);
  return r;
}

// ---------------------------------------------------------------------------
// The neighbouring steps of a decode layer fused into these GEMVs (the same
// epilogues as the lane-per-row kernels, see GemvEpilogue): per row, in the
// lane that holds the row's sum, the input RMSN scale, the residual add and
// norm_out = y * norm_w; per 64-row group, once every row of the group is
// stored (a count per group, agent-scope stores and loads), the next RMSN's
// partial sum ss_out (the same fixed butterfly of squares as the standalone
// preparation kernel) or, for a gate/up pair, act = SiLU(gate) * up.
// ---------------------------------------------------------------------------
struct LkEp {
  GemvEpilogue e;
  float scale;       // input RMSN factor (1 without kEpScale)
  int gflags;        // group work: kEpSs or kEpPair (not both), else 0
};

// The lane's share of the input RMSN's partial sums (kEpScale; at most 256
// of them): scale_ss[lane + 64 k], k = 0..3, added in k order. The four loads
// go out unconditionally before the block's other loads (indices past the
// end re-read the last sum; without kEpScale they read the block's x), and
// they are added only where the scale is formed: loads under a condition went
// out one at a time, each waited for before the next, ahead of every
// activation and weight load of the launch.
struct LkSsLoads {
  float v[4];
};

__device__ __forceinline__ LkSsLoads lk_ep_ss_issue(int flags, int scale_n, const GQK_GLOBAL float* scale_ss,
                                                    const GQK_GLOBAL float* x, int lane) {
  const bool on = (flags & kEpScale) && scale_n > 0;
  const GQK_GLOBAL float* const p = on ? scale_ss : x;
  const int last = on ? scale_n - 1 : 0;
  LkSsLoads r;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = lane + 64 * k;
    r.v[k] = p[i < last ? i : last];
  }
  return r;
}

__device__ __forceinline__ float lk_ep_ss_sum(const LkBlock& B, int lane, const LkSsLoads& r) {
  float t = 0.f;
  if (B.ep_flags & kEpScale) {
#pragma unroll
    for (int k = 0; k < 4; ++k) t += lane + 64 * k < B.scale_n ? r.v[k] : 0.f;
  }
  return t;
}

// The block's epilogue; the scale is 1 / sqrt(S / K + eps) with S the lanes'
// shares added by a fixed butterfly, or (kEpScaleV) the block's sum of v^2,
// formed by the caller.
__device__ __forceinline__ LkEp lk_ep(const GemvEpilogue& e, float ss_share, float v_total = 0.f) {
  LkEp o;
  o.e = e;
  o.scale = 1.f;
  o.gflags = (o.e.flags & kEpPairInWave) ? 0 : o.e.flags & (kEpSs | kEpPair);
  if (o.e.flags & kEpScale) {
    const float S = (o.e.flags & kEpScaleV) ? v_total : wave_sum_fixed(ss_share);
    o.scale = 1.0f / sqrtf(S * o.e.inv_k + o.e.eps);
  }
  return o;
}

// Row `row`'s final sum v, in the lane that holds it.
__device__ __forceinline__ void lk_ep_row(const LkEp& E, float v, int64_t row, GQK_GLOBAL float* y) {
  if (E.e.flags & kEpScale) v *= E.scale;
  if (E.e.flags & kEpResidual) v += E.e.residual[row];
  if (E.gflags)
    __hip_atomic_store((float*)&y[row], v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    y[row] = v;
  if (E.e.flags & kEpNorm) E.e.norm_out[row] = v * E.e.norm_w[row];
}

// After the block's rows [rb0, rb1) are stored: count them per 64-row group;
// the block that completes a group does its group work. Called by the whole
// block (wave-uniform; a barrier inside).
__device__ __forceinline__ void lk_ep_groups(const LkEp& E, int64_t rb0, int64_t rb1, int64_t rows,
                                             const GQK_GLOBAL float* y, int wave, int lane) {
  if (!E.gflags) return;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  GQK_WAIT_VMCNT(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (wave != 0 || rb1 <= rb0) return;
  const bool pair = (E.gflags & kEpPair) != 0;
  int* cnt = pair ? E.e.pair_cnt : E.e.norm_cnt;
  for (int64_t rg = rb0 / 64; rg * 64 < rb1; ++rg) {
    const int64_t g0 = rg * 64;
    const int grows = (int)(rows - g0 < 64 ? rows - g0 : 64);
    const int count = (int)((rb1 < g0 + 64 ? rb1 : g0 + 64) - (rb0 > g0 ? rb0 : g0));
    int old = 0;
    if (lane == 0)
      old = __hip_atomic_fetch_add(&cnt[rg * kCounterStride], count, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
    old = __builtin_amdgcn_readfirstlane(old);
    if (old + count != (pair ? 2 * grows : grows)) continue;
    const bool live = lane < grows;
    const int64_t r = g0 + (live ? lane : 0);
    const float v = __hip_atomic_load((const float*)&y[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (pair) {
      if (live) {
        const float o = __hip_atomic_load(&E.e.partner_y[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const float gv = E.e.role == 0 ? v : o, uv = E.e.role == 0 ? o : v;
        E.e.act[r] = gv / (1.0f + expf(-gv)) * uv;
      }
    } else {
      // the square rounded on its own, then the fixed butterfly: the same bits
      // as the standalone preparation kernel
      float sq = live ? v * v : 0.f;
      asm volatile("" : "+v"(sq));
      const float ss = wave_sum_fixed(sq);
      if (lane == 0) E.e.ss_out[rg] = ss;
    }
    if (lane == 0)
      __hip_atomic_store(&cnt[rg * kCounterStride], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// One GEMV alone, its descriptor in scalar kernel arguments (which the
// dispatcher can place in SGPRs before the waves start).
template <int kW>
__device__ __forceinline__ LkBlock lk_block_single(const uint8_t* W, const float* x, float* y,
                                                   int rows, int q, int r, int nsb, int b,
                                                   int wave) {
  LkBlock o;
  o.W = (const GQK_GLOBAL uint8_t*)W;
  o.x = (const GQK_GLOBAL float*)x;
  o.y = (GQK_GLOBAL float*)y;
  o.rows = rows;
  o.nsb = nsb;
  o.g = 0;
  o.W2 = nullptr;
  o.y2 = nullptr;
  o.scale_ss = nullptr;
  o.scale_n = 0;
  o.ep_flags = 0;
  const int bn = q + (b < r ? 1 : 0);
  const int bs0 = b * q + (b < r ? b : r);
  o.st0 = bs0 + (wave * bn) / kW;
  o.n = ((wave + 1) * bn) / kW - (wave * bn) / kW;
  o.bs0 = bs0;
  o.bn = bn;
  return o;
}

// Two GEMVs of one x, their descriptors in 14 dwords of scalar kernel
// arguments (all preloaded into SGPRs: 14 is the most the dispatcher places;
// the grid size, a hidden argument, would be a memory load): blocks [0, bb1)
// take GEMV 0, blocks [bb1, bb1 + nb1) GEMV 1, and each GEMV's steps of kRps
// rows are split over its blocks as the host splits them (the first r blocks
// q + 1 steps, the others q), q and r formed here by one uniform division.
template <int kW, int kRps>
__device__ __forceinline__ LkBlock lk_block_two(const uint8_t* W0, const uint8_t* W1, const float* x,
                                                float* y0, float* y1, int rows0, int rows1, int bb1,
                                                int nb1, int nsb, int b, int wave) {
  const bool second = b >= bb1;
  const uint32_t rows = (uint32_t)(second ? rows1 : rows0);
  const uint32_t nb = (uint32_t)(second ? nb1 : bb1);
  const uint32_t steps = (rows + kRps - 1) / kRps;
  const uint32_t q = steps / nb, r = steps - q * nb;
  return lk_block_single<kW>(second ? W1 : W0, x, second ? y1 : y0, (int)rows, (int)q, (int)r, nsb,
                             second ? b - bb1 : b, wave);
}

// Three GEMVs of one x (the q, k and v of a layer) in the same 14 dwords:
// W1 and W2 as signed 32-bit offsets from W0 and y1 and y2 from y0, in
// 16-byte units (all of them 16-byte aligned; the allocator's pools for small
// and large tensors can lie gigabytes apart), rows1 | rows2 << 16 and bb1 | bb2 << 16
// packed (the host takes this form only where all of them fit). Blocks
// [0, bb1) take GEMV 0, [bb1, bb2) GEMV 1, [bb2, nb) GEMV 2, each with at
// least one block.
template <int kW, int kRps>
__device__ __forceinline__ LkBlock lk_block_three(const uint8_t* W0, int dW1, int dW2, const float* x,
                                                  float* y0, int dy1, int dy2, int rows0, int rows12,
                                                  int bb12, int nb, int nsb, int b, int wave) {
  const uint32_t bb1 = (uint32_t)bb12 & 0xFFFFu, bb2 = (uint32_t)bb12 >> 16;
  const uint32_t ub = (uint32_t)b;
  const int m = ub >= bb2 ? 2 : ub >= bb1 ? 1 : 0;
  const uint32_t rows = m == 0 ? (uint32_t)rows0 : m == 1 ? ((uint32_t)rows12 & 0xFFFFu) : ((uint32_t)rows12 >> 16);
  const uint32_t b0 = m == 0 ? 0u : m == 1 ? bb1 : bb2;
  const uint32_t nbm = (m == 0 ? bb1 : m == 1 ? bb2 : (uint32_t)nb) - b0;
  const uint32_t steps = (rows + kRps - 1) / kRps;
  const uint32_t q = steps / nbm, r = steps - q * nbm;
  const int64_t dw = 16 * (m == 0 ? 0 : m == 1 ? (int64_t)dW1 : (int64_t)dW2);
  const int64_t dy = 4 * (m == 0 ? 0 : m == 1 ? (int64_t)dy1 : (int64_t)dy2);
  LkBlock o = lk_block_single<kW>(W0 + dw, x, y0 + dy, (int)rows, (int)q, (int)r, nsb, (int)(ub - b0), wave);
  o.g = m;
  return o;
}

// LDS float index of x's float4 i in the staged layout: lane slice u (64
// floats) at 68 u, four floats of padding after each. Slice u holds weights
// 64 u .. 64 u + 63 in order, except for Q6_K, whose unit u holds weights
// 128 n + 32 m + 16 h + t of super-block u / 4 (n = (u / 2) % 2, h = u % 2)
// at position 16 m + t.
template <int kType>
__device__ __forceinline__ int lk_x_slot(int i) {
  if constexpr (kType == 14) {
    const int e = 4 * i, r = e & 255;
    const int u = 4 * (e >> 8) + 2 * (r >> 7) + ((r >> 4) & 1);
    return 68 * u + 16 * ((r >> 5) & 3) + (r & 15);
  } else {
    return 4 * i + (i >> 4) * 4;
  }
}

// kPair: whether the block computes an in-wave gate/up pair (kEpPairInWave):
// 0 from the block's flags, 1 never, 2 always (known when the kernel is
// chosen, so that the weight addresses wait for no epilogue argument).
template <int kNsb, int kDepth, int kW, bool kEp, int kType = 12, int kPair = 0>
__device__ __forceinline__ void lk_run(const LkBlock& B, float* xl, const GemvEpilogue* eps, TlStamps& tl,
                                       const void* tl_key);

// kType is the row format, a GGUF type id: 12 (Q4_K), 2 (Q4_0: the same
// 0.5625 bytes per weight, a lane's quarter two 18-byte blocks read as nine
// aligned words, 36 u being a multiple of 4, the first block's codes
// re-aligned with v_alignbyte) or 8 (Q8_0: a quarter two 34-byte blocks, 17
// aligned words at 68 u). Epilogues on Q4_K only.
template <int kType, int kNsb, int kDepth, int kW, bool kEp>
__global__ __launch_bounds__(kW * 64) void gemv_lk_kernel(LkGroup grp) {
  // x in LDS with 4 floats of padding after every 64: the slice of lane u
  // starts at float 68 u, i.e. on bank 4 u mod 32 (16-byte reads conflict-free)
  __shared__ __attribute__((aligned(16))) float xl[256 * kNsb + 16 * kNsb];
  TlStamps tl;
  tl.stamp(0);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  lk_run<kNsb, kDepth, kW, kEp, kType>(lk_block<kW>(grp, (int)blockIdx.x, wave), xl, grp.ep, tl, grp.d[0].W);
}

// One GEMV, its descriptor as (preloaded) scalar arguments.
template <int kType, int kNsb, int kDepth, int kW>
__global__ __launch_bounds__(kW * 64) void gemv_lk1_kernel(const uint8_t* W, const float* x, float* y,
                                                           int rows, int q, int r) {
  __shared__ __attribute__((aligned(16))) float xl[256 * kNsb + 16 * kNsb];
  TlStamps tl;
  tl.stamp(0);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  lk_run<kNsb, kDepth, kW, false, kType>(lk_block_single<kW>(W, x, y, rows, q, r, kNsb, (int)blockIdx.x, wave),
                                         xl, nullptr, tl, W);
}

// One Q4_K GEMV with an epilogue: the descriptor and what the first loads
// need of the epilogue (its flags, the input RMSN's partial sums) as
// preloaded scalar arguments (13 dwords), the rest of the epilogue in memory,
// read after the last step.
template <int kNsb, int kDepth, int kW>
__global__ __launch_bounds__(kW * 64) void gemv_lk1e_kernel(const uint8_t* W, const float* x, float* y,
                                                            int rows, int q, int r, int ep_flags, int scale_n,
                                                            const float* scale_ss, GemvEpilogue ep) {
  __shared__ __attribute__((aligned(16))) float xl[256 * kNsb + 16 * kNsb];
  TlStamps tl;
  tl.stamp(0);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  LkBlock B = lk_block_single<kW>(W, x, y, rows, q, r, kNsb, (int)blockIdx.x, wave);
  B.ep_flags = ep_flags;
  B.scale_n = scale_n;
  B.scale_ss = (const GQK_GLOBAL float*)scale_ss;
  lk_run<kNsb, kDepth, kW, true, 12>(B, xl, &ep, tl, W);
}

// A gate/up pair with epilogue (input RMSN scale, SiLU(gate) up) computed in
// one wave: gate rows in lanes 0..31, the same rows of up in lanes 32..63.
// The descriptors as preloaded scalar arguments (13 dwords; the blocks split
// the gate's row steps), the epilogue in memory: it is first needed by the
// input RMSN's partial-sum loads, which go out after the first weight loads.
template <int kNsb, int kDepth, int kW>
__global__ __launch_bounds__(kW * 64) void gemv_lk2e_kernel(const uint8_t* W0, const uint8_t* W1, const float* x,
                                                            float* y0, float* y1, int rows, int q, int r,
                                                            GemvEpilogue ep) {
  __shared__ __attribute__((aligned(16))) float xl[256 * kNsb + 16 * kNsb];
  TlStamps tl;
  tl.stamp(0);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  LkBlock B = lk_block_single<kW>(W0, x, y0, rows, q, r, kNsb, (int)blockIdx.x, wave);
  B.W2 = (const GQK_GLOBAL uint8_t*)W1;
  B.y2 = (GQK_GLOBAL float*)y1;
  B.ep_flags = ep.flags;
  B.scale_n = ep.scale_n;
  B.scale_ss = (const GQK_GLOBAL float*)ep.scale_ss;
  lk_run<kNsb, kDepth, kW, true, 12, 2>(B, xl, &ep, tl, W0);
}

// Three GEMVs of one x (stages without epilogues), the descriptors packed into
// preloaded scalar arguments.
template <int kType, int kNsb, int kDepth, int kW>
__global__ __launch_bounds__(kW * 64) void gemv_lk3_kernel(const uint8_t* W0, int dW1, int dW2,
                                                           const float* x, float* y0, int dy1, int dy2,
                                                           int rows0, int rows12, int bb12, int nb) {
  __shared__ __attribute__((aligned(16))) float xl[256 * kNsb + 16 * kNsb];
  TlStamps tl;
  tl.stamp(0);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  lk_run<kNsb, kDepth, kW, false, kType>(lk_block_three<kW, 16 / kNsb>(W0, dW1, dW2, x, y0, dy1, dy2, rows0,
                                                                       rows12, bb12, nb, kNsb,
                                                                       (int)blockIdx.x, wave),
                                         xl, nullptr, tl, W0);
}

// Three GEMVs of one x with epilogues (the fused q/k/v: the input RMSN scale),
// the descriptors packed into the preloaded arguments as above, the three
// epilogues in memory (first needed by the input RMSN's partial-sum loads,
// which go out after the first weight loads).
struct LkEp3 {
  GemvEpilogue e[3];
};

template <int kNsb, int kDepth, int kW>
__global__ __launch_bounds__(kW * 64) void gemv_lk3e_kernel(const uint8_t* W0, int dW1, int dW2, const float* x,
                                                            float* y0, int dy1, int dy2, int rows0, int rows12,
                                                            int bb12, int nb, LkEp3 ep) {
  __shared__ __attribute__((aligned(16))) float xl[256 * kNsb + 16 * kNsb];
  TlStamps tl;
  tl.stamp(0);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  LkBlock B = lk_block_three<kW, 16 / kNsb>(W0, dW1, dW2, x, y0, dy1, dy2, rows0, rows12, bb12, nb, kNsb,
                                            (int)blockIdx.x, wave);
  const GemvEpilogue& e = ep.e[B.g];
  B.ep_flags = e.flags;
  B.scale_n = e.scale_n;
  B.scale_ss = (const GQK_GLOBAL float*)e.scale_ss;
  lk_run<kNsb, kDepth, kW, true, 12, 1>(B, xl, ep.e, tl, W0);
}

// Two GEMVs of one x (stages without epilogues), the descriptors as preloaded
// scalar arguments.
template <int kType, int kNsb, int kDepth, int kW>
__global__ __launch_bounds__(kW * 64) void gemv_lk2_kernel(const uint8_t* W0, const uint8_t* W1,
                                                           const float* x, float* y0, float* y1,
                                                           int rows0, int rows1, int bb1, int nb1) {
  __shared__ __attribute__((aligned(16))) float xl[256 * kNsb + 16 * kNsb];
  TlStamps tl;
  tl.stamp(0);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  lk_run<kNsb, kDepth, kW, false, kType>(
      lk_block_two<kW, 16 / kNsb>(W0, W1, x, y0, y1, rows0, rows1, bb1, nb1, kNsb, (int)blockIdx.x, wave),
      xl, nullptr, tl, W0);
}

template <int kNsb, int kDepth, int kW, bool kEp, int kType, int kPair>
__device__ __forceinline__ void lk_run(const LkBlock& B, float* xl, const GemvEpilogue* eps, TlStamps& tl,
                                       const void* tl_key) {
  static_assert(kType == 12 || kType == 2 || kType == 8 || kType == 14, "Q4_K, Q4_0, Q8_0 or Q6_K rows");
  static_assert(kType == 12 || !kEp, "epilogues on Q4_K only");
  constexpr bool kQ40 = kType == 2, kQ80 = kType == 8, kQ6 = kType == 14;
  using Load = typename LkLoadOf<kType>::type;
  constexpr int kU = 4 * kNsb;                 // lanes per row
  constexpr int kRps = 64 / kU;                // rows per step
  constexpr int kK = 256 * kNsb;
  // bytes per 256 weights: 144 (Q4_K, Q4_0), 272 (Q8_0) or 210 (Q6_K)
  constexpr uint32_t kRowBytes =
      (uint32_t)kNsb * (kQ80 ? 8u * kQ80BlockBytes : kQ6 ? (uint32_t)kQ6KBlockBytes : (uint32_t)kQ4KBlockBytes);
  constexpr int kXF4 = kK / 4;                 // float4 of x
  static_assert(kU >= 4 && kU <= 64 && 64 % kU == 0, "rows of 1 to 16 super-blocks");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const GQK_GLOBAL uint8_t* const W = B.W;
  const GQK_GLOBAL float* const x = B.x;
  GQK_GLOBAL float* const y = B.y;
  const int64_t rows = B.rows;
  const int64_t st0 = B.st0;
  const int n = B.n;

  const int u = lane % kU;
  const int s = u >> 2, gq = u & 3;
  const uint32_t hoff = (uint32_t)s * kQ4KBlockBytes;
  const uint32_t qoff = 16u + 32u * (uint32_t)gq;
  const uint32_t sh = 16u * (uint32_t)(gq & 1);
  const uint32_t hi_mask = gq >= 2 ? 0xFFFFFFFFu : 0u;
  // rows per step of each matrix: kRps, or kRps / 2 of the gate (lanes 0..31)
  // and the same rows of the up matrix (lanes 32..63) for an in-wave pair
  const bool paired = kEp && kRps >= 2 && (kPair == 2 || (kPair == 0 && (B.ep_flags & kEpPairInWave)));
  const int rpm = paired ? kRps / 2 : kRps;
  const int rsub = (lane / kU) % rpm;
  const GQK_GLOBAL uint8_t* const Wl = (paired && lane >= 32) ? B.W2 : W;
  LkSsLoads ssl;
  GemvEpilogue epl;
  if constexpr (kEp) {
    epl = eps[B.g];
  }

  // x: every thread loads its float4s first ...
  constexpr int kXIt = (kXF4 + kW * 64 - 1) / (kW * 64);
  lk_f32x4 xg[kXIt];
#pragma unroll
  for (int j = 0; j < kXIt; ++j) {
    const int i = tid + j * kW * 64;
    if (kXF4 % (kW * 64) == 0 || i < kXF4) xg[j] = reinterpret_cast<const GQK_GLOBAL lk_f32x4*>(x)[i];
  }
  // (kEpScaleV) and the float4s of v at the same indices, for the block's sum
  // of v^2, right behind x: the loads complete in order, so issued after the
  // first weight loads they held the x-staging barrier back until those
  // arrived. They read x when the flag is off, so they go out on every path.
  lk_f32x4 vg[kXIt];
  if constexpr (kEp) {
    const GQK_GLOBAL lk_f32x4* const vb = reinterpret_cast<const GQK_GLOBAL lk_f32x4*>(
        (B.ep_flags & kEpScaleV) ? (const GQK_GLOBAL float*)B.scale_ss : x);
#pragma unroll
    for (int j = 0; j < kXIt; ++j) {
      const int i = tid + j * kW * 64;
      vg[j] = vb[kXF4 % (kW * 64) == 0 || i < kXF4 ? i : 0];
    }
  }

  // ... then the weight loads of the first kDepth steps. A wave's steps are
  // consecutive rows: step st reads rows [st kRps, st kRps + kRps) at base
  // W + st kRps kRowBytes plus a 32-bit lane offset. Loads for steps past the
  // wave's last re-read that step's bytes (every step issues the same loads,
  // so the in-order load counter stays exact), and rows past the matrix
  // re-read its last row; neither is ever stored. A wave without steps
  // (n = 0) re-reads step max(st0 - 1, 0), which exists.
  const int64_t last = st0 + n - 1 > 0 ? st0 + n - 1 : 0;
  auto issue = [&](int64_t st, Load& L) {
    st = st < last ? st : last;
    const int64_t r0 = st * rpm;
    const int64_t lim = rows - 1 - r0;
    const uint32_t rr = lim < rpm - 1 ? (uint32_t)((int64_t)rsub < lim ? rsub : lim) : (uint32_t)rsub;
    const uint32_t off = rr * kRowBytes + hoff;
    const GQK_GLOBAL uint8_t* base = Wl + r0 * (int64_t)kRowBytes;
    if constexpr (kQ6) {
      q6k_unit_issue(base + rr * kRowBytes, (uint32_t)u, L);
    } else if constexpr (kQ80) {
      // blocks 2 u, 2 u + 1 of the row: bytes [68 u, 68 u + 68) as 17 words
      const GQK_GLOBAL uint32_t* w =
          reinterpret_cast<const GQK_GLOBAL uint32_t*>(base + (rr * kRowBytes + 68u * (uint32_t)u));
      L.a = lk_u32x4{w[0], w[1], w[2], w[3]};
      L.b = lk_u32x4{w[4], w[5], w[6], w[7]};
      L.c = lk_u32x4{w[8], w[9], w[10], w[11]};
      L.d = lk_u32x4{w[12], w[13], w[14], w[15]};
      L.e = w[16];
    } else if constexpr (kQ40) {
      // blocks 2 u, 2 u + 1 of the row: bytes [36 u, 36 u + 36) as 9 words
      const GQK_GLOBAL uint32_t* w =
          reinterpret_cast<const GQK_GLOBAL uint32_t*>(base + (rr * kRowBytes + 36u * (uint32_t)u));
      L.h = lk_u32x4{w[0], w[1], w[2], w[3]};
      L.qa = lk_u32x4{w[4], w[5], w[6], w[7]};
      L.qb = lk_u32x4{w[8], 0u, 0u, 0u};
    } else {
      L.h = *reinterpret_cast<const GQK_GLOBAL lk_u32x4*>(base + off);
      L.qa = *reinterpret_cast<const GQK_GLOBAL lk_u32x4*>(base + (off + qoff));
      L.qb = *reinterpret_cast<const GQK_GLOBAL lk_u32x4*>(base + (off + qoff + 16));
    }
  };
  // At most two steps go out before x is staged, the rest right after: the
  // block's x loads then queue behind at most two steps of every wave's
  // weight loads (with a four-step ring x arrived 1.2 us later), and the
  // loads keep their order, so the in-order waits stay exact.
  constexpr int kEarly = kDepth < 2 ? kDepth : 2;
  Load ring[kDepth];
#pragma unroll
  for (int p = 0; p < kEarly; ++p) issue(st0 + p, ring[p]);
  // the input RMSN's partial sums after the first weight loads: where the
  // epilogue comes from argument memory, only they wait for it (the empty asm
  // keeps the scheduler from moving their address work, and with it the
  // wait, above the weight loads)
  if constexpr (kEp) {
    int f = B.ep_flags, sn = B.scale_n;
    const float* sp = (const float*)B.scale_ss;
    asm volatile("" : "+s"(f), "+s"(sn), "+s"(sp));
    ssl = lk_ep_ss_issue(f, sn, (const GQK_GLOBAL float*)sp, B.x, lane);
  }
  tl.stamp(1);

#pragma unroll
  for (int j = 0; j < kXIt; ++j) {
    const int i = tid + j * kW * 64;
    if (kXF4 % (kW * 64) == 0 || i < kXF4)
      *reinterpret_cast<lk_f32x4*>(&xl[lk_x_slot<kType>(i)]) = xg[j];
  }
  // (kEpScaleV) the block's sum of v^2 in a fixed order: each thread its
  // float4s in order, the wave's lanes by a fixed butterfly, the waves in
  // wave order after the barrier
  __shared__ float lk_vsum[kW];
  if constexpr (kEp) {
    float sq = 0.f;
#pragma unroll
    for (int j = 0; j < kXIt; ++j) {
      const int i = tid + j * kW * 64;
      if (kXF4 % (kW * 64) == 0 || i < kXF4) {
        sq = fmaf(vg[j].x, vg[j].x, sq);
        sq = fmaf(vg[j].y, vg[j].y, sq);
        sq = fmaf(vg[j].z, vg[j].z, sq);
        sq = fmaf(vg[j].w, vg[j].w, sq);
      }
    }
    const float ws = wave_sum_fixed(sq);
    if (lane == 0) lk_vsum[tid >> 6] = ws;
  }
  __syncthreads();
#pragma unroll
  for (int p = kEarly; p < kDepth; ++p) issue(st0 + p, ring[p]);
  tl.stamp(2);
  LkEp E;
  if constexpr (kEp) {
    float vtot = 0.f;
#pragma unroll
    for (int w = 0; w < kW; ++w) vtot += lk_vsum[w];
    E = lk_ep(epl, lk_ep_ss_sum(B, lane, ssl), vtot);
  }
  if (n > 0) {

  float xv[64];
  {
    const float4* xp = reinterpret_cast<const float4*>(&xl[68 * u]);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float4 t = xp[i];
      xv[4 * i + 0] = t.x;
      xv[4 * i + 1] = t.y;
      xv[4 * i + 2] = t.z;
      xv[4 * i + 3] = t.w;
    }
  }
  float xs0 = 0.f, xs1 = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    xs0 += xv[i];
    xs1 += xv[32 + i];
  }
  float xq[4] = {0.f, 0.f, 0.f, 0.f};   // Q6_K: sums over the slice's four runs of 16
  if constexpr (kQ6) {
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int t = 0; t < 16; ++t) xq[m] += xv[16 * m + t];
  }

  // Step i: the dot products of the lane's 64 weights of rows
  // (st0 + i) kRps .. + kRps - 1, summed per row and stored.
  auto step = [&](const Load& L) {
    if constexpr (kQ6) {
      return q6k_unit_dot(L, (uint32_t)u & 1u, [&](int i) { return xv[i]; }, xq);
    } else if constexpr (kQ80) {
      // words: d0 | q 0..1, q 2..29 (7 words), q 30..31 | d1, then block 1's
      // 32 codes; w = q d, two independent sums per block
      const uint32_t w[17] = {L.a.x, L.a.y, L.a.z, L.a.w, L.b.x, L.b.y, L.b.z, L.b.w, L.c.x,
                              L.c.y, L.c.z, L.c.w, L.d.x, L.d.y, L.d.z, L.d.w, L.e};
      const float d0 = half_lo(w[0]), d1 = half_hi(w[8]);
      float s0a = 0.f, s0b = 0.f, s1a = 0.f, s1b = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint32_t c0 = __builtin_amdgcn_alignbyte(w[k + 1], w[k], 2);   // block 0, q 4k .. 4k + 3
        const uint32_t c1 = w[9 + k];                                         // block 1
        float& a0 = (k & 1) ? s0b : s0a;
        float& a1 = (k & 1) ? s1b : s1a;
        a0 = fmaf(sbyte0(c0), xv[4 * k + 0], a0);
        a0 = fmaf(sbyte1(c0), xv[4 * k + 1], a0);
        a0 = fmaf(sbyte2(c0), xv[4 * k + 2], a0);
        a0 = fmaf(sbyte3(c0), xv[4 * k + 3], a0);
        a1 = fmaf(sbyte0(c1), xv[32 + 4 * k + 0], a1);
        a1 = fmaf(sbyte1(c1), xv[32 + 4 * k + 1], a1);
        a1 = fmaf(sbyte2(c1), xv[32 + 4 * k + 2], a1);
        a1 = fmaf(sbyte3(c1), xv[32 + 4 * k + 3], a1);
      }
      return fmaf(d1, s1a + s1b, d0 * (s0a + s0b));
    } else if constexpr (kQ40) {
      return q40_quarter_dot(L, xv, xs0, xs1);
    } else {
      return q4k_quarter_dot(L, sh, hi_mask, xv, xs0, xs1);
    }
  };
  auto finish = [&](float r, int i) {
    r = lk_segment_sum<kU>(r);
    const int64_t row = (st0 + i) * rpm + rsub;
    if constexpr (kEp) {
      if (paired) {
        // lane 32 + l holds the up row whose gate row lane l holds
        const float gv = __shfl_xor(r, 32) * E.scale;
        const float v = r * E.scale;
        if (u == kU - 1 && row < rows) {
          if (lane < 32) {
            y[row] = v;
          } else {
            B.y2[row] = v;
            E.e.act[row] = gv / (1.0f + expf(-gv)) * v;
          }
        }
        return;
      }
    }
    if (u == kU - 1 && row < rows) {
      if constexpr (kEp)
        lk_ep_row(E, r, row, y);
      else
        y[row] = r;
    }
    if (i == 0) tl.stamp(3);
  };

  // Whole groups of kDepth steps: step i consumes ring slot i mod kDepth and
  // refills it with step i + kDepth, so kDepth - 1 later steps stay in flight
  // while it computes. Every pass of this loop issues the same loads in the
  // same order, so the wait before each step is exact.
  int i0 = 0;
  for (; i0 + kDepth <= n; i0 += kDepth) {
#pragma unroll
    for (int p = 0; p < kDepth; ++p) {
      const float r = step(ring[p]);
      issue(st0 + i0 + p + kDepth, ring[p]);
      finish(r, i0 + p);
    }
  }
  // The last n - i0 < kDepth steps, already in flight: no more loads.
#pragma unroll
  for (int p = 0; p < kDepth - 1; ++p)
    if (i0 + p < n) finish(step(ring[p]), i0 + p);
  }   // n > 0
  tl.stamp(4);
  if constexpr (kEp) {
    const int64_t rb0 = (int64_t)B.bs0 * rpm;
    const int64_t re = (int64_t)(B.bs0 + B.bn) * rpm;
    lk_ep_groups(E, rb0, re < rows ? re : rows, rows, y, __builtin_amdgcn_readfirstlane(tid >> 6), lane);
  }
  tl.stamp(5);
  tl_put(tl_key, tl);
}

// ---------------------------------------------------------------------------
// Rows of any number of super-blocks up to 128 (K up to 32768), Q4_K or Q4_0,
// with K split over the waves of a block: wave w of nw takes super-blocks
// [w nsb / nw, (w + 1) nsb / nw) of every row, and the block takes R
// consecutive rows of one GEMV. Within its slice a wave works as the
// lanes-along-K kernel above with 64 / kRps lanes per row and kRps rows per
// step: kRps = 4 (slices of at most 4 super-blocks), 2 (at most 8) or 1 (at
// most 16). Lane u of a row holds quarter u of the slice (lanes past the
// slice hold nothing and add zero), its 64 activations and their two
// sub-block sums kept in VGPRs for every row of the block. The wave stages
// only its own slice of x (through its own LDS window, no block barrier), so
// no lane reads x per row. Each step's slice sums (a fixed butterfly) go to
// LDS; after the last step the block adds the nw slice sums of each row in
// wave order and stores y. Nothing leaves the block but y: no scratch, no
// counters. The host picks kRps and nw so that the waves spread evenly over
// the four SIMDs (nw a multiple of 4 where it can) with the fewest row steps
// per SIMD; blocks of at most 12 waves (kRps 4 or 2) or 8 (kRps 1).
// ---------------------------------------------------------------------------
constexpr int kLksMaxNsb = 128;         // K up to 32768
constexpr int kLksMaxRows = 128;        // rows per block

// Super-blocks per slice at most, waves per block at most, and the LDS
// floats of one wave's padded x window, for kRps rows per step.
constexpr int lks_max_slice(int rps) { return 16 / rps; }
constexpr int lks_max_waves(int rps) { return rps == 1 ? 8 : 12; }
constexpr int lks_x_floats(int rps) { return lks_max_slice(rps) * 4 * 68; }

struct LksDesc {
  const uint8_t* W;
  float* y;
  int rows;
  int block_begin;   // first block of this GEMV in the launch
};

struct LksGroup {
  LksDesc d[kLkMaxGroup];
  const float* x;   // the one input of the group's GEMVs
  int n;
};

// Dynamic LDS bytes of a launch with nw waves and R rows per block.
constexpr size_t lks_lds_bytes(int rps, int nw, int R) {
  return (size_t)nw * lks_x_floats(rps) * 4 + (size_t)R * nw * 4;
}

// kType: GGUF type 12 (Q4_K) or 2 (Q4_0); both store 144 bytes per 256
// weights. kSingle: one GEMV whose pointers and rows come in the leading
// scalar arguments (preloaded into SGPRs), else the block's GEMV from grp.
// nw: the waves per block (blockDim.x / 64, passed so that it is preloaded
// too: blockDim.x is a kernel argument in memory, and its fetch held the
// first loads back by a round trip). kEp (one Q4_K GEMV): the residual add
// and the next norm's preparation of ep as the rows are stored (the output
// projection of a decode layer), read only after the last step.
template <int kType, int kDepth, bool kSingle, int kRps, bool kEp>
__global__ __launch_bounds__(lks_max_waves(kRps) * 64) void gemv_lks_kernel(const uint8_t* W1, const float* x,
                                                                     float* y1, int rows1, int nsb, int R,
                                                                     int nw, LksGroup grp, GemvEpilogue ep) {
  static_assert(kType == 12 || kType == 2, "Q4_K or Q4_0 rows");
  static_assert(!kEp || (kSingle && kType == 12), "epilogues on one Q4_K GEMV");
  static_assert(kRps == 1 || kRps == 2 || kRps == 4, "one, two or four rows per step");
  constexpr bool kQ40 = kType == 2;
  constexpr int kU = 64 / kRps;                 // lanes per row
  constexpr int kMaxSlice = lks_max_slice(kRps);
  constexpr int kXFloats = lks_x_floats(kRps);
  extern __shared__ __attribute__((aligned(16))) float lds[];
  TlStamps tl;
  tl.stamp(0);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const GQK_GLOBAL uint8_t* W;
  GQK_GLOBAL float* y;
  int rows, lb;
  if constexpr (kSingle) {
    W = (const GQK_GLOBAL uint8_t*)W1;
    y = (GQK_GLOBAL float*)y1;
    rows = rows1;
    lb = (int)blockIdx.x;
  } else {
    const int b = (int)blockIdx.x;
    const int g = (grp.n > 1 && b >= grp.d[1].block_begin) + (grp.n > 2 && b >= grp.d[2].block_begin) +
                  (grp.n > 3 && b >= grp.d[3].block_begin);
    const LksDesc& d = grp.d[g];
    W = (const GQK_GLOBAL uint8_t*)d.W;
    y = (GQK_GLOBAL float*)d.y;
    rows = d.rows;
    lb = b - d.block_begin;
  }
  const int64_t r0 = (int64_t)lb * R;
  const int nrows = (int)(rows - r0 < R ? rows - r0 : R);   // >= 1: the host gives no empty block
  const int n = (nrows + kRps - 1) / kRps;                 // row steps
  const int sa = (wave * nsb) / nw, sb = ((wave + 1) * nsb) / nw;
  const int S = sb - sa;                                   // 1 .. kMaxSlice super-blocks
  const int half = lane / kU;                              // row of the step
  const int u = lane % kU;
  const bool valid = u < 4 * S;
  const int uq = valid ? u : 4 * S - 1;                    // lanes past the slice re-read its last quarter
  const uint32_t row_bytes = (uint32_t)nsb * kQ4KBlockBytes;
  const uint32_t gq = (uint32_t)uq & 3u;
  const uint32_t hoff = kQ40 ? 36u * (uint32_t)(4 * sa + uq) : (uint32_t)(sa + (uq >> 2)) * kQ4KBlockBytes;
  const uint32_t qoff = hoff + 16u + 32u * gq;
  const uint32_t sh = 16u * (gq & 1u);
  const uint32_t hi_mask = gq >= 2 ? 0xFFFFFFFFu : 0u;

  // x: the wave's slice, S * 64 float4, lane l taking float4s l + 64 j. All
  // kMaxSlice loads are issued (those past the slice re-read its last float4
  // and land in the unread tail of the window): loads under a branch made the
  // compiler wait for each one in turn.
  const GQK_GLOBAL lk_f32x4* xs4 = (const GQK_GLOBAL lk_f32x4*)x + 64 * sa;
  lk_f32x4 xg[kMaxSlice];
#pragma unroll
  for (int j = 0; j < kMaxSlice; ++j) {
    const int i = lane + 64 * j;
    xg[j] = xs4[i < 64 * S ? i : 64 * S - 1];
  }

  // Step i reads rows r0 + kRps i + half (a row past the block's last
  // re-reads the last one; steps past the wave's last re-read that step:
  // every ring slot issues the same loads, so the in-order wait counts stay
  // exact).
  const int last = n - 1;
  auto issue = [&](int i, LkLoad& L) {
    i = i < last ? i : last;
    int rr = kRps * i + half;
    rr = rr < nrows ? rr : nrows - 1;
    const GQK_GLOBAL uint8_t* base = W + (r0 + rr) * (int64_t)row_bytes;
    if constexpr (kQ40) {
      const GQK_GLOBAL uint32_t* w = reinterpret_cast<const GQK_GLOBAL uint32_t*>(base + hoff);
      L.h = lk_u32x4{w[0], w[1], w[2], w[3]};
      L.qa = lk_u32x4{w[4], w[5], w[6], w[7]};
      L.qb = lk_u32x4{w[8], 0u, 0u, 0u};
    } else {
      L.h = *reinterpret_cast<const GQK_GLOBAL lk_u32x4*>(base + hoff);
      L.qa = *reinterpret_cast<const GQK_GLOBAL lk_u32x4*>(base + qoff);
      L.qb = *reinterpret_cast<const GQK_GLOBAL lk_u32x4*>(base + (qoff + 16));
    }
  };
  // The whole ring goes out with x (as in lk_run): the weights are in flight
  // from the start and x's wait overlaps them.
  LkLoad ring[kDepth];
#pragma unroll
  for (int p = 0; p < kDepth; ++p) issue(p, ring[p]);
  tl.stamp(1);

  // stage the slice in the wave's own LDS window (quarter v at float 68 v)
  // and take this lane's quarter back: a wave-level exchange, no block barrier
  float* xw = lds + wave * kXFloats;
#pragma unroll
  for (int j = 0; j < kMaxSlice; ++j) {
    const int i = lane + 64 * j;
    *reinterpret_cast<lk_f32x4*>(&xw[68 * (i >> 4) + 4 * (i & 15)]) = xg[j];
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  float xv[64];
  {
    const float4* xp = reinterpret_cast<const float4*>(&xw[68 * uq]);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float4 t = xp[i];
      xv[4 * i + 0] = t.x;
      xv[4 * i + 1] = t.y;
      xv[4 * i + 2] = t.z;
      xv[4 * i + 3] = t.w;
    }
  }
  float xs0 = 0.f, xs1 = 0.f;   // sums of x over the quarter's two halves of 32
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    xs0 += xv[i];
    xs1 += xv[32 + i];
  }
  tl.stamp(2);

  float* part = lds + nw * kXFloats;   // [row of the block][wave]
  auto step = [&](const LkLoad& L) {
    const float r = kQ40 ? q40_quarter_dot(L, xv, xs0, xs1) : q4k_quarter_dot(L, sh, hi_mask, xv, xs0, xs1);
    return valid ? r : 0.f;
  };
  auto finish = [&](float r, int i) {
    r = lk_segment_sum<kU>(r);
    const int rr = kRps * i + half;
    if (u == kU - 1 && rr < nrows) part[rr * nw + wave] = r;
    if (i == 0) tl.stamp(3);
  };
  int i0 = 0;
  for (; i0 + kDepth <= n; i0 += kDepth) {
#pragma unroll
    for (int p = 0; p < kDepth; ++p) {
      const float r = step(ring[p]);
      issue(i0 + p + kDepth, ring[p]);
      finish(r, i0 + p);
    }
  }
#pragma unroll
  for (int p = 0; p < kDepth - 1; ++p)
    if (i0 + p < n) finish(step(ring[p]), i0 + p);
  tl.stamp(4);

  // the rows' slice sums, added in wave order
  __syncthreads();
  if constexpr (kEp) {
    // residual, norm output and the 64-row groups' sums of squares, as in the
    // kernels above (no input scale on this path)
    const LkEp E = lk_ep(ep, 0.f);
    if (wave == 0) {
      for (int rr = lane; rr < nrows; rr += 64) {
        float v = 0.f;
        for (int w = 0; w < nw; ++w) v += part[rr * nw + w];
        lk_ep_row(E, v, r0 + rr, y);
      }
    }
    lk_ep_groups(E, r0, r0 + nrows, rows, y, wave, lane);
  } else {
    if (wave == 0) {
      for (int rr = lane; rr < nrows; rr += 64) {
        float v = 0.f;
        for (int w = 0; w < nw; ++w) v += part[rr * nw + w];
        y[r0 + rr] = v;
      }
    }
  }
  tl.stamp(5);
  tl_put(kSingle ? (const void*)W1 : (const void*)grp.d[0].W, tl);
}

// ---------------------------------------------------------------------------
// Long rows (K = 256 nsb > 4096, up to 12288): one row per step; lane l takes
// quarters l, l + 64, ... (kQ rounds, the last one partial), so a step reads
// a whole row. Too many activations per lane to keep in VGPRs: the block
// stages x in LDS (the same padded layout) together with the sums of x over
// each 32-weight sub-block, and every step reads each quarter's 64 values
// from LDS.
// ---------------------------------------------------------------------------
constexpr int kLkxMaxK = 12288;

struct LkxLoad {
  lk_u32x4 h, qa, qb;
};

template <int kType>
struct LkxLoadOf {
  using type = LkxLoad;
};
template <>
struct LkxLoadOf<14> {
  using type = LkLoad6;
};

//
// kType is the row format: GGUF type 12 (Q4_K: a quarter is one 32-byte nibble
// group plus its super-block's 16-byte header) or 2 (Q4_0, rows of 17 .. 48
// x 256 weights, the same 0.5625 bytes per weight: a quarter is two 18-byte
// blocks; no epilogues). kSingle: one GEMV whose descriptor comes in the
// leading scalar arguments (preloaded into SGPRs), else the group's. One
// kernel body for all: the compiler allocated about 100 more registers (and
// spilled) when the same body sat in an inlined function behind thin kernels.
template <int kType, int kQ, int kDepth, int kW, bool kEp, bool kSingle>
__global__ __launch_bounds__(kW * 64) void gemv_lkx_kernel(const uint8_t* W1, const float* x1, float* y1,
                                                           int rows1, int q1, int r1, int nsb1,
                                                           LkGroup grp) {
  static_assert(!(kSingle && kEp), "epilogues come with the group");
  static_assert(kType == 12 || kType == 2 || kType == 14, "Q4_K, Q4_0 or Q6_K rows");
  static_assert(kType == 12 || !kEp, "epilogues on Q4_K only");
  constexpr bool kQ40 = kType == 2, kQ6 = kType == 14;
  using XLoad = typename LkxLoadOf<kType>::type;
  // [K + K/16] padded x, then [K/32] sub-block sums ([K/16] sums of runs of
  // 16 for Q6_K)
  extern __shared__ __attribute__((aligned(16))) float xl[];
  TlStamps tl;
  tl.stamp(0);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const LkBlock B = kSingle ? lk_block_single<kW>(W1, x1, y1, rows1, q1, r1, nsb1, (int)blockIdx.x, wave)
                            : lk_block<kW>(grp, (int)blockIdx.x, wave);
  const int nsb = B.nsb;
  const int U = 4 * nsb;                    // quarters per row
  const int K = 256 * nsb;
  const int nxf4 = K / 4;
  const uint32_t row_bytes = (uint32_t)nsb * (kQ6 ? (uint32_t)kQ6KBlockBytes : (uint32_t)kQ4KBlockBytes);
  float* const xsum = xl + K + K / 16;
  LkSsLoads ssl;
  GemvEpilogue epl;
  if constexpr (kEp) {
    epl = grp.ep[B.g];
    ssl = lk_ep_ss_issue(B.ep_flags, B.scale_n, B.scale_ss, B.x, lane);
  }

  // x: the block's threads load it all first (at most 16 kQ / kW float4
  // each) ...
  constexpr int kXIt = 16 * kQ / kW;
  lk_f32x4 xg[kXIt];
#pragma unroll
  for (int j = 0; j < kXIt; ++j) {
    const int i = tid + j * kW * 64;
    if (i < nxf4) xg[j] = reinterpret_cast<const GQK_GLOBAL lk_f32x4*>(B.x)[i];
  }

  // ... then the weight loads of the first kDepth steps (rows). Quarter q of
  // the lane is uq = lane + 64 q; in the last round lanes past the row
  // re-read its last quarter and their sums are dropped.
  uint32_t hoff[kQ], qoff[kQ], sh[kQ], him[kQ];
  int uqc[kQ];
  bool val[kQ];
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    const int uq = lane + 64 * q;
    val[q] = uq < U;
    uqc[q] = val[q] ? uq : U - 1;
    const int gq = uqc[q] & 3;
    hoff[q] = (uint32_t)(uqc[q] >> 2) * kQ4KBlockBytes;
    qoff[q] = hoff[q] + 16u + 32u * (uint32_t)gq;
    sh[q] = 16u * (uint32_t)(gq & 1);
    him[q] = gq >= 2 ? 0xFFFFFFFFu : 0u;
  }
  const int64_t st0 = B.st0;
  const int n = B.n;
  const int64_t last = st0 + n - 1 > 0 ? st0 + n - 1 : 0;
  auto issue = [&](int64_t row, XLoad (&L)[kQ]) {
    row = row < last ? row : last;
    const GQK_GLOBAL uint8_t* base = B.W + row * (int64_t)row_bytes;
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      if constexpr (kQ6) {
        q6k_unit_issue(base, (uint32_t)uqc[q], L[q]);
      } else if constexpr (kQ40) {
        const GQK_GLOBAL uint32_t* w =
            reinterpret_cast<const GQK_GLOBAL uint32_t*>(base + 36u * (uint32_t)uqc[q]);
        L[q].h = lk_u32x4{w[0], w[1], w[2], w[3]};
        L[q].qa = lk_u32x4{w[4], w[5], w[6], w[7]};
        L[q].qb = lk_u32x4{w[8], 0u, 0u, 0u};
      } else {
        L[q].h = *reinterpret_cast<const GQK_GLOBAL lk_u32x4*>(base + hoff[q]);
        L[q].qa = *reinterpret_cast<const GQK_GLOBAL lk_u32x4*>(base + qoff[q]);
        L[q].qb = *reinterpret_cast<const GQK_GLOBAL lk_u32x4*>(base + (qoff[q] + 16));
      }
    }
  };
  XLoad ring[kDepth][kQ];
#pragma unroll
  for (int p = 0; p < kDepth; ++p) issue(st0 + p, ring[p]);
  tl.stamp(1);

  // store x; the eight threads 8m .. 8m + 7 hold the 32 values of
  // sub-block i / 8 (i = their float4 index) and add them with a fixed
  // butterfly, the first of them storing the sum
#pragma unroll
  for (int j = 0; j < kXIt; ++j) {
    const int i = tid + j * kW * 64;
    const bool in = i < nxf4;
    if constexpr (kQ6) {
      // the four threads 4m .. 4m + 3 hold one run of 16 (a unit's positions
      // 16 m' .. 16 m' + 15); the first stores its sum at 4 u + m'
      if (in) *reinterpret_cast<lk_f32x4*>(&xl[lk_x_slot<14>(i)]) = xg[j];
      float t = in ? (xg[j].x + xg[j].y) + (xg[j].z + xg[j].w) : 0.f;
      t += dpp_f32<0xB1>(t);    // quad_perm 1,0,3,2
      t += dpp_f32<0x4E>(t);    // quad_perm 2,3,0,1
      if (in && (tid & 3) == 0) xsum[lk_x_slot<14>(i) / 68 * 4 + ((lk_x_slot<14>(i) % 68) >> 4)] = t;
    } else {
      if (in) *reinterpret_cast<lk_f32x4*>(&xl[4 * i + (i >> 4) * 4]) = xg[j];
      float t = in ? (xg[j].x + xg[j].y) + (xg[j].z + xg[j].w) : 0.f;
      t += dpp_f32<0xB1>(t);    // quad_perm 1,0,3,2
      t += dpp_f32<0x4E>(t);    // quad_perm 2,3,0,1
      t += dpp_f32<0x141>(t);   // row_half_mirror
      if (in && (tid & 7) == 0) xsum[i >> 3] = t;
    }
  }
  __syncthreads();
  tl.stamp(2);
  LkEp E;
  if constexpr (kEp) E = lk_ep(epl, lk_ep_ss_sum(B, lane, ssl));
  if (n > 0) {
  float xs0[kQ], xs1[kQ];
  float xq6[kQ][4];
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    if constexpr (kQ6) {
#pragma unroll
      for (int m = 0; m < 4; ++m) xq6[q][m] = xsum[4 * uqc[q] + m];
    } else {
      xs0[q] = xsum[2 * uqc[q]];
      xs1[q] = xsum[2 * uqc[q] + 1];
    }
  }

  auto step = [&](const XLoad (&L)[kQ]) {
    float r = 0.f;
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      if constexpr (kQ6) {
        const float* xp = &xl[68 * uqc[q]];
        const float rq = q6k_unit_dot(L[q], (uint32_t)uqc[q] & 1u, [&](int i) { return xp[i]; }, xq6[q]);
        r += val[q] ? rq : 0.f;
        // one quarter at a time: left free, the scheduler hoisted the LDS
        // reads of all of them and spilled
        __builtin_amdgcn_sched_barrier(0);
      } else if constexpr (kQ40) {
        // two 18-byte blocks: block 0's codes re-aligned, block 1's aligned;
        // byte j of a block: low nibble weight j, high nibble weight j + 16
        const uint32_t w[9] = {L[q].h.x, L[q].h.y, L[q].h.z, L[q].h.w, L[q].qa.x,
                               L[q].qa.y, L[q].qa.z, L[q].qa.w, L[q].qb.x};
        const float d0 = half_lo(w[0]), d1 = half_hi(w[4]);
        const lk_f32x4* xp = reinterpret_cast<const lk_f32x4*>(&xl[68 * uqc[q]]);
        float s0a = 0.f, s0b = 0.f, s1a = 0.f, s1b = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t c0 = __builtin_amdgcn_alignbyte(w[k + 1], w[k], 2);
          const uint32_t c1 = w[5 + k];
          float l0[4], h0[4], l1[4], h1[4];
          nibbles_div512(opaque(c0 & 0x0F0F0F0Fu), l0);
          nibbles_div512(opaque((c0 >> 4) & 0x0F0F0F0Fu), h0);
          nibbles_div512(opaque(c1 & 0x0F0F0F0Fu), l1);
          nibbles_div512(opaque((c1 >> 4) & 0x0F0F0F0Fu), h1);
          const lk_f32x4 xa = xp[k], xb = xp[4 + k], xc = xp[8 + k], xd = xp[12 + k];
          s0a = fmaf(l0[0], xa.x, s0a); s0a = fmaf(l0[1], xa.y, s0a);
          s0a = fmaf(l0[2], xa.z, s0a); s0a = fmaf(l0[3], xa.w, s0a);
          s0b = fmaf(h0[0], xb.x, s0b); s0b = fmaf(h0[1], xb.y, s0b);
          s0b = fmaf(h0[2], xb.z, s0b); s0b = fmaf(h0[3], xb.w, s0b);
          s1a = fmaf(l1[0], xc.x, s1a); s1a = fmaf(l1[1], xc.y, s1a);
          s1a = fmaf(l1[2], xc.z, s1a); s1a = fmaf(l1[3], xc.w, s1a);
          s1b = fmaf(h1[0], xd.x, s1b); s1b = fmaf(h1[1], xd.y, s1b);
          s1b = fmaf(h1[2], xd.z, s1b); s1b = fmaf(h1[3], xd.w, s1b);
        }
        float rq = (d0 * 512.0f) * (s0a + s0b);
        rq = fmaf(d1 * 512.0f, s1a + s1b, rq);
        rq = fmaf(-8.0f * d0, xs0[q], rq);
        rq = fmaf(-8.0f * d1, xs1[q], rq);
        r += val[q] ? rq : 0.f;
      } else {
        float dsc0, dsc1, dmm0, dmm1;
        q4k_pair_scales(L[q].h.x, L[q].h.y, L[q].h.z, L[q].h.w, sh[q], him[q], dsc0, dsc1, dmm0, dmm1);
        const uint32_t qw[8] = {L[q].qa.x, L[q].qa.y, L[q].qa.z, L[q].qa.w,
                                L[q].qb.x, L[q].qb.y, L[q].qb.z, L[q].qb.w};
        const lk_f32x4* xp = reinterpret_cast<const lk_f32x4*>(&xl[68 * uqc[q]]);
        float la0 = 0.f, la1 = 0.f, ha0 = 0.f, ha1 = 0.f;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const lk_f32x4 xa = xp[t];       // x of sub-block 2 gq, weights 4t .. 4t + 3
          const lk_f32x4 xb = xp[8 + t];   // x of sub-block 2 gq + 1
          float ql[4], qh[4];
          nibbles_div512(opaque(qw[t] & 0x0F0F0F0Fu), ql);
          nibbles_div512(opaque((qw[t] >> 4) & 0x0F0F0F0Fu), qh);
          float& la = (t & 1) ? la1 : la0;
          float& ha = (t & 1) ? ha1 : ha0;
          la = fmaf(ql[0], xa.x, la);
          la = fmaf(ql[1], xa.y, la);
          la = fmaf(ql[2], xa.z, la);
          la = fmaf(ql[3], xa.w, la);
          ha = fmaf(qh[0], xb.x, ha);
          ha = fmaf(qh[1], xb.y, ha);
          ha = fmaf(qh[2], xb.z, ha);
          ha = fmaf(qh[3], xb.w, ha);
        }
        float rq = dsc0 * (la0 + la1);
        rq = fmaf(dsc1, ha0 + ha1, rq);
        rq = fmaf(-dmm0, xs0[q], rq);
        rq = fmaf(-dmm1, xs1[q], rq);
        r += val[q] ? rq : 0.f;
      }
    }
    return r;
  };
  auto finish = [&](float r, int i) {
    r = lk_segment_sum<64>(r);
    if (lane == 63) {
      if constexpr (kEp)
        lk_ep_row(E, r, st0 + i, B.y);
      else
        B.y[st0 + i] = r;
    }
    if (i == 0) tl.stamp(3);
  };

  int i0 = 0;
  for (; i0 + kDepth <= n; i0 += kDepth) {
#pragma unroll
    for (int p = 0; p < kDepth; ++p) {
      const float r = step(ring[p]);
      issue(st0 + i0 + p + kDepth, ring[p]);
      finish(r, i0 + p);
    }
  }
#pragma unroll
  for (int p = 0; p < kDepth - 1; ++p)
    if (i0 + p < n) finish(step(ring[p]), i0 + p);
  }   // n > 0
  tl.stamp(4);
  if constexpr (kEp) {
    const int64_t rb0 = B.bs0;
    lk_ep_groups(E, rb0, rb0 + B.bn, B.rows, B.y, wave, lane);
  }
  tl.stamp(5);
  tl_put(kSingle ? (const void*)W1 : (const void*)grp.d[0].W, tl);
}

}  // namespace gqk
