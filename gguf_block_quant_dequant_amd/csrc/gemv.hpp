// Batch-1 fused dequant x vector kernels (decode GEMV) for gfx950.
//
// Work mapping ("lane per row"): a wave owns 64 consecutive rows and walks a
// range of blocks along K. Lane i computes row row0 + i, so every lane is at
// the same column k at the same time and the activation x[k] is wave-uniform:
// the compiler reads x with scalar loads into SGPRs and each multiply-add is
// one v_fmac with an SGPR operand, with no per-lane activation traffic at all.
//
// Weight bytes reach the wave through LDS: a "chunk" (one Q4_K super-block, or
// eight Q8_0 blocks, of each of the 64 rows) is copied with direct
// global->LDS 16-byte loads in which consecutive lanes fetch consecutive
// 16-byte pieces of each row segment (coalesced HBM reads), and lane i then
// reads its own row segment back from LDS. The row stride in LDS (144 B or
// 272 B = 36 or 68 dwords, 4 modulo 32 banks) makes those 16-byte reads
// conflict-free. Each wave keeps SLOTS chunks of its own in LDS and issues the
// next chunk's loads before computing the current one.
//
// Split-K: a row group may be cut into P ranges along K processed by different
// waves. Each writes its 64 partial sums to scratch, bumps a per-row-group
// counter, and the wave that arrives last adds the P partials in range order
// (so results do not depend on timing) and writes y. The counter is reset by
// that wave, leaving scratch ready for the next call.
#pragma once

#include "coherent.hpp"
#include "device_common.hpp"
#include "gemv_types.hpp"

namespace gqk {

constexpr int kQ4KChunk = 64 * kQ4KBlockBytes;                  // 9216 B = 9 x 1 KiB
constexpr int kQ80ChunkBlocks = 8;
constexpr int kQ80ChunkRowBytes = kQ80ChunkBlocks * kQ80BlockBytes;   // 272 B
constexpr int kQ80Chunk = 64 * kQ80ChunkRowBytes;               // 17408 B = 17 x 1 KiB

// Where lane `lane`'s 16-byte piece of DMA window j comes from: window j,
// lane i lands at chunk byte 1024 j + 16 i = (row r, byte b) of the
// [64][row_seg] chunk. Rows past the matrix are clamped to its last row (the
// loads stay in bounds; those lanes' results are never stored).
template <int kWindows, int kRowSeg>
__device__ __forceinline__ void dma_offsets(int lane, uint32_t row_bytes, int valid_rows,
                                            uint32_t (&off)[kWindows]) {
#pragma unroll
  for (int j = 0; j < kWindows; ++j) {
    const int o = 1024 * j + 16 * lane;
    int r = o / kRowSeg;
    const int b = o - r * kRowSeg;
    r = r < valid_rows ? r : valid_rows - 1;
    off[j] = (uint32_t)r * row_bytes + (uint32_t)b;
  }
}

template <int kWindows>
__device__ __forceinline__ void dma_chunk(const uint8_t* src, const uint32_t (&off)[kWindows],
                                          uint8_t* slot) {
#pragma unroll
  for (int j = 0; j < kWindows; ++j) dma16(src + off[j], slot + 1024 * j);
}

// 16 consecutive activations in SGPRs.
typedef float xreg16 __attribute__((ext_vector_type(16)));

// Activations stream through two 16-SGPR tuples: the 64-byte scalar load of
// the next 16 values is issued before the current 16 are multiplied and waited
// for after. Both the load and the wait are inline assembly with the loaded
// tuple threaded through the wait, so no use can be scheduled before the wait
// and the compiler cannot hoist every load of a block to the top (which
// exhausts the SGPR file and spills through lanes).
#define GQK_SLOAD16(dst, base, off) \
  asm volatile("s_load_dwordx16 %0, %1, %2" : "=s"(dst) : "s"(base), "n"(off))
#define GQK_SWAIT(reg) asm volatile("s_waitcnt lgkmcnt(0)" : "+s"(reg))

// Load x[0..15] of a 1 KiB activation range into xa and, in the same
// round trip, touch its other 15 64-byte lines (one scalar dword each) so
// that the step-by-step loads that follow hit the scalar cache instead of
// each paying a miss. The touched words are discarded; their registers are
// held until the wait so no late load can land in a reused register. Every
// output is early-clobber: a load's data may return while later loads of the
// block are still to issue, so no destination may share registers with the
// base address.
__device__ __forceinline__ void sload_first_with_touch(xreg16& xa, const float* xs) {
  uint32_t t[15];
  asm volatile(
      "s_load_dwordx16 %0, %16, 0\n"
      "s_load_dword %1, %16, 64\n"
      "s_load_dword %2, %16, 128\n"
      "s_load_dword %3, %16, 192\n"
      "s_load_dword %4, %16, 256\n"
      "s_load_dword %5, %16, 320\n"
      "s_load_dword %6, %16, 384\n"
      "s_load_dword %7, %16, 448\n"
      "s_load_dword %8, %16, 512\n"
      "s_load_dword %9, %16, 576\n"
      "s_load_dword %10, %16, 640\n"
      "s_load_dword %11, %16, 704\n"
      "s_load_dword %12, %16, 768\n"
      "s_load_dword %13, %16, 832\n"
      "s_load_dword %14, %16, 896\n"
      "s_load_dword %15, %16, 960\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&s"(xa), "=&s"(t[0]), "=&s"(t[1]), "=&s"(t[2]), "=&s"(t[3]), "=&s"(t[4]),
        "=&s"(t[5]), "=&s"(t[6]), "=&s"(t[7]), "=&s"(t[8]), "=&s"(t[9]), "=&s"(t[10]),
        "=&s"(t[11]), "=&s"(t[12]), "=&s"(t[13]), "=&s"(t[14])
      : "s"(xs));
}
// The wait for step h + 1's activations also takes step h's accumulators as
// inputs, which pins step h's multiply-adds before it (and, since volatile
// statements keep their order, before the load for step h + 2).
#define GQK_SWAIT_AFTER(reg, d0, d1) \
  asm volatile("s_waitcnt lgkmcnt(0)" : "+s"(reg) : "v"(d0), "v"(d1))

// ---------------------------------------------------------------------------
// Q4_K: dot product of one super-block of this lane's row with xs[0..255].
// c[0..3] = header words (d|dmin, S[0..3], S[4..7], S[8..11]); c[4..35] =
// quant words: word 4 + 8g + t holds bytes Qb[32g + 4t .. 32g + 4t + 3], whose
// low nibbles are weights 64g + 4t + 0..3 (sub-block 2g) and high nibbles
// weights 64g + 32 + 4t + 0..3 (sub-block 2g + 1).
//   sum_i w_i x_i = sum_j (d sc_j) (sum_{i in j} q_i x_i) - sum_j (dmin m_j) xsum_j
// Nibbles are masked into byte positions (high nibbles shifted down first)
// and converted two per instruction as q / 512 (nibbles_div512); the 512 is
// folded into d sc_j, an exact power-of-two scaling.
// 16 steps of 16 weights. On entry xa holds xs[0..15]; on exit, if `more`,
// it holds xs[256..271] (the next super-block's first step).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float q4k_superblock_dot(const uint32_t (&c)[36], const float* xs,
                                                    bool more, xreg16& xa,
                                                    const float (&xsum)[8]) {
  float dsc[8], dmm[8];
  q4k_scales(c[0], c[1], c[2], c[3], dsc, dmm);
  float acc = 0.f;
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int h = 0; h < 16; ++h) {
    xreg16 xb;
    if (h < 15) GQK_SLOAD16(xb, xs, 64 * (h + 1));
    else if (more) GQK_SLOAD16(xb, xs, 1024);
    const int u = h >> 1;                 // sub-block
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t v = c[4 + 8 * (u >> 1) + 4 * (h & 1) + t];
      const uint32_t nib = opaque((u & 1) ? ((v >> 4) & 0x0F0F0F0Fu) : (v & 0x0F0F0F0Fu));
      float q[4];
      nibbles_div512(nib, q);
      float& a = (t & 1) ? a1 : a0;
      a = fmaf(q[0], xa[4 * t + 0], a);
      a = fmaf(q[1], xa[4 * t + 1], a);
      a = fmaf(q[2], xa[4 * t + 2], a);
      a = fmaf(q[3], xa[4 * t + 3], a);
    }
    if (h < 15 || more) {
      GQK_SWAIT_AFTER(xb, a0, a1);
      xa = xb;
    }
    if (h & 1) {
      acc = fmaf(dsc[u] * 512.0f, a0 + a1, acc);
      a0 = 0.f;
      a1 = 0.f;
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) acc = fmaf(-dmm[j], xsum[j], acc);
  return acc;
}

// ---------------------------------------------------------------------------
// Q8_0: dot product of eight blocks (272 bytes = 68 words) of this lane's row
// with xs[0..255]. Block b starts at byte 34 b: a 2-byte scale, then 32 signed
// bytes; b even starts word-aligned, b odd starts at byte 2 of a word.
// Same activation streaming as above.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float q80_chunk_dot(const uint32_t (&c)[68], const float* xs, bool more,
                                               xreg16& xa) {
  float acc = 0.f;
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int h = 0; h < 2 * kQ80ChunkBlocks; ++h) {
    xreg16 xb;
    if (h < 15) GQK_SLOAD16(xb, xs, 64 * (h + 1));
    else if (more) GQK_SLOAD16(xb, xs, 1024);
    const int b = h >> 1;
    const int base = kQ80BlockBytes * b;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int o = base + 2 + 16 * (h & 1) + i;
      const uint32_t w = c[o >> 2];
      const int sel = o & 3;
      const float q = sel == 0 ? sbyte0(w) : sel == 1 ? sbyte1(w) : sel == 2 ? sbyte2(w) : sbyte3(w);
      float& a = (i & 1) ? a1 : a0;
      a = fmaf(q, xa[i], a);
    }
    if (h < 15 || more) {
      GQK_SWAIT_AFTER(xb, a0, a1);
      xa = xb;
    }
    if (h & 1) {
      const float d = (base & 3) ? half_hi(c[base >> 2]) : half_lo(c[base >> 2]);
      acc = fmaf(d, a0 + a1, acc);
      a0 = 0.f;
      a1 = 0.f;
    }
  }
  return acc;
}

// ---------------------------------------------------------------------------
// One wave task: rows [row0, row0 + 64) (valid_rows of them real) x chunks
// [c0, c1) along K. Returns this lane's partial dot product.
// ---------------------------------------------------------------------------
// Sums of x over the 8 sub-blocks of one super-block, from a float4 that lane
// l loaded from xs[4 l .. 4 l + 3] (lanes 8j .. 8j + 7 cover sub-block j):
// butterfly over each group of 8 lanes with DPP, then the 8 group sums are
// read into SGPRs.
__device__ __forceinline__ void q4k_xsums(const float4& q, float (&xsum)[8]) {
  float s = (q.x + q.y) + (q.z + q.w);
  s += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s), 0xB1, 0xF, 0xF, true));  // quad_perm 1,0,3,2
  s += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s), 0x4E, 0xF, 0xF, true));  // quad_perm 2,3,0,1
  s += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s), 0x12C, 0xF, 0xF, true)); // row_ror:12
#pragma unroll
  for (int j = 0; j < 8; ++j)
    xsum[j] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s), 8 * j));
}

template <int kSlots>
__device__ __forceinline__ float q4k_wave_task(const uint8_t* __restrict__ W, const float* x,
                                               uint32_t row_bytes, int64_t row0, int valid_rows,
                                               int c0, int c1, uint8_t* slots, int lane) {
  const uint8_t* tile = W + row0 * (int64_t)row_bytes;
  uint32_t off[9];
  dma_offsets<9, kQ4KBlockBytes>(lane, row_bytes, valid_rows, off);
  const int n = c1 - c0;
  const float* xs0 = x + (int64_t)c0 * kQ4KBlockWeights;
  // Issue order per super-block i: the float4 of x for its sub-block sums,
  // then its 9 direct loads. Waiting for chunk i therefore also covers its x.
  float4 xq = reinterpret_cast<const float4*>(xs0)[lane];
#pragma unroll
  for (int p = 0; p < kSlots; ++p)
    if (p < n) dma_chunk<9>(tile + (c0 + p) * kQ4KBlockBytes, off, slots + p * kQ4KChunk);
  float acc = 0.f;
  xreg16 xa;
  sload_first_with_touch(xa, xs0);
  for (int i = 0; i < n; ++i) {
    uint8_t* slot = slots + (i % kSlots) * kQ4KChunk;
    // with two slots, chunk i+1's 9 loads (issued after x of i) may stay in flight
    if (kSlots >= 2 && i + 1 < n) GQK_WAIT_VMCNT(9);
    else GQK_WAIT_VMCNT(0);
    uint32_t c[36];
    lds_read_9x16(lds_addr(slot + lane * kQ4KBlockBytes), c);
    float xsum[8];
    q4k_xsums(xq, xsum);
    if (i + 1 < n) xq = reinterpret_cast<const float4*>(xs0 + (int64_t)(i + 1) * kQ4KBlockWeights)[lane];
    if (i + kSlots < n) dma_chunk<9>(tile + (c0 + i + kSlots) * kQ4KBlockBytes, off, slot);
    acc += q4k_superblock_dot(c, xs0 + (int64_t)i * kQ4KBlockWeights, i + 1 < n, xa, xsum);
  }
  return acc;
}

template <int kSlots>
__device__ __forceinline__ float q80_wave_task(const uint8_t* __restrict__ W, const float* x,
                                               uint32_t row_bytes, int64_t row0, int valid_rows,
                                               int c0, int c1, uint8_t* slots, int lane) {
  const uint8_t* tile = W + row0 * (int64_t)row_bytes;
  uint32_t off[17];
  dma_offsets<17, kQ80ChunkRowBytes>(lane, row_bytes, valid_rows, off);
  const int n = c1 - c0;
  float acc = 0.f;
#pragma unroll
  for (int p = 0; p < kSlots; ++p)
    if (p < n) dma_chunk<17>(tile + (c0 + p) * kQ80ChunkRowBytes, off, slots + p * kQ80Chunk);
  const float* xs0 = x + (int64_t)c0 * 256;
  xreg16 xa;
  sload_first_with_touch(xa, xs0);
  for (int i = 0; i < n; ++i) {
    uint8_t* slot = slots + (i % kSlots) * kQ80Chunk;
    if (kSlots >= 2 && i + 1 < n) GQK_WAIT_VMCNT(17);
    else GQK_WAIT_VMCNT(0);
    uint32_t c[68];
    lds_read_17x16(lds_addr(slot + lane * kQ80ChunkRowBytes), c);
    if (i + kSlots < n) dma_chunk<17>(tile + (c0 + i + kSlots) * kQ80ChunkRowBytes, off, slot);
    acc += q80_chunk_dot(c, xs0 + (int64_t)i * 256, i + 1 < n, xa);
  }
  return acc;
}


// v: this lane's final sum for row row0 + lane (lanes >= valid hold garbage).
// Called by the whole wave (wave-uniform control flow). kEp false: plain store
// (the launch has no epilogue; nothing of it is compiled in).
template <bool kEp>
__device__ __forceinline__ void finish_rows(const GemvEpilogue& ep, float v, float* __restrict__ y,
                                            int64_t row0, int valid, int rg, int lane) {
  const int flags = kEp ? ep.flags : 0;
  if (flags == 0) {
    if (lane < valid) y[row0 + lane] = v;
    return;
  }
  const bool live = lane < valid;
  const int64_t r = row0 + (live ? lane : 0);
  if (flags & kEpScale) {
    // the partial sums (or, kEpScaleV, the squares of v) in order, eight
    // loads in flight at a time
    const bool sq = (flags & kEpScaleV) != 0;
    float S = 0.f;
    const int n = ep.scale_n;
    for (int i0 = 0; i0 < n; i0 += 8) {
      float t[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) t[i] = ep.scale_ss[(i0 + i) < n ? (i0 + i) : (n - 1)];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i0 + i < n) S += sq ? t[i] * t[i] : t[i];
    }
    v *= 1.0f / sqrtf(S * ep.inv_k + ep.eps);
  }
  if ((flags & kEpResidual) && live) v += ep.residual[r];
  if (live) {
    if (flags & kEpPair)
      __hip_atomic_store(&y[r], v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      y[r] = v;
  }
  if ((flags & kEpNorm) && live) ep.norm_out[r] = v * ep.norm_w[r];
  if (flags & kEpSs) {
    // the square rounded on its own (kept out of the butterfly's first add,
    // which could otherwise take it unrounded as an fma): the same bits as the
    // standalone preparation kernel
    float sq = live ? v * v : 0.f;
    asm volatile("" : "+v"(sq));
    const float ss = wave_sum_fixed(sq);
    if (lane == 0) ep.ss_out[rg] = ss;
  }
  if (flags & kEpPair) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    GQK_WAIT_VMCNT(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    int old = 0;
    if (lane == 0)
      old = __hip_atomic_fetch_add(&ep.pair_cnt[rg * kCounterStride], 1, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
    old = __builtin_amdgcn_readfirstlane(old);
    if (old == 1) {
      if (live) {
        const float o = __hip_atomic_load(&ep.partner_y[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const float gv = ep.role == 0 ? v : o, uv = ep.role == 0 ? o : v;
        ep.act[r] = gv / (1.0f + expf(-gv)) * uv;
      }
      if (lane == 0)
        __hip_atomic_store(&ep.pair_cnt[rg * kCounterStride], 0, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Store this lane's partial; the last of the P waves of the row group sums
// them in order 0..P-1 and hands the sums to finish_rows. Wave-uniform
// control flow.
//
// Hand-off between waves on different XCDs without L2-wide write-back or
// invalidation: partials are written and read with agent-scope atomic
// accesses, which bypass the per-XCD L2's non-coherent lines, and the
// counter increment is issued only after the partial stores have completed
// (vmcnt(0)); the last arriver's loads are issued after its increment returned.
template <bool kEp>
__device__ __forceinline__ void splitk_finish(float acc, float* __restrict__ y, int64_t rows,
                                              int64_t row0, int valid_rows, int rg, int part,
                                              int P, const SplitK& sk, int lane,
                                              const GemvEpilogue& ep) {
  if (P == 1) {
    finish_rows<kEp>(ep, acc, y, row0, valid_rows, rg, lane);
    return;
  }
  if (lane < valid_rows)
    __hip_atomic_store(&sk.partials[(int64_t)part * rows + row0 + lane], acc, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  GQK_WAIT_VMCNT(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  int old = 0;
  if (lane == 0)
    old = __hip_atomic_fetch_add(&sk.counters[rg * kCounterStride], 1, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
  old = __builtin_amdgcn_readfirstlane(old);
  if (old == P - 1) {
    float s = 0.f;
    if (lane < valid_rows) {
      // eight loads in flight at a time (indexes past P repeat the last
      // partial and are not added), added strictly in order 0..P-1
      for (int p0 = 0; p0 < P; p0 += 8) {
        const float* pp[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int p = (p0 + i) < P ? (p0 + i) : (P - 1);
          pp[i] = &sk.partials[(int64_t)p * rows + row0 + lane];
        }
        float v[8];
        coherent_load8(pp, v);
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (p0 + i < P) s += v[i];
      }
    }
    finish_rows<kEp>(ep, s, y, row0, valid_rows, rg, lane);
    if (lane == 0)
      __hip_atomic_store(&sk.counters[rg * kCounterStride], 0, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---------------------------------------------------------------------------
// GEMV kernels over a group of up to kMaxGroup same-format GEMVs (one GEMV, or
// the GEMVs of one decode stage that read the same input, such as q/k/v).
// ---------------------------------------------------------------------------
constexpr int kGemvWaves = 4;      // per-wave task kernel (Q8_0)
constexpr int kBlockWaves = 8;     // block task kernel (Q4_K)
constexpr int kMaxGroup = 4;

struct GemvDesc {
  const uint8_t* W;
  const float* x;
  float* y;
  int64_t rows;
  int64_t task_end;    // tasks of GEMVs 0..g, cumulative
  int64_t part_off;    // this GEMV's partial sums in scratch (floats)
  int nchunks;         // per row: super-blocks (Q4_K) or 8-block chunks (Q8_0)
  int P;               // K ranges per row group
  int cnt_off;         // this GEMV's row-group counters in scratch
  int pad;
};

struct GemvGroup {
  GemvDesc d[kMaxGroup];
  int n;
  GemvEpilogue ep[kMaxGroup];   // read only by the wave that finishes a row group
};

// Task t of a group: which GEMV (g) and its descriptor. Kernel arguments live
// in a buffer that is new, hence cold, at every launch; indexing d[] with a
// computed g would make the descriptor loads wait for the task_end loads. All
// kMaxGroup descriptors are therefore read at fixed offsets (one batch of
// scalar loads) and g picks among them with selects.
template <class T>
__device__ __forceinline__ T pick4(int g, T a0, T a1, T a2, T a3) {
  return g == 0 ? a0 : g == 1 ? a1 : g == 2 ? a2 : a3;
}

__device__ __forceinline__ int64_t group_tasks(const GemvDesc (&d)[kMaxGroup], int n) {
  return pick4(n - 1, d[0].task_end, d[1].task_end, d[2].task_end, d[3].task_end);
}

__device__ __forceinline__ void pick_desc(const GemvDesc (&d)[kMaxGroup], int n, int64_t t,
                                          int* g_out, int64_t* lt_out, GemvDesc* out) {
  const int g = (n > 1 && t >= d[0].task_end) + (n > 2 && t >= d[1].task_end) +
                (n > 3 && t >= d[2].task_end);
  const int64_t before = pick4<int64_t>(g, 0, d[0].task_end, d[1].task_end, d[2].task_end);
  out->W = pick4(g, d[0].W, d[1].W, d[2].W, d[3].W);
  out->x = pick4(g, d[0].x, d[1].x, d[2].x, d[3].x);
  out->y = pick4(g, d[0].y, d[1].y, d[2].y, d[3].y);
  out->rows = pick4(g, d[0].rows, d[1].rows, d[2].rows, d[3].rows);
  out->task_end = pick4(g, d[0].task_end, d[1].task_end, d[2].task_end, d[3].task_end);
  out->part_off = pick4(g, d[0].part_off, d[1].part_off, d[2].part_off, d[3].part_off);
  out->nchunks = pick4(g, d[0].nchunks, d[1].nchunks, d[2].nchunks, d[3].nchunks);
  out->P = pick4(g, d[0].P, d[1].P, d[2].P, d[3].P);
  out->cnt_off = pick4(g, d[0].cnt_off, d[1].cnt_off, d[2].cnt_off, d[3].cnt_off);
  *g_out = g;
  *lt_out = t - before;
}

// Copies the group's descriptors and count out of the kernel arguments in one
// batch of scalar loads: the empty asm consumes every loaded word, so no load
// can be sunk behind a branch that depends on another load.
__device__ __forceinline__ void load_group(const GemvGroup& grp, GemvDesc (&dl)[kMaxGroup],
                                           int* n) {
  typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));
  u32x16 w[kMaxGroup];
#pragma unroll
  for (int k = 0; k < kMaxGroup; ++k) w[k] = *reinterpret_cast<const u32x16*>(&grp.d[k]);
  int cnt = grp.n;
  asm volatile("" : "+s"(w[0]), "+s"(w[1]), "+s"(w[2]), "+s"(w[3]), "+s"(cnt));
#pragma unroll
  for (int k = 0; k < kMaxGroup; ++k) dl[k] = __builtin_bit_cast(GemvDesc, w[k]);
  *n = cnt;
}

// Per-wave tasks (each wave one row group x K range). Used for Q8_0.
template <int kSlots, bool kQ4K, bool kEp>
__global__ __launch_bounds__(kGemvWaves * 64) void gemv_group_kernel(GemvGroup grp, float* partials,
                                                                    int* counters) {
  constexpr int kChunk = kQ4K ? kQ4KChunk : kQ80Chunk;
  constexpr int kRowSeg = kQ4K ? kQ4KBlockBytes : kQ80ChunkRowBytes;
  __shared__ __attribute__((aligned(16))) uint8_t slots[kGemvWaves][kSlots * kChunk];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t T = grp.d[grp.n - 1].task_end;
  for (int64_t t = (int64_t)blockIdx.x * kGemvWaves + wave; t < T;
       t += (int64_t)gridDim.x * kGemvWaves) {
    int g = 0;
    while (g + 1 < grp.n && t >= grp.d[g].task_end) ++g;
    const GemvDesc& D = grp.d[g];
    const int64_t lt = t - (g ? grp.d[g - 1].task_end : 0);
    const int P = D.P;
    const int rg = (int)(lt / P), part = (int)(lt % P);
    const int n = D.nchunks;
    const int c0 = (int)((int64_t)part * n / P), c1 = (int)((int64_t)(part + 1) * n / P);
    const int64_t row0 = (int64_t)rg * 64;
    const int valid = (int)((D.rows - row0) < 64 ? (D.rows - row0) : 64);
    const uint32_t row_bytes = (uint32_t)n * kRowSeg;
    float acc;
    if constexpr (kQ4K)
      acc = q4k_wave_task<kSlots>(D.W, D.x, row_bytes, row0, valid, c0, c1, &slots[wave][0], lane);
    else
      acc = q80_wave_task<kSlots>(D.W, D.x, row_bytes, row0, valid, c0, c1, &slots[wave][0], lane);
    const SplitK sk{partials + D.part_off, counters + (int64_t)D.cnt_off * kCounterStride};
    splitk_finish<kEp>(acc, D.y, D.rows, row0, valid, rg, part, P, sk, lane, grp.ep[g]);
  }
}

// Block tasks for Q4_K: block t (one per task) has kBlockWaves waves and owns
// one row group and a range of up to kBlockWaves super-blocks along K, one per
// wave. The waves' 64 partial sums are added in LDS in wave order; a row group
// whose K is cut into P > 1 ranges (K > kBlockWaves super-blocks) finishes
// through the split-K hand-off between blocks.
template <bool kEp>
__global__ __launch_bounds__(kBlockWaves * 64) void gemv_q4k_block_kernel(GemvGroup grp,
                                                                          float* partials,
                                                                          int* counters) {
  __shared__ __attribute__((aligned(16))) uint8_t slots[kBlockWaves][kQ4KChunk];
  __shared__ float red[kBlockWaves][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t t = blockIdx.x;
  GemvDesc dl[kMaxGroup];
  int ng;
  load_group(grp, dl, &ng);
  int g;
  int64_t lt;
  GemvDesc D;
  pick_desc(dl, ng, t, &g, &lt, &D);
  const int P = D.P;
  const int rg = (int)(lt / P), part = (int)(lt % P);
  const int n = D.nchunks;
  const int c0 = (int)((int64_t)part * n / P), c1 = (int)((int64_t)(part + 1) * n / P);
  const int64_t row0 = (int64_t)rg * 64;
  const int valid = (int)((D.rows - row0) < 64 ? (D.rows - row0) : 64);
  const uint32_t row_bytes = (uint32_t)n * kQ4KBlockBytes;
  // wave w takes super-block c0 + w (a range holds at most kBlockWaves)
  float acc = 0.f;
  const int c = c0 + wave;
  if (c < c1) {
    uint8_t* slot = &slots[wave][0];
    uint32_t off[9];
    dma_offsets<9, kQ4KBlockBytes>(lane, row_bytes, valid, off);
    const float* xs = D.x + (int64_t)c * kQ4KBlockWeights;
    const float4 xq = reinterpret_cast<const float4*>(xs)[lane];
    dma_chunk<9>(D.W + row0 * (int64_t)row_bytes + (int64_t)c * kQ4KBlockBytes, off, slot);
    xreg16 xa;
    sload_first_with_touch(xa, xs);
    GQK_WAIT_VMCNT(0);
    uint32_t cw[36];
    lds_read_9x16(lds_addr(slot + lane * kQ4KBlockBytes), cw);
    float xsum[8];
    q4k_xsums(xq, xsum);
    acc = q4k_superblock_dot(cw, xs, false, xa, xsum);
  }
  red[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kBlockWaves; ++w) s += red[w][lane];
    const SplitK sk{partials + D.part_off, counters + (int64_t)D.cnt_off * kCounterStride};
    splitk_finish<kEp>(s, D.y, D.rows, row0, valid, rg, part, P, sk, lane, grp.ep[g]);
  }
}

// Q8_0 rows whose length is not a multiple of 256 weights (row bytes not a
// multiple of 16): a plain wave-per-row kernel. Lane l takes blocks l, l+64,
// ...; the block's 34 bytes are read as 17 half-words (blocks are 2-byte
// aligned); the wave sums its 64 lane partials with a butterfly.
__global__ __launch_bounds__(256) void gemv_q8_0_rowwise_kernel(const uint8_t* __restrict__ W,
                                                                const float* __restrict__ x,
                                                                float* __restrict__ y,
                                                                int64_t rows, int nblocks) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint8_t* r = W + row * (int64_t)nblocks * kQ80BlockBytes;
  float acc = 0.f;
  for (int b = lane; b < nblocks; b += 64) {
    const uint16_t* h = reinterpret_cast<const uint16_t*>(r + (int64_t)b * kQ80BlockBytes);
    const float d = half_lo(h[0]);
    const float* xb = x + 32 * (int64_t)b;
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t w = h[1 + i];
      a = fmaf(sbyte0(w), xb[2 * i], a);
      a = fmaf(sbyte1(w), xb[2 * i + 1], a);
    }
    acc = fmaf(d, a, acc);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  if (lane == 0) y[row] = acc;
}

}  // namespace gqk
