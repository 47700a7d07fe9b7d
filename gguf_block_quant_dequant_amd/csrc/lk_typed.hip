// The lanes-along-K kernel launches of one block type (and epilogue variant),
// instantiated in a translation unit of its own: this file is compiled once
// per (GQK_LK_TYPE, GQK_LK_EP) pair so that the kernel families build in
// parallel. The launch plan (row length, ring depth, waves per block) comes
// from launch_lk in lk.hip.
#include "launch.hpp"
#include "gemv_lk.hpp"

#ifndef GQK_LK_TYPE
#error "GQK_LK_TYPE (a GGUF type id) must be defined"
#endif
#ifndef GQK_LK_EP
#define GQK_LK_EP 0
#endif

namespace gqk {

// Two GEMVs of one x without epilogues: both descriptors as scalar arguments.
// (The kernel re-forms each GEMV's q and r from its rows and block count, so
// both GEMVs must have blocks.)
static bool lk_two(const LkGroup& grp) {
  return grp.n == 2 && grp.d[0].x == grp.d[1].x && grp.d[1].block_begin > 0 &&
         grp.d[1].block_begin < grp.total_blocks && tuning().lk_two;
}

// Three GEMVs of one x without epilogues, every one with blocks, whose
// packed descriptors fit (see lk_block_three).
struct Lk3Args {
  int dW1, dW2, dy1, dy2, rows12, bb12;
};
static bool fits_i32(int64_t v) { return v >= INT32_MIN && v <= INT32_MAX; }
static bool lk_three(const LkGroup& grp, Lk3Args* a) {
  if (grp.n != 3 || !tuning().lk_three) return false;
  const LkDesc *d = grp.d;
  if (d[1].x != d[0].x || d[2].x != d[0].x) return false;
  const int bb1 = d[1].block_begin, bb2 = d[2].block_begin;
  if (!(0 < bb1 && bb1 < bb2 && bb2 < grp.total_blocks && bb2 < 65536)) return false;
  if (d[1].rows >= 65536 || d[2].rows >= 65536) return false;
  const int64_t w0 = (int64_t)reinterpret_cast<intptr_t>(d[0].W);
  const int64_t dW1 = (int64_t)reinterpret_cast<intptr_t>(d[1].W) - w0;
  const int64_t dW2 = (int64_t)reinterpret_cast<intptr_t>(d[2].W) - w0;
  const int64_t y0 = (int64_t)reinterpret_cast<intptr_t>(d[0].y);
  const int64_t by1 = (int64_t)reinterpret_cast<intptr_t>(d[1].y) - y0;
  const int64_t by2 = (int64_t)reinterpret_cast<intptr_t>(d[2].y) - y0;
  // offsets in 16-byte units
  if ((w0 | dW1 | dW2 | y0 | by1 | by2) & 15) return false;
  if (!fits_i32(dW1 / 16) || !fits_i32(dW2 / 16) || !fits_i32(by1 / 16) || !fits_i32(by2 / 16)) return false;
  a->dW1 = (int)(dW1 / 16);
  a->dW2 = (int)(dW2 / 16);
  a->dy1 = (int)(by1 / 16);
  a->dy2 = (int)(by2 / 16);
  a->rows12 = (int)((uint32_t)d[1].rows | ((uint32_t)d[2].rows << 16));
  a->bb12 = (int)((uint32_t)bb1 | ((uint32_t)bb2 << 16));
  return true;
}

template <int kType, int kNsb, int kW>
static void launch_lk3(const LkGroup& grp, const Lk3Args& a, int depth, hipStream_t stream) {
  const dim3 grid((unsigned)grp.total_blocks), block(kW * 64);
  const LkDesc& d = grp.d[0];
  if (depth <= 2)
    hipLaunchKernelGGL((gemv_lk3_kernel<kType, kNsb, 2, kW>), grid, block, 0, stream, d.W, a.dW1, a.dW2, d.x,
                       d.y, a.dy1, a.dy2, d.rows, a.rows12, a.bb12, grp.total_blocks);
  else
    hipLaunchKernelGGL((gemv_lk3_kernel<kType, kNsb, 4, kW>), grid, block, 0, stream, d.W, a.dW1, a.dW2, d.x,
                       d.y, a.dy1, a.dy2, d.rows, a.rows12, a.bb12, grp.total_blocks);
}

template <int kNsb, int kW>
static void launch_lk3e(const LkGroup& grp, const Lk3Args& a, int depth, hipStream_t stream) {
  const dim3 grid((unsigned)grp.total_blocks), block(kW * 64);
  const LkDesc& d = grp.d[0];
  LkEp3 ep;
  for (int i = 0; i < 3; ++i) ep.e[i] = grp.ep[i];
  if (depth <= 2)
    hipLaunchKernelGGL((gemv_lk3e_kernel<kNsb, 2, kW>), grid, block, 0, stream, d.W, a.dW1, a.dW2, d.x, d.y,
                       a.dy1, a.dy2, d.rows, a.rows12, a.bb12, grp.total_blocks, ep);
  else
    hipLaunchKernelGGL((gemv_lk3e_kernel<kNsb, 4, kW>), grid, block, 0, stream, d.W, a.dW1, a.dW2, d.x, d.y,
                       a.dy1, a.dy2, d.rows, a.rows12, a.bb12, grp.total_blocks, ep);
}

template <int kType, int kNsb, int kW>
static void launch_lk2(const LkGroup& grp, int depth, hipStream_t stream) {
  const dim3 grid((unsigned)grp.total_blocks), block(kW * 64);
  const LkDesc &a = grp.d[0], &b = grp.d[1];
  if (depth <= 2)
    hipLaunchKernelGGL((gemv_lk2_kernel<kType, kNsb, 2, kW>), grid, block, 0, stream, a.W, b.W, a.x, a.y, b.y,
                       a.rows, b.rows, b.block_begin, grp.total_blocks - b.block_begin);
  else
    hipLaunchKernelGGL((gemv_lk2_kernel<kType, kNsb, 4, kW>), grid, block, 0, stream, a.W, b.W, a.x, a.y, b.y,
                       a.rows, b.rows, b.block_begin, grp.total_blocks - b.block_begin);
}

// One launch of the lanes-along-K kernels for rows of 256 kNsb weights of
// type kType: one GEMV, two of one x, or a group from the descriptors.
template <int kType, int kNsb, int kW, bool kEp>
static void launch_lk_nsb(const LkGroup& grp, int depth, hipStream_t stream) {
  const dim3 grid((unsigned)grp.total_blocks), block(kW * 64);
  if (kEp && grp.n == 1 && tuning().lk_single) {
    // one GEMV with an epilogue (the output projection: residual add, norm
    // preparation): descriptor and epilogue flags preloaded
    if constexpr (kEp && kType == GGUF_QK_TYPE_Q4_K) {
      g_last_launch = GGUF_QK_LAUNCH_LK_SINGLE;
      const LkDesc& d = grp.d[0];
      const GemvEpilogue& ep = grp.ep[0];
      if (depth <= 2)
        hipLaunchKernelGGL((gemv_lk1e_kernel<kNsb, 2, kW>), grid, block, 0, stream, d.W, d.x, d.y, d.rows, d.q,
                           d.r, ep.flags, ep.scale_n, ep.scale_ss, ep);
      else
        hipLaunchKernelGGL((gemv_lk1e_kernel<kNsb, 4, kW>), grid, block, 0, stream, d.W, d.x, d.y, d.rows, d.q,
                           d.r, ep.flags, ep.scale_n, ep.scale_ss, ep);
      return;
    }
  }
  if (kEp && grp.n == 2 && (grp.ep[0].flags & kEpPairInWave) && tuning().lk_two) {
    // a gate/up pair in one wave: both descriptors preloaded
    if constexpr (kEp && kType == GGUF_QK_TYPE_Q4_K) {
      g_last_launch = GGUF_QK_LAUNCH_LK_TWO;
      const LkDesc& d0 = grp.d[0];
      const LkDesc& d1 = grp.d[1];
      if (depth <= 2)
        hipLaunchKernelGGL((gemv_lk2e_kernel<kNsb, 2, kW>), grid, block, 0, stream, d0.W, d1.W, d0.x, d0.y, d1.y,
                           d0.rows, d0.q, d0.r, grp.ep[0]);
      else
        hipLaunchKernelGGL((gemv_lk2e_kernel<kNsb, 4, kW>), grid, block, 0, stream, d0.W, d1.W, d0.x, d0.y, d1.y,
                           d0.rows, d0.q, d0.r, grp.ep[0]);
      return;
    }
  }
  if (!kEp && grp.n == 1 && tuning().lk_single) {
    g_last_launch = GGUF_QK_LAUNCH_LK_SINGLE;
    const LkDesc& d = grp.d[0];
    if (depth <= 2)
      hipLaunchKernelGGL((gemv_lk1_kernel<kType, kNsb, 2, kW>), grid, block, 0, stream, d.W, d.x, d.y,
                         d.rows, d.q, d.r);
    else
      hipLaunchKernelGGL((gemv_lk1_kernel<kType, kNsb, 4, kW>), grid, block, 0, stream, d.W, d.x, d.y,
                         d.rows, d.q, d.r);
    return;
  }
  if (!kEp && lk_two(grp)) {
    g_last_launch = GGUF_QK_LAUNCH_LK_TWO;
    launch_lk2<kType, kNsb, kW>(grp, depth, stream);
    return;
  }
  Lk3Args a3;
  if (kEp && !(grp.ep[0].flags & kEpPairInWave) && !(grp.ep[1].flags & kEpPairInWave) && lk_three(grp, &a3)) {
    // three GEMVs of one x with epilogues (the fused q/k/v)
    if constexpr (kEp && kType == GGUF_QK_TYPE_Q4_K) {
      g_last_launch = GGUF_QK_LAUNCH_LK_THREE;
      launch_lk3e<kNsb, kW>(grp, a3, depth, stream);
      return;
    }
  }
  if (!kEp && lk_three(grp, &a3)) {
    g_last_launch = GGUF_QK_LAUNCH_LK_THREE;
    launch_lk3<kType, kNsb, kW>(grp, a3, depth, stream);
    return;
  }
  g_last_launch = GGUF_QK_LAUNCH_LK_GROUP;
  if (depth <= 2)
    hipLaunchKernelGGL((gemv_lk_kernel<kType, kNsb, 2, kW, kEp>), grid, block, 0, stream, grp);
  else
    hipLaunchKernelGGL((gemv_lk_kernel<kType, kNsb, 4, kW, kEp>), grid, block, 0, stream, grp);
}

template <int kType, bool kEp, int kQ, int kW>
static void launch_lkx_t(const LkGroup& grp, size_t lds, hipStream_t stream) {
  g_last_launch = GGUF_QK_LAUNCH_LK_LONG;
  const dim3 grid((unsigned)grp.total_blocks), block(kW * 64);
  // one GEMV without epilogue: its descriptor as (preloaded) scalar arguments
  const bool single = grp.n == 1 && !kEp && tuning().lk_single;
  const LkDesc& d = grp.d[0];
  const uint8_t* W = single ? d.W : nullptr;
  const float* x = single ? d.x : nullptr;
  float* y = single ? d.y : nullptr;
  const int rows = single ? d.rows : 0, q = single ? d.q : 0, r = single ? d.r : 0;
  const int nsb = single ? d.nsb : 0;
  if constexpr (kType == GGUF_QK_TYPE_Q6_K && kQ == 3 && kW == 8) {
    return;   // three rounds of Q6_K quarters run in 4-wave blocks only (the plan never asks)
  } else if constexpr (kEp) {
    hipLaunchKernelGGL((gemv_lkx_kernel<kType, kQ, 2, kW, true, false>), grid, block, lds, stream, W, x, y,
                       rows, q, r, nsb, grp);
  } else {
    if (single)
      hipLaunchKernelGGL((gemv_lkx_kernel<kType, kQ, 2, kW, false, true>), grid, block, lds, stream, W, x, y,
                         rows, q, r, nsb, grp);
    else
      hipLaunchKernelGGL((gemv_lkx_kernel<kType, kQ, 2, kW, false, false>), grid, block, lds, stream, W, x, y,
                         rows, q, r, nsb, grp);
  }
}

template <int kType, bool kEp, int kNsb>
static void launch_lk_nsb_t(const LkGroup& grp, int depth, int bw, hipStream_t stream) {
  if constexpr (kType == GGUF_QK_TYPE_Q4_K && !kEp) {
    if (bw == 8) {
      launch_lk_nsb<kType, kNsb, 8, false>(grp, depth, stream);
      return;
    }
  }
  launch_lk_nsb<kType, kNsb, 4, kEp>(grp, depth, stream);
}

template <int kType, bool kEp>
void launch_lk_typed(const LkGroup& grp, const LkPlan& p, hipStream_t stream) {
  if (p.longrow) {
    if constexpr (kType != GGUF_QK_TYPE_Q8_0) {
      const int kq = (4 * p.nsb + 63) / 64;
      if (p.bw == 8) {
        if (kq == 2)
          launch_lkx_t<kType, kEp, 2, 8>(grp, p.lds, stream);
        else
          launch_lkx_t<kType, kEp, 3, 8>(grp, p.lds, stream);
      } else {
        if (kq == 2)
          launch_lkx_t<kType, kEp, 2, 4>(grp, p.lds, stream);
        else
          launch_lkx_t<kType, kEp, 3, 4>(grp, p.lds, stream);
      }
    }
    return;
  }
  switch (p.nsb) {
    case 1: launch_lk_nsb_t<kType, kEp, 1>(grp, p.depth, p.bw, stream); break;
    case 2: launch_lk_nsb_t<kType, kEp, 2>(grp, p.depth, p.bw, stream); break;
    case 4: launch_lk_nsb_t<kType, kEp, 4>(grp, p.depth, p.bw, stream); break;
    case 8: launch_lk_nsb_t<kType, kEp, 8>(grp, p.depth, p.bw, stream); break;
    default: launch_lk_nsb_t<kType, kEp, 16>(grp, p.depth, p.bw, stream); break;
  }
}

template void launch_lk_typed<GQK_LK_TYPE, (GQK_LK_EP != 0)>(const LkGroup&, const LkPlan&, hipStream_t);

template <int kType, int kDepth, bool kSingle, int kRps, bool kEp>
static void launch_lks_k(const LksGroup& grp, const GemvEpilogue& ep, int nsb, int R, int nw, int blocks,
                         hipStream_t stream) {
  g_last_launch = GGUF_QK_LAUNCH_LKS;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&gemv_lks_kernel<kType, kDepth, kSingle, kRps, kEp>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lks_lds_bytes(kRps, lks_max_waves(kRps), kLksMaxRows));
  (void)attr;
  const LksDesc& d = grp.d[0];
  hipLaunchKernelGGL((gemv_lks_kernel<kType, kDepth, kSingle, kRps, kEp>), dim3((unsigned)blocks),
                     dim3(64 * nw), lks_lds_bytes(kRps, nw, R), stream, d.W, grp.x, d.y, d.rows, nsb, R, nw,
                     grp, ep);
}

template <int kType, int kRps>
static void launch_lks_r(const LksGroup& grp, const GemvEpilogue* ep, int nsb, int R, int nw, int depth,
                         int blocks, hipStream_t stream) {
  const GemvEpilogue none{};
  if (grp.n == 1 && ep) {
    // (the host takes this path for one Q4_K GEMV only)
    if constexpr (kType == GGUF_QK_TYPE_Q4_K) {
      if (depth <= 2)
        launch_lks_k<kType, 2, true, kRps, true>(grp, *ep, nsb, R, nw, blocks, stream);
      else
        launch_lks_k<kType, 4, true, kRps, true>(grp, *ep, nsb, R, nw, blocks, stream);
    }
  } else if (grp.n == 1) {
    if (depth <= 2)
      launch_lks_k<kType, 2, true, kRps, false>(grp, none, nsb, R, nw, blocks, stream);
    else
      launch_lks_k<kType, 4, true, kRps, false>(grp, none, nsb, R, nw, blocks, stream);
  } else {
    if (depth <= 2)
      launch_lks_k<kType, 2, false, kRps, false>(grp, none, nsb, R, nw, blocks, stream);
    else
      launch_lks_k<kType, 4, false, kRps, false>(grp, none, nsb, R, nw, blocks, stream);
  }
}

template <int kType>
void launch_lks_typed(const LksGroup& grp, const GemvEpilogue* ep, int nsb, int R, int nw, int rps, int depth,
                      int blocks, hipStream_t stream) {
  if constexpr (kType == GGUF_QK_TYPE_Q4_K || kType == GGUF_QK_TYPE_Q4_0) {
    if (rps == 4)
      launch_lks_r<kType, 4>(grp, ep, nsb, R, nw, depth, blocks, stream);
    else if (rps == 2)
      launch_lks_r<kType, 2>(grp, ep, nsb, R, nw, depth, blocks, stream);
    else
      launch_lks_r<kType, 1>(grp, ep, nsb, R, nw, depth, blocks, stream);
  }
}

#if GQK_LK_EP == 0
template void launch_lks_typed<GQK_LK_TYPE>(const LksGroup&, const GemvEpilogue*, int, int, int, int, int, int,
                                            hipStream_t);
#endif

}  // namespace gqk
