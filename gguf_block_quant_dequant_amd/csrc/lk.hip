// Lanes-along-K GEMV launch plans (kernels in gemv_lk.hpp): blocks per GEMV,
// ring depth and waves per block; the launch itself is in lk_typed.hip, one
// translation unit per block type.
#include "launch.hpp"
#include "gemv_lk.hpp"

namespace gqk {

// Q4_K GEMVs whose rows hold 1, 2, 4, 8 or 16 super-blocks (lanes hold x), or
// 17 to 48 (x read from LDS), all the same: the lanes-along-K kernels take
// them, with any epilogue except norm preparation and a gate/up pair together
// on one GEMV, and at most 256 partial sums for an input RMSN (or the input
// vector itself, rows of at most 16 super-blocks).
bool lk_fits(const gguf_qk_gemv* const* v, const GemvEpilogue* const* e, int n) {
  const int64_t c = v[0]->cols;
  if (c % 256 || (c != 256 && c != 512 && c != 1024 && c != 2048 && c != 4096 && (c <= 4096 || c > kLkxMaxK)))
    return false;
  for (int i = 0; i < n; ++i) {
    if (v[i]->cols != c || v[i]->rows > (int64_t(1) << 30)) return false;
    if (e && e[i]) {
      const int f = e[i]->flags;
      if ((f & kEpNorm) && (f & kEpPair)) return false;
      if ((f & kEpScale) && !(f & kEpScaleV) && e[i]->scale_n > 256) return false;
      if ((f & kEpScaleV) && c > 4096) return false;
      if ((f & kEpSs) && !e[i]->norm_cnt) return false;
    }
  }
  return true;
}

// Q4_K or Q4_0 GEMVs whose rows the kernels above do not take as they are (a
// number of super-blocks other than 1, 2, 4, 8, 16, up to 128): the
// split-K-in-block kernel. Epilogues: one Q4_K GEMV with a residual add and
// norm preparation (row-group counters assigned for the partial sums), nothing else.
bool lks_fits(const gguf_qk_gemv* const* v, const GemvEpilogue* const* e, int n, int type) {
  if (type != GGUF_QK_TYPE_Q4_K && type != GGUF_QK_TYPE_Q4_0) return false;
  const int64_t c = v[0]->cols;
  if (c % 256) return false;
  const int64_t nsb = c / 256;
  if (nsb > kLksMaxNsb || nsb == 1 || nsb == 2 || nsb == 4 || nsb == 8 || nsb == 16) return false;
  for (int i = 0; i < n; ++i) {
    if (v[i]->cols != c || v[i]->rows > (int64_t(1) << 30)) return false;
    if (e && e[i] && e[i]->flags) {
      const int f = e[i]->flags;
      if (n != 1 || type != GGUF_QK_TYPE_Q4_K || (f & ~(kEpResidual | kEpNorm | kEpSs))) return false;
      if ((f & kEpSs) && !e[i]->norm_cnt) return false;
    }
  }
  return true;
}

// The split of a launch: rows per step (rps), waves per block (nw). Cost =
// row steps per SIMD (waves on the busiest SIMD times steps per wave; a SIMD
// runs its waves' steps one after another), ties to fewer waves.
static void lks_shape(int nsb, int R, int* rps_out, int* nw_out) {
  int best = -1, brps = 2, bnw = 1;
  for (int rps : {4, 2, 1}) {
    const int ms = lks_max_slice(rps);
    for (int nw = (nsb + ms - 1) / ms; nw <= lks_max_waves(rps); ++nw) {
      if (nw > nsb) break;
      const int cost = ((nw + 3) / 4) * ((R + rps - 1) / rps);
      if (best < 0 || cost < best || (cost == best && nw < bnw)) {
        best = cost;
        brps = rps;
        bnw = nw;
      }
    }
  }
  *rps_out = brps;
  *nw_out = bnw;
}

// One launch per run of GEMVs of one x (at most kLkMaxGroup): each block takes
// R rows of one GEMV, R a multiple of 4 chosen so that the launch has about
// one block per compute unit (at most kLksMaxRows).
int launch_lks(const gguf_qk_gemv* const* v, const GemvEpilogue* const* e, int n, hipStream_t stream,
               int type) {
  const int nsb = (int)(v[0]->cols / 256);
  for (int i0 = 0; i0 < n;) {
    int i1 = i0 + 1;
    while (i1 < n && v[i1]->x == v[i0]->x) ++i1;
    int64_t total = 0;
    for (int i = i0; i < i1; ++i) total += v[i]->rows;
    int64_t R = 4 * ((total + 4 * 256 - 1) / (4 * 256));   // whole steps of 1, 2 or 4 rows
    if (R > kLksMaxRows) R = kLksMaxRows;
    int rps = 2, nw = 1;
    lks_shape(nsb, (int)R, &rps, &nw);
    LksGroup grp{};
    grp.x = v[i0]->x;
    grp.n = i1 - i0;
    int64_t blocks = 0;
    for (int i = i0; i < i1; ++i) {
      LksDesc& d = grp.d[i - i0];
      d.W = static_cast<const uint8_t*>(v[i]->W);
      d.y = v[i]->y;
      d.rows = (int)v[i]->rows;
      d.block_begin = (int)blocks;
      blocks += (v[i]->rows + R - 1) / R;
    }
    if (blocks > INT32_MAX) return GGUF_QK_ERR_LIMIT;
    const int depth = R / rps <= 2 ? 2 : 4;
    // an epilogue only on a run of one GEMV (lks_fits)
    const GemvEpilogue* ep = (e && i1 - i0 == 1 && e[i0] && e[i0]->flags) ? e[i0] : nullptr;
    if (type == GGUF_QK_TYPE_Q4_0)
      launch_lks_typed<GGUF_QK_TYPE_Q4_0>(grp, nullptr, nsb, (int)R, nw, rps, depth, (int)blocks, stream);
    else
      launch_lks_typed<GGUF_QK_TYPE_Q4_K>(grp, ep, nsb, (int)R, nw, rps, depth, (int)blocks, stream);
    const int st = launch_status();
    if (st) return st;
    i0 = i1;
  }
  return GGUF_QK_OK;
}

// Lanes-along-K launch: blocks go to the GEMVs in proportion to their rows
// (at least one, at most one per row step); a shallow load ring when a wave
// has only a few steps.
int launch_lk(const gguf_qk_gemv* const* v, const GemvEpilogue* const* e, int n,
                     hipStream_t stream, int type) {
  const int nsb = (int)(v[0]->cols / 256);
  const bool longrow = nsb > 16;
  const int rps = longrow ? 1 : 64 / (4 * nsb);
  bool ep = false;
  for (int i = 0; i < n; ++i) ep = ep || (e && e[i] && e[i]->flags != 0);
  int bw = longrow ? tuning().lkx_bw : (ep || type != GGUF_QK_TYPE_Q4_K) ? 4 : tuning().lk_bw;
  // Q6_K rows of three rounds hold 20 words per quarter in the load ring:
  // only 4-wave blocks (512 registers a lane) fit them without scratch
  if (longrow && type == GGUF_QK_TYPE_Q6_K && nsb > 32) bw = 4;
  LkGroup grp{};
  grp.n = n;
  int64_t total_rows = 0;
  for (int i = 0; i < n; ++i) total_rows += v[i]->rows;
  // (Q6_K long rows: two rows per wave halve the x staging of 4-wave blocks)
  const int lkx_waves = type == GGUF_QK_TYPE_Q6_K ? tuning().lkx_waves_q6 : tuning().lkx_waves;
  // (a launch of up to twice the wave target's row steps gets one step per
  // wave, so that no wave runs a second step after the others are done: q+k+v
  // 3.36 -> 3.28 us)
  int64_t target_waves = longrow ? lkx_waves : tuning().lk_waves;
  if (!longrow) {
    int64_t steps = 0;
    for (int i = 0; i < n; ++i) steps += (v[i]->rows + rps - 1) / rps;
    if (steps > target_waves && steps <= 2 * target_waves) target_waves = steps;
  }
  const int64_t target_blocks = (target_waves + bw - 1) / bw;
  // gate/up pairs computed in the same wave (the gate's rows in lanes 0..31,
  // the up's in 32..63): the gate's descriptor takes both matrices' blocks,
  // the up's gets none
  bool in_wave[kLkMaxGroup] = {false, false, false, false};
  for (int i = 0; i + 1 < n; ++i)
    if (!longrow && rps >= 2 && e && e[i] && e[i + 1] && (e[i]->flags & kEpPair) && e[i]->role == 0 &&
        (e[i + 1]->flags & kEpPair) && e[i + 1]->role == 1 &&
        !((e[i]->flags | e[i + 1]->flags) & (kEpNorm | kEpResidual)) &&
        (e[i]->flags & kEpScale) == (e[i + 1]->flags & kEpScale) &&
        e[i]->scale_ss == e[i + 1]->scale_ss && e[i]->scale_n == e[i + 1]->scale_n &&
        e[i]->eps == e[i + 1]->eps && v[i]->x == v[i + 1]->x && v[i + 1]->rows == v[i]->rows &&
        tuning().lk_pair_in_wave)
      in_wave[i] = true;
  // Each GEMV's share of the target block count, rounded down, then the
  // blocks left over to the largest remainders, so that the launch has the
  // target count (one block per compute unit) where the row steps allow.
  int64_t want_of[kLkMaxGroup] = {0, 0, 0, 0}, steps_of[kLkMaxGroup] = {0, 0, 0, 0};
  double frac_of[kLkMaxGroup] = {0, 0, 0, 0};
  int64_t assigned = 0;
  for (int i = 0; i < n; ++i) {
    const bool up_half = i > 0 && in_wave[i - 1];
    const int rpm = in_wave[i] ? rps / 2 : rps;
    steps_of[i] = (v[i]->rows + rpm - 1) / rpm;
    if (up_half) continue;
    const double share = (in_wave[i] ? 2.0 : 1.0) * (double)v[i]->rows / (double)total_rows;
    const double exact = (double)target_blocks * share;
    want_of[i] = (int64_t)exact;
    frac_of[i] = exact - (double)want_of[i];
    if (want_of[i] < 1) {
      want_of[i] = 1;
      frac_of[i] = -1.0;
    }
    if (want_of[i] > steps_of[i]) want_of[i] = steps_of[i];
    assigned += want_of[i];
  }
  while (assigned < target_blocks) {
    int best = -1;
    for (int i = 0; i < n; ++i)
      if (want_of[i] > 0 && want_of[i] < steps_of[i] && (best < 0 || frac_of[i] > frac_of[best])) best = i;
    if (best < 0 || frac_of[best] < 0.0) break;
    ++want_of[best];
    frac_of[best] = -1.0;
    ++assigned;
  }
  int64_t bb = 0, max_wave_steps = 0;
  for (int i = 0; i < n; ++i) {
    const int64_t steps = steps_of[i];
    const int64_t want = want_of[i];
    LkDesc& d = grp.d[i];
    d.W = static_cast<const uint8_t*>(v[i]->W);
    d.x = v[i]->x;
    d.y = v[i]->y;
    d.rows = (int)v[i]->rows;
    d.block_begin = (int)bb;
    d.q = want ? (int)(steps / want) : 0;
    d.r = want ? (int)(steps % want) : 0;
    d.nsb = nsb;
    if (e && e[i]) {
      grp.ep[i] = *e[i];
      if (in_wave[i]) grp.ep[i].flags |= kEpPairInWave;
      d.ep_flags = grp.ep[i].flags;
      d.scale_ss = e[i]->scale_ss;
      d.scale_n = e[i]->scale_n;
    }
    bb += want;
    if (want) {
      const int64_t ws = ((steps + want - 1) / want + bw - 1) / bw;
      if (ws > max_wave_steps) max_wave_steps = ws;
    }
  }
  grp.total_blocks = (int)bb;
  LkPlan p;
  p.nsb = nsb;
  p.longrow = longrow;
  p.depth = max_wave_steps <= 2 ? 2 : 4;
  p.bw = bw;
  // long rows: x padded, then the sums of x per 32-weight sub-block (per run
  // of 16 for Q6_K)
  p.lds = longrow ? (size_t)(256 * nsb) * 4 * (type == GGUF_QK_TYPE_Q6_K ? 36 : 35) / 32 : 0;
  if (type == GGUF_QK_TYPE_Q4_0)
    launch_lk_typed<GGUF_QK_TYPE_Q4_0, false>(grp, p, stream);
  else if (type == GGUF_QK_TYPE_Q6_K)
    launch_lk_typed<GGUF_QK_TYPE_Q6_K, false>(grp, p, stream);
  else if (type == GGUF_QK_TYPE_Q8_0)
    launch_lk_typed<GGUF_QK_TYPE_Q8_0, false>(grp, p, stream);
  else if (ep)
    launch_lk_typed<GGUF_QK_TYPE_Q4_K, true>(grp, p, stream);
  else
    launch_lk_typed<GGUF_QK_TYPE_Q4_K, false>(grp, p, stream);
  return launch_status();
}

}  // namespace gqk
