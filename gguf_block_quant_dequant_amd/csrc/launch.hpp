// Internal host interface between the C ABI layer (gguf_qk.hip) and the
// translation units that hold kernel launches: fixed launch-shape choices
// and the launch functions each unit exports.
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/gguf_qk.h"
#include "gemv_types.hpp"

namespace gqk {

// Launch-shape choices (the measured best on the decode, prefill and small
// batch shapes).
struct Tuning {
  int target_tasks = 2048;   // wave tasks a split-K GEMV aims for
  int gemm_blocks = 0;       // blocks a split prefill GEMM aims for (0: 256, one per CU)
  int gemm_max_split = 0;    // largest K split of a prefill GEMM (0: by K)
  int sb_blocks = 512;       // blocks a small-batch product aims for
  int sb_max_split = 8;      // largest K split of a small-batch product
  int q4k_slots = 1;         // LDS chunks in flight per wave, Q4_K
  int q80_slots = 1;         // LDS chunks in flight per wave, Q8_0
  int q4k_lk = 1;            // Q4_K GEMVs without epilogue: lanes-along-K kernels
  int lk_waves = 1024;       // waves a lanes-along-K launch aims for
  int lkx_waves = 2048;      // the same for rows longer than 16 super-blocks
  int lkx_waves_q6 = 1024;   // the same for Q6_K rows longer than 16 super-blocks
  int lk_single = 1;         // one-GEMV launches take their descriptor as scalar arguments
  int lk_bw = 4;             // waves per block, rows of <= 16 super-blocks (4 or 8)
  int lkx_bw = 8;            // waves per block, longer rows (4 or 8)
  int lk_pair_in_wave = 1;   // gate/up pairs: both rows of an index in one wave
  int lk_two = 1;            // two GEMVs of one x: descriptors as scalar arguments
  int lk_three = 1;          // three GEMVs of one x: packed descriptors as scalar arguments
  int q4_0_lk = 1;           // Q4_0 rows of 256 .. 12288 weights: lanes-along-K kernels
  int q8_0_lk = 1;           // Q8_0 rows of 256 .. 4096 weights: lanes-along-K kernels
  int q6_k_lk = 1;           // Q6_K rows of 256 .. 12288 weights: lanes-along-K kernels
  int gemm_db = 1;           // prefill: the double-buffered GEMM
  int gemm_wide = 1;         // prefill: 256-token blocks where they fill the device
  int gemm_wide_tiles = 256; // ... i.e. give at least this many tiles unsplit
  int gemm_wide_target = 256;  // 256-token blocks resident at once (one per CU)
};

inline const Tuning& tuning() {
  static const Tuning t;
  return t;
}

// Kernel family of the calling thread's most recent GEMV launch (the values of
// GGUF_QK_LAUNCH_* in include/gguf_qk.h), for gguf_qk_last_launch.
extern thread_local int g_last_launch;

inline int launch_status() {
  return hipGetLastError() == hipSuccess ? GGUF_QK_OK : GGUF_QK_ERR_LAUNCH;
}

// lk.hip: the lanes-along-K kernels. lk_fits says whether they take a group
// of n GEMVs of one row length (with these epilogues); launch_lk launches it.
bool lk_fits(const gguf_qk_gemv* const* v, const GemvEpilogue* const* e, int n);
int launch_lk(const gguf_qk_gemv* const* v, const GemvEpilogue* const* e, int n, hipStream_t stream,
              int type);
// The split-K-in-block kernel (rows of other lengths, up to 128 super-blocks;
// Q4_K and Q4_0, no epilogues).
bool lks_fits(const gguf_qk_gemv* const* v, const GemvEpilogue* const* e, int n, int type);
int launch_lks(const gguf_qk_gemv* const* v, const GemvEpilogue* const* e, int n, hipStream_t stream,
               int type);

}  // namespace gqk
