// libgguf_qk: C ABI over the gfx950 kernels (declarations and contract in
// include/gguf_qk.h). Host code only validates, picks launch shapes and
// launches; every arithmetic step runs in the kernels.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/gguf_file.h"
#include "../../include/gguf_qk.h"
#include "dequant.hpp"
#include "gemm.hpp"
#include "gemv.hpp"
#include "gemv_lk.hpp"
#include "gemv_other.hpp"
#include "gemv_small_batch.hpp"
#include "layer_ops.hpp"
#include "probe.hpp"

namespace gqk {

// Per-device scratch for split-K partial sums and row-group counters. It is a
// static device array (each GPU the library runs on holds its own copy for the
// life of the process); nothing is allocated at call time. Counters are zero
// at load and every kernel that uses one returns it to zero.
constexpr int64_t kScratchPartials = int64_t(2) << 20;   // floats (8 MiB)
constexpr int64_t kScratchCounters = int64_t(1) << 14;   // row-group counters
constexpr int kMaxSplits = 16;                            // K ranges per row group
// Prefill split K: fp32 partial tiles (32 MiB) and one counter per tile.
constexpr int64_t kGemmScratchFloats = int64_t(8) << 20;
constexpr int64_t kGemmMaxTiles = int64_t(1) << 12;
constexpr int kGemmMaxSplits = 8;
// Gate/up pair counters of the fused SiLU(gate) * up epilogue (row groups of
// the pairs of one step).
constexpr int64_t kPairCounters = int64_t(1) << 12;
struct ScratchArea {
  float partials[kScratchPartials];
  int counters[kScratchCounters * kCounterStride];
  float gemm_partials[kGemmScratchFloats];
  int gemm_counters[kGemmMaxTiles * kGemmCounterStride];
  int pair_counters[kPairCounters * kCounterStride];
};
static __device__ __attribute__((aligned(256))) ScratchArea g_scratch;

constexpr int kMaxDevices = 64;

// Launch-shape knobs. Defaults are the measured best; GGUF_QK_TUNE (for
// sweeps, e.g. "tasks=2048,q4k_slots=1,q80_slots=1") overrides them.
struct Tuning {
  int target_tasks = 2048;   // wave tasks a split-K GEMV aims for
  int gemm_blocks = 0;       // blocks a prefill GEMM aims for (0: by K, see gguf_qmatmul_q4_k)
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
};

static const Tuning& tuning() {
  static const Tuning t = [] {
    Tuning r;
    const char* e = std::getenv("GGUF_QK_TUNE");
    if (!e) return r;
    const char* p = e;
    while (*p) {
      const char* eq = std::strchr(p, '=');
      if (!eq) break;
      const std::string key(p, eq - p);
      const int v = std::atoi(eq + 1);
      if (key == "tasks" && v > 0) r.target_tasks = v;
      if (key == "gemm_blocks" && v >= 0) r.gemm_blocks = v;
      if (key == "gemm_max_split" && v >= 0 && v <= kGemmMaxSplits) r.gemm_max_split = v;
      if (key == "sb_blocks" && v > 0) r.sb_blocks = v;
      if (key == "sb_max_split" && v > 0 && v <= 8) r.sb_max_split = v;
      if (key == "q4k_slots" && (v == 1 || v == 2)) r.q4k_slots = v;
      if (key == "q80_slots" && (v == 1 || v == 2)) r.q80_slots = v;
      if (key == "q4k_lk" && (v == 0 || v == 1)) r.q4k_lk = v;
      if (key == "lk_waves" && v > 0) r.lk_waves = v;
      if (key == "lkx_waves" && v > 0) r.lkx_waves = v;
      if (key == "lkx_waves_q6" && v > 0) r.lkx_waves_q6 = v;
      if (key == "lk_single" && (v == 0 || v == 1)) r.lk_single = v;
      if (key == "lk_bw" && (v == 4 || v == 8)) r.lk_bw = v;
      if (key == "lkx_bw" && (v == 4 || v == 8)) r.lkx_bw = v;
      if (key == "lk_pair_in_wave" && (v == 0 || v == 1)) r.lk_pair_in_wave = v;
      if (key == "lk_two" && (v == 0 || v == 1)) r.lk_two = v;
      if (key == "lk_three" && (v == 0 || v == 1)) r.lk_three = v;
      if (key == "q4_0_lk" && (v == 0 || v == 1)) r.q4_0_lk = v;
      if (key == "q8_0_lk" && (v == 0 || v == 1)) r.q8_0_lk = v;
      if (key == "q6_k_lk" && (v == 0 || v == 1)) r.q6_k_lk = v;
      if (key == "gemm_db" && (v == 0 || v == 1)) r.gemm_db = v;
      const char* comma = std::strchr(eq, ',');
      if (!comma) break;
      p = comma + 1;
    }
    return r;
  }();
  return t;
}

struct DeviceState {
  std::atomic<int> checked{0};   // 0 unknown, 1 gfx950, -1 unsupported
  ScratchArea* scratch = nullptr;
  std::mutex mu;
};
static DeviceState g_dev[kMaxDevices];

// Returns GGUF_QK_OK and the scratch of the current device, or an error.
static int current_device(ScratchArea** scratch) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return GGUF_QK_ERR_DEVICE;
  }
  DeviceState& st = g_dev[dev];
  int c = st.checked.load(std::memory_order_acquire);
  if (c == 0) {
    std::lock_guard<std::mutex> lk(st.mu);
    c = st.checked.load(std::memory_order_relaxed);
    if (c == 0) {
      hipDeviceProp_t prop;
      bool ok = hipGetDeviceProperties(&prop, dev) == hipSuccess &&
                std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
      void* p = nullptr;
      if (ok) ok = hipGetSymbolAddress(&p, HIP_SYMBOL(g_scratch)) == hipSuccess && p != nullptr;
      (void)hipGetLastError();
      st.scratch = static_cast<ScratchArea*>(p);
      c = ok ? 1 : -1;
      st.checked.store(c, std::memory_order_release);
    }
  }
  if (c != 1) return GGUF_QK_ERR_DEVICE;
  if (scratch) *scratch = st.scratch;
  return GGUF_QK_OK;
}

static int launch_status() {
  return hipGetLastError() == hipSuccess ? GGUF_QK_OK : GGUF_QK_ERR_LAUNCH;
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

static bool overlap(const void* a, int64_t an, const void* b, int64_t bn) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return an > 0 && bn > 0 && a0 < b0 + (uintptr_t)bn && b0 < a0 + (uintptr_t)an;
}

// Byte size of rows x row_bytes without overflow, or -1.
static int64_t mat_bytes(int64_t rows, int64_t row_bytes) {
  if (rows < 0 || row_bytes <= 0) return -1;
  if (rows > 0 && row_bytes > INT64_MAX / rows) return -1;
  return rows * row_bytes;
}

static int64_t row_bytes_of(int type, int64_t cols) {
  if (cols <= 0) return GGUF_QK_ERR_SHAPE;
  if (type == GGUF_QK_TYPE_Q8_0) {
    if (cols % kQ80BlockWeights) return GGUF_QK_ERR_SHAPE;
    if (cols / kQ80BlockWeights > INT64_MAX / kQ80BlockBytes) return GGUF_QK_ERR_SHAPE;
    return cols / kQ80BlockWeights * kQ80BlockBytes;
  }
  if (type == GGUF_QK_TYPE_Q4_K) {
    if (cols % kQ4KBlockWeights) return GGUF_QK_ERR_SHAPE;
    if (cols / kQ4KBlockWeights > INT64_MAX / kQ4KBlockBytes) return GGUF_QK_ERR_SHAPE;
    return cols / kQ4KBlockWeights * kQ4KBlockBytes;
  }
  if (type == GGUF_QK_TYPE_Q4_0) {
    if (cols % kQ40BlockWeights) return GGUF_QK_ERR_SHAPE;
    if (cols / kQ40BlockWeights > INT64_MAX / kQ40BlockBytes) return GGUF_QK_ERR_SHAPE;
    return cols / kQ40BlockWeights * kQ40BlockBytes;
  }
  if (type == GGUF_QK_TYPE_Q6_K) {
    if (cols % kQ6KBlockWeights) return GGUF_QK_ERR_SHAPE;
    if (cols / kQ6KBlockWeights > INT64_MAX / kQ6KBlockBytes) return GGUF_QK_ERR_SHAPE;
    return cols / kQ6KBlockWeights * kQ6KBlockBytes;
  }
  return GGUF_QK_ERR_SHAPE;
}

// Common validation of (W, out-ish) element ranges for a [rows x cols] matrix.
static int check_matrix(int type, const void* W, int64_t rows, int64_t cols, int64_t* wbytes) {
  if (!W) return GGUF_QK_ERR_NULL;
  if (rows < 0) return GGUF_QK_ERR_SHAPE;
  const int64_t rb = row_bytes_of(type, cols);
  if (rb < 0) return (int)rb;
  const int64_t wb = mat_bytes(rows, rb);
  if (wb < 0) return GGUF_QK_ERR_SHAPE;
  if (!aligned16(W)) return GGUF_QK_ERR_ALIGN;
  *wbytes = wb;
  return GGUF_QK_OK;
}

static int grid_1d(int64_t n, int per) { return (int)((n + per - 1) / per); }

}  // namespace gqk

using namespace gqk;

extern "C" {

int gguf_qk_abi_version(void) { return GGUF_QK_ABI_VERSION; }

const char* gguf_qk_strerror(int status) {
  switch (status) {
    case GGUF_QK_OK: return "ok";
    case GGUF_QK_ERR_NULL: return "null pointer argument";
    case GGUF_QK_ERR_SHAPE: return "invalid shape (rows/n_tokens < 0, cols <= 0, cols not a multiple of the block, or size overflow)";
    case GGUF_QK_ERR_ALIGN: return "pointer not 16-byte aligned";
    case GGUF_QK_ERR_ALIAS: return "output overlaps an input";
    case GGUF_QK_ERR_DEVICE: return "no HIP device, or the current device is not gfx950";
    case GGUF_QK_ERR_LAUNCH: return "kernel launch failed";
    case GGUF_QK_ERR_LIMIT: return "request exceeds a library limit";
    case GGUF_QK_ERR_FORMAT: return "the file does not follow the GGUF layout";
    case GGUF_QK_ERR_IO: return "the file cannot be opened or mapped";
    case GGUF_QK_ERR_NOT_FOUND: return "no tensor or key of that name, or index out of range";
    default: return "unknown status";
  }
}

int64_t gguf_row_bytes(int type, int64_t cols) { return row_bytes_of(type, cols); }

static int dequant_common(int type, const void* W, void* out, int64_t out_elem_bytes,
                          int64_t rows, int64_t cols, hipStream_t stream, int kind) {
  int64_t wb = 0;
  int st = check_matrix(type, W, rows, cols, &wb);
  if (st) return st;
  if (!out) return GGUF_QK_ERR_NULL;
  if (!aligned16(out)) return GGUF_QK_ERR_ALIGN;
  if (rows > 0 && cols > INT64_MAX / out_elem_bytes / rows) return GGUF_QK_ERR_SHAPE;
  const int64_t ob = rows * cols * out_elem_bytes;
  if (overlap(W, wb, out, ob)) return GGUF_QK_ERR_ALIAS;
  if (rows == 0) return GGUF_QK_OK;
  st = current_device(nullptr);
  if (st) return st;
  const int64_t quads = rows * cols / 4;
  if (grid_1d(quads, 256) <= 0 || quads / 256 >= INT32_MAX) return GGUF_QK_ERR_LIMIT;
  const dim3 grid(grid_1d(quads, 256)), block(256);
  const uint8_t* w = static_cast<const uint8_t*>(W);
  if (kind == 0)
    hipLaunchKernelGGL(dequant_q8_0_kernel, grid, block, 0, stream, w, static_cast<float4*>(out), quads);
  else if (kind == 1)
    hipLaunchKernelGGL(dequant_q4_k_kernel, grid, block, 0, stream, w, static_cast<float4*>(out), quads);
  else
    hipLaunchKernelGGL(dequant_q4_k_bf16_kernel, grid, block, 0, stream, w, static_cast<uint2*>(out), quads);
  return launch_status();
}

int dequant_q8_0(const void* W, float* out, int64_t rows, int64_t cols, hipStream_t stream) {
  return dequant_common(GGUF_QK_TYPE_Q8_0, W, out, 4, rows, cols, stream, 0);
}

int dequant_q4_k(const void* W, float* out, int64_t rows, int64_t cols, hipStream_t stream) {
  return dequant_common(GGUF_QK_TYPE_Q4_K, W, out, 4, rows, cols, stream, 1);
}

int dequant_q4_k_bf16(const void* W, uint16_t* out, int64_t rows, int64_t cols, hipStream_t stream) {
  return dequant_common(GGUF_QK_TYPE_Q4_K, W, out, 2, rows, cols, stream, 2);
}

// Validates one GEMV (type, W, x, y, rows, cols). Returns its weight bytes.
static int check_gemv(int type, const void* W, const float* x, const float* y, int64_t rows,
                      int64_t cols, int64_t* wbytes) {
  int st = check_matrix(type, W, rows, cols, wbytes);
  if (st) return st;
  if (!x || !y) return GGUF_QK_ERR_NULL;
  if (!aligned16(x) || !aligned16(y)) return GGUF_QK_ERR_ALIGN;
  if (rows > INT64_MAX / 4 || cols > INT64_MAX / 4) return GGUF_QK_ERR_SHAPE;
  if (overlap(y, rows * 4, W, *wbytes) || overlap(y, rows * 4, x, cols * 4)) return GGUF_QK_ERR_ALIAS;
  if (row_bytes_of(type, cols) * 64 > INT32_MAX) return GGUF_QK_ERR_LIMIT;   // 32-bit tile offsets
  return GGUF_QK_OK;
}

// Lays out one group of same-format GEMVs (already validated, rows > 0) as
// tasks: Q4_K as block tasks (8 waves per row group and up to 8 super-blocks,
// partials added in LDS), Q8_0 as per-wave tasks with split-K sized to the
// task target. Returns the task count. Q8_0 GEMVs with cols % 256 != 0 are
// never grouped (see launch_step).
static int64_t plan_group(int type, const gguf_qk_gemv* const* v, const GemvEpilogue* const* e,
                          int n, GemvGroup* grp) {
  *grp = GemvGroup{};
  grp->n = n;
  for (int i = 0; i < n; ++i)
    if (e && e[i]) grp->ep[i] = *e[i];
  int64_t total_bytes = 0;
  for (int i = 0; i < n; ++i) total_bytes += v[i]->rows * row_bytes_of(type, v[i]->cols);
  int64_t tasks = 0, part_off = 0, cnt_off = 0;
  for (int i = 0; i < n; ++i) {
    const gguf_qk_gemv& g = *v[i];
    const int nch = (int)(g.cols / 256);   // Q4_K super-blocks or Q8_0 8-block chunks
    const int64_t RG = (g.rows + 63) / 64;
    int64_t P;
    if (type == GGUF_QK_TYPE_Q4_K) {
      P = (nch + kBlockWaves - 1) / kBlockWaves;
    } else {
      const int64_t bytes = g.rows * row_bytes_of(type, g.cols);
      int64_t want = (int64_t)((double)tuning().target_tasks * (double)bytes / (double)total_bytes);
      if (want < 1) want = 1;
      // nearest, not up: a GEMV with about as many row groups as the task
      // target is not cut (cutting puts the two halves of each row, which
      // share a 128-byte line, on different XCDs: 64.0 vs 60.0 us for the
      // 128256 x 2048 head)
      P = (want + RG / 2) / RG;
      if (P > nch) P = nch;
      if (P > kMaxSplits) P = kMaxSplits;
      if (P < 1) P = 1;
    }
    while (P > 1 && part_off + P * g.rows > kScratchPartials) --P;
    if (P > 1 && cnt_off + RG > kScratchCounters) P = 1;
    GemvDesc& d = grp->d[i];
    d.W = static_cast<const uint8_t*>(g.W);
    d.x = g.x;
    d.y = g.y;
    d.rows = g.rows;
    d.nchunks = nch;
    d.P = (int)P;
    d.part_off = part_off;
    d.cnt_off = (int)cnt_off;
    tasks += RG * P;
    d.task_end = tasks;
    if (P > 1) {
      part_off += P * g.rows;
      cnt_off += RG;
    }
  }
  return tasks;
}

extern "C++" {
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
  if (!kEp && grp.n == 1 && tuning().lk_single) {
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
    launch_lk2<kType, kNsb, kW>(grp, depth, stream);
    return;
  }
  Lk3Args a3;
  if (!kEp && lk_three(grp, &a3)) {
    launch_lk3<kType, kNsb, kW>(grp, a3, depth, stream);
    return;
  }
  if (depth <= 2)
    hipLaunchKernelGGL((gemv_lk_kernel<kType, kNsb, 2, kW, kEp>), grid, block, 0, stream, grp);
  else
    hipLaunchKernelGGL((gemv_lk_kernel<kType, kNsb, 4, kW, kEp>), grid, block, 0, stream, grp);
}

template <int kNsb>
static void launch_lk_nsb(const LkGroup& grp, int depth, int waves, bool ep, int type,
                          hipStream_t stream) {
  if (type == GGUF_QK_TYPE_Q4_0)
    launch_lk_nsb<GGUF_QK_TYPE_Q4_0, kNsb, 4, false>(grp, depth, stream);
  else if (type == GGUF_QK_TYPE_Q6_K)
    launch_lk_nsb<GGUF_QK_TYPE_Q6_K, kNsb, 4, false>(grp, depth, stream);
  else if (type == GGUF_QK_TYPE_Q8_0)
    launch_lk_nsb<GGUF_QK_TYPE_Q8_0, kNsb, 4, false>(grp, depth, stream);
  else if (ep)
    launch_lk_nsb<GGUF_QK_TYPE_Q4_K, kNsb, 4, true>(grp, depth, stream);
  else if (waves == 8)
    launch_lk_nsb<GGUF_QK_TYPE_Q4_K, kNsb, 8, false>(grp, depth, stream);
  else
    launch_lk_nsb<GGUF_QK_TYPE_Q4_K, kNsb, 4, false>(grp, depth, stream);
}

template <int kQ, int kW>
static void launch_lkx(const LkGroup& grp, size_t lds, bool ep, int type, hipStream_t stream) {
  const bool q40 = type == GGUF_QK_TYPE_Q4_0, q6 = type == GGUF_QK_TYPE_Q6_K;
  const dim3 grid((unsigned)grp.total_blocks), block(kW * 64);
  // one GEMV without epilogue: its descriptor as (preloaded) scalar arguments
  const bool single = grp.n == 1 && !ep && tuning().lk_single;
  const LkDesc& d = grp.d[0];
  const uint8_t* W = single ? d.W : nullptr;
  const float* x = single ? d.x : nullptr;
  float* y = single ? d.y : nullptr;
  const int rows = single ? d.rows : 0, q = single ? d.q : 0, r = single ? d.r : 0;
  const int nsb = single ? d.nsb : 0;
  if (q6) {
    // (three rounds of Q6_K quarters run in 4-wave blocks only)
    if constexpr (!(kQ == 3 && kW == 8)) {
      if (single)
        hipLaunchKernelGGL((gemv_lkx_kernel<GGUF_QK_TYPE_Q6_K, kQ, 2, kW, false, true>), grid, block, lds,
                           stream, W, x, y, rows, q, r, nsb, grp);
      else
        hipLaunchKernelGGL((gemv_lkx_kernel<GGUF_QK_TYPE_Q6_K, kQ, 2, kW, false, false>), grid, block, lds,
                           stream, W, x, y, rows, q, r, nsb, grp);
    }
    return;
  }
  if (q40 && single)
    hipLaunchKernelGGL((gemv_lkx_kernel<GGUF_QK_TYPE_Q4_0, kQ, 2, kW, false, true>), grid, block, lds, stream,
                       W, x, y, rows, q, r, nsb, grp);
  else if (q40)
    hipLaunchKernelGGL((gemv_lkx_kernel<GGUF_QK_TYPE_Q4_0, kQ, 2, kW, false, false>), grid, block, lds, stream,
                       W, x, y, rows, q, r, nsb, grp);
  else if (single)
    hipLaunchKernelGGL((gemv_lkx_kernel<GGUF_QK_TYPE_Q4_K, kQ, 2, kW, false, true>), grid, block, lds, stream,
                       W, x, y, rows, q, r, nsb, grp);
  else if (ep)
    hipLaunchKernelGGL((gemv_lkx_kernel<GGUF_QK_TYPE_Q4_K, kQ, 2, kW, true, false>), grid, block, lds, stream,
                       W, x, y, rows, q, r, nsb, grp);
  else
    hipLaunchKernelGGL((gemv_lkx_kernel<GGUF_QK_TYPE_Q4_K, kQ, 2, kW, false, false>), grid, block, lds, stream,
                       W, x, y, rows, q, r, nsb, grp);
}
}

// Q4_K GEMVs whose rows hold 1, 2, 4, 8 or 16 super-blocks (lanes hold x), or
// 17 to 48 (x read from LDS), all the same: the lanes-along-K kernels take
// them, with any epilogue except norm preparation and a gate/up pair together
// on one GEMV, and at most 256 partial sums for an input RMSN.
static bool lk_fits(const gguf_qk_gemv* const* v, const GemvEpilogue* const* e, int n) {
  const int64_t c = v[0]->cols;
  if (c % 256 || (c != 256 && c != 512 && c != 1024 && c != 2048 && c != 4096 && (c <= 4096 || c > kLkxMaxK)))
    return false;
  for (int i = 0; i < n; ++i) {
    if (v[i]->cols != c || v[i]->rows > (int64_t(1) << 30)) return false;
    if (e && e[i]) {
      const int f = e[i]->flags;
      if ((f & kEpNorm) && (f & kEpPair)) return false;
      if ((f & kEpScale) && e[i]->scale_n > 256) return false;
      if ((f & kEpNorm) && !e[i]->norm_cnt) return false;
    }
  }
  return true;
}

// Lanes-along-K launch: blocks go to the GEMVs in proportion to their rows
// (at least one, at most one per row step); a shallow load ring when a wave
// has only a few steps.
static int launch_lk(const gguf_qk_gemv* const* v, const GemvEpilogue* const* e, int n,
                     hipStream_t stream, int type = GGUF_QK_TYPE_Q4_K) {
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
  const int64_t target_blocks = ((longrow ? lkx_waves : tuning().lk_waves) + bw - 1) / bw;
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
  int64_t bb = 0, max_wave_steps = 0;
  for (int i = 0; i < n; ++i) {
    const bool up_half = i > 0 && in_wave[i - 1];
    const int rpm = in_wave[i] ? rps / 2 : rps;
    const int64_t steps = (v[i]->rows + rpm - 1) / rpm;
    const double share = (in_wave[i] ? 2.0 : 1.0) * (double)v[i]->rows / (double)total_rows;
    int64_t want = (int64_t)((double)target_blocks * share + 0.5);
    if (want < 1) want = 1;
    if (want > steps) want = steps;
    if (up_half) want = 0;
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
  const int depth = max_wave_steps <= 2 ? 2 : 4;
  if (longrow) {
    const int kq = (4 * nsb + 63) / 64;
    // x padded, then the sums of x per 32-weight sub-block (per run of 16 for Q6_K)
    const size_t lds = (size_t)(256 * nsb) * 4 * (type == GGUF_QK_TYPE_Q6_K ? 36 : 35) / 32;
    if (bw == 8) {
      if (kq == 2)
        launch_lkx<2, 8>(grp, lds, ep, type, stream);
      else
        launch_lkx<3, 8>(grp, lds, ep, type, stream);
    } else {
      if (kq == 2)
        launch_lkx<2, 4>(grp, lds, ep, type, stream);
      else
        launch_lkx<3, 4>(grp, lds, ep, type, stream);
    }
    return launch_status();
  }
  switch (nsb) {
    case 1: launch_lk_nsb<1>(grp, depth, bw, ep, type, stream); break;
    case 2: launch_lk_nsb<2>(grp, depth, bw, ep, type, stream); break;
    case 4: launch_lk_nsb<4>(grp, depth, bw, ep, type, stream); break;
    case 8: launch_lk_nsb<8>(grp, depth, bw, ep, type, stream); break;
    default: launch_lk_nsb<16>(grp, depth, bw, ep, type, stream); break;
  }
  return launch_status();
}

static int launch_other(int type, const void* W, const float* x, float* y, int64_t rows,
                        int64_t cols, hipStream_t stream);

// Launches one planned group.
static int launch_group(int type, const gguf_qk_gemv* const* v, const GemvEpilogue* const* e, int n,
                        const ScratchArea* scratch, hipStream_t stream) {
  if (type == GGUF_QK_TYPE_Q4_K && tuning().q4k_lk && lk_fits(v, e, n)) return launch_lk(v, e, n, stream);
  if (type == GGUF_QK_TYPE_Q4_0 || type == GGUF_QK_TYPE_Q6_K) {
    // rows of 256 .. 12288 weights in multiples of 256 (no epilogues on
    // these types): the lanes-along-K kernels; else the lane-quad kernel, one
    // launch each
    const bool on = type == GGUF_QK_TYPE_Q4_0 ? tuning().q4_0_lk : tuning().q6_k_lk;
    if (on && lk_fits(v, nullptr, n)) return launch_lk(v, nullptr, n, stream, type);
    for (int i = 0; i < n; ++i) {
      const int st = launch_other(type, v[i]->W, v[i]->x, v[i]->y, v[i]->rows, v[i]->cols, stream);
      if (st) return st;
    }
    return GGUF_QK_OK;
  }
  if (type == GGUF_QK_TYPE_Q8_0 && tuning().q8_0_lk && v[0]->cols <= 4096 && lk_fits(v, nullptr, n)) {
    // Q8_0 rows of 256 .. 4096 weights (multiples of 256) without epilogues:
    // the lanes-along-K kernels; else the lane-per-row kernel below
    bool ep = false;
    for (int i = 0; i < n; ++i) ep = ep || (e && e[i] && e[i]->flags != 0);
    if (!ep) return launch_lk(v, nullptr, n, stream, type);
  }
  GemvGroup grp;
  const int64_t tasks = plan_group(type, v, e, n, &grp);
  float* partials = const_cast<float*>(scratch->partials);
  int* counters = const_cast<int*>(scratch->counters);
  const int64_t blocks = type == GGUF_QK_TYPE_Q4_K ? tasks : (tasks + kGemvWaves - 1) / kGemvWaves;
  if (blocks > INT32_MAX) return GGUF_QK_ERR_LIMIT;
  bool ep = false;   // any epilogue in this launch: the kernel variant that has them
  for (int i = 0; i < n; ++i) ep = ep || grp.ep[i].flags != 0;
  if (type == GGUF_QK_TYPE_Q4_K) {
    if (ep)
      hipLaunchKernelGGL(gemv_q4k_block_kernel<true>, dim3((unsigned)blocks), dim3(kBlockWaves * 64), 0,
                         stream, grp, partials, counters);
    else
      hipLaunchKernelGGL(gemv_q4k_block_kernel<false>, dim3((unsigned)blocks), dim3(kBlockWaves * 64),
                         0, stream, grp, partials, counters);
    return launch_status();
  }
  const dim3 grid((unsigned)blocks), block(kGemvWaves * 64);
  if (ep)
    hipLaunchKernelGGL((gemv_group_kernel<1, false, true>), grid, block, 0, stream, grp, partials,
                       counters);
  else if (tuning().q80_slots == 2)
    hipLaunchKernelGGL((gemv_group_kernel<2, false, false>), grid, block, 0, stream, grp, partials,
                       counters);
  else
    hipLaunchKernelGGL((gemv_group_kernel<1, false, false>), grid, block, 0, stream, grp, partials,
                       counters);
  return launch_status();
}

static int launch_rowwise_q8_0(const gguf_qk_gemv& g, hipStream_t stream) {
  const int64_t blocks = (g.rows + 3) / 4;
  if (blocks > INT32_MAX || g.cols / kQ80BlockWeights > INT32_MAX) return GGUF_QK_ERR_LIMIT;
  hipLaunchKernelGGL(gemv_q8_0_rowwise_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<const uint8_t*>(g.W), g.x, g.y, g.rows,
                     (int)(g.cols / kQ80BlockWeights));
  return launch_status();
}

// Launches the GEMVs of one step: same-format GEMVs go together, kMaxGroup at
// a time; each launch follows the previous one on the stream.
static int launch_other(int type, const void* W, const float* x, float* y, int64_t rows,
                        int64_t cols, hipStream_t stream);

static int launch_step(const gguf_qk_gemv* list, const GemvEpilogue* eps, int n,
                       const ScratchArea* scratch, hipStream_t stream) {
  for (int type : {GGUF_QK_TYPE_Q4_K, GGUF_QK_TYPE_Q4_0, GGUF_QK_TYPE_Q6_K, GGUF_QK_TYPE_Q8_0}) {
    const gguf_qk_gemv* grp[kMaxGroup];
    const GemvEpilogue* ge[kMaxGroup];
    int k = 0;
    for (int i = 0; i < n; ++i) {
      const gguf_qk_gemv& g = list[i];
      if (g.type != type || g.rows == 0) continue;
      if (type == GGUF_QK_TYPE_Q8_0 && g.cols % 256) {
        const int st = launch_rowwise_q8_0(g, stream);
        if (st) return st;
        continue;
      }
      // the two GEMVs of a gate/up pair go into one launch: a gate that would
      // take the last place of a group opens the next one
      if (k == kMaxGroup - 1 && eps && (eps[i].flags & kEpPair) && eps[i].role == 0) {
        const int st = launch_group(type, grp, ge, k, scratch, stream);
        if (st) return st;
        k = 0;
      }
      ge[k] = eps ? &eps[i] : nullptr;
      grp[k++] = &g;
      if (k == kMaxGroup) {
        const int st = launch_group(type, grp, ge, k, scratch, stream);
        if (st) return st;
        k = 0;
      }
    }
    if (k) {
      const int st = launch_group(type, grp, ge, k, scratch, stream);
      if (st) return st;
    }
  }
  return GGUF_QK_OK;
}

static int matvec_common(int type, const void* W, const float* x, float* y, int64_t rows,
                         int64_t cols, hipStream_t stream) {
  int64_t wb = 0;
  int st = check_gemv(type, W, x, y, rows, cols, &wb);
  if (st) return st;
  if (rows == 0) return GGUF_QK_OK;
  ScratchArea* scratch = nullptr;
  st = current_device(&scratch);
  if (st) return st;
  const gguf_qk_gemv g{W, x, y, rows, cols, type, 0, {0}};
  return launch_step(&g, nullptr, 1, scratch, stream);
}

// Validates entry i's epilogue (the whole list is in view for pairs) and
// fills the device form; the pair counters are attached later (pair_rg: the
// first pair counter row group of the entry's pair, else -1). pair_off: next
// free pair counter row group of the step.
static int make_epilogue(const gguf_qk_gemv* list, const gguf_qk_gemv_ep* ep, int32_t n, int32_t i,
                         int64_t* pair_off, int64_t* pair_rg, int64_t* norm_rg, GemvEpilogue* out) {
  *pair_rg = -1;
  *norm_rg = -1;
  *out = GemvEpilogue{};
  const gguf_qk_gemv& g = list[i];
  const gguf_qk_gemv_ep& e = ep[i];
  const int64_t RG = (g.rows + 63) / 64;
  auto al4 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; };
  int flags = 0;
  if (e.scale_ss) {
    if (e.scale_n < 1 || e.scale_n > INT32_MAX || !(e.eps >= 0.f) || e.eps > 3.0e38f || !al4(e.scale_ss))
      return GGUF_QK_ERR_SHAPE;
    flags |= kEpScale;
  }
  if (e.residual) {
    if (!al4(e.residual)) return GGUF_QK_ERR_ALIGN;
    if (e.residual != g.y && overlap(e.residual, g.rows * 4, g.y, g.rows * 4)) return GGUF_QK_ERR_ALIAS;
    flags |= kEpResidual;
  }
  if (e.norm_w || e.norm_out || e.ss_out) {
    if (!e.norm_w || !e.norm_out || !e.ss_out) return GGUF_QK_ERR_NULL;
    if (!al4(e.norm_w) || !al4(e.norm_out) || !al4(e.ss_out)) return GGUF_QK_ERR_ALIGN;
    flags |= kEpNorm;
    // row-group counters for kernels whose blocks do not own whole row groups
    // (taken from the step's group counters when there are enough left)
    if (*pair_off + RG <= kPairCounters) {
      *norm_rg = *pair_off;
      *pair_off += RG;
    }
  }
  if (e.pair != 0) {
    if (e.pair != 1 && e.pair != 2) return GGUF_QK_ERR_SHAPE;
    const int32_t j = e.pair == 1 ? i + 1 : i - 1;   // the partner
    if (j < 0 || j >= n) return GGUF_QK_ERR_SHAPE;
    const gguf_qk_gemv& h = list[j];
    if (ep[j].pair != 3 - e.pair || h.stage != g.stage || h.rows != g.rows || h.type != g.type ||
        ep[j].act != e.act)
      return GGUF_QK_ERR_SHAPE;
    if (!e.act) return GGUF_QK_ERR_NULL;
    if (!al4(e.act)) return GGUF_QK_ERR_ALIGN;
    if (e.pair == 1) {                              // counters are taken once per pair
      if (*pair_off + RG > kPairCounters) return GGUF_QK_ERR_LIMIT;
      *pair_rg = *pair_off;
      *pair_off += RG;
    }
    out->partner_y = h.y;
    out->role = e.pair - 1;
    out->act = e.act;
    flags |= kEpPair;
  }
  // outputs written by the epilogue may not overlap what the step reads or writes
  const void* outs[3] = {e.norm_out, e.ss_out, e.act};
  const int64_t outn[3] = {g.rows * 4, RG * 4, g.rows * 4};
  for (int a = 0; a < 3; ++a) {
    if (!outs[a]) continue;
    for (int32_t b = 0; b < n; ++b) {
      if (list[b].stage != g.stage) continue;
      const int64_t wb = list[b].rows * row_bytes_of(list[b].type, list[b].cols);
      if (overlap(outs[a], outn[a], list[b].y, list[b].rows * 4) ||
          overlap(outs[a], outn[a], list[b].x, list[b].cols * 4) ||
          overlap(outs[a], outn[a], list[b].W, wb))
        return GGUF_QK_ERR_ALIAS;
    }
    if (overlap(outs[a], outn[a], e.residual, e.residual ? g.rows * 4 : 0) ||
        overlap(outs[a], outn[a], e.norm_w, e.norm_w ? g.rows * 4 : 0) ||
        overlap(outs[a], outn[a], e.scale_ss, e.scale_ss ? e.scale_n * 4 : 0))
      return GGUF_QK_ERR_ALIAS;
  }
  if (flags && ((g.type == GGUF_QK_TYPE_Q8_0 && g.cols % 256) || g.type == GGUF_QK_TYPE_Q4_0 ||
                g.type == GGUF_QK_TYPE_Q6_K))
    return GGUF_QK_ERR_SHAPE;
  out->scale_ss = e.scale_ss;
  out->residual = e.residual;
  out->norm_w = e.norm_w;
  out->norm_out = e.norm_out;
  out->ss_out = e.ss_out;
  out->scale_n = (int)e.scale_n;
  out->eps = e.eps;
  out->inv_k = 1.0f / (float)g.cols;
  out->flags = flags;
  return GGUF_QK_OK;
}

static int batch_common(const gguf_qk_gemv* list, const gguf_qk_gemv_ep* ep, int32_t n,
                        hipStream_t stream) {
  if (n < 0) return GGUF_QK_ERR_SHAPE;
  if (n == 0) return GGUF_QK_OK;
  if (!list) return GGUF_QK_ERR_NULL;
  // validate everything before any HIP call
  for (int32_t i = 0; i < n; ++i) {
    int64_t wb = 0;
    const gguf_qk_gemv& g = list[i];
    if (g.type != GGUF_QK_TYPE_Q8_0 && g.type != GGUF_QK_TYPE_Q4_K && g.type != GGUF_QK_TYPE_Q4_0 &&
        g.type != GGUF_QK_TYPE_Q6_K)
      return GGUF_QK_ERR_SHAPE;
    const int st = check_gemv(g.type, g.W, g.x, g.y, g.rows, g.cols, &wb);
    if (st) return st;
  }
  // inside a step, no output may overlap another entry's output or input
  for (int32_t i = 0; i < n;) {
    int32_t j = i;
    while (j < n && list[j].stage == list[i].stage) ++j;
    for (int32_t a = i; a < j; ++a)
      for (int32_t b = i; b < j; ++b) {
        if (a == b) continue;
        const int64_t wb = list[b].rows * row_bytes_of(list[b].type, list[b].cols);
        if (overlap(list[a].y, list[a].rows * 4, list[b].y, list[b].rows * 4) ||
            overlap(list[a].y, list[a].rows * 4, list[b].x, list[b].cols * 4) ||
            overlap(list[a].y, list[a].rows * 4, list[b].W, wb))
          return GGUF_QK_ERR_ALIAS;
      }
    i = j;
  }
  std::vector<GemvEpilogue> eps;
  std::vector<int64_t> pair_rg, norm_rg;
  if (ep) {
    eps.resize(n);
    pair_rg.resize(n);
    norm_rg.resize(n);
    int64_t pair_off = 0;
    for (int32_t i = 0; i < n; ++i) {
      if (i > 0 && list[i].stage != list[i - 1].stage) pair_off = 0;   // a step has finished
      const int st = make_epilogue(list, ep, n, i, &pair_off, &pair_rg[i], &norm_rg[i], &eps[i]);
      if (st) return st;
      if (ep[i].pair == 2) pair_rg[i] = pair_rg[i - 1];   // the gate's counters
    }
  }
  ScratchArea* scratch = nullptr;
  int st = current_device(&scratch);
  if (st) return st;
  for (int32_t i = 0; i < (int32_t)eps.size(); ++i) {
    if (pair_rg[i] >= 0) eps[i].pair_cnt = scratch->pair_counters + pair_rg[i] * kCounterStride;
    if (norm_rg[i] >= 0) eps[i].norm_cnt = scratch->pair_counters + norm_rg[i] * kCounterStride;
  }
  for (int32_t i = 0; i < n;) {
    int32_t j = i;
    while (j < n && list[j].stage == list[i].stage) ++j;
    st = launch_step(list + i, ep ? eps.data() + i : nullptr, j - i, scratch, stream);
    if (st) return st;
    i = j;
  }
  return GGUF_QK_OK;
}

int gguf_qmatvec_batch(const gguf_qk_gemv* list, int32_t n, hipStream_t stream) {
  return batch_common(list, nullptr, n, stream);
}

int gguf_qmatvec_batch_ep(const gguf_qk_gemv* list, const gguf_qk_gemv_ep* ep, int32_t n,
                          hipStream_t stream) {
  return batch_common(list, ep, n, stream);
}

int gguf_qmatvec_q8_0(const void* W, const float* x, float* y, int64_t rows, int64_t cols,
                      hipStream_t stream) {
  return matvec_common(GGUF_QK_TYPE_Q8_0, W, x, y, rows, cols, stream);
}

int gguf_qmatvec_q4_k(const void* W, const float* x, float* y, int64_t rows, int64_t cols,
                      hipStream_t stream) {
  return matvec_common(GGUF_QK_TYPE_Q4_K, W, x, y, rows, cols, stream);
}

// Q4_0 / Q6_K: dequant (one thread per Q4_0 block or Q6_K quad of 16
// weights) and the batch-1 GEMV (kOtherRows rows per wave).
static int dequant_other(int type, const void* W, float* out, int64_t rows, int64_t cols,
                         hipStream_t stream) {
  int64_t wb = 0;
  int st = check_matrix(type, W, rows, cols, &wb);
  if (st) return st;
  if (!out) return GGUF_QK_ERR_NULL;
  if (!aligned16(out)) return GGUF_QK_ERR_ALIGN;
  if (rows > 0 && cols > INT64_MAX / 4 / rows) return GGUF_QK_ERR_SHAPE;
  if (overlap(W, wb, out, rows * cols * 4)) return GGUF_QK_ERR_ALIAS;
  if (rows == 0) return GGUF_QK_OK;
  st = current_device(nullptr);
  if (st) return st;
  const uint8_t* w = static_cast<const uint8_t*>(W);
  if (type == GGUF_QK_TYPE_Q4_0) {
    const int64_t units = rows * (cols / kQ40BlockWeights);
    if (units / 256 >= INT32_MAX) return GGUF_QK_ERR_LIMIT;
    hipLaunchKernelGGL(dequant_q4_0_kernel, dim3(grid_1d(units, 256)), dim3(256), 0, stream, w, out,
                       units);
  } else {
    const int64_t units = rows * (cols / kQ6KBlockWeights) * 16;
    if (units / 256 >= INT32_MAX) return GGUF_QK_ERR_LIMIT;
    hipLaunchKernelGGL(dequant_q6_k_kernel, dim3(grid_1d(units, 256)), dim3(256), 0, stream, w, out,
                       units);
  }
  return launch_status();
}

static int launch_other(int type, const void* W, const float* x, float* y, int64_t rows,
                        int64_t cols, hipStream_t stream);

static int matvec_other(int type, const void* W, const float* x, float* y, int64_t rows,
                        int64_t cols, hipStream_t stream) {
  int64_t wb = 0;
  int st = check_gemv(type, W, x, y, rows, cols, &wb);
  if (st) return st;
  if (rows == 0) return GGUF_QK_OK;
  st = current_device(nullptr);
  if (st) return st;
  if (type == GGUF_QK_TYPE_Q4_0 || type == GGUF_QK_TYPE_Q6_K) {
    ScratchArea* scratch = nullptr;
    st = current_device(&scratch);
    if (st) return st;
    const gguf_qk_gemv g{W, x, y, rows, cols, type, 0, {0}};
    return launch_step(&g, nullptr, 1, scratch, stream);
  }
  return launch_other(type, W, x, y, rows, cols, stream);
}

static int launch_other(int type, const void* W, const float* x, float* y, int64_t rows,
                        int64_t cols, hipStream_t stream) {
  const int64_t per_block = (int64_t)kOtherRows * kOtherWaves;
  const int64_t blocks = (rows + per_block - 1) / per_block;
  if (blocks > INT32_MAX) return GGUF_QK_ERR_LIMIT;
  const uint8_t* w = static_cast<const uint8_t*>(W);
  if (type == GGUF_QK_TYPE_Q4_0)
    hipLaunchKernelGGL(gemv_q4_0_kernel, dim3((unsigned)blocks), dim3(kOtherWaves * 64), 0, stream,
                       w, x, y, rows, cols / kQ40BlockWeights);
  else
    hipLaunchKernelGGL(gemv_q6_k_kernel, dim3((unsigned)blocks), dim3(kOtherWaves * 64), 0, stream,
                       w, x, y, rows, cols / kQ6KBlockWeights);
  return launch_status();
}

int dequant_q4_0(const void* W, float* out, int64_t rows, int64_t cols, hipStream_t stream) {
  return dequant_other(GGUF_QK_TYPE_Q4_0, W, out, rows, cols, stream);
}

int dequant_q6_k(const void* W, float* out, int64_t rows, int64_t cols, hipStream_t stream) {
  return dequant_other(GGUF_QK_TYPE_Q6_K, W, out, rows, cols, stream);
}

int gguf_qmatvec_q4_0(const void* W, const float* x, float* y, int64_t rows, int64_t cols,
                      hipStream_t stream) {
  return matvec_other(GGUF_QK_TYPE_Q4_0, W, x, y, rows, cols, stream);
}

int gguf_qmatvec_q6_k(const void* W, const float* x, float* y, int64_t rows, int64_t cols,
                      hipStream_t stream) {
  return matvec_other(GGUF_QK_TYPE_Q6_K, W, x, y, rows, cols, stream);
}

// Prefill of n (1 .. 4) Q4_K matrices sharing X (validated as a whole before
// any launch; one launch of the double-buffered kernel, the matrices' row
// tiles end to end along grid x).
static int matmul_q4_k_group(const void* const* W, uint16_t* const* Y, const int64_t* rows, int n,
                             const uint16_t* X, int64_t n_tokens, int64_t cols, hipStream_t stream) {
  if (!W || !Y || !rows) return GGUF_QK_ERR_NULL;
  if (n < 1 || n > kGemmMaxGroup) return GGUF_QK_ERR_SHAPE;
  int64_t wb[kGemmMaxGroup] = {0, 0, 0, 0};
  for (int m = 0; m < n; ++m) {
    if (rows[m] < 0) return GGUF_QK_ERR_SHAPE;
    if (rows[m] == 0 && n > 1) {   // skipped: its W and Y are not touched (may be null)
      const int64_t rb = row_bytes_of(GGUF_QK_TYPE_Q4_K, cols);
      if (rb < 0) return (int)rb;
      continue;
    }
    const int st = check_matrix(GGUF_QK_TYPE_Q4_K, W[m], rows[m], cols, &wb[m]);
    if (st) return st;
    if (!Y[m]) return GGUF_QK_ERR_NULL;
    if (!aligned16(Y[m])) return GGUF_QK_ERR_ALIGN;
  }
  if (!X) return GGUF_QK_ERR_NULL;
  if (n_tokens < 0) return GGUF_QK_ERR_SHAPE;
  if (!aligned16(X)) return GGUF_QK_ERR_ALIGN;
  for (int m = 0; m < n; ++m)
    if (n_tokens > 0 && (cols > INT64_MAX / 2 / n_tokens || rows[m] > INT64_MAX / 2 / n_tokens))
      return GGUF_QK_ERR_SHAPE;
  const int64_t xb = n_tokens * cols * 2;
  for (int m = 0; m < n; ++m) {
    if (rows[m] == 0) continue;
    const int64_t yb = n_tokens * rows[m] * 2;
    if (overlap(Y[m], yb, X, xb)) return GGUF_QK_ERR_ALIAS;
    for (int o = 0; o < n; ++o) {
      if (rows[o] == 0) continue;
      if (overlap(Y[m], yb, W[o], wb[o])) return GGUF_QK_ERR_ALIAS;
      if (o != m && overlap(Y[m], yb, Y[o], n_tokens * rows[o] * 2)) return GGUF_QK_ERR_ALIAS;
    }
  }
  if (n_tokens == 0) return GGUF_QK_OK;
  const int64_t gy = (n_tokens + kGemmBM - 1) / kGemmBM;
  GemmGroup G{};
  int64_t gx = 0;
  for (int m = 0; m < n; ++m) {
    if (rows[m] == 0) continue;   // nothing to compute, nothing written
    G.W[G.n] = static_cast<const uint8_t*>(W[m]);
    G.Y[G.n] = Y[m];
    G.rows[G.n] = rows[m];
    G.tile_begin[G.n] = (int)gx;
    ++G.n;
    gx += (rows[m] + kGemmBN - 1) / kGemmBN;
    if (gx > INT32_MAX) return GGUF_QK_ERR_LIMIT;
  }
  if (G.n == 0) return GGUF_QK_OK;
  if (gy > 65535) return GGUF_QK_ERR_LIMIT;
  ScratchArea* scratch = nullptr;
  int st = current_device(&scratch);
  if (st) return st;
  // Split K over whole super-blocks when there are too few tiles to fill the
  // device, as far as the scratch for the fp32 partial tiles allows.
  // Measured on the 2048-hidden shapes: long K (down, 43 super-blocks) gains
  // from up to 8 ranges and two blocks per CU; short K (8 super-blocks) from
  // at most 4 ranges and one block per CU, past which the last block's sum
  // over the partial tiles costs more than the extra blocks save.
  const int64_t tiles = gx * gy, nsb = cols / kQ4KBlockWeights;
  const bool long_k = nsb >= 32;
  const int64_t target = tuning().gemm_blocks ? tuning().gemm_blocks : (long_k ? 512 : 256);
  const int64_t max_split = tuning().gemm_max_split ? tuning().gemm_max_split : (long_k ? 8 : 4);
  int64_t S = target / tiles;
  if (S > max_split) S = max_split;
  if (S > nsb) S = nsb;
  while (S > 1 && S * tiles * kGemmTileFloats > kGemmScratchFloats) --S;
  if (S < 1 || tiles > kGemmMaxTiles) S = 1;
  if (tuning().gemm_db && xb < (int64_t(1) << 32)) {   // 32-bit X offsets
    hipLaunchKernelGGL(gemm_q4_k_db_kernel, dim3((unsigned)gx, (unsigned)gy, (unsigned)S), dim3(256), 0,
                       stream, G, X, n_tokens, (int)nsb, scratch->gemm_partials, scratch->gemm_counters);
    return launch_status();
  }
  // the single-buffered kernel, one launch per matrix (its own split)
  for (int m = 0; m < G.n; ++m) {
    const int64_t gxm = (G.rows[m] + kGemmBN - 1) / kGemmBN, tm = gxm * gy;
    int64_t Sm = target / tm;
    if (Sm > max_split) Sm = max_split;
    if (Sm > nsb) Sm = nsb;
    while (Sm > 1 && Sm * tm * kGemmTileFloats > kGemmScratchFloats) --Sm;
    if (Sm < 1 || tm > kGemmMaxTiles) Sm = 1;
    hipLaunchKernelGGL(gemm_q4_k_kernel, dim3((unsigned)gxm, (unsigned)gy, (unsigned)Sm), dim3(256), 0,
                       stream, G.W[m], X, G.Y[m], n_tokens, G.rows[m], (int)nsb, scratch->gemm_partials,
                       scratch->gemm_counters);
    st = launch_status();
    if (st) return st;
  }
  return GGUF_QK_OK;
}

int gguf_qmatmul_q4_k(const void* W, const uint16_t* X, uint16_t* Y, int64_t n_tokens,
                      int64_t rows, int64_t cols, hipStream_t stream) {
  return matmul_q4_k_group(&W, &Y, &rows, 1, X, n_tokens, cols, stream);
}

int gguf_qmatmul_q4_k_multi(const void* const* W, uint16_t* const* Y, const int64_t* rows, int32_t n,
                            const uint16_t* X, int64_t n_tokens, int64_t cols, hipStream_t stream) {
  return matmul_q4_k_group(W, Y, rows, n, X, n_tokens, cols, stream);
}

// Small batch (fp32 X and Y, 32 tokens x 128 rows per block, K in steps of
// 256). Shares the prefill GEMM's partial-tile scratch and tile counters.
static_assert(kSbCounterStride == kGemmCounterStride, "shared tile counters");

static int small_batch_group(int type, const void* const* W, float* const* Y, const int64_t* rows, int n,
                             const float* X, int64_t n_tokens, int64_t cols, hipStream_t stream) {
  if (!W || !Y || !rows) return GGUF_QK_ERR_NULL;
  if (n < 1 || n > kSbMaxGroup) return GGUF_QK_ERR_SHAPE;
  int64_t wb[kSbMaxGroup] = {0, 0, 0, 0};
  for (int m = 0; m < n; ++m) {
    if (rows[m] < 0) return GGUF_QK_ERR_SHAPE;
    if (rows[m] == 0 && n > 1) {   // skipped: its W and Y are not touched (may be null)
      const int64_t rb = row_bytes_of(type, cols);
      if (rb < 0) return (int)rb;
      continue;
    }
    const int st = check_matrix(type, W[m], rows[m], cols, &wb[m]);
    if (st) return st;
    if (!Y[m]) return GGUF_QK_ERR_NULL;
    if (!aligned16(Y[m])) return GGUF_QK_ERR_ALIGN;
  }
  if (!X) return GGUF_QK_ERR_NULL;
  if (n_tokens < 0 || cols % kSbK) return GGUF_QK_ERR_SHAPE;
  if (!aligned16(X)) return GGUF_QK_ERR_ALIGN;
  for (int m = 0; m < n; ++m)
    if (n_tokens > 0 && (cols > INT64_MAX / 4 / n_tokens || rows[m] > INT64_MAX / 4 / n_tokens))
      return GGUF_QK_ERR_SHAPE;
  const int64_t xb = n_tokens * cols * 4;
  for (int m = 0; m < n; ++m) {
    if (rows[m] == 0) continue;
    const int64_t yb = n_tokens * rows[m] * 4;
    if (overlap(Y[m], yb, X, xb)) return GGUF_QK_ERR_ALIAS;
    for (int o = 0; o < n; ++o) {
      if (rows[o] == 0) continue;
      if (overlap(Y[m], yb, W[o], wb[o])) return GGUF_QK_ERR_ALIAS;
      if (o != m && overlap(Y[m], yb, Y[o], n_tokens * rows[o] * 4)) return GGUF_QK_ERR_ALIAS;
    }
  }
  if (n_tokens == 0) return GGUF_QK_OK;
  const int64_t steps = cols / kSbK;
  if (row_bytes_of(type, cols) * kSbRows > INT32_MAX || n_tokens > INT32_MAX || steps > INT32_MAX)
    return GGUF_QK_ERR_LIMIT;   // 32-bit offsets inside a block's rows
  SbGroup G{};
  int64_t gx = 0;
  for (int m = 0; m < n; ++m) {
    if (rows[m] == 0) continue;
    G.W[G.n] = static_cast<const uint8_t*>(W[m]);
    G.Y[G.n] = Y[m];
    G.rows[G.n] = rows[m];
    G.tile_begin[G.n] = (int)gx;
    ++G.n;
    gx += (rows[m] + kSbRows - 1) / kSbRows;
    if (gx > INT32_MAX) return GGUF_QK_ERR_LIMIT;
  }
  if (G.n == 0) return GGUF_QK_OK;
  const int64_t gy = (n_tokens + kSbTokens - 1) / kSbTokens;
  if (gy > 65535) return GGUF_QK_ERR_LIMIT;
  ScratchArea* scratch = nullptr;
  const int st = current_device(&scratch);
  if (st) return st;
  // Split K over whole steps when the tiles alone do not fill the device, as
  // far as the partial-tile scratch allows.
  const int64_t tiles = gx * gy;
  int64_t S = tuning().sb_blocks / tiles;
  if (S > tuning().sb_max_split) S = tuning().sb_max_split;
  if (S > steps) S = steps;
  while (S > 1 && S * tiles * kSbTileFloats > kGemmScratchFloats) --S;
  if (S < 1 || tiles > kGemmMaxTiles) S = 1;
  const dim3 grid((unsigned)gx, (unsigned)gy, (unsigned)S), block(256);
  if (type == GGUF_QK_TYPE_Q4_K)
    hipLaunchKernelGGL(gemv_small_batch_kernel<true>, grid, block, 0, stream, G, X, (int)n_tokens,
                       (int)steps, scratch->gemm_partials, scratch->gemm_counters);
  else
    hipLaunchKernelGGL(gemv_small_batch_kernel<false>, grid, block, 0, stream, G, X, (int)n_tokens,
                       (int)steps, scratch->gemm_partials, scratch->gemm_counters);
  return launch_status();
}

static int small_batch_common(int type, const void* W, const float* X, float* Y, int64_t n_tokens,
                              int64_t rows, int64_t cols, hipStream_t stream) {
  return small_batch_group(type, &W, &Y, &rows, 1, X, n_tokens, cols, stream);
}

int gguf_qmatmul_f32_q8_0(const void* W, const float* X, float* Y, int64_t n_tokens, int64_t rows,
                          int64_t cols, hipStream_t stream) {
  return small_batch_common(GGUF_QK_TYPE_Q8_0, W, X, Y, n_tokens, rows, cols, stream);
}

int gguf_qmatmul_f32_q4_k(const void* W, const float* X, float* Y, int64_t n_tokens, int64_t rows,
                          int64_t cols, hipStream_t stream) {
  return small_batch_common(GGUF_QK_TYPE_Q4_K, W, X, Y, n_tokens, rows, cols, stream);
}

int gguf_qmatmul_f32_q8_0_multi(const void* const* W, float* const* Y, const int64_t* rows, int32_t n,
                                const float* X, int64_t n_tokens, int64_t cols, hipStream_t stream) {
  return small_batch_group(GGUF_QK_TYPE_Q8_0, W, Y, rows, n, X, n_tokens, cols, stream);
}

int gguf_qmatmul_f32_q4_k_multi(const void* const* W, float* const* Y, const int64_t* rows, int32_t n,
                                const float* X, int64_t n_tokens, int64_t cols, hipStream_t stream) {
  return small_batch_group(GGUF_QK_TYPE_Q4_K, W, Y, rows, n, X, n_tokens, cols, stream);
}

// Standalone layer steps (vectors of n fp32).
static int vec_check(std::initializer_list<const void*> ptrs, int64_t n) {
  for (const void* p : ptrs) {
    if (!p) return GGUF_QK_ERR_NULL;
    if (!aligned16(p)) return GGUF_QK_ERR_ALIGN;
  }
  if (n < 0 || n > INT64_MAX / 4) return GGUF_QK_ERR_SHAPE;
  return GGUF_QK_OK;
}

int gguf_rmsnorm_prep_f32(const float* v, const float* norm_w, float* vw, float* ss, int64_t n,
                          hipStream_t stream) {
  int st = vec_check({v, norm_w, vw, ss}, n);
  if (st) return st;
  const int64_t groups = (n + 63) / 64;
  if (overlap(vw, n * 4, v, n * 4) || overlap(vw, n * 4, norm_w, n * 4) ||
      overlap(ss, groups * 4, v, n * 4) || overlap(ss, groups * 4, norm_w, n * 4) ||
      overlap(ss, groups * 4, vw, n * 4))
    return GGUF_QK_ERR_ALIAS;
  if (n == 0) return GGUF_QK_OK;
  st = current_device(nullptr);
  if (st) return st;
  if ((groups + 3) / 4 > INT32_MAX) return GGUF_QK_ERR_LIMIT;
  hipLaunchKernelGGL(rmsnorm_prep_kernel, dim3((unsigned)((groups + 3) / 4)), dim3(256), 0, stream,
                     v, norm_w, vw, ss, n);
  return launch_status();
}

int gguf_rmsnorm_f32(const float* v, const float* norm_w, float eps, float* out, int64_t n,
                     hipStream_t stream) {
  int st = vec_check({v, norm_w, out}, n);
  if (st) return st;
  if (!(eps >= 0.f) || eps > 3.0e38f) return GGUF_QK_ERR_SHAPE;
  if (overlap(out, n * 4, v, n * 4) || overlap(out, n * 4, norm_w, n * 4)) return GGUF_QK_ERR_ALIAS;
  if (n == 0) return GGUF_QK_OK;
  st = current_device(nullptr);
  if (st) return st;
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(1), dim3(1024), 0, stream, v, norm_w, eps, out, n);
  return launch_status();
}

static int elementwise2(int kind, const float* a, const float* b, float* out, int64_t n,
                        hipStream_t stream) {
  int st = vec_check({a, b, out}, n);
  if (st) return st;
  // out may be a or b exactly (each element is read before it is written by
  // the same thread), not a partial overlap
  if ((out != a && overlap(out, n * 4, a, n * 4)) || (out != b && overlap(out, n * 4, b, n * 4)))
    return GGUF_QK_ERR_ALIAS;
  if (n == 0) return GGUF_QK_OK;
  st = current_device(nullptr);
  if (st) return st;
  if ((n + 255) / 256 > INT32_MAX) return GGUF_QK_ERR_LIMIT;
  const dim3 grid((unsigned)((n + 255) / 256)), block(256);
  if (kind == 0)
    hipLaunchKernelGGL(swiglu_kernel, grid, block, 0, stream, a, b, out, n);
  else
    hipLaunchKernelGGL(add_kernel, grid, block, 0, stream, a, b, out, n);
  return launch_status();
}

int gguf_swiglu_f32(const float* g, const float* u, float* out, int64_t n, hipStream_t stream) {
  return elementwise2(0, g, u, out, n, stream);
}

int gguf_add_f32(const float* a, const float* b, float* out, int64_t n, hipStream_t stream) {
  return elementwise2(1, a, b, out, n, stream);
}

int gguf_qk_probe_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  if (!buf || !sink) return GGUF_QK_ERR_NULL;
  if (bytes < 0 || bytes % 16) return GGUF_QK_ERR_SHAPE;
  if (!aligned16(buf) || !aligned16(sink)) return GGUF_QK_ERR_ALIGN;
  if (overlap(sink, 4, buf, bytes)) return GGUF_QK_ERR_ALIAS;
  if (bytes == 0) return GGUF_QK_OK;
  int st = current_device(nullptr);
  if (st) return st;
  int cus = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();
    return GGUF_QK_ERR_DEVICE;
  }
  const int64_t n16 = bytes / 16;
  int64_t blocks = (int64_t)cus * 8;
  const int64_t need = (n16 + kProbeThreads - 1) / kProbeThreads;
  if (blocks > need) blocks = need;
  hipLaunchKernelGGL(probe_read_kernel, dim3((unsigned)blocks), dim3(kProbeThreads), 0, stream,
                     static_cast<const u32x4*>(buf), n16, sink);
  return launch_status();
}

}  // extern "C"
