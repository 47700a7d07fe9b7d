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
#include <thread>
#include <vector>

#include "../../include/gguf_file.h"
#include "../../include/gguf_qk.h"
#include "launch.hpp"
#include "dequant.hpp"
#include "gemm.hpp"
#include "gemv.hpp"
#include "gemv_other.hpp"
#include "gemv_small_batch.hpp"
#include "gemv_sbw.hpp"
#include "layer_ops.hpp"
#include "probe.hpp"
#include "timeline.hpp"

namespace gqk {

// Scratch for split-K partial sums and row-group counters, in slots: each
// stream that runs kernels needing scratch holds one slot of the device for
// the life of the process (or until gguf_qk_stream_release), so calls on
// different streams may overlap in time. The slots are a static device array
// (each GPU the library runs on holds its own copy for the life of the
// process); nothing is allocated at call time. Counters are zero at load and
// every kernel that uses one returns it to zero.
constexpr int64_t kScratchPartials = int64_t(2) << 20;   // floats (8 MiB)
constexpr int64_t kScratchCounters = int64_t(1) << 14;   // row-group counters
constexpr int kMaxSplits = 16;                            // K ranges per row group
// Prefill split K: fp32 partial tiles (32 MiB) and one counter per tile.
constexpr int64_t kGemmScratchFloats = int64_t(8) << 20;
constexpr int64_t kGemmMaxTiles = int64_t(1) << 12;
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
static_assert(GGUF_QK_STREAM_SLOTS >= 1, "at least one scratch slot");
static __device__ __attribute__((aligned(256))) ScratchArea g_scratch[GGUF_QK_STREAM_SLOTS];

constexpr int kMaxDevices = 64;

struct DeviceState {
  std::atomic<int> checked{0};   // 0 unknown, 1 gfx950, -1 unsupported
  ScratchArea* scratch = nullptr;   // this device's slot array
  std::mutex mu;
  // slot i is held by (stream[i], thread[i]) when held[i]; thread is only
  // part of the key for the per-thread default stream
  bool held[GGUF_QK_STREAM_SLOTS] = {};
  hipStream_t stream[GGUF_QK_STREAM_SLOTS] = {};
  std::thread::id thread[GGUF_QK_STREAM_SLOTS];
};
static DeviceState g_dev[kMaxDevices];

thread_local int g_last_launch = GGUF_QK_LAUNCH_NONE;

// Returns GGUF_QK_OK and the current device's index, or an error.
static int current_device(int* dev_out = nullptr) {
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
  if (dev_out) *dev_out = dev;
  return GGUF_QK_OK;
}

static bool same_holder(const DeviceState& st, int i, hipStream_t stream) {
  return st.held[i] && st.stream[i] == stream &&
         (stream != hipStreamPerThread || st.thread[i] == std::this_thread::get_id());
}

// The scratch slot of `stream` on the current device: the slot the stream
// already holds, else a free one (taken for it). GGUF_QK_ERR_LIMIT when every
// slot is held by another stream.
static int stream_scratch(hipStream_t stream, ScratchArea** out) {
  int dev = -1;
  const int st0 = current_device(&dev);
  if (st0) return st0;
  DeviceState& st = g_dev[dev];
  std::lock_guard<std::mutex> lk(st.mu);
  int free_slot = -1;
  for (int i = 0; i < GGUF_QK_STREAM_SLOTS; ++i) {
    if (same_holder(st, i, stream)) {
      *out = st.scratch + i;
      return GGUF_QK_OK;
    }
    if (!st.held[i] && free_slot < 0) free_slot = i;
  }
  if (free_slot < 0) return GGUF_QK_ERR_LIMIT;
  st.held[free_slot] = true;
  st.stream[free_slot] = stream;
  st.thread[free_slot] = std::this_thread::get_id();
  *out = st.scratch + free_slot;
  return GGUF_QK_OK;
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
  st = current_device();
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


static int launch_other(int type, const void* W, const float* x, float* y, int64_t rows,
                        int64_t cols, hipStream_t stream);

// Kernel family of one group: the lanes-along-K launches (no scratch) or the
// fallback GEMV kernels (split-K partials and counters in scratch).
enum class GroupKind { kLks, kLk, kOther, kFallback };

static GroupKind group_kind(int type, const gguf_qk_gemv* const* v, const GemvEpilogue* const* e, int n) {
  if (lks_fits(v, e, n, type)) return GroupKind::kLks;
  if (type == GGUF_QK_TYPE_Q4_K && tuning().q4k_lk && lk_fits(v, e, n)) return GroupKind::kLk;
  if (type == GGUF_QK_TYPE_Q4_0 || type == GGUF_QK_TYPE_Q6_K) {
    // rows of 256 .. 12288 weights in multiples of 256 (no epilogues on
    // these types): the lanes-along-K kernels; else the lane-quad kernel, one
    // launch each
    const bool on = type == GGUF_QK_TYPE_Q4_0 ? tuning().q4_0_lk : tuning().q6_k_lk;
    return on && lk_fits(v, nullptr, n) ? GroupKind::kLk : GroupKind::kOther;
  }
  if (type == GGUF_QK_TYPE_Q8_0 && tuning().q8_0_lk && v[0]->cols <= 4096 && lk_fits(v, nullptr, n)) {
    // Q8_0 rows of 256 .. 4096 weights (multiples of 256) without epilogues:
    // the lanes-along-K kernels; else the lane-per-row kernel
    bool ep = false;
    for (int i = 0; i < n; ++i) ep = ep || (e && e[i] && e[i]->flags != 0);
    if (!ep) return GroupKind::kLk;
  }
  return GroupKind::kFallback;
}

// Launches one planned group. scratch: the stream's slot; only the fallback
// kernels use it (null where no group of the call needs it).
static int launch_group(int type, const gguf_qk_gemv* const* v, const GemvEpilogue* const* e, int n,
                        ScratchArea* scratch, hipStream_t stream) {
  switch (group_kind(type, v, e, n)) {
    case GroupKind::kLks: return launch_lks(v, type == GGUF_QK_TYPE_Q4_K ? e : nullptr, n, stream, type);
    case GroupKind::kLk: return launch_lk(v, type == GGUF_QK_TYPE_Q4_K ? e : nullptr, n, stream, type);
    case GroupKind::kOther:
      g_last_launch = GGUF_QK_LAUNCH_OTHER;
      for (int i = 0; i < n; ++i) {
        const int st = launch_other(type, v[i]->W, v[i]->x, v[i]->y, v[i]->rows, v[i]->cols, stream);
        if (st) return st;
      }
      return GGUF_QK_OK;
    case GroupKind::kFallback: break;
  }
  if (!scratch) return GGUF_QK_ERR_LIMIT;
  g_last_launch = GGUF_QK_LAUNCH_SPLIT_K;
  GemvGroup grp;
  const int64_t tasks = plan_group(type, v, e, n, &grp);
  float* partials = scratch->partials;
  int* counters = scratch->counters;
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
  g_last_launch = GGUF_QK_LAUNCH_ROWWISE;
  const int64_t blocks = (g.rows + 3) / 4;
  if (blocks > INT32_MAX || g.cols / kQ80BlockWeights > INT32_MAX) return GGUF_QK_ERR_LIMIT;
  hipLaunchKernelGGL(gemv_q8_0_rowwise_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<const uint8_t*>(g.W), g.x, g.y, g.rows,
                     (int)(g.cols / kQ80BlockWeights));
  return launch_status();
}

// Groups the GEMVs of one step: same-format GEMVs go together, kMaxGroup at a
// time, in a fixed order; fn(type, group, epilogues, count) is called per
// group and single(g) for each Q8_0 GEMV whose rows are not a multiple of
// 256 weights. Stops at the first nonzero status.
extern "C++" {
template <class GroupFn, class SingleFn>
static int for_each_group(const gguf_qk_gemv* list, const GemvEpilogue* eps, int n, GroupFn&& fn,
                          SingleFn&& single) {
  for (int type : {GGUF_QK_TYPE_Q4_K, GGUF_QK_TYPE_Q4_0, GGUF_QK_TYPE_Q6_K, GGUF_QK_TYPE_Q8_0}) {
    const gguf_qk_gemv* grp[kMaxGroup];
    const GemvEpilogue* ge[kMaxGroup];
    int k = 0;
    for (int i = 0; i < n; ++i) {
      const gguf_qk_gemv& g = list[i];
      if (g.type != type || g.rows == 0) continue;
      if (type == GGUF_QK_TYPE_Q8_0 && g.cols % 256) {
        const int st = single(g);
        if (st) return st;
        continue;
      }
      // the two GEMVs of a gate/up pair go into one launch: a gate that would
      // take the last place of a group opens the next one
      if (k == kMaxGroup - 1 && eps && (eps[i].flags & kEpPair) && eps[i].role == 0) {
        const int st = fn(type, grp, ge, k);
        if (st) return st;
        k = 0;
      }
      ge[k] = eps ? &eps[i] : nullptr;
      grp[k++] = &g;
      if (k == kMaxGroup) {
        const int st = fn(type, grp, ge, k);
        if (st) return st;
        k = 0;
      }
    }
    if (k) {
      const int st = fn(type, grp, ge, k);
      if (st) return st;
    }
  }
  return GGUF_QK_OK;
}

}  // extern "C++"

// Whether any group of the step runs a kernel that needs scratch.
static bool step_needs_scratch(const gguf_qk_gemv* list, const GemvEpilogue* eps, int n) {
  bool need = false;
  for_each_group(
      list, eps, n,
      [&](int type, const gguf_qk_gemv* const* v, const GemvEpilogue* const* e, int k) {
        need = need || group_kind(type, v, e, k) == GroupKind::kFallback;
        return GGUF_QK_OK;
      },
      [](const gguf_qk_gemv&) { return GGUF_QK_OK; });
  return need;
}

// Launches the GEMVs of one step, each launch after the previous one on the
// stream. scratch: the stream's slot, or null when step_needs_scratch is false.
static int launch_step(const gguf_qk_gemv* list, const GemvEpilogue* eps, int n, ScratchArea* scratch,
                       hipStream_t stream) {
  return for_each_group(
      list, eps, n,
      [&](int type, const gguf_qk_gemv* const* v, const GemvEpilogue* const* e, int k) {
        return launch_group(type, v, e, k, scratch, stream);
      },
      [&](const gguf_qk_gemv& g) { return launch_rowwise_q8_0(g, stream); });
}

// Launches one step, taking the stream's scratch slot first when a kernel of
// the step needs it (so a step that cannot get one enqueues nothing).
static int run_step(const gguf_qk_gemv* list, const GemvEpilogue* eps, int n, ScratchArea* scratch,
                    hipStream_t stream) {
  if (!scratch && step_needs_scratch(list, eps, n)) {
    const int st = stream_scratch(stream, &scratch);
    if (st) return st;
  }
  return launch_step(list, eps, n, scratch, stream);
}

static int matvec_common(int type, const void* W, const float* x, float* y, int64_t rows,
                         int64_t cols, hipStream_t stream) {
  int64_t wb = 0;
  int st = check_gemv(type, W, x, y, rows, cols, &wb);
  if (st) return st;
  if (rows == 0) return GGUF_QK_OK;
  st = current_device();
  if (st) return st;
  const gguf_qk_gemv g{W, x, y, rows, cols, type, 0, {0}};
  return run_step(&g, nullptr, 1, nullptr, stream);
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
  if (e.scale_ss && e.scale_v) return GGUF_QK_ERR_SHAPE;
  if (e.scale_ss) {
    if (e.scale_n < 1 || e.scale_n > INT32_MAX || !(e.eps >= 0.f) || e.eps > 3.0e38f || !al4(e.scale_ss))
      return GGUF_QK_ERR_SHAPE;
    flags |= kEpScale;
  }
  if (e.scale_v) {
    if (!(e.eps >= 0.f) || e.eps > 3.0e38f || g.cols > INT32_MAX) return GGUF_QK_ERR_SHAPE;
    if (!aligned16(e.scale_v)) return GGUF_QK_ERR_ALIGN;
    // v is read while the step runs: no output of the step may overlap it
    for (int32_t b = 0; b < n; ++b)
      if (list[b].stage == g.stage && overlap(e.scale_v, g.cols * 4, list[b].y, list[b].rows * 4))
        return GGUF_QK_ERR_ALIAS;
    flags |= kEpScale | kEpScaleV;
  }
  if (e.residual) {
    if (!al4(e.residual)) return GGUF_QK_ERR_ALIGN;
    if (e.residual != g.y && overlap(e.residual, g.rows * 4, g.y, g.rows * 4)) return GGUF_QK_ERR_ALIAS;
    flags |= kEpResidual;
  }
  if (e.norm_w || e.norm_out || e.ss_out) {
    if (!e.norm_w || !e.norm_out) return GGUF_QK_ERR_NULL;
    if (!al4(e.norm_w) || !al4(e.norm_out) || (e.ss_out && !al4(e.ss_out))) return GGUF_QK_ERR_ALIGN;
    flags |= kEpNorm;
    if (e.ss_out) {
      flags |= kEpSs;
      // row-group counters for kernels whose blocks do not own whole row groups
      // (taken from the step's group counters when there are enough left)
      if (*pair_off + RG <= kPairCounters) {
        *norm_rg = *pair_off;
        *pair_off += RG;
      }
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
        overlap(outs[a], outn[a], e.scale_ss, e.scale_ss ? e.scale_n * 4 : 0) ||
        overlap(outs[a], outn[a], e.scale_v, e.scale_v ? g.cols * 4 : 0))
      return GGUF_QK_ERR_ALIAS;
  }
  if (flags && ((g.type == GGUF_QK_TYPE_Q8_0 && g.cols % 256) || g.type == GGUF_QK_TYPE_Q4_0 ||
                g.type == GGUF_QK_TYPE_Q6_K))
    return GGUF_QK_ERR_SHAPE;
  out->scale_ss = e.scale_v ? e.scale_v : e.scale_ss;
  out->residual = e.residual;
  out->norm_w = e.norm_w;
  out->norm_out = e.norm_out;
  out->ss_out = e.ss_out;
  out->scale_n = e.scale_v ? (int)g.cols : (int)e.scale_n;
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
  int st = current_device();
  if (st) return st;
  // the stream's scratch slot, taken before anything is enqueued when a pair
  // or norm epilogue counts row groups or a step runs a fallback kernel
  bool need = false;
  for (int32_t i = 0; i < (int32_t)eps.size(); ++i) need = need || pair_rg[i] >= 0 || norm_rg[i] >= 0;
  for (int32_t i = 0; i < n && !need;) {
    int32_t j = i;
    while (j < n && list[j].stage == list[i].stage) ++j;
    need = step_needs_scratch(list + i, ep ? eps.data() + i : nullptr, j - i);
    i = j;
  }
  ScratchArea* scratch = nullptr;
  if (need) {
    st = stream_scratch(stream, &scratch);
    if (st) return st;
  }
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
  st = current_device();
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
  st = current_device();
  if (st) return st;
  if (type == GGUF_QK_TYPE_Q4_0 || type == GGUF_QK_TYPE_Q6_K) {
    const gguf_qk_gemv g{W, x, y, rows, cols, type, 0, {0}};
    return run_step(&g, nullptr, 1, nullptr, stream);
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
  ScratchArea* scratch = nullptr;
  int st = stream_scratch(stream, &scratch);
  if (st) return st;
  const int64_t nsb = cols / kQ4KBlockWeights;
  // Split K over whole super-blocks when there are too few tiles to fill the
  // device, as far as the scratch for the fp32 partial tiles allows; the
  // split is then evened out (the fewest ranges that give the same longest
  // range). `target` blocks, at most `max_split` ranges.
  auto split_for = [&](int64_t tiles, int64_t tile_floats, int64_t target, int64_t max_split) {
    int64_t S = target / tiles;
    if (S > max_split) S = max_split;
    if (S > nsb) S = nsb;
    while (S > 1 && S * tiles * tile_floats > kGemmScratchFloats) --S;
    if (S < 1 || tiles > kGemmMaxTiles) S = 1;
    if (S > 1) {
      const int64_t per = (nsb + S - 1) / S;
      S = (nsb + per - 1) / per;
    }
    return S;
  };
  // Measured on the 2048-hidden shapes with 128-token blocks (one block per
  // CU: 288 registers a lane): about one round of blocks, K split into at
  // most 8 (long K: down, 43 super-blocks) or 4 (short K: 8 super-blocks)
  // ranges; down took 2 us less in one round of 4 ranges than in two rounds
  // of 8, and short K slows past 4 ranges, where the last block's sum over
  // the partial tiles costs more than the extra blocks save.
  const bool long_k = nsb >= 32;
  const int64_t target = tuning().gemm_blocks ? tuning().gemm_blocks : 256;
  const int64_t max_split = tuning().gemm_max_split ? tuning().gemm_max_split : (long_k ? 8 : 4);
  if (tuning().gemm_db && xb < (int64_t(1) << 32)) {   // 32-bit X offsets
    // Tiles [0, nfull) over all of K, the rest split S ways; the fp32 partial
    // tiles of the split ones must fit the scratch.
    auto launch_db = [&](auto kernel, int threads, int64_t tiles, int64_t nfull, int64_t S, int64_t tile_floats) {
      while (S > 1 && ((tiles - nfull) * S * tile_floats > kGemmScratchFloats || tiles - nfull > kGemmMaxTiles)) --S;
      if (S <= 1) {
        S = 1;
        nfull = tiles;
      }
      const int64_t blocks = nfull + (tiles - nfull) * S;
      if (blocks > INT32_MAX) return (int)GGUF_QK_ERR_LIMIT;
      hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(threads), 0, stream, G, X, n_tokens, (int)nsb,
                         (int)gx, (int)nfull, (int)S, scratch->gemm_partials, scratch->gemm_counters);
      return launch_status();
    };
    // The K ranges for tiles that would otherwise leave the device partly
    // idle: as many as fill `slots` blocks (at most max_split, at most one
    // super-block each), then evened out (the fewest ranges with the same
    // longest range).
    auto even_split = [&](int64_t tiles, int64_t slots) {
      int64_t S = slots / (tiles > 0 ? tiles : 1);
      if (S > max_split) S = max_split;
      if (S > nsb) S = nsb;
      if (S < 1) S = 1;
      const int64_t per = (nsb + S - 1) / S;
      return (nsb + per - 1) / per;
    };
    // 256-token blocks (half the weight decoding per MFMA of 128-token ones)
    // where they give at least a block per CU unsplit: whole rounds of one
    // block per CU (a 110 KB LDS tile) take all of K, and the tiles past the
    // last whole round are split so that they fill one short round instead
    // of a mostly idle full one (the prefill gate/up launch: 344 tiles, 256
    // whole + 88 split in two, 1.5 rounds of a whole tile's time instead of 2)
    const int64_t gy4 = (n_tokens + gdb_bm(4) - 1) / gdb_bm(4);
    const int64_t slots = tuning().gemm_wide_target;
    if (tuning().gemm_wide && n_tokens > gdb_bm(2) && gx * gy4 >= tuning().gemm_wide_tiles) {
      const int64_t tiles = gx * gy4;
      const int64_t nfull = tiles >= slots ? tiles / slots * slots : 0;
      return launch_db(gemm_q4_k_db_kernel<4>, 512, tiles, nfull, even_split(tiles - nfull, slots),
                       gdb_tile_floats(4));
    }
    // 128-token blocks: every tile split alike
    const int64_t gy = (n_tokens + gdb_bm(2) - 1) / gdb_bm(2);
    const int64_t S = split_for(gx * gy, gdb_tile_floats(2), target, max_split);
    return launch_db(gemm_q4_k_db_kernel<2>, 256, gx * gy, S > 1 ? 0 : gx * gy, S, gdb_tile_floats(2));
  }
  const int64_t gy = (n_tokens + kGemmBM - 1) / kGemmBM;
  if (gy > 65535) return GGUF_QK_ERR_LIMIT;
  // the single-buffered kernel, one launch per matrix (its own split)
  for (int m = 0; m < G.n; ++m) {
    const int64_t gxm = (G.rows[m] + kGemmBN - 1) / kGemmBN, tm = gxm * gy;
    const int64_t Sm = split_for(tm, kGemmTileFloats, target, max_split);
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

extern "C++" {
// Q4_K small batch on the matrix-core kernel of gemv_sbw.hpp: up to 16
// tokens per block (grid y past 16), one wave per super-block of a K range
// (K split over blocks so that a range has at most kSbwMaxWaves
// super-blocks), the split and the row tiles per block chosen below.
static int launch_sbw(const SbGroup& G, const float* X, int64_t n_tokens, int64_t nsb, hipStream_t stream) {
  int64_t tiles_of[kSbMaxGroup];
  for (int m = 0; m < G.n; ++m) {
    if (G.rows[m] > INT32_MAX) return GGUF_QK_ERR_LIMIT;
    tiles_of[m] = (G.rows[m] + 15) / 16;
  }
  const int64_t gy = (n_tokens + kSbwMaxTokens - 1) / kSbwMaxTokens;
  if (gy > 65535) return GGUF_QK_ERR_LIMIT;
  // K ranges: as few as the waves of a block allow (a split costs a round
  // trip of partial tiles through memory that is coherent across the XCDs,
  // several microseconds); row tiles per block rt by a cost model of the
  // launch's time: rounds of blocks (a compute unit holds 8 / nw blocks of nw
  // waves) times a block's bytes per wave (rt tiles of 2304 weight bytes, the
  // super-block's activations at 1 KiB per token), scaled up when fewer than
  // 256 blocks or 1024 waves leave compute units or load slots idle; ties to
  // fewer tiles
  const int64_t s_min = (nsb + kSbwMaxWaves - 1) / kSbwMaxWaves;
  const int64_t ntok = n_tokens < kSbwMaxTokens ? n_tokens : kSbwMaxTokens;
  const bool pair = ntok <= 8;   // the paired layout (staging and sums side by side in LDS)
  int64_t S = s_min, rt = 1;
  {
    const int64_t nw = (nsb + S - 1) / S, per_cu = kSbwMaxWaves / nw;
    double best = -1.0;
    for (int64_t r = 1; r <= kSbwMaxTiles; ++r) {
      if (sbw_lds_bytes((int)r, (int)nw, pair ? 8 : 16, pair) > kSbwLdsLimit) break;
      int64_t blocks = 0;
      for (int m = 0; m < G.n; ++m) blocks += (tiles_of[m] + r - 1) / r;
      blocks *= gy * S;
      const int64_t rounds = (blocks + 256 * per_cu - 1) / (256 * per_cu);
      double cost = (double)rounds * (double)(23 * r + 10 * ntok);
      if (blocks < 256) cost *= 256.0 / (double)blocks;
      if (blocks * nw < 1024) cost *= 1024.0 / (double)(blocks * nw);
      if (best < 0 || cost < best) {
        best = cost;
        rt = r;
      }
    }
  }
  if (S > 65535) return GGUF_QK_ERR_LIMIT;
  const uint8_t* Wm[kSbMaxGroup] = {nullptr, nullptr, nullptr, nullptr};
  int rows_m[kSbMaxGroup] = {0, 0, 0, 0};
  SbwRest rest{};
  int64_t gx = 0;   // (the kernel finds each matrix's first block the same way)
  for (int m = 0; m < G.n; ++m) {
    Wm[m] = static_cast<const uint8_t*>(G.W[m]);
    rest.Y[m] = G.Y[m];
    rows_m[m] = (int)G.rows[m];
    gx += (tiles_of[m] + rt - 1) / rt;
    if (gx > INT32_MAX) return GGUF_QK_ERR_LIMIT;
  }
  rest.W3 = Wm[3];
  rest.rows3 = rows_m[3];
  const int64_t ntiles = gx * gy, tile_floats = rt * 256;
  if (S > 1 && (S * ntiles * tile_floats > kGemmScratchFloats || ntiles > kGemmMaxTiles)) return GGUF_QK_ERR_LIMIT;
  const int nw = (int)((nsb + S - 1) / S);   // the longest range
  ScratchArea* scratch = nullptr;
  if (S > 1) {
    const int st = stream_scratch(stream, &scratch);
    if (st) return st;
  }
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemv_sbw_kernel<false>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSbwLdsLimit);
  static const hipError_t attr_pair = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemv_sbw_kernel<true>),
                                                          hipFuncAttributeMaxDynamicSharedMemorySize,
                                                          (int)kSbwLdsLimit);
  if (attr != hipSuccess || attr_pair != hipSuccess) return GGUF_QK_ERR_LAUNCH;
  // (the scratch is only touched when S > 1)
  rest.partials = scratch ? scratch->gemm_partials : nullptr;
  rest.counters = scratch ? scratch->gemm_counters : nullptr;
  const dim3 grid((unsigned)gx, (unsigned)gy, (unsigned)S), block(64 * nw);
  const size_t lds = sbw_lds_bytes((int)rt, nw, pair ? 8 : 16, pair);
  static_assert(sbw_lds_bytes(kSbwMaxTiles, kSbwMaxWaves, 16, false) <= kSbwLdsLimit, "shared staging fits");
  if (lds > kSbwLdsLimit) return GGUF_QK_ERR_LIMIT;
  const uint32_t shape = sbw_shape(nw, (int)rt, G.n, (int)S);
  if (pair)
    hipLaunchKernelGGL(gemv_sbw_kernel<true>, grid, block, lds, stream, Wm[0], Wm[1], Wm[2], X, (int)nsb,
                       (int)n_tokens, shape, rows_m[0], rows_m[1], rows_m[2], rest);
  else
    hipLaunchKernelGGL(gemv_sbw_kernel<false>, grid, block, lds, stream, Wm[0], Wm[1], Wm[2], X, (int)nsb,
                       (int)n_tokens, shape, rows_m[0], rows_m[1], rows_m[2], rest);
  return launch_status();
}
}  // extern "C++"

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
  // Q4_K up to 32 tokens: the super-block-per-wave kernel (16 tokens per
  // block, weights read once per 16 tokens); more tokens and Q8_0 below
  // (measured at 64 tokens: 4.05 ms per pass there against 3.21 below)
  if (type == GGUF_QK_TYPE_Q4_K && n_tokens <= kSbwRouteTokens) return launch_sbw(G, X, n_tokens, steps, stream);
  const int64_t gy = (n_tokens + kSbTokens - 1) / kSbTokens;
  if (gy > 65535) return GGUF_QK_ERR_LIMIT;
  ScratchArea* scratch = nullptr;
  const int st = stream_scratch(stream, &scratch);
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
  st = current_device();
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
  st = current_device();
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
  st = current_device();
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

#if GQK_TIMELINE
extern "C++" {
namespace gqk {
std::vector<TlBindFn>& tl_registry() {
  static std::vector<TlBindFn> r;
  return r;
}
}  // namespace gqk
}
static TlRec* g_tl_recs_dev = nullptr;
#endif

int gguf_qk_timeline_setup(uint64_t mult) {
#if GQK_TIMELINE
  if (mult && !(mult & 1u)) return GGUF_QK_ERR_SHAPE;
  int st = current_device();
  if (st) return st;
  const size_t bytes = sizeof(TlRec) * (size_t)kTlSlots * kTlWaves;
  // the instrumented build's own record buffer (the default build allocates nothing)
  if (!g_tl_recs_dev && hipMalloc(&g_tl_recs_dev, bytes) != hipSuccess) {
    (void)hipGetLastError();
    return GGUF_QK_ERR_DEVICE;
  }
  if (hipMemset(g_tl_recs_dev, 0, bytes) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
    (void)hipGetLastError();
    return GGUF_QK_ERR_DEVICE;
  }
  const TlState s{mult, g_tl_recs_dev};
  for (TlBindFn f : tl_registry())
    if (f(s)) return GGUF_QK_ERR_DEVICE;
  return GGUF_QK_OK;
#else
  (void)mult;
  return GGUF_QK_ERR_LIMIT;
#endif
}

int gguf_qk_timeline_fetch(void* host_out, int64_t bytes) {
#if GQK_TIMELINE
  if (!host_out) return GGUF_QK_ERR_NULL;
  if (bytes != (int64_t)(sizeof(TlRec) * (size_t)kTlSlots * kTlWaves)) return GGUF_QK_ERR_SHAPE;
  if (!g_tl_recs_dev) return GGUF_QK_ERR_LIMIT;
  if (hipMemcpy(host_out, g_tl_recs_dev, (size_t)bytes, hipMemcpyDeviceToHost) != hipSuccess) {
    (void)hipGetLastError();
    return GGUF_QK_ERR_DEVICE;
  }
  return GGUF_QK_OK;
#else
  (void)host_out;
  (void)bytes;
  return GGUF_QK_ERR_LIMIT;
#endif
}

int gguf_qk_last_launch(void) { return g_last_launch; }

int gguf_qk_stream_release(hipStream_t stream) {
  int dev = -1;
  const int st = current_device(&dev);
  if (st) return st;
  DeviceState& ds = g_dev[dev];
  std::lock_guard<std::mutex> lk(ds.mu);
  for (int i = 0; i < GGUF_QK_STREAM_SLOTS; ++i)
    if (same_holder(ds, i, stream)) ds.held[i] = false;
  return GGUF_QK_OK;
}

int gguf_qk_probe_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  if (!buf || !sink) return GGUF_QK_ERR_NULL;
  if (bytes < 0 || bytes % 16) return GGUF_QK_ERR_SHAPE;
  if (!aligned16(buf) || !aligned16(sink)) return GGUF_QK_ERR_ALIGN;
  if (overlap(sink, 4, buf, bytes)) return GGUF_QK_ERR_ALIAS;
  if (bytes == 0) return GGUF_QK_OK;
  int st = current_device();
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

int gguf_qk_probe_latency(const uint32_t* next, int64_t n, int64_t steps, uint64_t* out, hipStream_t stream) {
  if (!next || !out) return GGUF_QK_ERR_NULL;
  if (n < 64 || n > (int64_t(1) << 31) || (n & (n - 1)) || steps < 1) return GGUF_QK_ERR_SHAPE;
  if (!aligned16(next) || !aligned16(out)) return GGUF_QK_ERR_ALIGN;
  if (overlap(out, 16, next, n * 4)) return GGUF_QK_ERR_ALIAS;
  const int st = current_device();
  if (st) return st;
  hipLaunchKernelGGL(probe_chase_kernel, dim3(1), dim3(64), 0, stream, next, (uint32_t)(n - 1), steps, out);
  return launch_status();
}

}  // extern "C"
