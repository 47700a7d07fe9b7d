// Per-wave stage timelines of the decode GEMV kernels, compiled in only when
// GQK_TIMELINE is set (the instrumented library, libgguf_qk_timeline.so; the
// default build has none of it).
//
// A kernel wave takes up to six time stamps of the device's constant 100 MHz
// clock (s_memrealtime) at fixed points of its work and lane 0 writes them,
// with its hardware wave id and XCD, to a record. Records are addressed by a
// hash of the launch's key (the first weight pointer of the launch: slot =
// the top 12 bits of key * mult, mult chosen by the host so that the traced
// keys take distinct slots) and the wave's index in the grid, so a pass of
// the decode stream fills one slot per (launch, wave) with no atomics and no
// lookups; a replay overwrites the previous pass's records.
//   t0 kernel entry          t3 first row step computed and stored
//   t1 loads issued          t4 last row step computed
//   t2 activations staged    t5 epilogue done (end)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#if GQK_TIMELINE
#include <vector>
#endif

namespace gqk {

constexpr int kTlSlots = 4096;   // launch slots (12-bit hash)
constexpr int kTlWaves = 2048;   // waves tracked per launch

struct TlRec {
  uint32_t t[6];
  uint32_t hwid;   // HW_ID register: wave, SIMD, CU, shader array, shader engine
  uint32_t xcc;    // XCD of the wave
};

struct TlState {
  uint64_t mult;   // slot of key k: (k * mult) >> 52; 0: nothing is traced
  TlRec* recs;     // [kTlSlots][kTlWaves]
};

struct TlStamps {
#if GQK_TIMELINE
  uint32_t t[6] = {0, 0, 0, 0, 0, 0};
  __device__ __forceinline__ void stamp(int i) { t[i] = (uint32_t)__builtin_amdgcn_s_memrealtime(); }
#else
  __device__ __forceinline__ void stamp(int) {}
#endif
};

#if GQK_TIMELINE
// One copy per translation unit (no relocatable device code): the host binds
// every unit's copy to the same buffers (tl_registry).
static __device__ TlState g_tl;

__device__ __forceinline__ void tl_put(const void* key, const TlStamps& s) {
  const uint64_t mult = g_tl.mult;
  const int slot = (int)(((uint64_t)(uintptr_t)key * mult) >> 52);
  const int gw = (int)blockIdx.x * (int)(blockDim.x >> 6) + (int)(threadIdx.x >> 6);
  if (mult == 0 || gw >= kTlWaves || (threadIdx.x & 63) != 0) return;
  TlRec r;
#pragma unroll
  for (int i = 0; i < 6; ++i) r.t[i] = s.t[i];
  r.hwid = (uint32_t)__builtin_amdgcn_s_getreg((31 << 11) | 4);    // HW_REG_HW_ID, 32 bits
  r.xcc = (uint32_t)__builtin_amdgcn_s_getreg((15 << 11) | 20);    // HW_REG_XCC_ID, 16 bits
  g_tl.recs[(int64_t)slot * kTlWaves + gw] = r;
}

using TlBindFn = int (*)(const TlState&);
std::vector<TlBindFn>& tl_registry();

namespace {
struct TlRegister {
  TlRegister() {
    tl_registry().push_back(+[](const TlState& s) -> int {
      return hipMemcpyToSymbol(HIP_SYMBOL(g_tl), &s, sizeof s) == hipSuccess ? 0 : -1;
    });
  }
};
static TlRegister tl_register_;
}  // namespace
#else
__device__ __forceinline__ void tl_put(const void*, const TlStamps&) {}
#endif

}  // namespace gqk
