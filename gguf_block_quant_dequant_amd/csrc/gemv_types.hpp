// Plain types and helpers shared by the GEMV kernel families (lane per row,
// lanes along K) and the host code that launches them.
#pragma once

#include "device_common.hpp"

namespace gqk {

constexpr int kQ40BlockBytes = 18;   // fp16 d + 16 bytes of 4-bit codes
constexpr int kQ40BlockWeights = 32;

// Row-group counters sit one per 128-byte line: atomics on one line are
// serialized where they execute (about 12 ns each on this device), so
// counters sharing a line would queue behind each other.
constexpr int kCounterStride = 32;   // ints

struct SplitK {
  float* partials;   // [P][rows] floats
  int* counters;     // [row groups] ints at stride kCounterStride, zero between calls
};

// What the wave that holds a row group's final sums does with them (the steps
// either side of the decode GEMVs, "GGUF Inferencer in R", section 5.2, fused
// into the GEMV that produces or consumes their vector). flags == 0: store y.
//  kEpScale    y = s * (W x), s = 1 / sqrt(sum(scale_ss[0..scale_n)) * inv_k + eps):
//              RMSN of the input when x holds v * norm and scale_ss the partial
//              sums of v^2 (the scalar factor of RMSN moves past the product)
//  kEpResidual y += residual (the residual add)
//  kEpNorm     also norm_out = y * norm_w: the next RMSN's input
//  kEpSs       (with kEpNorm) also ss_out[rg] = sum of y^2 over the row group's
//              rows (fixed butterfly order): the next RMSN's partial sums
//  kEpScaleV   (with kEpScale) scale_ss is v itself (scale_n = cols floats) and
//              the kernel forms sum(v^2) in a fixed order
//  kEpPair     one of a gate/up pair: the second of the pair to finish a row
//              group writes act = SiLU(gate) * up for it (y stores and the
//              partner's loads are agent-scope; a counter per row group)
constexpr int kEpScale = 1, kEpResidual = 2, kEpNorm = 4, kEpPair = 8;
// A gate/up pair whose rows the lanes-along-K kernel computes in the same
// wave (the gate's descriptor carries both; set by the host, never by users).
constexpr int kEpPairInWave = 16;
constexpr int kEpSs = 32, kEpScaleV = 64;

struct GemvEpilogue {
  const float* scale_ss;
  const float* residual;
  const float* norm_w;
  float* norm_out;
  float* ss_out;
  float* act;
  const float* partner_y;
  int* pair_cnt;       // [row groups] at stride kCounterStride, zero between calls
  int scale_n;
  float eps;
  float inv_k;         // 1 / length of the normalized vector
  int flags;
  int role;            // pair: 0 gate, 1 up
  int* norm_cnt;       // [row groups] at stride kCounterStride, zero between calls: the
                       // lanes-along-K kernels count finished rows of a row group before
                       // its ss_out sum (a block kernel owns whole row groups, no count)
};

__device__ __forceinline__ float wave_sum_fixed(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

}  // namespace gqk
