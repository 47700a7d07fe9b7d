// Loads of split-K partial sums stored by other blocks.
#pragma once

#include <hip/hip_runtime.h>

namespace gqk {

// Eight fp32 loads of values that other blocks stored with agent-scope
// stores (split-K partial sums), in the form of the agent-scope relaxed atomic
// load (global_load_dword sc1), all eight in flight together: written as
// atomic loads, the compiler issued each one after the previous one had
// returned, a memory round trip per value. The block waits for the eight.
__device__ __forceinline__ void coherent_load8(const float* const (&p)[8], float (&v)[8]) {
  asm volatile(
      "global_load_dword %0, %8, off sc1\n"
      "global_load_dword %1, %9, off sc1\n"
      "global_load_dword %2, %10, off sc1\n"
      "global_load_dword %3, %11, off sc1\n"
      "global_load_dword %4, %12, off sc1\n"
      "global_load_dword %5, %13, off sc1\n"
      "global_load_dword %6, %14, off sc1\n"
      "global_load_dword %7, %15, off sc1\n"
      "s_waitcnt vmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
      : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]), "v"(p[4]), "v"(p[5]), "v"(p[6]), "v"(p[7])
      : "memory");
}

}  // namespace gqk
