// Definitions shared by the decode kernels (score, select, attend, combine).
#pragma once

#include "append_items.h"

namespace spla {
namespace {

__device__ __forceinline__ int n_blocks(const DecodeArgs& a, int b) { return (a.lens[b] + a.bk - 1) / a.bk; }

// Kernel arguments live in memory and are read with scalar loads.  Left to
// itself the compiler issues each load next to its first use, so a kernel that
// branches on one argument before it needs the next pays one memory round trip
// per step.  Passing the values through an empty asm statement makes it issue
// all of their loads as one batch ahead of it (one round trip).
#define SPLA_SCALARS_READY(...) asm volatile("" ::__VA_ARGS__)

}  // namespace
}  // namespace spla


// each launcher returns the status of its own launch (hipLaunchKernel /
// hipExtLaunchKernel report it directly, so an error left behind by an
// unrelated earlier HIP call is never attributed to it)
#define SPLA_DISPATCH_D(D_, ...)                                     \
  switch (D_) {                                                     \
    case 64: { constexpr int DD = 64; return __VA_ARGS__; }         \
    case 128: { constexpr int DD = 128; return __VA_ARGS__; }       \
    default: return hipErrorInvalidValue;                           \
  }
#define SPLA_DISPATCH_RD(R_, D_, ...)                                         \
  switch (R_) {                                                              \
    case 1: { constexpr int RR = 1; SPLA_DISPATCH_D(D_, __VA_ARGS__) }       \
    case 2: { constexpr int RR = 2; SPLA_DISPATCH_D(D_, __VA_ARGS__) }       \
    case 4: { constexpr int RR = 4; SPLA_DISPATCH_D(D_, __VA_ARGS__) }       \
    case 8: { constexpr int RR = 8; SPLA_DISPATCH_D(D_, __VA_ARGS__) }       \
    default: return hipErrorInvalidValue;                                    \
  }

