// Hand-offs between the workgroups of one (sequence, KV head) pair inside
// one kernel, through a counter in the L2 of the XCD they all run on
// (workgroups go to the XCDs in turn by linear id, so ids equal modulo 8
// share an XCD).  A waiting workgroup only ever waits on workgroups with
// smaller linear ids, which are dispatched before it and never wait
// themselves; the wait is bounded all the same.  Counter line of a pair:
// [0] producers done, [1] attend workgroups past their wait (one-kernel
// step), [2] the producers' XCD mask.
#pragma once

#include "decode_common.h"

namespace spla {
namespace {

constexpr int kSpinLimit = 1 << 20;
constexpr int kPollSleep = 1;  // s_sleep units (64 clocks) between polls

// producer: this workgroup's stores have reached the L2, then the count
// (and the producers' XCD mask, which the attend workgroups check)
__device__ __forceinline__ void step_signal(int32_t* ctr) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_or(ctr + 2, 1 << xcc_id(), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
}

// attend: wait until the pair's producer count reaches `target`.  The poll
// is an atomic (performed in the L2, where the producers' adds are); a load
// would not do: even a load marked to skip the CU's L1 has been seen to
// return a stale count from it for as long as the wait lasted.
__device__ __forceinline__ void step_wait(int32_t* ctr, int target, uint32_t* err) {
  if (threadIdx.x == 0) {
    // an add of a zero the compiler cannot see as one (an add of a known zero
    // would become a load)
    int zero;
    asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
    int n = 0;
    for (int spin = 0;; ++spin) {
      n = __hip_atomic_fetch_add(ctr, zero, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      if (n >= target) break;
      if (spin >= kSpinLimit) {
        atomicOr(err, kErrStepWait);
        break;
      }
      __builtin_amdgcn_s_sleep(kPollSleep);
    }
    if (n > target) atomicOr(err, kErrStepCount);  // a count the previous call did not clear
  }
  __syncthreads();
}

// the pair's XCD mask as the L2 holds it (an or of a zero the compiler cannot
// see as one: an or of a known zero would become a load)
__device__ __forceinline__ int step_mask(int32_t* ctr) {
  int zero;
  asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
  return __hip_atomic_fetch_or(ctr + 2, zero, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

}  // namespace
}  // namespace spla
