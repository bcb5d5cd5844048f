// Device-side signal primitives: the HIP meaning of the pages' wait / notify /
// consume_token (Triton-distributed semantics page, "Signal-based
// synchronization" and "Token-based data dependency"; paper summary, "Method":
// set / check / spin-lock signal operations on flag words).
//
// notify(set)    -> flag_release: all prior stores of the calling thread (and,
//                   through a preceding __syncthreads, of its workgroup) are
//                   made visible at agent scope, then the flag word is stored.
//                   On gfx950 the compiler emits an L2 write-back (buffer_wbl2
//                   sc1) before the store, which also covers the XCD-private L2.
// wait(ptr, n)   -> wait_flags: one thread polls n consecutive flag words with
//                   relaxed agent-scope loads (they bypass the stale L2 copy),
//                   sleeping between polls, until each holds the call's epoch.
// consume_token  -> the acquire fence after the poll (L2/L1 invalidate, so no
//                   stale line of the tile survives) followed by __syncthreads():
//                   no load of the tile can be issued before the wait ends,
//                   which is what the token's data dependency guarantees on the
//                   pages.
//
// Every wait is bounded by a tick budget of the 100 MHz constant clock; on
// expiry the first failing workgroup records the flag, the value seen and the
// value expected in the device status word, and the caller returns early.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace sgt {

__device__ __forceinline__ uint64_t clock_ticks() { return wall_clock64(); }

__device__ __forceinline__ bool flag_is_set(uint32_t v, uint32_t epoch) { return (int32_t)(v - epoch) >= 0; }

__device__ __forceinline__ uint32_t flag_peek(const uint32_t* f) {
  return __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void flag_release(uint32_t* f, uint32_t epoch) {
  __hip_atomic_store(f, epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void acquire_agent() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

__device__ inline void report_timeout(uint32_t* status, int64_t flag, uint32_t seen, uint32_t expected) {
  if (atomicCAS(status, 0u, kStatusTimeout) == 0u) {
    status[1] = (uint32_t)flag;
    status[2] = seen;
    status[3] = expected;
    __threadfence();
  }
}

// Single-thread wait for flags[f0 .. f1) (pages' wait(ptr, n) with n = f1 - f0).
// Returns true when all are set; false after the time budget (status recorded).
__device__ inline bool wait_flags_one_thread(const uint32_t* flags, int64_t f0, int64_t f1, uint32_t epoch,
                                             uint64_t timeout_ticks, uint32_t* status) {
  const uint64_t t0 = clock_ticks();
  for (int64_t f = f0; f < f1; ++f) {
    uint32_t v = flag_peek(flags + f);
    while (!flag_is_set(v, epoch)) {
      if (clock_ticks() - t0 > timeout_ticks) {
        report_timeout(status, f, v, epoch);
        return false;
      }
      __builtin_amdgcn_s_sleep(2);
      v = flag_peek(flags + f);
    }
  }
  acquire_agent();
  return true;
}

// Workgroup-wide wait: thread 0 polls, then every thread passes a barrier.
// `ok` must be a __shared__ int.  Returns the shared verdict.
__device__ inline bool wait_flags_block(const uint32_t* flags, int64_t f0, int64_t f1, uint32_t epoch,
                                        uint64_t timeout_ticks, uint32_t* status, int* ok) {
  if (threadIdx.x == 0) *ok = wait_flags_one_thread(flags, f0, f1, epoch, timeout_ticks, status) ? 1 : 0;
  __syncthreads();
  return *ok != 0;
}

// Workgroup-wide release of flags[f0 .. f1): every thread's prior global stores
// are ordered before the flag stores.
__device__ inline void release_flags_block(uint32_t* flags, int64_t f0, int64_t f1, uint32_t epoch) {
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0)
    for (int64_t f = f0; f < f1; ++f) flag_release(flags + f, epoch);
}

}  // namespace sgt
