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
//                   flag_publish_coherent is the cheaper form for data written
//                   with device-scope (sc1) stores.
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

// Producer workgroup, at its end: once every wave's stores are acknowledged,
// count the workgroup finished (a release, so its plain stores go with it).
__device__ __forceinline__ void count_finished(uint32_t* finished) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(finished, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// Cache-policy bits of the buffer load/store builtins on gfx950.
constexpr int kCpolSc0 = 1, kCpolNt = 2, kCpolSc1 = 16;

// notify(set) for data that was itself stored at device scope (sc1, written
// through to the device coherence point) and whose stores every wave of the
// workgroup has waited on (s_waitcnt vmcnt(0)) before a workgroup barrier:
// nothing dirty remains in the XCD's L2 to write back, so the flag is a
// device-scope store without the release's full L2 write-back.
__device__ __forceinline__ void flag_publish_coherent(uint32_t* f, uint32_t epoch) {
  __hip_atomic_store(f, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline void report_timeout(uint32_t* status, int64_t flag, uint32_t seen, uint32_t expected) {
  if (atomicCAS(status, 0u, kStatusTimeout) == 0u) {
    status[1] = (uint32_t)flag;
    status[2] = seen;
    status[3] = expected;
    __threadfence();
  }
}

// Consumer workgroup of an overlapped call, at its end: thread 0 waits until
// the producer's finished count (cumulative over calls, compared as a wrapping
// difference) reaches `all`, then the acquire.  Bounded: on expiry the status
// records flag index 0xFFFFFFFF (no flag) with the count seen.
__device__ inline void wait_producer_done(const uint32_t* done, uint32_t all, uint64_t timeout_ticks,
                                          uint32_t* status) {
  if (!done || threadIdx.x != 0) return;
  const uint64_t t0 = clock_ticks();
  uint32_t v = __hip_atomic_load(done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  while ((int32_t)(v - all) < 0) {
    if (clock_ticks() - t0 > timeout_ticks) {
      report_timeout(status, 0xFFFFFFFFll, v, all);
      return;
    }
    __builtin_amdgcn_s_sleep(2);
    v = __hip_atomic_load(done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  acquire_agent();
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

// Wave-parallel wait for flags[f0 .. f1), called by all 64 lanes of one wave:
// lane i polls flag f0 + i (64 at a time), so n flags cost one memory latency
// per poll instead of n.  Returns true when all are set (after an acquire
// fence), false after the time budget (status recorded).
__device__ inline bool wait_flags_wave(const uint32_t* flags, int64_t f0, int64_t f1, uint32_t epoch,
                                       uint64_t timeout_ticks, uint32_t* status) {
  const int lane = threadIdx.x & 63;
  const uint64_t t0 = clock_ticks();
  for (int64_t base = f0; base < f1; base += 64) {
    const int64_t f = base + lane;
    bool mine = f >= f1;
    uint32_t v = 0;
    while (true) {
      if (!mine) {
        v = flag_peek(flags + f);
        mine = flag_is_set(v, epoch);
      }
      if (__all(mine)) break;
      if (clock_ticks() - t0 > timeout_ticks) {
        if (!mine) report_timeout(status, f, v, epoch);
        return false;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  acquire_agent();
  return true;
}

// Workgroup-wide wait: wave 0 polls, then every thread passes a barrier.
// `ok` must be a __shared__ int.  Returns the shared verdict.
__device__ inline bool wait_flags_block(const uint32_t* flags, int64_t f0, int64_t f1, uint32_t epoch,
                                        uint64_t timeout_ticks, uint32_t* status, int* ok) {
  if (threadIdx.x < 64) {
    const bool good = wait_flags_wave(flags, f0, f1, epoch, timeout_ticks, status);
    if (threadIdx.x == 0) *ok = good ? 1 : 0;
  }
  __syncthreads();
  return *ok != 0;
}

// Workgroup-wide release of flags[f0 .. f1): every thread's prior global stores
// are ordered before the flag stores.  Each wave only waits for its stores to
// be acknowledged (no cache write-back per wave); after the barrier the one
// agent-scope release writes back the XCD's L2 once for all of them.
__device__ inline void release_flags_block(uint32_t* flags, int64_t f0, int64_t f1, uint32_t epoch) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0)
    for (int64_t f = f0; f < f1; ++f) flag_release(flags + f, epoch);
}

}  // namespace sgt
