// One rank's share of a signal-gated ring AllReduce (Triton-distributed
// semantics page, "Example: ring AllReduce with overlap": a ReduceScatter
// phase and an AllGather phase of W - 1 steps each, every tile synchronized
// on its own with wait / notify, a tile reduced as soon as it arrives, no
// barrier between steps, sending the next tile overlapped with reducing this
// one).
//
// The vector x (N fp32) is cut into W chunks of C = N / W elements, chunk c
// at [c * C, (c + 1) * C), and each chunk into T tiles.  Rank r receives from
// rank r - 1 and sends to rank r + 1 (mod W):
//   ReduceScatter step s (0 .. W-2): it sends chunk r - s and receives chunk
//     r - s - 1, adding its own x to it; what it sends at step s > 0 is what
//     it reduced at step s - 1, and after the last step it holds the full sum
//     of chunk r + 1.
//   AllGather step s (0 .. W-2): it sends chunk r + 1 - s (first the chunk it
//     just finished, then each chunk it received the step before) and
//     receives the full chunk r - s into the result.
// Messages are numbered k = s for the ReduceScatter steps and k = W - 1 + s
// for the AllGather steps.  inbox[k] is where the left neighbour's message k
// lands (its flags: in_flags[k][tile]); outbox[k] is this rank's message k
// to its right neighbour (out_flags[k][tile], published after device-scope
// stores).
//
// Work items, in arrival order: the T tiles of message 0 (chunk r of x, sent
// without waiting), then (k, tile) for every received message, step-major.
// Workgroup g takes items g, g + G, ...; an item waits only on its own tile's
// flag.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "ring.hpp"
#include "signal.hpp"

namespace sgt {

namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRingThreads = 256;
constexpr int kRingUnroll = 4;  // float4 accesses per thread per pass: 16 KiB of each operand per pass

__device__ inline __amdgpu_buffer_rsrc_t ring_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ int wrap(int v, int W) { return ((v % W) + W) % W; }

__global__ void __launch_bounds__(kRingThreads) ring_allreduce_kernel(RingArgs a) {
  __shared__ int ok;
  const int W = a.W, r = a.rank;
  const int64_t n_items = (int64_t)a.T * (2 * W - 1);
  for (int64_t it = blockIdx.x; it < n_items; it += gridDim.x) {
    // k: the received message (-1: the first send), j: the tile
    const int k = (int)(it / a.T) - 1, j = (int)(it % a.T);
    const int64_t e0 = (int64_t)j * a.tile;
    const int64_t n_el = a.C - e0 < a.tile ? a.C - e0 : a.tile;
    const uint32_t bytes = (uint32_t)(n_el * 4);
    uint64_t t_wait = 0;
    if (a.trace && threadIdx.x == 0) t_wait = clock_ticks();
    if (k >= 0) {
      const int64_t f = (int64_t)k * a.T + j;
      if (!wait_flags_block(a.in_flags, f, f + 1, a.epoch, a.timeout_ticks, a.status, &ok)) return;  // uniform
    }
    if (a.trace && threadIdx.x == 0) {
      a.trace[it * 3 + 0] = t_wait;
      a.trace[it * 3 + 1] = clock_ticks();
    }
    // operands of this item (uniform): src0 (+ src1) -> dst_out and/or dst_send
    const float* src0;
    const float* src1 = nullptr;
    float* dst_out = nullptr;
    int send = -1;  // outbox message written, or -1
    if (k < 0 && W == 1) {             // a ring of one: the sum is x itself
      src0 = a.x + e0;
      dst_out = a.out + e0;
    } else if (k < 0) {                // first send: chunk r of x
      src0 = a.x + (int64_t)r * a.C + e0;
      send = 0;
    } else if (k <= W - 2) {           // ReduceScatter step k: chunk r - k - 1
      const int c = wrap(r - k - 1, W);
      src0 = a.x + (int64_t)c * a.C + e0;
      src1 = a.inbox + (int64_t)k * a.C + e0;
      send = k + 1;                    // the next ReduceScatter send, or (k = W - 2) the first AllGather send
      if (k == W - 2) dst_out = a.out + (int64_t)c * a.C + e0;
    } else {                           // AllGather step s: full chunk r - s
      const int s = k - (W - 1);
      src0 = a.inbox + (int64_t)k * a.C + e0;
      dst_out = a.out + (int64_t)wrap(r - s, W) * a.C + e0;
      send = s < W - 2 ? k + 1 : -1;
    }
    const __amdgpu_buffer_rsrc_t r0 = ring_rsrc(src0, bytes);
    const __amdgpu_buffer_rsrc_t r1 = ring_rsrc(src1 ? src1 : src0, bytes);
    const __amdgpu_buffer_rsrc_t ro = ring_rsrc(dst_out ? dst_out : a.out, dst_out ? bytes : 0u);
    float* sendp = send >= 0 ? a.outbox + (int64_t)send * a.C + e0 : a.outbox;
    const __amdgpu_buffer_rsrc_t rs = ring_rsrc(sendp, send >= 0 ? bytes : 0u);
    const uint32_t lane = threadIdx.x * 16u, step = kRingThreads * 16u;
    // offsets past the tile read zero and their stores are dropped (range
    // check), so the passes need no bounds tests
    for (uint32_t b = 0; b < bytes; b += step * kRingUnroll) {
      f32x4_t v[kRingUnroll];
#pragma unroll
      for (int u = 0; u < kRingUnroll; ++u)
        v[u] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r0, b + lane + u * step, 0, kCpolNt));
      if (src1) {
#pragma unroll
        for (int u = 0; u < kRingUnroll; ++u)
          v[u] += __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r1, b + lane + u * step, 0, kCpolNt));
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < kRingUnroll; ++u) {
        const u32x4 w = __builtin_bit_cast(u32x4, v[u]);
        __builtin_amdgcn_raw_buffer_store_b128(w, ro, b + lane + u * step, 0, kCpolNt);
        __builtin_amdgcn_raw_buffer_store_b128(w, rs, b + lane + u * step, 0, kCpolSc1);
      }
    }
    // notify the right neighbour: every wave's device-scope stores are
    // acknowledged before one lane stores the tile's flag
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
      if (send >= 0) flag_publish_coherent(a.out_flags + (int64_t)send * a.T + j, a.epoch);
      if (a.trace) a.trace[it * 3 + 2] = clock_ticks();
    }
  }
  // the join with an overlapped producer: its workgroups count themselves
  // finished, and the kernel ends after all of them
  wait_producer_done(a.prod_done, a.prod_done_all, a.timeout_ticks, a.status);
}

}  // namespace

hipError_t launch_ring_allreduce(const RingArgs& a, int grid, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(ring_allreduce_kernel, dim3(grid), dim3(kRingThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sgt
