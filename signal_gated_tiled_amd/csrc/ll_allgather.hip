// Low-latency (LL) AllGather and its flag-based counterpart (paper summary,
// "Method": for short messages the inter-node AllGather stores data and flag
// together in 8-byte blocks and spins on them to detect arrival, which saves
// the separate signal operation of every transfer; Triton-distributed
// semantics page, "Producer-consumer model" and "Signal-based
// synchronization" for the flag-based form).
//
// LL packet: one aligned 8-byte word, payload dword first, flag dword second
// (little-endian: bits 0..31 data, 32..63 the call's epoch).  A peer writes
// its shard's payload as packets into its slot of the receiver's LL buffer;
// the receiver polls the packets themselves: a packet whose flag holds the
// epoch carries valid data in the same word, so no flag store, no store
// acknowledgement and no acquire fence sit between data and use.  The cost is
// twice the bytes on the link and an unpacking pass on the receiver.
//
// On one GPU the peers are simulated: the producer below writes each peer's
// packets no earlier than that peer's link would deliver them (paced, as the
// flag-based producer releases its flags).  Device-scope (sc1) stores write
// the packets through to the device coherence point; the receiver's
// device-scope (sc1) loads read them there, whatever XCD wrote them.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "signal.hpp"

namespace sgt {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kLlThreads = 256;
constexpr int kLlUnroll = 8;  // 16-byte loads per thread per pass: 32 KiB of packets per workgroup pass

__device__ inline __amdgpu_buffer_rsrc_t ll_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Paced packing of the remote chunks.  items[i]: src = a peer's payload chunk
// (chunk_bytes), dst = its packets in the LL buffer (2 * chunk_bytes); the
// writes start `lead` ticks before the item's release so that the chunk lands
// about when the peer's link would have delivered it.  trace_issue (optional):
// trace_issue[2 * chunk] = the tick the chunk's writes began.
__device__ __forceinline__ void ll_produce(int first, int stride, const ProdItem* __restrict__ items, int n_items,
                                           int64_t chunk_bytes, uint32_t epoch, int withhold_peer, uint64_t lead,
                                           uint64_t* trace_issue) {
  __shared__ uint64_t t0;
  if (threadIdx.x == 0) t0 = clock_ticks();
  __syncthreads();
  const uint32_t cb = (uint32_t)chunk_bytes;
  const uint32_t lane = threadIdx.x * 16u, step = kLlThreads * 16u;
  for (int it = first; it < n_items; it += stride) {
    const ProdItem item = items[it];
    if ((int)item.peer == withhold_peer) continue;  // uniform: the item is the workgroup's
    if (threadIdx.x == 0) {
      // the schedule is finite, so this wait always ends
      if (item.release > lead)
        while (clock_ticks() < t0 + item.release - lead) __builtin_amdgcn_s_sleep(4);
      if (trace_issue) trace_issue[2 * (int64_t)item.flag0] = clock_ticks();
    }
    __syncthreads();
    const __amdgpu_buffer_rsrc_t rs = ll_rsrc(item.src, cb), rd = ll_rsrc(item.dst, 2u * cb);
    // 16 payload bytes -> two 16-byte lines of two packets each; offsets past
    // the chunk read zero and their stores are dropped by the range check
    for (uint32_t b = 0; b < cb; b += step * kLlUnroll) {
      u32x4 v[kLlUnroll];
#pragma unroll
      for (int u = 0; u < kLlUnroll; ++u)
        v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, b + lane + (uint32_t)u * step, 0, kCpolNt);
#pragma unroll
      for (int u = 0; u < kLlUnroll; ++u) {
        const uint32_t o = 2u * (b + lane + (uint32_t)u * step);
        const u32x4 lo = {v[u].x, epoch, v[u].y, epoch};
        const u32x4 hi = {v[u].z, epoch, v[u].w, epoch};
        __builtin_amdgcn_raw_buffer_store_b128(lo, rd, o, 0, kCpolSc1);
        __builtin_amdgcn_raw_buffer_store_b128(hi, rd, o + 16u, 0, kCpolSc1);
      }
    }
    __syncthreads();  // the next item's stamp is taken after this one's writes were issued
  }
}

// Plain workgroup copy of `bytes` (a multiple of 16) for the local shard.
__device__ inline void ll_copy_local(char* dst, const char* src, uint32_t bytes) {
  const __amdgpu_buffer_rsrc_t rs = ll_rsrc(src, bytes), rd = ll_rsrc(dst, bytes);
  const uint32_t lane = threadIdx.x * 16u, stride = kLlThreads * 16u;
  for (uint32_t b = 0; b < bytes; b += stride * kLlUnroll) {
    u32x4 v[kLlUnroll];
#pragma unroll
    for (int u = 0; u < kLlUnroll; ++u)
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, b + lane + (uint32_t)u * stride, 0, kCpolNt);
#pragma unroll
    for (int u = 0; u < kLlUnroll; ++u) __builtin_amdgcn_raw_buffer_store_b128(v[u], rd, b + lane + (uint32_t)u * stride, 0, 0);
  }
}

// LL receiver.  items[i]: the chunks in arrival order (local ones first);
// workgroup g takes items g, g + G, ...  A remote item's src is its packets,
// dst its rows of the gathered buffer.  Each wave polls its own lines of a
// pass (two packets per 16-byte device-scope load) until every packet's flag
// holds the epoch, then stores the payload; the waves of a workgroup need no
// barrier inside an item, since each lane stores only what it has checked.
// A wave whose budget expires records the packet in the status word; the
// workgroup then stops at the item's end.  trace_seen (optional):
// trace_seen[2 * chunk + 1] = the tick the whole chunk had been seen.
__device__ __forceinline__ void ll_receive(int first, int stride, const ProdItem* __restrict__ items, int n_items,
                                           int64_t chunk_bytes, uint32_t epoch, int rank, uint64_t timeout_ticks,
                                           uint32_t* status, uint64_t* trace) {
  __shared__ int failed;
  if (threadIdx.x == 0) failed = 0;
  __syncthreads();
  const uint32_t cb = (uint32_t)chunk_bytes, pb = 2u * cb;
  const uint32_t lane = threadIdx.x * 16u, step = kLlThreads * 16u;
  for (int it = first; it < n_items; it += stride) {
    const ProdItem item = items[it];
    const int64_t chunk = item.flag0;
    if ((int)item.peer == rank) {
      ll_copy_local(item.dst, item.src, cb);
      if (trace && threadIdx.x == 0) trace[2 * chunk] = trace[2 * chunk + 1] = clock_ticks();
      continue;
    }
    const __amdgpu_buffer_rsrc_t rs = ll_rsrc(item.src, pb), rd = ll_rsrc(item.dst, cb);
    const uint64_t t0 = clock_ticks();
    bool good = true;
    for (uint32_t b = 0; b < pb; b += step * kLlUnroll) {
      u32x4 v[kLlUnroll];
      // Two phases keep the polling traffic low while the chunk is still on
      // its way: first each lane polls one line of its pass, then it loads
      // all of them and re-polls until every packet holds the epoch.
      for (int phase = 0; phase < 2 && good; ++phase) {
        while (true) {
          bool ready = true;
#pragma unroll
          for (int u = 0; u < kLlUnroll; ++u) {
            if (phase == 0 && u > 0) break;
            const uint32_t o = b + lane + (uint32_t)u * step;
            v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, o, 0, kCpolSc1);
            // past the chunk: nothing to wait for (the load read zero); bitwise
            // operators keep the checks free of branches and per-load waits
            ready = ready & ((o >= pb) | (flag_is_set(v[u].y, epoch) & flag_is_set(v[u].w, epoch)));
          }
          if (__all(ready)) break;
          if (clock_ticks() - t0 > timeout_ticks ||
              __hip_atomic_load(&failed, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) {
            if (!ready) {
              // the first packet of this lane still missing, as an 8-byte word index into the LL buffer
              int64_t at = -1;
              uint32_t seen = 0;
              for (int u = (phase == 0 ? 0 : kLlUnroll - 1); u >= 0; --u) {
                const uint32_t o = b + lane + (uint32_t)u * step;
                if (o < pb && !flag_is_set(v[u].y, epoch)) {
                  at = o;
                  seen = v[u].y;
                } else if (o < pb && !flag_is_set(v[u].w, epoch)) {
                  at = o + 8;
                  seen = v[u].w;
                }
              }
              report_timeout(status, (chunk * (int64_t)pb + at) / 8, seen, epoch);
            }
            __hip_atomic_store(&failed, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            good = false;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
      }
      if (!good) break;
#pragma unroll
      for (int u = 0; u < kLlUnroll; ++u) {
        const u32x2 d = {v[u].x, v[u].z};
        __builtin_amdgcn_raw_buffer_store_b64(d, rd, (b + lane + (uint32_t)u * step) >> 1, 0, 0);
      }
    }
    __syncthreads();
    if (failed) return;  // uniform after the barrier
    if (trace && threadIdx.x == 0) trace[2 * chunk + 1] = clock_ticks();
  }
}

// Stand-alone LL AllGather in one launch: workgroups [0, n_prod_blocks) are
// the simulated peers (items[0, n_prod)), the others the receiver
// (items[n_prod, n_prod + n_recv)).  A launch with n_prod_blocks equal to its
// grid is the peers alone, one with 0 the receiver alone.
__global__ void __launch_bounds__(kLlThreads) ll_allgather_kernel(const ProdItem* __restrict__ items, int n_prod,
                                                                  int n_recv, int n_prod_blocks, int64_t chunk_bytes,
                                                                  uint32_t epoch, int withhold_peer, uint64_t lead,
                                                                  int rank, uint64_t timeout_ticks, uint32_t* status,
                                                                  uint64_t* trace) {
  if ((int)blockIdx.x < n_prod_blocks)
    ll_produce(blockIdx.x, n_prod_blocks, items, n_prod, chunk_bytes, epoch, withhold_peer, lead, trace);
  else
    ll_receive(blockIdx.x - n_prod_blocks, gridDim.x - n_prod_blocks, items + n_prod, n_recv, chunk_bytes, epoch,
               rank, timeout_ticks, status, trace);
}

}  // namespace

hipError_t launch_ll_allgather(const ProdItem* items, int n_prod, int n_recv, int n_prod_blocks, int grid,
                               int64_t chunk_bytes, uint32_t epoch, int withhold_peer, uint64_t lead, int rank,
                               uint64_t timeout_ticks, uint32_t* status, uint64_t* trace, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(ll_allgather_kernel, dim3(grid), dim3(kLlThreads), 0, stream, items, n_prod, n_recv,
                     n_prod_blocks, chunk_bytes, epoch, withhold_peer, lead, rank, timeout_ticks, status, trace);
  return hipGetLastError();
}

}  // namespace sgt
