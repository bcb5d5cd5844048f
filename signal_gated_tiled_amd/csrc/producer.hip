// AllGather producer: moves the peers' shards into the gathered buffer one
// signal tile at a time and releases each tile's flag (Triton-distributed
// semantics page, "Producer-consumer model" and "AllGather + GEMM overlap";
// paper summary, "Method": intra-node AllGather in pull mode, the local side
// choosing the order; resource partitioning keeps communication on units of
// its own).
//
// On one GPU a peer's link is simulated: each tile is copied HBM to HBM at full
// speed and its flag is released no earlier than the time a link of the
// configured per-peer rate would have delivered it (plus seeded jitter).  The
// host builds the item list sorted by release time; workgroup g takes items
// g, g + G, g + 2G, ...
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "signal.hpp"

namespace sgt {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ inline void copy_bytes(char* __restrict__ dst, const char* __restrict__ src, int64_t bytes) {
  const bool v16 = ((bytes | (int64_t)(uintptr_t)dst | (int64_t)(uintptr_t)src) & 15) == 0;
  if (v16) {
    constexpr int U = 8;
    const int64_t n = bytes >> 4;
    const u32x4* s = reinterpret_cast<const u32x4*>(src);
    u32x4* d = reinterpret_cast<u32x4*>(dst);
    const int64_t step = (int64_t)blockDim.x * U;
    for (int64_t base = threadIdx.x; base < n; base += step) {
      u32x4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t i = base + (int64_t)u * blockDim.x;
        if (i < n) v[u] = __builtin_nontemporal_load(s + i);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t i = base + (int64_t)u * blockDim.x;
        if (i < n) d[i] = v[u];
      }
    }
  } else {  // 4-byte elements (fp32 rows of any length)
    const int64_t n = bytes >> 2;
    const uint32_t* s = reinterpret_cast<const uint32_t*>(src);
    uint32_t* d = reinterpret_cast<uint32_t*>(dst);
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) d[i] = s[i];
  }
}

__global__ void __launch_bounds__(256) ag_producer_kernel(PtrTable shards, char* gathered, uint32_t* flags,
                                                          const ProdItem* items, int n_items, int64_t tile_bytes,
                                                          int tiles_per_shard, uint32_t epoch, int withhold_peer,
                                                          uint64_t* trace_release) {
  __shared__ uint64_t t0;
  if (threadIdx.x == 0) t0 = clock_ticks();
  __syncthreads();
  for (int it = blockIdx.x; it < n_items; it += gridDim.x) {
    const ProdItem item = items[it];
    const int p = (int)item.peer;
    const int64_t local_tile = (int64_t)item.tile - (int64_t)p * tiles_per_shard;
    copy_bytes(gathered + (int64_t)item.tile * tile_bytes,
               static_cast<const char*>(shards.p[p]) + local_tile * tile_bytes, tile_bytes);
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
      // Pace: the link of this peer delivers the tile at t0 + release.  The
      // schedule is finite, so this wait always ends.
      const uint64_t target = t0 + item.release;
      while (clock_ticks() < target) __builtin_amdgcn_s_sleep(4);
      if (p != withhold_peer) flag_release(flags + item.tile, epoch);
      if (trace_release) trace_release[item.tile] = clock_ticks();
    }
  }
}

// Sets n flags to the epoch (pre-resident data, or the peers' flags of a
// GEMM+RS call whose partials are already in place).  Plain stores: the kernel
// boundary orders them before the consumer launched after it on the stream.
__global__ void fill_u32_kernel(uint32_t* p, int64_t n, uint32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

}  // namespace

hipError_t launch_ag_producer(const PtrTable& shards, void* gathered, uint32_t* flags, const ProdItem* items,
                              int n_items, int64_t tile_bytes, int tiles_per_shard, uint32_t epoch,
                              int withhold_peer, uint64_t* trace_release, int grid, hipStream_t stream) {
  if (n_items <= 0) return hipSuccess;
  if (grid > n_items) grid = n_items;
  hipLaunchKernelGGL(ag_producer_kernel, dim3(grid), dim3(256), 0, stream, shards, static_cast<char*>(gathered),
                     flags, items, n_items, tile_bytes, tiles_per_shard, epoch, withhold_peer, trace_release);
  return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n, v);
  return hipGetLastError();
}

}  // namespace sgt
