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

__device__ inline __amdgpu_buffer_rsrc_t rsrc_of(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Copy `bytes` (< 2^31) from src to dst with the whole workgroup; returns true
// when the device-coherent path was used.  16-byte multiples use buffer
// loads (non-temporal: the source is read once) and device-scope stores (sc1:
// written through to the coherence point) with 32-bit offsets: past the end,
// loads read zero and stores are dropped by the hardware range check, so the
// unrolled body needs no bounds tests.
template <int U>
__device__ inline bool copy_bytes(char* __restrict__ dst, const char* __restrict__ src, int64_t bytes) {
  const bool v16 = ((bytes | (int64_t)(uintptr_t)dst | (int64_t)(uintptr_t)src) & 15) == 0;
  if (v16) {
    const __amdgpu_buffer_rsrc_t rs = rsrc_of(src, (uint32_t)bytes), rd = rsrc_of(dst, (uint32_t)bytes);
    const uint32_t lane = threadIdx.x * 16u, stride = blockDim.x * 16u;
    for (uint32_t b = 0; b < (uint32_t)bytes; b += stride * U) {
      u32x4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, b + lane + (uint32_t)u * stride, 0, kCpolNt);
      // all U loads in flight before the first store: left to itself the
      // scheduler pairs each store with its load to save registers, which
      // leaves one 16-byte load in flight per lane
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < U; ++u)
        __builtin_amdgcn_raw_buffer_store_b128(v[u], rd, b + lane + (uint32_t)u * stride, 0, kCpolSc1);
    }
    return true;
  }
  // 4-byte elements (fp32 rows of any length): plain stores, published by a release
  const int64_t n = bytes >> 2;
  const uint32_t* s = reinterpret_cast<const uint32_t*>(src);
  uint32_t* d = reinterpret_cast<uint32_t*>(dst);
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) d[i] = s[i];
  return false;
}

// Copy `rows` rows of `seg` bytes (a multiple of 16), `stride` bytes apart in
// both buffers (a column block of row-major matrices of the same width), with
// the loads and stores of copy_bytes; (rows - 1) * stride + seg < 2^31.
template <int U>
__device__ inline void copy_rows(char* __restrict__ dst, const char* __restrict__ src, uint32_t rows, uint32_t seg,
                                 uint32_t stride) {
  const uint32_t span = (rows - 1) * stride + seg;
  const __amdgpu_buffer_rsrc_t rs = rsrc_of(src, span), rd = rsrc_of(dst, span);
  const uint32_t upr = seg >> 4, total = rows * upr;
  for (uint32_t u0 = threadIdx.x; u0 < total; u0 += blockDim.x * U) {
    u32x4 v[U];
    uint32_t off[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t unit = u0 + (uint32_t)u * blockDim.x;
      const uint32_t r = unit / upr;
      off[u] = unit < total ? r * stride + (unit - r * upr) * 16u : 0x80000000u;
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, off[u], 0, kCpolNt);
    }
    __builtin_amdgcn_sched_barrier(0);  // every load in flight before the first store
#pragma unroll
    for (int u = 0; u < U; ++u) __builtin_amdgcn_raw_buffer_store_b128(v[u], rd, off[u], 0, kCpolSc1);
  }
}

// 256 threads x 32 loads of 16 bytes = 128 KiB in flight per workgroup: a copy
// is latency-bound, so bytes in flight set each workgroup's bandwidth.
constexpr int kProdThreads = 256;

// A simulated link delivers a tile's bytes over the tile's transfer time, not
// in one burst: a workgroup starts each paced tile's copy only `lead` ticks
// before its release, `lead` being twice the workgroup's last measured copy
// time (so the copy is done by the release), which keeps the producer's HBM
// traffic close to the links' rate instead of front-loading it.
// Producer role: this workgroup takes items first, first + stride, ...
// seg_rows > 0: each item is a column block of seg_rows rows of seg_bytes,
// row_stride apart (K-chunked signal tiles); else tile_bytes contiguous bytes.
__device__ __forceinline__ void produce_items(int first, int stride, uint32_t* flags,
                                              const ProdItem* __restrict__ items, int n_items, int64_t tile_bytes,
                                              uint32_t epoch, int withhold_peer, uint64_t* trace_release,
                                              uint64_t lead0, uint32_t* started, uint64_t* trace_issue,
                                              uint32_t seg_rows = 0, uint32_t seg_bytes = 0,
                                              uint32_t row_stride = 0) {
  __shared__ uint64_t t0, lead;
  if (threadIdx.x == 0) {
    t0 = clock_ticks();
    lead = lead0;
    // counts this workgroup as running, for a consumer launched later that
    // may only take the producer's CUs once every producer workgroup holds one
    if (started) __hip_atomic_fetch_add(started, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  for (int it = first; it < n_items; it += stride) {
    const ProdItem item = items[it];
    const int p = (int)item.peer;
    uint64_t c0 = 0;
    if (threadIdx.x == 0) {
      // the schedule is finite, so this wait always ends
      if (item.release > lead)
        while (clock_ticks() < t0 + item.release - lead) __builtin_amdgcn_s_sleep(4);
      c0 = clock_ticks();
      if (trace_issue) trace_issue[2 * (int64_t)item.flag0] = c0;
    }
    __syncthreads();
    bool coherent = true;
    if (seg_rows > 0) copy_rows<32>(item.dst, item.src, seg_rows, seg_bytes, row_stride);
    else coherent = copy_bytes<32>(item.dst, item.src, tile_bytes);
    // Every wave waits until its stores are acknowledged; after the barrier one
    // lane publishes the flag.  Device-scope stores leave nothing in the XCD's
    // L2 to write back, so the flag needs no release write-back; the plain
    // 4-byte path takes the full release.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
      const uint64_t d = clock_ticks() - c0;
      lead = 2 * d > 100 ? 2 * d : 100;
      // Pace: the link of this peer delivers the tile at t0 + release.  The
      // schedule is finite, so this wait always ends.
      const uint64_t target = t0 + item.release;
      while (clock_ticks() < target) __builtin_amdgcn_s_sleep(4);
      if (p != withhold_peer) {
        if (coherent) {
          for (uint32_t f = 0; f < item.nflags; ++f) flag_publish_coherent(flags + item.flag0 + f, epoch);
        } else {
          flag_release(flags + item.flag0, epoch);
          for (uint32_t f = 1; f < item.nflags; ++f) flag_publish_coherent(flags + item.flag0 + f, epoch);
        }
      }
      if (trace_release) trace_release[item.flag0] = clock_ticks();
    }
  }
}

// Releaser of the copy-engine producer (one thread): the copy engines move the
// data on their own; a copy unit's mark word takes the call's epoch once its
// bytes are written (a dependent 4-byte copy on the same engine, started
// after the data copy has completed).  For each item, in release order: wait
// until its unit's mark holds the epoch (system-scope loads: the mark is
// written by the copy engine, not through this XCD's L2), then until its
// release time, then publish its flags.  Every wait is bounded.
__device__ void release_items(uint32_t* flags, const RelItem* __restrict__ rel, int n_rel,
                              const uint32_t* marks, uint32_t epoch, int withhold_peer, uint64_t* trace_release,
                              uint64_t timeout_ticks, uint32_t* status, uint32_t* started) {
  if (threadIdx.x != 0) return;
  // counted as running, like the copying workgroups (see produce_items)
  if (started) __hip_atomic_fetch_add(started, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t t0 = clock_ticks();
  for (int i = 0; i < n_rel; ++i) {
    const RelItem r = rel[i];
    uint32_t v = __hip_atomic_load(marks + r.mark, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    while (!flag_is_set(v, epoch)) {
      if (clock_ticks() - t0 > timeout_ticks) {
        report_timeout(status, r.flag0, v, epoch);
        return;
      }
      __builtin_amdgcn_s_sleep(2);
      v = __hip_atomic_load(marks + r.mark, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
    // pace: the link delivers the item at t0 + release (a finite schedule, so this ends)
    while (clock_ticks() < t0 + r.release) __builtin_amdgcn_s_sleep(4);
    if ((int)r.peer != withhold_peer)
      for (uint32_t f = 0; f < r.nflags; ++f) flag_publish_coherent(flags + r.flag0 + f, epoch);
    if (trace_release) trace_release[r.flag0] = clock_ticks();
  }
}

// Workgroups [0, gridDim - (n_rel > 0)) copy items (CU producer); with
// copy-engine items (n_rel > 0) the last workgroup is their releaser.
__global__ void __launch_bounds__(kProdThreads) ag_producer_kernel(uint32_t* flags,
                                                                   const ProdItem* __restrict__ items, int n_items,
                                                                   int64_t tile_bytes, uint32_t epoch,
                                                                   int withhold_peer, uint64_t* trace_release,
                                                                   uint64_t lead0, uint32_t* started,
                                                                   uint64_t* trace_issue, uint32_t seg_rows,
                                                                   uint32_t seg_bytes, uint32_t row_stride,
                                                                   const RelItem* __restrict__ rel, int n_rel,
                                                                   const uint32_t* marks, uint64_t timeout_ticks,
                                                                   uint32_t* status, uint32_t* finished) {
  const int pwg = (int)gridDim.x - (n_rel > 0 ? 1 : 0);
  if ((int)blockIdx.x >= pwg) {
    release_items(flags, rel, n_rel, marks, epoch, withhold_peer, trace_release, timeout_ticks, status, started);
    return;
  }
  produce_items(blockIdx.x, pwg, flags, items, n_items, tile_bytes, epoch, withhold_peer, trace_release, lead0,
                started, trace_issue, seg_rows, seg_bytes, row_stride);
  if (finished) count_finished(finished);
}

// Stand-alone flag-based AllGather in one launch: workgroups [0, n_prod_blocks)
// are the producer (items[0, n_prod)), the others the receiving side, which
// waits for the flags of items[n_prod, n_prod + n_recv) in arrival order
// (wave 0 polls, then the acquire).  A launch with n_prod_blocks equal to its
// grid is the producer alone, one with 0 the receiver alone.  trace
// (optional, 2 words per chunk): {producer began the chunk, receiver saw its flag}.
__global__ void __launch_bounds__(kProdThreads) ag_allgather_kernel(uint32_t* flags, const ProdItem* __restrict__ items,
                                                                    int n_prod, int n_recv, int n_prod_blocks,
                                                                    int64_t tile_bytes, uint32_t epoch,
                                                                    int withhold_peer, uint64_t lead0,
                                                                    uint64_t timeout_ticks, uint32_t* status,
                                                                    uint64_t* trace) {
  if ((int)blockIdx.x < n_prod_blocks) {
    produce_items(blockIdx.x, n_prod_blocks, flags, items, n_prod, tile_bytes, epoch, withhold_peer, nullptr, lead0,
                  nullptr, trace);
    return;
  }
  __shared__ int ok;
  const ProdItem* __restrict__ recv = items + n_prod;
  const int stride = gridDim.x - n_prod_blocks;
  for (int it = blockIdx.x - n_prod_blocks; it < n_recv; it += stride) {
    const int64_t f = recv[it].flag0;
    if (!wait_flags_block(flags, f, f + 1, epoch, timeout_ticks, status, &ok)) return;  // uniform
    if (trace && threadIdx.x == 0) trace[2 * f + 1] = clock_ticks();
  }
}

// Sets n flags to the epoch (pre-resident data, or the peers' flags of a
// GEMM+RS call whose partials are already in place).  Plain stores: the kernel
// boundary orders them before the consumer launched after it on the stream.
__global__ void fill_u32_kernel(uint32_t* p, int64_t n, uint32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// GEMM+RS set-up in one launch: the resident peers' flags take the epoch and
// the reduction-claim counter restarts at zero.
__global__ void rs_prepare_kernel(uint32_t* pflags, int64_t n, uint32_t v, uint32_t* counter) {
  const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i0 == 0) *counter = 0u;
  for (int64_t i = i0; i < n; i += (int64_t)gridDim.x * blockDim.x) pflags[i] = v;
}

}  // namespace

hipError_t launch_rs_prepare(uint32_t* pflags, int64_t n, uint32_t v, uint32_t* counter, hipStream_t stream) {
  int64_t blocks = (n + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(rs_prepare_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, pflags, n, v, counter);
  return hipGetLastError();
}

hipError_t launch_ag_producer(uint32_t* flags, const ProdItem* items, int n_items,
                              int64_t tile_bytes, uint32_t epoch, int withhold_peer, uint64_t* trace_release, int grid,
                              hipStream_t stream, uint32_t* started, uint64_t* trace_issue, uint32_t seg_rows,
                              uint32_t seg_bytes, uint32_t row_stride, const RelItem* rel, int n_rel,
                              const uint32_t* marks, uint64_t timeout_ticks, uint32_t* status, uint32_t* finished) {
  if (n_items <= 0 && n_rel <= 0) return hipSuccess;
  if (grid > n_items) grid = n_items > 0 ? n_items : 0;
  if (n_rel > 0) grid += 1;  // the releaser
  // first estimate of a tile's copy time: at 16 GB/s per workgroup (100 MHz ticks)
  const uint64_t lead0 = (uint64_t)(tile_bytes / 160) + 100;
  hipLaunchKernelGGL(ag_producer_kernel, dim3(grid), dim3(kProdThreads), 0, stream, flags, items, n_items, tile_bytes,
                     epoch, withhold_peer, trace_release, lead0, started, trace_issue, seg_rows, seg_bytes,
                     row_stride, rel, n_rel, marks, timeout_ticks, status, finished);
  return hipGetLastError();
}

hipError_t launch_ag_allgather(uint32_t* flags, const ProdItem* items, int n_prod, int n_recv, int n_prod_blocks,
                               int grid, int64_t tile_bytes, uint32_t epoch, int withhold_peer,
                               uint64_t timeout_ticks, uint32_t* status, uint64_t* trace, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  const uint64_t lead0 = (uint64_t)(tile_bytes / 160) + 100;
  hipLaunchKernelGGL(ag_allgather_kernel, dim3(grid), dim3(kProdThreads), 0, stream, flags, items, n_prod, n_recv,
                     n_prod_blocks, tile_bytes, epoch, withhold_peer, lead0, timeout_ticks, status, trace);
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
