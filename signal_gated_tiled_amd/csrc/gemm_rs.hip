// GEMM + ReduceScatter (Triton-distributed semantics page, "GEMM +
// ReduceScatter overlap": the GEMM produces output tiles and signals each one;
// the ReduceScatter consumer waits for a tile and reduces it; paper summary,
// "Method": intra-node ReduceScatter in push mode, the reduction running in
// parallel and synchronized by signals).
//
// One persistent kernel holds both roles.  Its work list is
//   [0, n_gemm)            GEMM tiles of P = A_local * B, row block `rank`
//                          first, then rank+1, rank+2, ... (start from local
//                          data); each stores its fp32 tile and releases the
//                          flags of the rs_tile x rs_tile signal tiles it covers;
//   [n_gemm, n_gemm+n_red) reduction items, one per signal tile of the local
//                          block: wait for the GEMM flag and the W-1 peer flags,
//                          then C_shard = P[local] + sum of peer partials
//                          (fixed order: local, then peers by ascending rank).
// GEMM tiles are assigned statically; reduction tiles are claimed from an
// atomic counter, so they land in the workgroups left idle by the last, partial
// round of GEMM tiles.  Dependencies only point from reduction to GEMM, and a
// workgroup claims reduction tiles only after all of its own GEMM tiles, so the
// kernel cannot deadlock; every wait is still bounded.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "mfma_tile.hpp"
#include "sched.hpp"
#include "rs_reduce.hpp"
#include "signal.hpp"

namespace sgt {

namespace {

// GEMM m-tiles never straddle row blocks: block b holds tm_b = ceil(block_rows / 256)
// m-tiles, the last one possibly short.
__device__ __forceinline__ void gemm_tile_coords(const RsArgs& a, int t, int64_t* m0, int64_t* m_end, int64_t* n0) {
  const int tm_b = (int)((a.block_rows + kBM - 1) / kBM);
  const int per_block = tm_b * a.tiles_n;
  const int bi = t / per_block, rem = t % per_block;
  const int blk = (a.rank + bi) % a.W;
  const int mi = rem / a.tiles_n, ni = rem % a.tiles_n;
  *m0 = (int64_t)blk * a.block_rows + (int64_t)mi * kBM;
  const int64_t blk_end = (int64_t)(blk + 1) * a.block_rows;
  *m_end = *m0 + kBM < blk_end ? *m0 + kBM : blk_end;
  *n0 = (int64_t)ni * kBN;
}

template <int kW, bool kBNK>
__device__ void do_gemm_item(const RsArgs& a, int t) {
  int64_t m0, m_end, n0;
  gemm_tile_coords(a, t, &m0, &m_end, &n0);
  const uint16_t* A = static_cast<const uint16_t*>(a.A);
  const uint16_t* B = static_cast<const uint16_t*>(a.B);
  const KRows ka = krows_strided<kW>(A + m0 * a.K, m_end - m0, a.K);
  KRows kb = ka;
  if constexpr (kBNK) kb = krows_strided<kW>(B + n0 * a.K, a.N - n0, a.K);
  MfmaAcc<kW> acc;
  gemm_tile<kW, kBNK>(ka, kb, B, a.N, n0, a.K, acc);
  // rows past m_end belong to the next block's tile: clip to m_end
  store_tile<kW, false, kCpolSc1>(a.P, m_end, a.N, m0, n0, acc);
  // release the covered signal tiles (rs_tile divides 256 and the block rows)
  const int64_t n_end = n0 + kBN < a.N ? n0 + kBN : a.N;
  const int64_t gtn = (a.N + a.rs_tile - 1) / a.rs_tile;
  // The tile went out with device-scope stores: once every wave's stores are
  // acknowledged, one lane publishes the covered flags (no L2 write-back).
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0)
    for (int64_t mi = m0 / a.rs_tile; mi <= (m_end - 1) / a.rs_tile; ++mi)
      for (int64_t nj = n0 / a.rs_tile; nj <= (n_end - 1) / a.rs_tile; ++nj)
        flag_publish_coherent(a.gflags + mi * gtn + nj, a.epoch);
}

template <int kW, bool kBNK>
__global__ void __launch_bounds__(Tile<kW>::kThreads, 1) gemm_rs_kernel(RsArgs a) {
  __shared__ int ok;
  __shared__ int claimed;
  const int G = gridDim.x;
  // GEMM tiles: static, XCD-grouped round robin (tiles sharing operands run on
  // one XCD at the same time).
  for (int t = xcd_remap(blockIdx.x, G); t < a.n_gemm_tiles; t += G) {
    const uint64_t t_start = clock_ticks();
    do_gemm_item<kW, kBNK>(a, t);
    __syncthreads();
    if (a.trace && threadIdx.x == 0) {
      a.trace[3 * t + 0] = t_start;
      a.trace[3 * t + 1] = clock_ticks();
      a.trace[3 * t + 2] = blockIdx.x;
    }
  }
  // Reduction items: claimed one at a time by whichever workgroups finish their
  // GEMM tiles first (the ones with one tile fewer in the last partial round).
  // One item ahead: while the workgroup streams item j, thread 0 claims the
  // item after the next one and wave 0 peeks at the next one's flags, so the
  // round trips of the claim and of the flags overlap the stream.
  if (threadIdx.x == 0) claimed = (int)atomicAdd(a.red_counter, 1u);
  __syncthreads();
  int j = claimed;
  __syncthreads();
  if (j >= a.n_red_items) return;
  if (threadIdx.x < 64) {
    const RedFlag rf = red_flag(a, j, threadIdx.x);
    const bool good = red_wait(a, rf, rf.f ? flag_peek(rf.f) : 0u);
    if (threadIdx.x == 0) {
      ok = good ? 1 : 0;
      claimed = (int)atomicAdd(a.red_counter, 1u);
    }
  }
  __syncthreads();
  if (!ok) return;
  int jn = claimed;  // claimed, flags not yet seen
  __syncthreads();
  while (true) {
    RedFlag rf{nullptr, 0};
    uint32_t v = 0;
    int jnn = 0;
    if (jn < a.n_red_items && threadIdx.x < 64) {
      rf = red_flag(a, jn, threadIdx.x);
      if (rf.f) v = flag_peek(rf.f);
      if (threadIdx.x == 0) jnn = (int)atomicAdd(a.red_counter, 1u);
    }
    const uint64_t t_start = clock_ticks();
    red_stream(a, j);
    if (a.trace && threadIdx.x == 0) {
      const int t = a.n_gemm_tiles + j;
      a.trace[3 * t + 0] = t_start;
      a.trace[3 * t + 1] = clock_ticks();
      a.trace[3 * t + 2] = blockIdx.x;
    }
    if (jn >= a.n_red_items) break;
    if (threadIdx.x < 64) {
      const bool good = red_wait(a, rf, v);
      if (threadIdx.x == 0) {
        ok = good ? 1 : 0;
        claimed = jnn;
      }
    }
    __syncthreads();
    if (!ok) return;
    j = jn;
    jn = claimed;
    __syncthreads();  // every thread has read `claimed` before thread 0 writes it again
  }
  // paced peers: the join with the producer (its workgroups count themselves finished)
  wait_producer_done(a.prod_done, a.prod_done_all, a.timeout_ticks, a.status);
}

}  // namespace

int rs_gemm_tile() { return kBM; }

// `done`, when given, is recorded by the launch itself at the kernel's end (no
// separate marker on the stream).
hipError_t launch_gemm_rs(const RsArgs& a, int grid, hipStream_t stream, hipEvent_t done) {
  const bool nk = a.b_layout == 1;
  auto go = [&](auto kernel, int threads) {
    hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(threads), 0, stream, nullptr, done, 0, a);
  };
  if (a.tile_waves == 4) {
    if (nk) go(gemm_rs_kernel<4, true>, Tile<4>::kThreads);
    else go(gemm_rs_kernel<4, false>, Tile<4>::kThreads);
  } else {
    if (nk) go(gemm_rs_kernel<8, true>, Tile<8>::kThreads);
    else go(gemm_rs_kernel<8, false>, Tile<8>::kThreads);
  }
  return hipGetLastError();
}

}  // namespace sgt
