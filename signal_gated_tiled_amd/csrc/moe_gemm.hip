// MoE AllGather + grouped GEMM consumer (paper summary, "Experiments": MoE
// routing kernels; Triton-distributed semantics page, "AllGather + GEMM
// overlap": wait for the data a tile reads, then compute it; DITRON article,
// "three-level tiling": device-level tiles sized by each expert's token count).
//
// Work item = (grouped row tile, column tile): rows [r0, r0 + kR) of one
// expert's group (clipped to the group; kR = 128 or 256) times 256 columns of that expert's
// weight.  Persistent workgroups claim items from the readiness-ordered list
// with an atomic counter.  Before loading, wave 0 polls, lane by lane, the
// flag of the signal tile that holds each row's token (a tile waits for
// exactly the tokens it reads); then the rows are gathered straight into LDS
// (the DMA takes one row offset per load) and the MFMA tile core computes
// Y[r0 .., n0 ..] = X[row_token[r0 ..]] * W_e[:, n0 ..].
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "mfma_tile.hpp"
#include "signal.hpp"

namespace sgt {

namespace {

// Wait until every row of the tile has arrived: lane l of wave 0 watches the
// signal tiles of rows l, l + 64, ... (kR / 64 rows).  Returns the workgroup's
// verdict (false after a timeout, recorded in the status word).
template <int kR>
__device__ __forceinline__ bool wait_tile_rows(const MoeArgs& a, const int32_t* tok, int rows_valid, int* ok) {
  constexpr int Q = kR / 64;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int64_t f[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int r = lane + 64 * q;
      f[q] = r < rows_valid ? (int64_t)(tok[r] / a.flag_rows) : -1;
    }
    const uint64_t t0 = clock_ticks();
    bool good = true;
    while (true) {
      bool mine = true;
      uint32_t seen = 0;
      int64_t which = -1;
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        if (f[q] >= 0) {
          const uint32_t v = flag_peek(a.flags + f[q]);
          if (flag_is_set(v, a.epoch)) {
            f[q] = -1;
          } else {
            mine = false;
            seen = v;
            which = f[q];
          }
        }
      }
      if (__all(mine)) break;
      if (clock_ticks() - t0 > a.timeout_ticks) {
        if (!mine) report_timeout(a.status, which, seen, a.epoch);
        good = false;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    if (good) acquire_agent();
    if (lane == 0) *ok = good ? 1 : 0;
  }
  __syncthreads();
  return *ok != 0;
}

template <int kW, int kR, bool kBNK, bool kOutBf16>
__global__ void __launch_bounds__(Tile<kW>::kThreads, 1) moe_consumer_bf16(MoeArgs a) {
  __shared__ int item_s, ok;
  if (a.late_blocks > 0 && (int)blockIdx.x >= (int)gridDim.x - a.late_blocks) {
    // a workgroup that may sit on a CU the producer needs: run only if every
    // producer workgroup is already running (one check, no wait)
    if (threadIdx.x == 0)
      ok = __hip_atomic_load(a.started, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.started_all ? 1 : 0;
    __syncthreads();
    if (!ok) return;
  }
  const uint32_t nt = *a.n_tiles;
  const int64_t n_items = (int64_t)(nt < a.tiles_cap ? nt : a.tiles_cap) * a.tiles_n;
  while (true) {
    if (threadIdx.x == 0) item_s = (int)atomicAdd(a.claim, 1u);
    __syncthreads();
    const int64_t item = item_s;
    if (item >= n_items) break;
    const MoeTile mt = a.order[item / a.tiles_n];
    const int64_t n0 = (item % a.tiles_n) * kBN;
    const int e = mt.expert;
    const int64_t r0 = mt.r0;
    int64_t r_end = a.expert_off[e + 1];
    r_end = r_end < a.rows ? r_end : a.rows;  // the tables are exact; this only bounds every access
    if (r0 >= r_end) {  // (uniform) the barrier keeps item_s from being overwritten before all read it
      __syncthreads();
      continue;
    }
    const int rows_valid = (int)(r_end - r0 < kR ? r_end - r0 : kR);
    const int32_t* tok = a.row_token + r0;
    uint64_t t_wait = 0;
    if (a.trace && threadIdx.x == 0) t_wait = clock_ticks();
    if (!wait_tile_rows<kR>(a, tok, rows_valid, &ok)) return;
    if (a.trace && threadIdx.x == 0) {
      a.trace[item * 4 + 0] = t_wait;
      a.trace[item * 4 + 1] = clock_ticks();
      a.trace[item * 4 + 3] = blockIdx.x;
    }

    // A: gathered rows of X (row offsets < T * H * 2 < 2^31).
    KRows ka;
    ka.rsrc = make_rsrc(a.X, (uint64_t)a.T * (uint64_t)a.H * 2u);
#pragma unroll
    for (int i = 0; i < kR / kW / 8; ++i) {
      const int r = dma_row<kW, kR>(i);
      ka.row_off[i] = r < rows_valid ? (uint32_t)((int64_t)tok[r] * a.H * 2) : kOOB;
    }
    krows_chunks<kW, kR>(ka);
    // B: expert e's weight, H x I (KN) or I x H (NK).
    const uint16_t* Be = a.We + (int64_t)e * a.H * a.I;
    KRows kb = ka;
    if constexpr (kBNK) kb = krows_strided<kW>(Be + n0 * a.H, a.I - n0, a.H);
    MfmaAcc<kW, kR> acc;
    gemm_tile<kW, kBNK, kR>(ka, kb, Be, a.I, n0, a.H, acc);
    store_tile<kW, kOutBf16, 0, kR>(a.Y, r0 + rows_valid, a.I, r0, n0, acc);
    if (a.trace && threadIdx.x == 0) a.trace[item * 4 + 2] = clock_ticks();
  }
}

}  // namespace

template <int kW, int kR>
static void launch_moe(const MoeArgs& a, bool nk, bool ob, int grid, hipStream_t stream) {
  const dim3 blk(Tile<kW>::kThreads);
  if (nk && ob) hipLaunchKernelGGL((moe_consumer_bf16<kW, kR, true, true>), dim3(grid), blk, 0, stream, a);
  if (nk && !ob) hipLaunchKernelGGL((moe_consumer_bf16<kW, kR, true, false>), dim3(grid), blk, 0, stream, a);
  if (!nk && ob) hipLaunchKernelGGL((moe_consumer_bf16<kW, kR, false, true>), dim3(grid), blk, 0, stream, a);
  if (!nk && !ob) hipLaunchKernelGGL((moe_consumer_bf16<kW, kR, false, false>), dim3(grid), blk, 0, stream, a);
}

hipError_t launch_moe_consumer(const MoeArgs& a, int b_layout, int out_dtype, int tile_rows, int tile_waves, int grid,
                               hipStream_t stream) {
  const bool nk = b_layout == 1, ob = out_dtype == 1;
  if (tile_rows == 256) {
    if (tile_waves == 4) launch_moe<4, 256>(a, nk, ob, grid, stream);
    else launch_moe<8, 256>(a, nk, ob, grid, stream);
  } else {
    if (tile_waves == 4) launch_moe<4, 128>(a, nk, ob, grid, stream);
    else launch_moe<8, 128>(a, nk, ob, grid, stream);
  }
  return hipGetLastError();
}

}  // namespace sgt
