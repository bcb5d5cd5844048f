// MoE AllGather + grouped GEMM consumer (paper summary, "Experiments": MoE
// routing kernels; Triton-distributed semantics page, "AllGather + GEMM
// overlap": wait for the data a tile reads, then compute it; DITRON article,
// "three-level tiling": device-level tiles sized by each expert's token count).
//
// Work item = (grouped row tile, column tile): rows [r0, r0 + kR) of one
// expert's group (clipped to the group; kR = 128 or 256) times 256 columns of that expert's
// weight.  Persistent workgroups claim items from their XCD's share of the
// expert-major list with an atomic counter per XCD (the column tiles of a row
// tile are consecutive items, and so are an expert's row tiles, so they run
// side by side on one XCD and read the gathered rows and the expert's weight
// columns from its L2), then help the other XCDs.  Before
// loading, wave 0 polls, lane by lane, the flag of the signal tile that holds
// each row's token (a tile waits for exactly the tokens it reads); then the
// rows are gathered straight into LDS
// (the DMA takes one row offset per load) and the MFMA tile core computes
// Y[r0 .., n0 ..] = X[row_token[r0 ..]] * W_e[:, n0 ..].
#include <hip/hip_ext.h>
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

// The 8-wave tile with W_e stored I x H runs on the five-slot ring with the
// expert weights leading (loaded two steps ahead): they are the first touches
// here (each expert's slab is read by its few row tiles), while the gathered
// token rows are read by up to eight experts' tiles and mostly hit the caches.
constexpr bool kMoeRingLeadA = false;

// One tile of rows [r0, r0 + rows_valid) of expert e's group (rows_valid <= kR)
// times 256 columns of W_e, on the workgroup's LDS stages; between() runs after
// the K loop, before the results are stored.
template <int kW, int kR, bool kBNK, bool kOutBf16, class Between>
__device__ __forceinline__ void moe_tile(const MoeArgs& a, const int32_t* tok, int rows_valid, int e, int64_t r0,
                                         int64_t n0, uint8_t* s0, uint8_t* s1, uint8_t* s2, uint8_t* s3,
                                         uint8_t* s4, Between&& between) {
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
  acc_zero<kW, kR>(acc);
  if constexpr (kW == 8 && kBNK) gemm_tile_range_r5<kR, kMoeRingLeadA>(ka, kb, 0, a.H, acc, s0, s1, s2, s3, s4);
  else gemm_tile_range_lds<kW, kBNK, kR>(ka, kb, Be, a.I, n0, a.H, 0, a.H, acc, s0, s1, s2, s3);
  between();
  store_tile<kW, kOutBf16, 0, kR>(a.Y, r0 + rows_valid, a.I, r0, n0, acc);
}

// The next work item for wave 0 (the same value in all its lanes), or -1 once
// every list is used up: one atomic on the home XCD's list while it has items;
// after that, every list's counter read at once (one lane each) and an atomic
// only on those that still show items.  home_left is wave 0's record that its
// home list may still have items.
__device__ __forceinline__ int claim_item(const MoeArgs& a, uint32_t nt, int home, bool& home_left) {
  const int lane = threadIdx.x & 63;
  const uint32_t tn = (uint32_t)a.tiles_n;
  int item = -1;
  if (home_left) {
    if (lane == 0) {
      const uint32_t len = xcd_list_len(nt, home) * tn;
      const uint32_t c = len ? atomicAdd(a.xcd_claim + home * kXcdClaimStride, 1u) : len;
      if (c < len) item = (int)(xcd_list_start(nt, home) * tn + c);
    }
    item = __shfl(item, 0);
    home_left = item >= 0;
    if (home_left) return item;
  }
  const uint32_t len = lane < kXcds ? xcd_list_len(nt, lane) * tn : 0u;
  const uint32_t seen = lane < kXcds && lane != home
                            ? __hip_atomic_load(a.xcd_claim + lane * kXcdClaimStride, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT)
                            : len;
  const uint64_t open = __ballot(seen < len);
  if (lane == 0) {
    for (int k = 1; k < kXcds && item < 0; ++k) {
      const int x = (home + k) % kXcds;
      if (!((open >> x) & 1u)) continue;
      const uint32_t lx = xcd_list_len(nt, x) * tn;
      const uint32_t c = atomicAdd(a.xcd_claim + x * kXcdClaimStride, 1u);
      if (c < lx) item = (int)(xcd_list_start(nt, x) * tn + c);
    }
  }
  return __shfl(item, 0);
}

// kRmax = 256: a row tile of more than 128 valid rows runs as a 256-row tile,
// a shorter one (the tail of a group) as a 128-row tile, so short groups do
// not pay for 256 rows; kRmax = 128: every tile is 128 rows.  Both tile
// heights share the workgroup's four LDS stages.
template <int kW, int kRmax, bool kBNK, bool kOutBf16>
__global__ void __launch_bounds__(Tile<kW>::kThreads, 1) moe_consumer_bf16(MoeArgs a) {
  // LDS: the K loop's stages (the step loop's four, or the ring's five slots of
  // 32 KiB).  With the ring the two shared words live at the start of the fifth
  // slot: they are used only between tiles, when no load is in flight, and the
  // ring writes that slot first in its first step, after a barrier every wave
  // passes once it has read them.
  constexpr bool kRing = kW == 8 && kBNK;
  struct Words {
    int item_s, ok;
  };
  __shared__ __attribute__((aligned(1024))) uint8_t s0[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t s1[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t s2[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t s3[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t s4[kRing ? kStageBytes : sizeof(Words)];
  Words* const wd = reinterpret_cast<Words*>(s4);
  int& item_s = wd->item_s;
  int& ok = wd->ok;
  if (a.late_blocks > 0 && (int)blockIdx.x >= (int)gridDim.x - a.late_blocks) {
    // a workgroup that may sit on a CU the producer needs: run only if every
    // producer workgroup is already running (one check, no wait)
    if (threadIdx.x == 0)
      ok = __hip_atomic_load(a.started, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.started_all ? 1 : 0;
    __syncthreads();
    if (!ok) return;
  }
  const uint32_t nt_raw = *a.n_tiles;
  const uint32_t nt = nt_raw < a.tiles_cap ? nt_raw : a.tiles_cap;
  // Work items come from the list of this workgroup's XCD (workgroup b runs on
  // XCD b % kXcds), then, once it is used up, from the other XCDs' lists.  The
  // claim of the next item goes out while the current tile's results are
  // stored; item_s hands it to every wave.
  const int home = (int)(blockIdx.x % kXcds);
  bool home_left = true;
  if (threadIdx.x < 64) {
    const int first = claim_item(a, nt, home, home_left);
    if (threadIdx.x == 0) item_s = first;
  }
  __syncthreads();
  int item = item_s;
  while (item >= 0) {
    const MoeTile mt = a.order[item / a.tiles_n];
    const int64_t n0 = (int64_t)(item % a.tiles_n) * kBN;
    const int e = mt.expert;
    const int64_t r0 = mt.r0;
    // (the tables are exact; the clamps only bound every access)
    int64_t rv = mt.rows < kRmax ? mt.rows : kRmax;
    rv = r0 + rv <= a.rows ? rv : a.rows - r0;
    int next = -1;
    auto claim_next = [&]() {
      if (threadIdx.x < 64) next = claim_item(a, nt, home, home_left);
    };
    if (rv > 0 && e >= 0 && e < a.E) {  // (uniform)
      const int rows_valid = (int)rv;
      const int32_t* tok = a.row_token + r0;
      uint64_t t_wait = 0, cyc0 = 0;
      if (a.trace && threadIdx.x == 0) {
        t_wait = clock_ticks();
        cyc0 = __builtin_amdgcn_s_memtime();
      }
      if (!wait_tile_rows<kRmax>(a, tok, rows_valid, &ok)) return;
      if (a.trace && threadIdx.x == 0) {
        a.trace[item * 4 + 0] = t_wait;
        a.trace[item * 4 + 1] = clock_ticks();
      }
      if (kRmax == 256 && rows_valid > 128)
        moe_tile<kW, kRmax, kBNK, kOutBf16>(a, tok, rows_valid, e, r0, n0, s0, s1, s2, s3, s4, claim_next);
      else
        moe_tile<kW, 128, kBNK, kOutBf16>(a, tok, rows_valid, e, r0, n0, s0, s1, s2, s3, s4, claim_next);
      if (a.trace && threadIdx.x == 0) {  // end time; workgroup and engine-clock cycles since the wait began
        a.trace[item * 4 + 2] = clock_ticks();
        a.trace[item * 4 + 3] = (uint64_t)blockIdx.x | ((__builtin_amdgcn_s_memtime() - cyc0) << 16);
      }
    } else {
      __syncthreads();  // every wave has read item_s before it is written again
      claim_next();
    }
    // (with a tile, the barriers of its K loop lie between every wave's read of
    // item_s and this write)
    if (threadIdx.x == 0) item_s = next;
    __syncthreads();
    item = item_s;
  }
  wait_producer_done(a.prod_done, a.prod_done_all, a.timeout_ticks, a.status);
}

}  // namespace

// `done`, when given, is recorded by the launch itself at the kernel's end
// (no separate marker on the stream).
template <int kW, int kR>
static void launch_moe(const MoeArgs& a, bool nk, bool ob, int grid, hipStream_t stream, hipEvent_t done) {
  auto go = [&](auto kernel) {
    hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(Tile<kW>::kThreads), 0, stream, nullptr, done, 0, a);
  };
  if (nk && ob) go(moe_consumer_bf16<kW, kR, true, true>);
  if (nk && !ob) go(moe_consumer_bf16<kW, kR, true, false>);
  if (!nk && ob) go(moe_consumer_bf16<kW, kR, false, true>);
  if (!nk && !ob) go(moe_consumer_bf16<kW, kR, false, false>);
}

hipError_t launch_moe_consumer(const MoeArgs& a, int b_layout, int out_dtype, int tile_rows, int tile_waves, int grid,
                               hipStream_t stream, hipEvent_t done) {
  const bool nk = b_layout == 1, ob = out_dtype == 1;
  if (tile_rows == 256) {
    if (tile_waves == 4) launch_moe<4, 256>(a, nk, ob, grid, stream, done);
    else launch_moe<8, 256>(a, nk, ob, grid, stream, done);
  } else {
    if (tile_waves == 4) launch_moe<4, 128>(a, nk, ob, grid, stream, done);
    else launch_moe<8, 128>(a, nk, ob, grid, stream, done);
  }
  return hipGetLastError();
}

}  // namespace sgt
