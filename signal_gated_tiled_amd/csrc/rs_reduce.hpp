// The signal-gated reduction item of a ReduceScatter (Triton-distributed
// semantics page, "GEMM + ReduceScatter overlap": the reduction of a tile waits
// for the signals of every contribution to it; paper summary, "Method":
// ReduceScatter with the reduction synchronized by signals), shared by the
// dense GEMM+ReduceScatter and the MoE combine kernels.
//
// Item j is row band j % red_split of signal tile j / red_split of this
// rank's row block: wait for the tile's flag in gflags (the local partial P)
// and for its W-1 peer flags, then C_shard = P[local] + sum of the peers'
// partials over the band's rows, in fixed order (local, then peers by
// ascending rank).  Bands of a few tens of rows keep the items small enough
// to spread evenly over the workgroups (each streams at a bounded rate).
#pragma once

#include <hip/hip_runtime.h>

#include "common.hpp"
#include "mfma_tile.hpp"
#include "signal.hpp"

namespace sgt {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// The flag lane `lane` of wave 0 watches for item j: lane `rank` the GEMM flag
// of the local tile (in gflags), lane p < W peer p's flag of the tile (in
// pflags), the other lanes none.  `idx` is the flag's index for a timeout
// report.
struct RedFlag {
  const uint32_t* f;
  int64_t idx;
};

__device__ inline RedFlag red_flag(const RsArgs& a, int j, int lane) {
  const int jt = j / a.red_split;
  const int ti = jt / a.rs_tn, tj = jt % a.rs_tn;
  const int64_t gtn = (a.N + a.rs_tile - 1) / a.rs_tile;
  const int64_t row0 = (int64_t)a.rank * a.block_rows + (int64_t)ti * a.rs_tile;  // row in P
  const int64_t per = (int64_t)a.rs_tm * a.rs_tn;
  const int64_t gidx = (row0 / a.rs_tile) * gtn + tj, pidx = lane * per + jt;
  if (lane >= a.W) return RedFlag{nullptr, 0};
  return lane == a.rank ? RedFlag{a.gflags + gidx, gidx} : RedFlag{a.pflags + pidx, pidx};
}

// Wave 0: wait until every flag of an item is set, given `v`, the value of a
// peek already taken (so a peek issued early costs no round trip here); then
// the acquire.  False after a timeout (recorded in the status word).
__device__ inline bool red_wait(const RsArgs& a, RedFlag rf, uint32_t v) {
  bool mine = rf.f == nullptr || flag_is_set(v, a.epoch);
  const uint64_t t0 = clock_ticks();
  while (!__all(mine)) {
    if (clock_ticks() - t0 > a.timeout_ticks) {  // the clock is a scalar read: uniform over the wave
      if (!mine) report_timeout(a.status, rf.idx, v, a.epoch);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
    if (!mine) {
      v = flag_peek(rf.f);
      mine = flag_is_set(v, a.epoch);
    }
  }
  acquire_agent();
  return true;
}

// The workgroup's part of item j once its flags are in: row band j % red_split
// of signal tile j / red_split, C_shard = P[local] + the peers' partials.
__device__ inline void red_stream(const RsArgs& a, int j) {
  const int jt = j / a.red_split, rband = j % a.red_split;
  const int ti = jt / a.rs_tn, tj = jt % a.rs_tn;
  const int64_t row0 = (int64_t)a.rank * a.block_rows + (int64_t)ti * a.rs_tile;  // row in P
  // float4 columns: rs_tile / 4 per row; a pass of the workgroup covers
  // blockDim / (rs_tile / 4) rows.  Four passes are issued together so each
  // thread has 4 x W loads in flight (the reduction is bound by HBM latency
  // times bytes in flight per workgroup).  Every access is a buffer access
  // whose record range is the rs_tile x N band of its operand: a row past the
  // tile or a column past N gets an out-of-range offset (loads read zero,
  // stores are dropped), so the loop has no branches and the compiler issues
  // all of a pass's loads before waiting (a guarded load would wait for each).
  const int cols4 = a.rs_tile / 4;
  const int rows_per_pass = (int)blockDim.x / cols4;
  const int c4 = threadIdx.x % cols4, rr = threadIdx.x / cols4;
  const int64_t col = (int64_t)tj * a.rs_tile + 4 * c4;
  const bool col_ok = col < a.N;  // N % 4 == 0: a float4 is either fully in or out
  const uint64_t band = (uint64_t)a.rs_tile * (uint64_t)a.N * 4u;  // < 2^31 (checked by the host)
  const __amdgpu_buffer_rsrc_t rP = make_rsrc(a.P + row0 * a.N, band);
  const __amdgpu_buffer_rsrc_t rC = make_rsrc(a.C_shard + (int64_t)ti * a.rs_tile * a.N, band);
  constexpr int R = 4;
  const int band_rows = a.rs_tile / a.red_split, rb_end = (rband + 1) * band_rows;
  for (int r0 = rband * band_rows + rr; r0 < rb_end; r0 += R * rows_per_pass) {
    uint32_t off[R];
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int r = r0 + u * rows_per_pass;
      off[u] = (col_ok && r < rb_end) ? (uint32_t)(((int64_t)r * a.N + col) * 4) : kOOB;
    }
    f32x4_t s[R];
#pragma unroll
    for (int u = 0; u < R; ++u)
      s[u] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rP, off[u], 0, 0));
    // peers in ascending rank, skipping this rank by index arithmetic
#pragma unroll 8
    for (int q = 0; q < a.W - 1; ++q) {
      const int p = q + (q >= a.rank ? 1 : 0);
      const float* part = static_cast<const float*>(a.partials.p[p]) + (int64_t)ti * a.rs_tile * a.N;
      const __amdgpu_buffer_rsrc_t rq = make_rsrc(part, band);
#pragma unroll
      for (int u = 0; u < R; ++u)
        s[u] += __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rq, off[u], 0, kCpolNt));
    }
#pragma unroll
    for (int u = 0; u < R; ++u)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, s[u]), rC, off[u], 0, kCpolNt);
  }
}

// Item j, whole: wave 0 polls the item's W flags at once (one lane per
// contribution), then the workgroup streams the band.  *ok = 0 after a timeout.
__device__ inline void do_reduce_item(const RsArgs& a, int j, int* ok) {
  if (threadIdx.x < 64) {
    const RedFlag rf = red_flag(a, j, threadIdx.x);
    const bool good = red_wait(a, rf, rf.f ? flag_peek(rf.f) : 0u);
    if (threadIdx.x == 0) *ok = good ? 1 : 0;
  }
  __syncthreads();
  if (!*ok) return;
  red_stream(a, j);
}

}  // namespace sgt
