// The signal-gated reduction item of a ReduceScatter (Triton-distributed
// semantics page, "GEMM + ReduceScatter overlap": the reduction of a tile waits
// for the signals of every contribution to it; paper summary, "Method":
// ReduceScatter with the reduction synchronized by signals), shared by the
// dense GEMM+ReduceScatter and the MoE combine kernels.
//
// Item j is signal tile j of this rank's row block: wait for its flag in
// gflags (the local partial P) and for the W-1 peer flags, then
// C_shard = P[local] + sum of the peers' partials, in fixed order (local, then
// peers by ascending rank).
#pragma once

#include <hip/hip_runtime.h>

#include "common.hpp"
#include "mfma_tile.hpp"
#include "signal.hpp"

namespace sgt {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ inline void do_reduce_item(const RsArgs& a, int j, int* ok) {
  const int ti = j / a.rs_tn, tj = j % a.rs_tn;
  const int64_t gtn = (a.N + a.rs_tile - 1) / a.rs_tile;
  const int64_t row0 = (int64_t)a.rank * a.block_rows + (int64_t)ti * a.rs_tile;  // row in P
  if (threadIdx.x == 0) {
    bool good = wait_flags_one_thread(a.gflags, (row0 / a.rs_tile) * gtn + tj, (row0 / a.rs_tile) * gtn + tj + 1,
                                      a.epoch, a.timeout_ticks, a.status);
    const int64_t per = (int64_t)a.rs_tm * a.rs_tn;
    for (int p = 0; p < a.W && good; ++p)
      if (p != a.rank)
        good = wait_flags_one_thread(a.pflags, p * per + j, p * per + j + 1, a.epoch, a.timeout_ticks, a.status);
    *ok = good ? 1 : 0;
  }
  __syncthreads();
  if (!*ok) return;
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
  for (int r0 = rr; r0 < a.rs_tile; r0 += R * rows_per_pass) {
    uint32_t off[R];
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int r = r0 + u * rows_per_pass;
      off[u] = (col_ok && r < a.rs_tile) ? (uint32_t)(((int64_t)r * a.N + col) * 4) : kOOB;
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

}  // namespace sgt
