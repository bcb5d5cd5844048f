// MoE GEMM + ReduceScatter, the combine side of an MoE layer (paper summary,
// "Experiments": MoE ReduceScatter among the kernels measured; Triton-distributed
// semantics page, "GEMM + ReduceScatter overlap": the GEMM signals each output
// tile and the reduction waits for exactly the tiles it reads).
//
//   Y[r]  = Hg[r] * W2[e(r)]                      grouped rows x expert weight
//   P[t]  = sum_j gate[t][j] * Y[row(t, j)]       per-token combine, pick order
//   C     = P[rank block] + sum_p partial_p       the ReduceScatter of GEMM+RS
//
// A prologue kernel builds the inverse routing table row(t, j), the list of
// 256-row tiles of the expert groups, and clears the counters.  One persistent
// kernel then holds three kinds of work:
//   GEMM tiles      static, column-major over (256-row group tile, 256-column
//                   tile); each stores its Y tile with device-scope stores and
//                   counts itself done in its column;
//   combine tiles   claimed in column-major order: a 128-token x 128-column tile
//                   of P waits until every group tile of its GEMM column is
//                   done, sums each token's k rows with its gates, stores P and
//                   publishes the tile's flag (the GEMM+RS flag layout);
//   reduction tiles claimed after every combine tile: the dense GEMM+RS
//                   reduction item (this rank's block of P plus the peers').
// Dependencies point only from later kinds to earlier ones and a workgroup
// claims only after its own GEMM tiles, with at most one workgroup per CU, so
// the kernel cannot deadlock; every wait is bounded.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "mfma_tile.hpp"
#include "rs_reduce.hpp"
#include "sched.hpp"
#include "signal.hpp"

namespace sgt {

namespace {

constexpr int kCombTile = 128;  // combine tile: tokens x columns (the GEMM+RS signal tile)
constexpr int kCombPicks = 8;   // picks of a token whose rows are loaded together

// One workgroup of kPrepThreads (>= the 256 experts the host allows).
constexpr int kPrepThreads = 256;

__global__ void __launch_bounds__(kPrepThreads) moe_rs_prep_kernel(MoeRsArgs a) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  if (blockIdx.x == 0) {
    for (int c = threadIdx.x; c < a.tiles_n; c += blockDim.x) a.col_done[c] = 0u;
    if (threadIdx.x == 0) *a.claim = 0u;
    // 256-row tiles of each expert's group, experts in order: thread e counts
    // expert e's tiles, an exclusive prefix sum over the threads gives its
    // first entry, and it writes its own tiles (entries past tiles_cap are
    // dropped, as the host sized the table for every routing).
    __shared__ int scan[kPrepThreads];
    const int e = threadIdx.x;
    const int64_t g0 = e < a.E ? a.expert_off[e] : 0, g1 = e < a.E ? a.expert_off[e + 1] : 0;
    const int mine = g1 > g0 ? (int)((g1 - g0 + kBM - 1) / kBM) : 0;
    scan[e] = mine;
    __syncthreads();
    for (int d = 1; d < kPrepThreads; d <<= 1) {  // inclusive Hillis-Steele scan
      const int v = e >= d ? scan[e - d] : 0;
      __syncthreads();
      scan[e] += v;
      __syncthreads();
    }
    const int first = scan[e] - mine;
    for (int i = 0; i < mine; ++i)
      if (first + i < a.tiles_cap) {
        const int64_t r0 = g0 + (int64_t)i * kBM;
        a.tiles[first + i] = MoeTile{e, (int32_t)r0, (int32_t)(g1 - r0 < kBM ? g1 - r0 : kBM)};
      }
    if (e == kPrepThreads - 1) *a.n_row_tiles = (uint32_t)(scan[e] < a.tiles_cap ? scan[e] : a.tiles_cap);
  }
  // inverse routing: the row holding pick (t, j) is the row of group topk_ids[t][j] whose token is t
  for (int64_t r = gid; r < a.rows; r += stride) {
    const int32_t t = a.row_token[r];
    if (t < 0 || t >= a.T) continue;
    int lo = 0, hi = a.E;  // expert of row r: the last e with expert_off[e] <= r
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.expert_off[mid] <= r) lo = mid;
      else hi = mid;
    }
    for (int j = 0; j < a.k; ++j)
      if (a.topk_ids[(int64_t)t * a.k + j] == lo) a.row_of[(int64_t)t * a.k + j] = (int32_t)r;
  }
}

// Four columns of grouped row `row` of Y as fp32 (an fp32 Y: one 16-byte
// load; a bf16 Y: one 8-byte load of four bf16, widened exactly).
template <bool kYbf16>
__device__ __forceinline__ f32x4_t load_y4(__amdgpu_buffer_rsrc_t rY, int32_t row, int64_t H, int64_t col,
                                           bool col_ok) {
  if constexpr (kYbf16) {
    const uint32_t off = col_ok ? (uint32_t)(((int64_t)row * H + col) * 2) : kOOB;
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    const u32x2_t w = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rY, off, 0, 0));
    const f32x4_t v = {__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                       __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u)};
    return v;
  } else {
    const uint32_t off = col_ok ? (uint32_t)(((int64_t)row * H + col) * 4) : kOOB;
    return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rY, off, 0, 0));
  }
}

// Combine tile c of P: 128 tokens x 128 columns, column-major.
template <bool kYbf16>
__device__ void do_combine_item(const MoeRsArgs& a, int64_t c, uint32_t n_rt, int* ok) {
  const int64_t ptm = a.T / kCombTile;
  const int64_t cn = c / ptm, cm = c % ptm;
  const int64_t ct = cn * kCombTile / kBN;  // the GEMM column tile holding these columns
  if (threadIdx.x == 0) {
    const uint64_t t0 = clock_ticks();
    bool good = true;
    uint32_t v = __hip_atomic_load(a.col_done + ct, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    while (v < n_rt) {
      if (clock_ticks() - t0 > a.rs.timeout_ticks) {
        report_timeout(a.rs.status, ct, v, n_rt);
        good = false;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
      v = __hip_atomic_load(a.col_done + ct, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (good) acquire_agent();
    *ok = good ? 1 : 0;
  }
  __syncthreads();
  if (!*ok) return;
  // float4 columns as in the reduction; every access is a buffer access with
  // an out-of-range offset for a column past H, so the loop has no branches.
  const int cols4 = kCombTile / 4;
  const int rows_per_pass = (int)blockDim.x / cols4;
  const int c4 = threadIdx.x % cols4, rr = threadIdx.x / cols4;
  const int64_t col = cn * kCombTile + 4 * c4;
  const bool col_ok = col < a.H;
  const __amdgpu_buffer_rsrc_t rY = make_rsrc(a.Y, (uint64_t)a.rows * (uint64_t)a.H * (kYbf16 ? 2u : 4u));
  const __amdgpu_buffer_rsrc_t rP = make_rsrc(a.rs.P, (uint64_t)a.T * (uint64_t)a.H * 4u);
  const __amdgpu_buffer_rsrc_t rG = make_rsrc(a.gate, (uint64_t)a.T * (uint64_t)a.k * 4u);
  const __amdgpu_buffer_rsrc_t rR = make_rsrc(a.row_of, (uint64_t)a.T * (uint64_t)a.k * 4u);
  // Per pass, two memory round trips per group of kCombPicks picks: the
  // group's gates and rows first, then all of its Y rows (picks past k read
  // zero through out-of-range offsets and are not added).
  for (int r0 = rr; r0 < kCombTile; r0 += rows_per_pass) {
    const int64_t t = cm * kCombTile + r0;  // < T: T is a multiple of the tile
    f32x4_t s = {0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < a.k; j0 += kCombPicks) {
      float g[kCombPicks];
      int32_t row[kCombPicks];
#pragma unroll
      for (int j = 0; j < kCombPicks; ++j) {
        const uint32_t pick = j0 + j < a.k ? (uint32_t)((t * a.k + j0 + j) * 4) : kOOB;
        g[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rG, pick, 0, 0));
        row[j] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(rR, pick, 0, 0);
      }
      f32x4_t y[kCombPicks];
#pragma unroll
      for (int j = 0; j < kCombPicks; ++j) y[j] = load_y4<kYbf16>(rY, row[j], a.H, col, col_ok && j0 + j < a.k);
#pragma unroll
      for (int j = 0; j < kCombPicks; ++j) {
        // the sum starts from pick 0's term (not from +0, which would turn a -0 term into +0)
        if (j0 + j == 0) s = g[0] * y[0];
        else if (j0 + j < a.k) s += g[j] * y[j];
      }
    }
    const uint32_t off = col_ok ? (uint32_t)((t * a.H + col) * 4) : kOOB;
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, s), rP, off, 0, kCpolSc1);
  }
  // every wave's device-scope stores acknowledged, then one lane publishes the tile
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const int64_t gtn = (a.H + kCombTile - 1) / kCombTile;
    flag_publish_coherent(a.rs.gflags + cm * gtn + cn, a.rs.epoch);
  }
}

template <bool kBNK, bool kYbf16>
__global__ void __launch_bounds__(Tile<8>::kThreads, 1) moe_rs_kernel(MoeRsArgs a) {
  constexpr int kW = 8;
  __shared__ int ok;
  __shared__ int claimed;
  const int G = gridDim.x;
  uint32_t n_rt = *a.n_row_tiles;
  n_rt = n_rt < (uint32_t)a.tiles_cap ? n_rt : (uint32_t)a.tiles_cap;
  const int64_t n_gemm = (int64_t)n_rt * a.tiles_n;
  const uint16_t* Hg = a.Hg;
  for (int64_t g = xcd_remap(blockIdx.x, G); g < n_gemm; g += G) {
    const int64_t ct = g / n_rt, rt = g % n_rt;
    const MoeTile mt = a.tiles[rt];
    const int e = mt.expert;
    const int64_t r0 = mt.r0;
    int64_t r_end = a.expert_off[e + 1];
    r_end = r_end < a.rows ? r_end : a.rows;  // the tables are exact; this only bounds every access
    const int64_t n0 = ct * kBN;
    if (r0 < r_end) {  // (uniform)
      const uint16_t* Be = a.W2 + (int64_t)e * a.I * a.H;
      const KRows ka = krows_strided<kW>(Hg + r0 * a.I, r_end - r0, a.I);
      KRows kb = ka;
      if constexpr (kBNK) kb = krows_strided<kW>(Be + n0 * a.I, a.H - n0, a.I);
      MfmaAcc<kW> acc;
      gemm_tile<kW, kBNK>(ka, kb, Be, a.H, n0, a.I, acc);
      store_tile<kW, kYbf16, kCpolSc1>(a.Y, r_end, a.H, r0, n0, acc);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_fetch_add(a.col_done + ct, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  const int64_t n_comb = (a.T / kCombTile) * ((a.H + kCombTile - 1) / kCombTile);
  const int64_t n_red = a.rs.n_red_items;
  while (true) {
    if (threadIdx.x == 0) claimed = (int)atomicAdd(a.claim, 1u);
    __syncthreads();
    const int64_t j = claimed;
    __syncthreads();
    if (j >= n_comb + n_red) break;
    if (j < n_comb) do_combine_item<kYbf16>(a, j, n_rt, &ok);
    else do_reduce_item(a.rs, (int)(j - n_comb), &ok);
    if (!ok) return;
    __syncthreads();
  }
  // paced peers: the join with the producer (its workgroups count themselves finished)
  wait_producer_done(a.rs.prod_done, a.rs.prod_done_all, a.rs.timeout_ticks, a.rs.status);
}

}  // namespace

// `done`, when given, is recorded by the main kernel's launch at its end (no
// separate marker on the stream).
hipError_t launch_moe_rs(const MoeRsArgs& a, int grid, hipStream_t stream, hipEvent_t done) {
  int64_t pb = (a.rows + 255) / 256;
  if (pb < 1) pb = 1;
  if (pb > 1024) pb = 1024;
  hipLaunchKernelGGL(moe_rs_prep_kernel, dim3((unsigned)pb), dim3(kPrepThreads), 0, stream, a);
  auto go = [&](auto kernel) {
    hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(Tile<8>::kThreads), 0, stream, nullptr, done, 0, a);
  };
  if (a.b_layout == 1) {
    if (a.y_bf16) go(moe_rs_kernel<true, true>);
    else go(moe_rs_kernel<true, false>);
  } else {
    if (a.y_bf16) go(moe_rs_kernel<false, true>);
    else go(moe_rs_kernel<false, false>);
  }
  return hipGetLastError();
}

}  // namespace sgt
