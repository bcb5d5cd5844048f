// AllGather + GEMM consumer: a persistent GEMM that waits on each row panel's
// flags before reading it (Triton-distributed semantics page, "AllGather + GEMM
// overlap": the consumer waits for each tile, then computes it at once;
// "Threadblock swizzle": start on local data; paper summary, "Method": the GEMM
// gains wait + consume_token before its loads, and AMD persistent kernels).
//
// Two kernels share the schedule and the wait:
//  * ag_consumer_bf16: bf16 inputs on the matrix cores (mfma_tile.hpp), 256 x 256
//    tiles, one workgroup (4 or 8 wave64s) per CU.
//  * ag_consumer_f32: fp32 inputs with fp32 FMAs (64 x 64 tiles), for fp32
//    workloads where a bf16 downcast would lose the required accuracy.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "mfma_tile.hpp"
#include "sched.hpp"
#include "signal.hpp"

namespace sgt {

namespace {

// Wait for flags [f0, f1) and record trace stamps.
__device__ __forceinline__ bool gate_flags(const AgArgs& a, int64_t f0, int64_t f1, int* ok, int64_t tile_id) {
  const uint64_t t_wait = a.trace && threadIdx.x == 0 ? clock_ticks() : 0;
  const bool good = wait_flags_block(a.flags, f0, f1, a.epoch, a.timeout_ticks, a.status, ok);
  if (a.trace && threadIdx.x == 0) {
    a.trace[tile_id * 4 + 0] = t_wait;
    a.trace[tile_id * 4 + 1] = clock_ticks();
    a.trace[tile_id * 4 + 3] = blockIdx.x;
  }
  return good;
}

// Wait for the flags covering rows [m0, m1) (signal tiles of flag_rows rows x all K).
__device__ __forceinline__ bool gate_rows(const AgArgs& a, int64_t m0, int64_t m1, int* ok, int64_t tile_id) {
  return gate_flags(a, m0 / a.flag_rows, (m1 - 1) / a.flag_rows + 1, ok, tile_id);
}

// K-chunked signal tiles: are all n_kc chunk flags of panel pm set?  One peek
// per chunk (lane q of wave 0), no waiting; when they are, the acquire follows
// and the trace records the tile as ready at once.
__device__ __forceinline__ bool panel_chunks_in(const AgArgs& a, int64_t pm, int* ok, int64_t tile_id) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const bool in = lane >= a.n_kc || flag_is_set(flag_peek(a.flags + pm * a.n_kc + lane), a.epoch);
    const bool all = __all(in);
    if (all) acquire_agent();
    if (lane == 0) {
      *ok = all ? 1 : 0;
      if (a.trace) {
        const uint64_t now = clock_ticks();
        a.trace[tile_id * 4 + 0] = now;
        a.trace[tile_id * 4 + 1] = now;
        a.trace[tile_id * 4 + 3] = blockIdx.x;
      }
    }
  }
  __syncthreads();
  return *ok != 0;
}

// K-chunked signal tiles: how many chunks q0, q0 + 1, ... of panel pm are
// already in, counted up to the first that is not (one peek per lane of wave
// 0, no waiting; an acquire when any is).  `n` must be a __shared__ int.
__device__ __forceinline__ int chunks_in_after(const AgArgs& a, int64_t pm, int q0, int* n) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x, q = q0 + lane;
    const bool in = q < a.n_kc && flag_is_set(flag_peek(a.flags + pm * a.n_kc + q), a.epoch);
    const uint64_t missing = __ballot(!in);  // lanes past the panel's chunks count as missing
    const int run = missing ? __builtin_ctzll(missing) : 64;
    if (run > 0) acquire_agent();
    if (lane == 0) *n = run;
  }
  __syncthreads();
  return *n;
}

// A traced tile's end: its end time, and in the last word the workgroup
// (bits 0..15) with the engine-clock cycles since cyc0 (bits 16..63).
__device__ __forceinline__ void trace_tile_end(uint64_t* rec, uint64_t cyc0) {
  rec[2] = clock_ticks();
  rec[3] = (uint64_t)blockIdx.x | ((__builtin_amdgcn_s_memtime() - cyc0) << 16);
}

// The next tile of this workgroup, or -1: the static schedule (tile t, then
// t + G, ...) or, with dynamic claiming, the next claim from this XCD's list
// and then from the other XCDs' lists (thread 0 claims; `x`, `left` and
// `next` are its state; the result goes through a shared word).
__device__ __forceinline__ int next_tile(const AgArgs& a, int total, int* x, int* left, int* next, int* tile_s) {
  if (!a.xcd_claim) {
    const int t = *next;
    *next += gridDim.x;
    return t < total ? t : -1;
  }
  if (threadIdx.x == 0) {
    int t = -1;
    while (*left > 0) {
      const uint32_t c = atomicAdd(a.xcd_claim + *x * kXcdClaimStride, 1u);
      t = (int)xcd_seq_tile(*x, c, a.base_grid, total);
      if (t >= 0) break;
      *x = (*x + 1) % kXcds;
      --*left;
    }
    *tile_s = t;
  }
  __syncthreads();
  const int t = *tile_s;
  __syncthreads();  // every thread has read tile_s before thread 0 may claim again
  return t;
}

// The workgroup's shared words.  all_in and n_more have words of their own:
// the chunk waits that may follow rewrite `ok` with no barrier between.
struct AgWords {
  int ok, all_in, n_more, tile_s;
};

template <int kW, bool kBNK, bool kOutBf16>
__global__ void __launch_bounds__(Tile<kW>::kThreads, 1) ag_consumer_bf16(AgArgs a) {
  // LDS: the K loop's stages (the step loop's four, or the ring's five slots
  // of 32 KiB, 160 KiB in all).  With the ring the shared words live at the
  // start of the fifth slot: they are used only between K ranges, when no
  // load is in flight, and the ring writes that slot first in its first step,
  // after a barrier every wave passes once it has read them.
  constexpr bool kRing = kW == 8 && kBNK;
  __shared__ __attribute__((aligned(1024))) uint8_t s0[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t s1[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t s2[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t s3[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t s4[kRing ? kStageBytes : sizeof(AgWords)];
  AgWords* const wd = reinterpret_cast<AgWords*>(s4);
  int& ok = wd->ok;
  const int total = a.tiles_m * a.tiles_n;
  const uint16_t* A = static_cast<const uint16_t*>(a.A);
  const uint16_t* B = static_cast<const uint16_t*>(a.B);
  // the next launch's claim counters start at zero (stream order publishes them)
  if (a.xcd_claim_next && blockIdx.x == 0 && threadIdx.x < kXcds) a.xcd_claim_next[threadIdx.x * kXcdClaimStride] = 0u;
  if (a.late_blocks > 0 && (int)blockIdx.x >= (int)gridDim.x - a.late_blocks) {
    // a workgroup that may sit on a CU the producer needs: run only if every
    // producer workgroup is already running (one check, no wait); it then
    // claims tiles like the others
    if (threadIdx.x == 0)
      ok = __hip_atomic_load(a.started, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.started_all ? 1 : 0;
    __syncthreads();
    if (!ok) return;
  }
  int xq = (int)(blockIdx.x % kXcds), left = kXcds, next = xcd_remap(blockIdx.x, gridDim.x);
  // K steps [k0, k1) of the tile at column n0 into acc
  auto k_range = [&](const KRows& ka, const KRows& kb, int64_t n0, int64_t k0, int64_t k1, MfmaAcc<kW>& acc) {
    if constexpr (kRing) gemm_tile_range_r5<kBM, true>(ka, kb, k0, k1, acc, s0, s1, s2, s3, s4);
    else gemm_tile_range_lds<kW, kBNK, kBM>(ka, kb, B, a.N, n0, a.K, k0, k1, acc, s0, s1, s2, s3);
  };
  for (int t = next_tile(a, total, &xq, &left, &next, &wd->tile_s); t >= 0;
       t = next_tile(a, total, &xq, &left, &next, &wd->tile_s)) {
    // traced: the tile's engine-clock cycles (waits included) go beside the
    // workgroup in its last trace word, so a trace also gives the clock
    const uint64_t cyc0 = a.trace && threadIdx.x == 0 ? __builtin_amdgcn_s_memtime() : 0;
    int64_t seq_m, pn;
    tile_at(t, a.tiles_m, a.tiles_n, &seq_m, &pn);
    const int64_t pm = panel_at(seq_m, a.tiles_m, a.rows_per_shard, kBM, a.W, a.rank, a.order);
    const int64_t m0 = pm * kBM, n0 = pn * kBN;
    const int64_t m1 = m0 + kBM < a.M ? m0 + kBM : a.M;
    const int64_t tile_id = (int64_t)pm * a.tiles_n + pn;
    // A panel that lies inside the local shard is read from the shard itself
    // and needs no wait; any other panel waits for its flags and is read from
    // the gathered buffer.
    const int64_t l0 = (int64_t)a.rank * a.rows_per_shard;
    const bool local = m0 >= l0 && m1 <= l0 + a.rows_per_shard;
    const uint16_t* Abase = A + m0 * a.K;
    int64_t rows_valid = a.M - m0;
    if (local) {
      Abase = static_cast<const uint16_t*>(a.A_local) + (m0 - l0) * a.K;
      rows_valid = l0 + a.rows_per_shard - m0;
      if (a.trace && threadIdx.x == 0) {
        const uint64_t now = clock_ticks();
        a.trace[tile_id * 4 + 0] = now;
        a.trace[tile_id * 4 + 1] = now;
        a.trace[tile_id * 4 + 3] = blockIdx.x;
      }
    } else if (a.n_kc > 0) {
      // K-chunked signal tiles: when every chunk of the panel is in, the tile
      // runs at once; otherwise it takes the chunks in order as they land (the
      // 8-wave tile with B stored N x K, the one whose registers leave room for
      // a second K loop; the other variants wait for the whole panel).
      if constexpr (kW != 8 || !kBNK) {
        if (!gate_flags(a, pm * a.n_kc, (pm + 1) * a.n_kc, &ok, tile_id)) return;
      } else if (!panel_chunks_in(a, pm, &wd->all_in, tile_id)) {
        const KRows ka = krows_strided<kW>(Abase, rows_valid, a.K);
        KRows kb = ka;
        if constexpr (kBNK) kb = krows_strided<kW>(B + n0 * a.K, a.N - n0, a.K);
        MfmaAcc<kW> acc;
        acc_zero<kW>(acc);
        // each range: wait for the next chunk, then take it with every later
        // chunk already in (a range pays one pipeline start, so few and long)
        for (int q = 0; q < a.n_kc;) {
          const int64_t f = pm * a.n_kc + q;
          if (!wait_flags_block(a.flags, f, f + 1, a.epoch, a.timeout_ticks, a.status, &ok)) return;
          if (q == 0 && a.trace && threadIdx.x == 0) a.trace[tile_id * 4 + 1] = clock_ticks();
          const int q_end = q + 1 + chunks_in_after(a, pm, q + 1, &wd->n_more);
          k_range(ka, kb, n0, (int64_t)q * a.kc_cols, (int64_t)q_end * a.kc_cols, acc);
          q = q_end;
        }
        store_tile<kW, kOutBf16>(a.C, a.M, a.N, m0, n0, acc);
        if (a.trace && threadIdx.x == 0) trace_tile_end(a.trace + tile_id * 4, cyc0);
        continue;
      }
    } else if (!gate_rows(a, m0, m1, &ok, tile_id)) {
      return;
    }

    const KRows ka = krows_strided<kW>(Abase, rows_valid, a.K);
    KRows kb = ka;
    if constexpr (kBNK) kb = krows_strided<kW>(B + n0 * a.K, a.N - n0, a.K);
    MfmaAcc<kW> acc;
    acc_zero<kW>(acc);
    k_range(ka, kb, n0, 0, a.K, acc);
    store_tile<kW, kOutBf16>(a.C, a.M, a.N, m0, n0, acc);
    if (a.trace && threadIdx.x == 0) trace_tile_end(a.trace + tile_id * 4, cyc0);
  }
  wait_producer_done(a.prod_done, a.prod_done_all, a.timeout_ticks, a.status);
}

// fp32 path: 64 x 64 tiles, BK = 16, each thread a 4 x 4 block of outputs.
constexpr int kF32BM = 64, kF32BN = 64, kF32BK = 16;

__global__ void __launch_bounds__(256) ag_consumer_f32(AgArgs a) {
  __shared__ float As[kF32BK][kF32BM + 4];
  __shared__ float Bs[kF32BK][kF32BN + 4];
  __shared__ int ok;
  const float* A = static_cast<const float*>(a.A);
  const float* B = static_cast<const float*>(a.B);
  const int total = a.tiles_m * a.tiles_n;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int G = gridDim.x;
  for (int t = xcd_remap(blockIdx.x, G); t < total; t += G) {
    const int64_t pn = t % a.tiles_n;
    const int64_t pm = panel_at(t / a.tiles_n, a.tiles_m, a.rows_per_shard, kF32BM, a.W, a.rank, a.order);
    const int64_t m0 = pm * kF32BM, n0 = pn * kF32BN;
    const int64_t m1 = m0 + kF32BM < a.M ? m0 + kF32BM : a.M;
    const int64_t tile_id = pm * a.tiles_n + pn;
    if (!gate_rows(a, m0, m1, &ok, tile_id)) return;

    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

    for (int64_t k0 = 0; k0 < a.K; k0 += kF32BK) {
      {  // A tile: row tid / 4, k (tid % 4) * 4 + u
        const int r = tid >> 2, kq = (tid & 3) * 4;
        const int64_t m = m0 + r;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int64_t k = k0 + kq + u;
          As[kq + u][r] = (m < a.M && k < a.K) ? A[m * a.K + k] : 0.f;
        }
      }
      if (a.b_layout == 0) {  // K x N: k tid / 16, n (tid % 16) * 4 + u
        const int kk = tid >> 4, nq = (tid & 15) * 4;
        const int64_t k = k0 + kk;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int64_t n = n0 + nq + u;
          Bs[kk][nq + u] = (k < a.K && n < a.N) ? B[k * a.N + n] : 0.f;
        }
      } else {  // N x K: n tid / 4, k (tid % 4) * 4 + u
        const int nn = tid >> 2, kq = (tid & 3) * 4;
        const int64_t n = n0 + nn;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int64_t k = k0 + kq + u;
          Bs[kq + u][nn] = (k < a.K && n < a.N) ? B[n * a.K + k] : 0.f;
        }
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < kF32BK; ++kk) {
        float av[4], bv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) av[i] = As[kk][ty * 4 + i];
#pragma unroll
        for (int j = 0; j < 4; ++j) bv[j] = Bs[kk][tx * 4 + j];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(av[i], bv[j], acc[i][j]);
      }
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = m0 + ty * 4 + i;
      if (m >= a.M) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t n = n0 + tx * 4 + j;
        if (n >= a.N) continue;
        if (a.out_dtype == 0)
          static_cast<float*>(a.C)[m * a.N + n] = acc[i][j];
        else
          static_cast<uint16_t*>(a.C)[m * a.N + n] = f32_to_bf16_rne(acc[i][j]);
      }
    }
    if (a.trace && threadIdx.x == 0) a.trace[tile_id * 4 + 2] = clock_ticks();
  }
}

}  // namespace

int ag_panel_rows(int in_dtype) { return in_dtype == 1 ? kBM : kF32BM; }
int ag_panel_cols(int in_dtype) { return in_dtype == 1 ? kBN : kF32BN; }

// `done`, when given, is recorded by the launch itself at the kernel's end (no
// separate marker on the stream).
template <int kW>
static void launch_bf16(const AgArgs& a, int grid, hipStream_t stream, hipEvent_t done) {
  const bool nk = a.b_layout == 1, ob = a.out_dtype == 1;
  auto go = [&](auto kernel) {
    hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(Tile<kW>::kThreads), 0, stream, nullptr, done, 0, a);
  };
  if (nk && ob) go(ag_consumer_bf16<kW, true, true>);
  if (nk && !ob) go(ag_consumer_bf16<kW, true, false>);
  if (!nk && ob) go(ag_consumer_bf16<kW, false, true>);
  if (!nk && !ob) go(ag_consumer_bf16<kW, false, false>);
}

hipError_t launch_ag_consumer(const AgArgs& a, int in_dtype, int grid, hipStream_t stream, hipEvent_t done) {
  if (in_dtype == 1) {
    if (a.tile_waves == 4) launch_bf16<4>(a, grid, stream, done);
    else launch_bf16<8>(a, grid, stream, done);
  } else {
    hipExtLaunchKernelGGL(ag_consumer_f32, dim3(grid), dim3(256), 0, stream, nullptr, done, 0, a);
  }
  return hipGetLastError();
}

}  // namespace sgt
