// MoE routing on the GPU: top-k experts per token, rows grouped by expert, and
// the grouped consumer's work list ordered by when its rows can arrive
// (paper summary, "Experiments": MoE routing operations among the
// communication-bound kernels; DITRON article, "three-level tiling": the
// device-level tiles of an MoE layer take their sizes from how many tokens each
// expert receives, known only at run time).
//
// Three launches after the per-expert counters are cleared:
//  1. moe_topk_kernel  -- one wave per token: k rounds of a wave-wide argmax
//     over the token's logits (largest logit first, equal logits: lower expert
//     id), each pick counted per expert.
//  2. moe_place_kernel -- one workgroup per expert: prefix sums of the counts
//     give the expert's first row (expert_off) and first row tile; a pass over
//     the tokens in ascending order places each token that chose the expert at
//     the next row of its group, and the readiness key of each 256-row tile is
//     the latest arrival rank among the signal tiles its rows come from.
//  3. moe_sort_kernel  -- one workgroup: a stable counting sort of the row tiles
//     by readiness key, so the consumer claims first the tiles whose rows land
//     first.
// Every table the consumer reads is an integer result that does not depend on
// the order of atomic updates: the counts are sums, and positions come from
// prefix sums over tokens in ascending order.
#include <hip/hip_runtime.h>

#include "common.hpp"

namespace sgt {

namespace {

constexpr int kRouteRows = 256;        // rows per grouped row tile (the MFMA tile height)
constexpr int kMaxTilesPerExpert = 4096;
constexpr int kSortBuckets = 1024;

// Order-preserving map of an fp32 value to uint32 (total order; -0 and +0
// compare equal, as floating-point comparison has them).
__device__ __forceinline__ uint32_t sort_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, m, 64);
    const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), m, 64);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

// One wave per token.  Lane l holds experts l, l + 64, l + 128, l + 192 as
// (key << 32) | (0xFFFFFFFF - e): the wave maximum is the largest logit and,
// among equal logits, the lowest expert id.  A taken expert's entry becomes 0,
// below every live entry.
__global__ void __launch_bounds__(256) moe_topk_kernel(const float* __restrict__ logits, int64_t T, int E, int k,
                                                       int32_t* __restrict__ topk_ids, uint32_t* __restrict__ counts) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* l = logits + t * E;
  uint64_t v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    v[j] = e < E ? ((uint64_t)sort_key(l[e]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e) : 0ull;
  }
  for (int s = 0; s < k; ++s) {
    uint64_t m = v[0];
#pragma unroll
    for (int j = 1; j < 4; ++j) m = v[j] > m ? v[j] : m;
    m = wave_max_u64(m);
    const int e = (int)(0xFFFFFFFFu - (uint32_t)m);
    if ((e & 63) == lane) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j == (e >> 6)) v[j] = 0ull;
    }
    if (lane == 0) {
      topk_ids[t * k + s] = e;
      atomicAdd(counts + e, 1u);
    }
  }
}

// Exclusive prefix sum over one value per thread of a 256-thread workgroup.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t x, uint32_t* sh /* 256 */, uint32_t* total) {
  const int t = threadIdx.x;
  sh[t] = x;
  __syncthreads();
  for (int d = 1; d < 256; d <<= 1) {
    const uint32_t y = t >= d ? sh[t - d] : 0u;
    __syncthreads();
    sh[t] += y;
    __syncthreads();
  }
  const uint32_t incl = sh[t];
  *total = sh[255];
  __syncthreads();
  return incl - x;
}

// One workgroup (256 threads) per expert.
__global__ void __launch_bounds__(256) moe_place_kernel(const int32_t* __restrict__ topk_ids, int64_t T, int E, int k,
                                                        const uint32_t* __restrict__ rank_of_flag, int32_t flag_rows,
                                                        MoeTables tb, int32_t* __restrict__ expert_off,
                                                        int32_t* __restrict__ row_token) {
  __shared__ uint32_t sh[256];
  __shared__ uint32_t wave_cnt[4];
  __shared__ uint32_t keys[kMaxTilesPerExpert];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int e = blockIdx.x;

  // First row and first row tile of every expert: prefix sums of the counts.
  const uint32_t c = tid < E ? tb.counts[tid] : 0u;
  uint32_t rows_total, tiles_total;
  const uint32_t row0 = block_exclusive_scan(c, sh, &rows_total);
  const uint32_t tiles = (c + kRouteRows - 1) / kRouteRows;
  const uint32_t tile0 = block_exclusive_scan(tiles, sh, &tiles_total);
  __shared__ uint32_t my_row0, my_tile0, my_count;
  if (tid == e) {
    my_row0 = row0;
    my_tile0 = tile0;
    my_count = c;
  }
  if (e == 0) {
    if (tid < E) expert_off[tid] = (int32_t)row0;
    if (tid == 0) {
      expert_off[E] = (int32_t)rows_total;
      *tb.n_tiles = tiles_total;
      *tb.claim = 0u;
    }
  }
  __syncthreads();
  const uint32_t n_e = my_count, base_row = my_row0, base_tile = my_tile0;
  const uint32_t nt_e = (n_e + kRouteRows - 1) / kRouteRows;
  for (uint32_t j = tid; j < nt_e; j += 256) keys[j] = 0u;
  __syncthreads();

  // Place the tokens that chose e, in ascending token order.
  uint32_t placed = 0;
  for (int64_t r = 0; r < T; r += 256) {
    const int64_t t = r + tid;
    bool match = false;
    if (t < T) {
      const int32_t* ids = topk_ids + t * k;
      for (int s = 0; s < k; ++s) match |= ids[s] == e;
    }
    const uint64_t ballot = __ballot(match);
    const uint32_t below = (uint32_t)__popcll(ballot & ((1ull << lane) - 1ull));
    if (lane == 0) wave_cnt[wv] = (uint32_t)__popcll(ballot);
    __syncthreads();
    uint32_t wbase = placed;
    for (int w = 0; w < wv; ++w) wbase += wave_cnt[w];
    if (match) {
      const uint32_t pos = wbase + below;
      row_token[base_row + pos] = (int32_t)t;
      const uint32_t key = rank_of_flag ? rank_of_flag[t / flag_rows] : 0u;
      atomicMax(&keys[pos / kRouteRows], key);
    }
    placed += wave_cnt[0] + wave_cnt[1] + wave_cnt[2] + wave_cnt[3];
    __syncthreads();
  }
  for (uint32_t j = tid; j < nt_e; j += 256) {
    tb.tiles[base_tile + j] = MoeTile{e, (int32_t)(base_row + j * kRouteRows)};
    tb.keys[base_tile + j] = keys[j];
  }
}

// One workgroup of 1024 threads: stable counting sort of the row tiles by
// readiness key (keys < n_keys, folded into kSortBuckets buckets).
__global__ void __launch_bounds__(1024) moe_sort_kernel(MoeTables tb, uint32_t n_keys) {
  __shared__ uint32_t base[kSortBuckets];
  __shared__ uint32_t chunk_b[1024];
  const int tid = threadIdx.x;
  const uint32_t n = *tb.n_tiles;
  auto bucket = [&](uint32_t key) -> uint32_t {
    if (n_keys <= kSortBuckets) return key < n_keys ? key : n_keys - 1;
    const uint64_t b = (uint64_t)key * kSortBuckets / n_keys;
    return b < kSortBuckets ? (uint32_t)b : kSortBuckets - 1;
  };
  base[tid] = 0u;
  __syncthreads();
  for (uint32_t i = tid; i < n; i += 1024) atomicAdd(&base[bucket(tb.keys[i])], 1u);
  __syncthreads();
  // exclusive scan of the 1024 bucket counts (Hillis-Steele in place)
  const uint32_t own = base[tid];
  for (int d = 1; d < 1024; d <<= 1) {
    const uint32_t y = tid >= d ? base[tid - d] : 0u;
    __syncthreads();
    base[tid] += y;
    __syncthreads();
  }
  base[tid] -= own;
  __syncthreads();
  // Stable placement, 1024 entries at a time: an entry's rank inside its bucket
  // is the number of earlier entries of the chunk with the same bucket.
  for (uint32_t c0 = 0; c0 < n; c0 += 1024) {
    const uint32_t i = c0 + tid;
    const uint32_t b = i < n ? bucket(tb.keys[i]) : 0xFFFFFFFFu;
    chunk_b[tid] = b;
    __syncthreads();
    if (i < n) {
      uint32_t rank = 0;
      for (int j = 0; j < tid; ++j) rank += chunk_b[j] == b;
      tb.order[base[b] + rank] = tb.tiles[i];
    }
    __syncthreads();
    if (i < n) atomicAdd(&base[b], 1u);
    __syncthreads();
  }
}

}  // namespace

int moe_route_rows() { return kRouteRows; }
int moe_max_tiles_per_expert() { return kMaxTilesPerExpert; }

hipError_t launch_moe_route(const float* logits, int64_t T, int E, int k, const uint32_t* rank_of_flag,
                            int32_t flag_rows, uint32_t n_flags, const MoeTables& tb, int32_t* expert_off,
                            int32_t* row_token, int32_t* topk_ids, hipStream_t stream) {
  hipLaunchKernelGGL(moe_topk_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, stream, logits, T, E, k, topk_ids,
                     tb.counts);
  hipLaunchKernelGGL(moe_place_kernel, dim3((unsigned)E), dim3(256), 0, stream, topk_ids, T, E, k, rank_of_flag,
                     flag_rows, tb, expert_off, row_token);
  hipLaunchKernelGGL(moe_sort_kernel, dim3(1), dim3(1024), 0, stream, tb, n_flags);
  return hipGetLastError();
}

}  // namespace sgt
