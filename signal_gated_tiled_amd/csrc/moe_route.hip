// MoE routing on the GPU: top-k experts per token, rows grouped by expert, and
// the grouped consumer's work list ordered by when its rows can arrive
// (paper summary, "Experiments": MoE routing operations among the
// communication-bound kernels; DITRON article, "three-level tiling": the
// device-level tiles of an MoE layer take their sizes from how many tokens each
// expert receives, known only at run time).
//
// Three launches:
//  1. top-k (largest logit first, equal logits: lower expert id).  For
//     k <= 8, one thread per token keeps its 8 best (logit, id) pairs sorted
//     in registers while it scans the logits in expert order; otherwise one
//     wave per token runs k rounds of a wave-wide argmax.  Each token's picks
//     also go to a bitmask (one bit per expert), and each workgroup writes how
//     many of its tokens chose each expert.
//  2. moe_place_kernel -- one workgroup per expert: the per-group counts give
//     every expert's size, and prefix sums over experts its first row
//     (expert_off) and first row tile; one pass over the tokens' mask words in
//     ascending token order (a prefix sum over threads) places each token that
//     chose the expert at the next row of its group.  Each group is cut into
//     row tiles of the consumer's tile height; the readiness key of a row tile
//     is the latest arrival rank among the signal tiles its rows come from.
//  3. moe_sort_kernel  -- one workgroup: a stable counting sort of the row tiles
//     by readiness key, so the consumer claims first the tiles whose rows land
//     first.
// No table depends on the order of concurrent updates (no global atomics):
// counts are per-workgroup sums, positions are prefix sums over tokens.
#include <hip/hip_runtime.h>

#include "common.hpp"

namespace sgt {

namespace {

constexpr int kMaxTilesPerExpert = 4096;
constexpr int kSortBuckets = 256;
constexpr int kRankCache = 4096;       // arrival ranks staged in LDS (signal tiles per call)

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

__device__ __forceinline__ uint64_t pack_choice(float logit, int e) {
  return ((uint64_t)sort_key(logit) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}

// One thread per token, k <= 8.  best[0..7] stays sorted in decreasing packed
// order: each new (logit, id) is bubbled in with max / min exchanges, so among
// equal logits the earlier (lower) id stays ahead, as k rounds of argmax with
// ties to the lower id would pick.  Workgroup g takes tokens [256 g, 256 g + 256).
__global__ void __launch_bounds__(256) moe_topk8_kernel(const float* __restrict__ logits, int64_t T, int E, int k,
                                                        int32_t* __restrict__ topk_ids, uint32_t* __restrict__ masks,
                                                        uint32_t* __restrict__ partials) {
  __shared__ uint32_t cnt[256];
  const int tid = threadIdx.x;
  cnt[tid] = 0u;
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * 256 + tid;
  if (t < T) {
    const float* l = logits + t * E;
    uint64_t best[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) best[j] = 0ull;
#pragma unroll 4
    for (int e = 0; e < E; ++e) {
      uint64_t x = pack_choice(l[e], e);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint64_t hi = best[j] > x ? best[j] : x;
        x = best[j] > x ? x : best[j];
        best[j] = hi;
      }
    }
    uint32_t words[8];
#pragma unroll
    for (int w = 0; w < 8; ++w) words[w] = 0u;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (s < k) {
        const int e = (int)(0xFFFFFFFFu - (uint32_t)best[s]);
        topk_ids[t * k + s] = e;
        atomicAdd(&cnt[e], 1u);
#pragma unroll
        for (int w = 0; w < 8; ++w)
          if (w == (e >> 5)) words[w] |= 1u << (e & 31);
      }
    }
    const int nw = (E + 31) >> 5;
#pragma unroll
    for (int w = 0; w < 8; ++w)
      if (w < nw) masks[(int64_t)w * T + t] = words[w];
  }
  __syncthreads();
  if (tid < E) partials[(int64_t)blockIdx.x * E + tid] = cnt[tid];
}

// Workgroup g (4 waves) takes tokens [g * tpg, (g + 1) * tpg); a wave takes
// every 4th of them.  Lane l holds experts l, l + 64, l + 128, l + 192 as
// (key << 32) | (0xFFFFFFFF - e): the wave maximum is the largest logit and,
// among equal logits, the lowest expert id.  A taken expert's entry becomes 0,
// below every live entry.
__global__ void __launch_bounds__(256) moe_topk_kernel(const float* __restrict__ logits, int64_t T, int E, int k,
                                                       int tpg, int32_t* __restrict__ topk_ids,
                                                       uint32_t* __restrict__ masks, uint32_t* __restrict__ partials) {
  __shared__ uint32_t cnt[256];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nw = (E + 31) >> 5;
  cnt[tid] = 0u;
  __syncthreads();
  for (int j = wv; j < tpg; j += 4) {
    const int64_t t = (int64_t)blockIdx.x * tpg + j;
    if (t >= T) break;
    const float* l = logits + t * E;
    uint64_t v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane + 64 * q;
      v[q] = e < E ? pack_choice(l[e], e) : 0ull;
    }
    uint32_t word = 0u;  // lane l < nw builds mask word l of this token
    for (int s = 0; s < k; ++s) {
      uint64_t m = v[0];
#pragma unroll
      for (int q = 1; q < 4; ++q) m = v[q] > m ? v[q] : m;
      m = wave_max_u64(m);
      const int e = (int)(0xFFFFFFFFu - (uint32_t)m);
      if ((e & 63) == lane) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (q == (e >> 6)) v[q] = 0ull;
      }
      if (lane == (e >> 5)) word |= 1u << (e & 31);
      if (lane == 0) {
        topk_ids[t * k + s] = e;
        atomicAdd(&cnt[e], 1u);
      }
    }
    if (lane < nw) masks[(int64_t)lane * T + t] = word;
  }
  __syncthreads();
  if (tid < E) partials[(int64_t)blockIdx.x * E + tid] = cnt[tid];
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
__global__ void __launch_bounds__(256) moe_place_kernel(const uint32_t* __restrict__ masks,
                                                        const uint32_t* __restrict__ partials, int n_groups,
                                                        int64_t T, int E, const uint32_t* __restrict__ rank_of_flag,
                                                        int32_t flag_rows, int tile_rows, MoeTables tb,
                                                        int32_t* __restrict__ expert_off,
                                                        int32_t* __restrict__ row_token) {
  __shared__ uint32_t sh[256];
  __shared__ uint32_t cnt[256];
  __shared__ uint32_t keys[kMaxTilesPerExpert];
  __shared__ uint32_t ranks[kRankCache];
  __shared__ uint32_t my_row0, my_tile0, my_count;
  const int tid = threadIdx.x;
  const int e = blockIdx.x;
  // The arrival ranks may live in host memory: read each once into LDS.
  const int64_t n_flags = (T + flag_rows - 1) / flag_rows;
  const bool cached = rank_of_flag && n_flags <= kRankCache;
  if (cached)
    for (int64_t f = tid; f < n_flags; f += 256) ranks[f] = rank_of_flag[f];

  // Every expert's token count: the top-k groups' counts summed, 256 / E
  // threads per expert each taking every (256 / E)-th group.
  cnt[tid] = 0u;
  __syncthreads();
  {
    const int q = 256 / E;
    if (tid < q * E) {
      const int x = tid % E, part = tid / E;
      uint32_t sum = 0u;
#pragma unroll 8
      for (int g = part; g < n_groups; g += q) sum += partials[(int64_t)g * E + x];
      atomicAdd(&cnt[x], sum);
    }
  }
  __syncthreads();

  // First row and first row tile of every expert: prefix sums over experts.
  const uint32_t c = tid < E ? cnt[tid] : 0u;
  uint32_t rows_total, tiles_total;
  const uint32_t row0 = block_exclusive_scan(c, sh, &rows_total);
  const uint32_t tiles = (c + tile_rows - 1) / tile_rows;
  const uint32_t tile0 = block_exclusive_scan(tiles, sh, &tiles_total);
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
  const uint32_t nt_e = (n_e + tile_rows - 1) / tile_rows;
  for (uint32_t j = tid; j < nt_e; j += 256) keys[j] = 0u;
  __syncthreads();

  // Place the tokens that chose e, in ascending token order: thread i takes
  // 16 consecutive tokens of each 4096-token round.
  const uint32_t* mw = masks + (int64_t)(e >> 5) * T;
  const int bit = e & 31;
  uint32_t placed = 0;
  for (int64_t rb = 0; rb < T; rb += 4096) {
    const int64_t t0 = rb + 16 * tid;
    uint32_t sel = 0u;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int64_t t = t0 + u;
      const uint32_t m = t < T ? mw[t] : 0u;
      sel |= ((m >> bit) & 1u) << u;
    }
    uint32_t total;
    uint32_t pos = placed + block_exclusive_scan((uint32_t)__popc(sel), sh, &total);
    while (sel) {
      const int u = __ffs(sel) - 1;
      sel &= sel - 1u;
      const int64_t t = t0 + u;
      row_token[base_row + pos] = (int32_t)t;
      const int64_t f = t / flag_rows;
      const uint32_t key = cached ? ranks[f] : (rank_of_flag ? rank_of_flag[f] : 0u);
      atomicMax(&keys[pos / tile_rows], key);
      ++pos;
    }
    placed += total;
  }
  __syncthreads();
  for (uint32_t j = tid; j < nt_e; j += 256) {
    tb.tiles[base_tile + j] = MoeTile{e, (int32_t)(base_row + j * tile_rows)};
    tb.keys[base_tile + j] = keys[j];
  }
}

// One workgroup of 256 threads: stable counting sort of the row tiles by
// readiness key (keys < n_keys, folded into 256 buckets).
__global__ void __launch_bounds__(256) moe_sort_kernel(MoeTables tb, uint32_t n_keys) {
  __shared__ uint32_t base[kSortBuckets];
  __shared__ uint32_t chunk_b[kSortBuckets];
  __shared__ uint32_t sh[256];
  const int tid = threadIdx.x;
  const uint32_t n = *tb.n_tiles;
  auto bucket = [&](uint32_t key) -> uint32_t {
    if (n_keys <= kSortBuckets) return key < n_keys ? key : n_keys - 1;
    const uint64_t b = (uint64_t)key * kSortBuckets / n_keys;
    return b < kSortBuckets ? (uint32_t)b : kSortBuckets - 1;
  };
  base[tid] = 0u;
  __syncthreads();
  for (uint32_t i = tid; i < n; i += 256) atomicAdd(&base[bucket(tb.keys[i])], 1u);
  __syncthreads();
  uint32_t total;
  const uint32_t first = block_exclusive_scan(base[tid], sh, &total);
  base[tid] = first;
  __syncthreads();
  // Stable placement, 256 entries at a time: an entry's rank inside its bucket
  // is the number of earlier entries of the chunk with the same bucket.
  for (uint32_t c0 = 0; c0 < n; c0 += 256) {
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

int moe_max_tiles_per_expert() { return kMaxTilesPerExpert; }

// Tokens per top-k workgroup: 256 (one per thread) when k <= 8; else 16 (four
// per wave), or more when that would make over 4096 groups.
int moe_tokens_per_group(int64_t T, int k) {
  if (k <= 8) return 256;
  int64_t tpg = 16;
  if ((T + tpg - 1) / tpg > 4096) tpg = ((T + 4095) / 4096 + 3) / 4 * 4;
  return (int)tpg;
}

hipError_t launch_moe_route(const float* logits, int64_t T, int E, int k, const uint32_t* rank_of_flag,
                            int32_t flag_rows, uint32_t n_flags, int tile_rows, const MoeTables& tb,
                            int32_t* expert_off, int32_t* row_token, int32_t* topk_ids, hipStream_t stream) {
  if (k <= 8)
    hipLaunchKernelGGL(moe_topk8_kernel, dim3((unsigned)tb.n_groups), dim3(256), 0, stream, logits, T, E, k, topk_ids,
                       tb.masks, tb.partials);
  else
    hipLaunchKernelGGL(moe_topk_kernel, dim3((unsigned)tb.n_groups), dim3(256), 0, stream, logits, T, E, k,
                       tb.tokens_per_group, topk_ids, tb.masks, tb.partials);
  hipLaunchKernelGGL(moe_place_kernel, dim3((unsigned)E), dim3(256), 0, stream, tb.masks, tb.partials, tb.n_groups,
                     T, E, rank_of_flag, flag_rows, tile_rows, tb, expert_off, row_token);
  hipLaunchKernelGGL(moe_sort_kernel, dim3(1), dim3(256), 0, stream, tb, n_flags);
  return hipGetLastError();
}

}  // namespace sgt
