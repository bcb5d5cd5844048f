// MoE routing on the GPU: top-k experts per token, rows grouped by expert, and
// the grouped consumer's work list (paper summary, "Experiments": MoE routing
// operations among the communication-bound kernels; DITRON article,
// "three-level tiling": the device-level tiles of an MoE layer take their
// sizes from how many tokens each expert receives, known only at run time).
//
// Two launches:
//  1. moe_topk_kernel  -- one wave per token, one lane per expert (up to four
//     experts a lane): k rounds of a wave-wide argmax (largest logit first,
//     equal logits: lower expert id).  Each token's picks also go to a bitmask
//     (one bit per expert), and each workgroup adds how many of its tokens
//     chose each expert to the call's counts.
//  2. moe_place_kernel -- one workgroup per expert: prefix sums of the counts
//     over experts give its first row (expert_off) and first row tile; one
//     pass over the tokens' mask words in ascending token order (a prefix sum
//     over threads) places each token that chose the expert at the next row of
//     its group.  Each group is cut into row tiles of the consumer's tile
//     height, and the workgroup writes its expert's tiles into the work list
//     in expert-major order, dealt out to per-XCD lists in chunks of a few
//     consecutive tiles (xcd_list_pos): the tiles of one expert that an XCD
//     runs side by side read the same weight columns through its L2.
// No table depends on the order of concurrent updates: counts are integer
// sums, positions are prefix sums over tokens.  The counts are double-buffered
// by call parity: each call's top-k kernel clears the next call's buffer.
#include <hip/hip_runtime.h>

#include "common.hpp"

namespace sgt {

namespace {

// Order-preserving map of an fp32 value to uint32 (total order; -0 and +0
// compare equal, as floating-point comparison has them).
__device__ __forceinline__ uint32_t sort_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Branch-free 32-bit loads: a buffer resource over [base, base + bytes) reads
// 0 for any offset past the end, so guarded loads need no branch (a branch per
// load would make each one wait for the previous).
constexpr uint32_t kNoLoad = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t words_rsrc(const void* base, uint64_t bytes) {
  const uint32_t n = bytes >= 0x80000000ull ? 0x7FFFFFFFu : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}

__device__ __forceinline__ uint32_t load_word(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0);
}

// Maximum over the 64 lanes of a wave, returned to every lane: DPP exchanges
// inside each row of 16 lanes (quad swaps, then half-row and row mirrors),
// then the four row results read out of lanes 15, 31, 47 and 63.
__device__ __forceinline__ uint32_t dpp_max(uint32_t v, uint32_t ctrl_result) { return v > ctrl_result ? v : ctrl_result; }

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = dpp_max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, true));   // quad_perm 1,0,3,2
  v = dpp_max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, true));   // quad_perm 2,3,0,1
  v = dpp_max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, true));  // row_half_mirror
  v = dpp_max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, true));  // row_mirror
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 15), r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 31);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 47), r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
  const uint32_t a = r0 > r1 ? r0 : r1, b = r2 > r3 ? r2 : r3;
  return a > b ? a : b;
}

// Workgroup g (8 waves) takes tokens [g * tpg, (g + 1) * tpg); a wave takes
// every 8th of them, their logits loaded up front.  Lane l holds the keys of
// experts l, l + 64, ... (kSlots = ceil(E / 64) of them).  Each of the k rounds
// takes the wave maximum of the live keys and then, with one ballot per slot,
// the lowest expert id holding it: the largest logit first and, among equal
// logits, the lowest id.  Round s's pick is kept by lane s % 64 (slot s / 64);
// the picks are written, counted and turned into mask words once per token.
// The workgroup's picks per expert are summed in LDS and added to the call's
// counts (integer sums: the order of the atomic updates does not matter).
constexpr int kTopkWaves = 8;
constexpr int kTopkPerWave = 4;

template <int kSlots>
__global__ void __launch_bounds__(64 * kTopkWaves) moe_topk_kernel(const float* __restrict__ logits, int64_t T, int E,
                                                                  int k, int tpg, int32_t* __restrict__ topk_ids,
                                                                  uint32_t* __restrict__ masks, uint32_t* counts,
                                                                  uint32_t* counts_next) {
  __shared__ uint32_t cnt[256];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  // all 256 entries: the next call may have more experts
  if (blockIdx.x == 0 && tid < 256) counts_next[tid] = 0u;
  const int nw = (E + 31) >> 5;
  if (tid < 256) cnt[tid] = 0u;
  __syncthreads();
  // this workgroup's logits (T * E * 4 < 2^31 bytes, checked by the host)
  const int64_t g0 = (int64_t)blockIdx.x * tpg;
  const int64_t g1 = g0 + tpg < T ? g0 + tpg : T;
  const __amdgpu_buffer_rsrc_t lr = words_rsrc(logits + g0 * E, (uint64_t)(g1 > g0 ? g1 - g0 : 0) * E * 4);
  for (int j0 = wv; j0 < tpg; j0 += kTopkWaves * kTopkPerWave) {
    // this wave's tokens of the pass, all their logits in flight at once
    uint32_t raw[kTopkPerWave][kSlots];
#pragma unroll
    for (int u = 0; u < kTopkPerWave; ++u) {
      const int j = j0 + u * kTopkWaves;
#pragma unroll
      for (int q = 0; q < kSlots; ++q) {
        const int e = lane + 64 * q;
        raw[u][q] = load_word(lr, (j < tpg && e < E) ? (uint32_t)(j * E + e) * 4u : kNoLoad);
      }
    }
#pragma unroll
    for (int u = 0; u < kTopkPerWave; ++u) {
      const int64_t t = g0 + j0 + u * kTopkWaves;
      if (!(j0 + u * kTopkWaves < tpg && t < T)) break;
      uint32_t v[kSlots];   // live keys; a taken or absent expert holds 0 and is not live
      bool live[kSlots];
#pragma unroll
      for (int q = 0; q < kSlots; ++q) {
        live[q] = lane + 64 * q < E;
        v[q] = live[q] ? sort_key(__uint_as_float(raw[u][q])) : 0u;
      }
      int pick[kSlots];
#pragma unroll
      for (int q = 0; q < kSlots; ++q) pick[q] = -1;
      uint32_t word = 0u;  // lane l < nw builds mask word l of this token
      for (int s = 0; s < k; ++s) {
        uint32_t lm = 0u;
#pragma unroll
        for (int q = 0; q < kSlots; ++q) lm = (live[q] && v[q] > lm) ? v[q] : lm;
        const uint32_t m = wave_max_u32(lm);
        int e = -1;
#pragma unroll
        for (int q = 0; q < kSlots; ++q) {
          const uint64_t b = __ballot(live[q] && v[q] == m);
          if (e < 0 && b) e = 64 * q + __ffsll((unsigned long long)b) - 1;
        }
        // k <= E keeps a live entry, so e >= 0 (all lanes agree on it)
#pragma unroll
        for (int q = 0; q < kSlots; ++q) {
          if (lane + 64 * q == e) live[q] = false;
          if (s == lane + 64 * q) pick[q] = e;
        }
        if (lane == (e >> 5)) word |= 1u << (e & 31);
      }
#pragma unroll
      for (int q = 0; q < kSlots; ++q) {
        if (pick[q] >= 0) {
          topk_ids[t * k + lane + 64 * q] = pick[q];
          atomicAdd(&cnt[pick[q]], 1u);
        }
      }
      if (lane < nw) masks[(int64_t)lane * T + t] = word;
    }
  }
  __syncthreads();
  if (tid < E && cnt[tid]) atomicAdd(counts + tid, cnt[tid]);
}

// Exclusive prefix sum over one value per thread of a 256-thread workgroup:
// an inclusive scan inside each wave with cross-lane shifts, then each wave
// adds the totals of the waves before it.  `sh` holds 4 words.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t x, uint32_t* sh, uint32_t* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  uint32_t incl = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = (uint32_t)__shfl_up((int)incl, d, 64);
    if (lane >= d) incl += y;
  }
  if (lane == 63) sh[wv] = incl;
  __syncthreads();
  uint32_t before = 0u;
  for (int w = 0; w < wv; ++w) before += sh[w];
  *total = sh[0] + sh[1] + sh[2] + sh[3];
  __syncthreads();
  return before + incl - x;
}

// One workgroup (256 threads) per expert.
__global__ void __launch_bounds__(256) moe_place_kernel(const uint32_t* __restrict__ masks, int64_t T, int E,
                                                        int tile_rows, int64_t rows_cap, MoeTables tb,
                                                        int32_t* __restrict__ expert_off,
                                                        int32_t* __restrict__ row_token) {
  __shared__ uint32_t sh[256];
  __shared__ uint32_t my_row0, my_tile0, my_count, n_tiles;
  const int tid = threadIdx.x;
  const int e = blockIdx.x;

  // First row and first row tile of every expert: prefix sums over experts.
  const uint32_t c = tid < E ? tb.counts[tid] : 0u;
  uint32_t rows_total, tiles_total;
  const uint32_t row0 = block_exclusive_scan(c, sh, &rows_total);
  const uint32_t tiles = (c + tile_rows - 1) / tile_rows;
  const uint32_t tile0 = block_exclusive_scan(tiles, sh, &tiles_total);
  if (tid == e) {
    my_row0 = row0;
    my_tile0 = tile0;
    my_count = c;
  }
  if (tid == 0) n_tiles = tiles_total;
  if (e == 0) {
    if (tid < E) expert_off[tid] = (int32_t)row0;
    if (tid == 0) {
      expert_off[E] = (int32_t)rows_total;
      *tb.n_tiles = tiles_total;
    }
    if (tid < kXcds) tb.xcd_claim[tid * kXcdClaimStride] = 0u;
  }
  __syncthreads();
  const uint32_t n_e = my_count, base_row = my_row0, base_tile = my_tile0, nt = n_tiles;

  // This expert's row tiles, in row order, at their places in the XCD lists.
  const uint32_t nt_e = (n_e + tile_rows - 1) / tile_rows;
  for (uint32_t j = tid; j < nt_e; j += 256) {
    const uint32_t q = xcd_list_pos(base_tile + j, nt);  // < nt (base_tile + j < nt)
    const uint32_t r = j * tile_rows, rows = n_e - r < (uint32_t)tile_rows ? n_e - r : (uint32_t)tile_rows;
    if (q < tb.tiles_cap) tb.order[q] = MoeTile{e, (int32_t)(base_row + r), (int32_t)rows};
  }

  // Place the tokens that chose e, in ascending token order: thread i takes
  // 16 consecutive tokens of each 4096-token round.
  const __amdgpu_buffer_rsrc_t mr = words_rsrc(masks + (int64_t)(e >> 5) * T, (uint64_t)T * 4);
  const int bit = e & 31;
  uint32_t placed = 0;
  for (int64_t rb = 0; rb < T; rb += 4096) {
    const int64_t t0 = rb + 16 * tid;
    uint32_t m[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) m[u] = load_word(mr, t0 + u < T ? (uint32_t)(t0 + u) * 4u : kNoLoad);
    uint32_t sel = 0u;
#pragma unroll
    for (int u = 0; u < 16; ++u) sel |= ((m[u] >> bit) & 1u) << u;
    uint32_t total;
    uint32_t pos = placed + block_exclusive_scan((uint32_t)__popc(sel), sh, &total);
    // (counts are exact by construction; the bound only keeps every store
    // inside row_token whatever the tables hold)
    while (sel) {
      const int u = __ffs(sel) - 1;
      sel &= sel - 1u;
      if ((int64_t)base_row + pos < rows_cap) row_token[base_row + pos] = (int32_t)(t0 + u);  // T <= 2^20
      ++pos;
    }
    placed += total;
  }
}

}  // namespace

// Tokens per top-k workgroup: 64 (four per wave), or more when that would
// make over 4096 groups.
int moe_tokens_per_group(int64_t T, int k) {
  (void)k;
  int64_t tpg = kTopkWaves * kTopkPerWave;
  if ((T + tpg - 1) / tpg > 4096) tpg = ((T + 4095) / 4096 + tpg - 1) / tpg * tpg;
  return (int)tpg;
}

hipError_t launch_moe_route(const float* logits, int64_t T, int E, int k, int tile_rows, const MoeTables& tb,
                            int32_t* expert_off, int32_t* row_token, int32_t* topk_ids, hipStream_t stream) {
  const dim3 g((unsigned)tb.n_groups), b(64 * kTopkWaves);
  const int slots = (E + 63) / 64;
  if (slots == 1)
    hipLaunchKernelGGL(moe_topk_kernel<1>, g, b, 0, stream, logits, T, E, k, tb.tokens_per_group, topk_ids, tb.masks,
                       tb.counts, tb.counts_next);
  else if (slots == 2)
    hipLaunchKernelGGL(moe_topk_kernel<2>, g, b, 0, stream, logits, T, E, k, tb.tokens_per_group, topk_ids, tb.masks,
                       tb.counts, tb.counts_next);
  else
    hipLaunchKernelGGL(moe_topk_kernel<4>, g, b, 0, stream, logits, T, E, k, tb.tokens_per_group, topk_ids, tb.masks,
                       tb.counts, tb.counts_next);
  hipLaunchKernelGGL(moe_place_kernel, dim3((unsigned)E), dim3(256), 0, stream, tb.masks, T, E, tile_rows, T * k, tb,
                     expert_off, row_token);
  return hipGetLastError();
}

}  // namespace sgt
