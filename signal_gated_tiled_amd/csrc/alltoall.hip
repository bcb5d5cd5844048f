// Expert-parallel AllToAll, one rank's share (paper summary, "Experiments":
// the AllToAll dispatch and combine of expert parallelism, measured against
// DeepEP; complete guide, §4.2: low-latency AllToAll for expert parallelism;
// semantics page, "Producer-consumer model" and "Signal-based
// synchronization" for the per-chunk flags).
//
// Experts are split over the W ranks in contiguous blocks of E_l = E / W.
// Dispatch: every rank p sends each of its tokens to the owner of every expert
// the token picked.  Rank r receives, for its local expert l and source p,
// the rows of p's tokens that picked expert r * E_l + l, in ascending token
// order, into fixed slots (T_r rows per (l, p) block, so no count exchange has
// to precede the data), with the count in a packet {epoch, count} and one
// flag per chunk of rows.  Combine: each expert's owner sends its outputs for
// this rank's tokens back in the same slot order; this rank's token t then
// sums gate[t, j] * (the row of its j-th pick) over its picks, each pick
// waiting only on the flag of the chunk that holds its row.
//
// On one GPU the other ranks are simulated: the senders of the blocks this
// rank receives (dispatch), or that come back to it (combine), run here as
// sender workgroups, one per (block, chunk), each publishing its chunk's flag
// no earlier than its link (one per peer, all concurrent, the local one
// unthrottled) would have delivered it.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "alltoall.hpp"
#include "common.hpp"
#include "signal.hpp"

namespace sgt {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kA2aThreads = 256;
constexpr int kA2aUnroll = 8;    // 16-byte loads in flight per thread in the copy
constexpr int kRecvUnits = 2;    // 16-byte units (8 bf16) per lane per pass of the combine
constexpr int kRecvPicks = 8;    // picks whose rows are loaded together
constexpr uint32_t kOob = 0x80000000u;  // past every buffer range (ranges are below 2^31 bytes)

__device__ inline __amdgpu_buffer_rsrc_t a2a_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Four expert ids at byte offset `off` of a routing table; an offset past the
// table (a token past T_r, or the second half of a row of four ids) gives -1s,
// which select no expert.  A value select, not a select of addresses: no
// stack copy of the -1s.
__device__ __forceinline__ int4 ids4(__amdgpu_buffer_rsrc_t rt, uint32_t off) {
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  const u4 w = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(rt, off, 0, 0));
  const bool in = off != kOob;
  return make_int4(in ? (int)w.x : -1, in ? (int)w.y : -1, in ? (int)w.z : -1, in ? (int)w.w : -1);
}

// Scan of one block's routing table (grid: one workgroup per block b).
// Finds, in ascending order, the tokens of the table that picked the block's
// expert: dispatch writes them to recv_token (the block's list) and the
// count packet; combine writes each such pick's position to slot_of (and
// workgroup 0 marks picks of ids outside [0, E) with -1).  Both write the
// block's count to the context's count table.
//
// A pass covers kScanSub x 256 tokens: every thread loads the ids of its
// kScanSub tokens first (16-byte loads when k is 4 or 8), so a pass costs
// one memory round trip; the positions then come from one ballot per
// sub-pass and one barrier for all of them.
constexpr int kScanSub = 4;

__device__ __forceinline__ void scan_mark(const A2aArgs& a, int b, int e, bool combine, int64_t t, int j, int v,
                                          int pos) {
  if (!combine) return;
  if (v == e) a.lists[t * a.k + j] = pos;
  else if (b == 0 && (v < 0 || v >= a.E)) a.lists[t * a.k + j] = -1;
}

__global__ void __launch_bounds__(kA2aThreads) a2a_scan_kernel(A2aArgs a) {
  __shared__ int wsum[kScanSub][kA2aThreads / 64];
  const int b = blockIdx.x;
  const bool combine = a.mode == 1;
  const int e = combine ? b : a.rank * a.E_l + b / a.W;
  const int32_t* tab = static_cast<const int32_t*>(combine ? a.table.p[0] : a.table.p[b % a.W]);
  const int k = a.k;
  const bool vec = (k == 4 || k == 8) && ((reinterpret_cast<uintptr_t>(tab) & 15u) == 0);
  const __amdgpu_buffer_rsrc_t rt = a2a_rsrc(tab, (uint32_t)(a.T_r * k * 4));
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int running = 0;
  for (int64_t t0 = 0; t0 < a.T_r; t0 += kA2aThreads * kScanSub) {
    bool hit[kScanSub];
    int4 v[kScanSub][2];
    if (vec) {
      // all loads of the pass in flight before any use
#pragma unroll
      for (int i = 0; i < kScanSub; ++i) {
        const int64_t t = t0 + i * kA2aThreads + threadIdx.x;
        v[i][0] = ids4(rt, t < a.T_r ? (uint32_t)(t * k * 4) : kOob);
        v[i][1] = ids4(rt, t < a.T_r && k == 8 ? (uint32_t)(t * k * 4 + 16) : kOob);
      }
#pragma unroll
      for (int i = 0; i < kScanSub; ++i) {
        hit[i] = false;
#pragma unroll
        for (int q = 0; q < 2; ++q)
          hit[i] |= (v[i][q].x == e) | (v[i][q].y == e) | (v[i][q].z == e) | (v[i][q].w == e);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kScanSub; ++i) {
        const int64_t t = t0 + i * kA2aThreads + threadIdx.x;
        hit[i] = false;
        if (t < a.T_r)
          for (int j = 0; j < k; ++j) hit[i] |= tab[t * k + j] == e;
      }
    }
    int pre[kScanSub];
#pragma unroll
    for (int i = 0; i < kScanSub; ++i) {
      const uint64_t bal = __ballot(hit[i]);
      pre[i] = __popcll(bal & ((1ull << lane) - 1ull));
      if (lane == 0) wsum[i][wave] = __popcll(bal);
    }
    __syncthreads();
    int base = running;
#pragma unroll
    for (int i = 0; i < kScanSub; ++i) {
      int off = base, tot = 0;
      for (int w = 0; w < kA2aThreads / 64; ++w) {
        if (w < wave) off += wsum[i][w];
        tot += wsum[i][w];
      }
      const int64_t t = t0 + i * kA2aThreads + threadIdx.x;
      const int pos = off + pre[i];
      if (hit[i] && !combine) a.lists[(int64_t)b * a.T_r + pos] = (int32_t)t;
      if (combine && t < a.T_r) {
        if (vec) {
          scan_mark(a, b, e, true, t, 0, v[i][0].x, pos);
          scan_mark(a, b, e, true, t, 1, v[i][0].y, pos);
          scan_mark(a, b, e, true, t, 2, v[i][0].z, pos);
          scan_mark(a, b, e, true, t, 3, v[i][0].w, pos);
          if (k == 8) {
            scan_mark(a, b, e, true, t, 4, v[i][1].x, pos);
            scan_mark(a, b, e, true, t, 5, v[i][1].y, pos);
            scan_mark(a, b, e, true, t, 6, v[i][1].z, pos);
            scan_mark(a, b, e, true, t, 7, v[i][1].w, pos);
          }
        } else {
          for (int j = 0; j < k; ++j) scan_mark(a, b, e, true, t, j, tab[t * k + j], pos);
        }
      }
      base += tot;
    }
    running = base;
    __syncthreads();  // wsum is rewritten by the next pass
  }
  if (threadIdx.x == 0) {
    a.counts[b] = running;
    if (!combine)
      __hip_atomic_store(a.count_sig + b, ((uint64_t)a.epoch << 32) | (uint32_t)running, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Sender workgroup: chunk c of block b.  Copies its rows (gathered by token
// for the dispatch, contiguous for the combine) into the block's slots with
// device-scope stores, waits until every wave's stores are acknowledged, and
// publishes the chunk's flag no earlier than the link's delivery time: the
// link carries its blocks in expert order, so the chunk lands once the rows
// of the link's earlier blocks and this block's rows through this chunk have
// crossed it.
__device__ __forceinline__ void a2a_send(const A2aArgs& a, int item) {
  __shared__ int32_t s_tok[kA2aMaxChunkRows];
  __shared__ uint64_t s_t0;
  __shared__ int s_rows, s_before;
  const int b = item / a.n_chunks, c = item % a.n_chunks;
  const bool combine = a.mode == 1;
  const int link = combine ? b / a.E_l : b % a.W;
  const int l = combine ? b % a.E_l : b / a.W;
  if (threadIdx.x == 0) {
    s_t0 = clock_ticks();
    const int count = a.counts[b];
    int before = 0;
    for (int m = 0; m < l; ++m) before += a.counts[combine ? link * a.E_l + m : m * a.W + link];
    const int rest = count - c * a.chunk_rows;
    s_rows = rest < a.chunk_rows ? rest : a.chunk_rows;
    s_before = before;
  }
  __syncthreads();
  const int rows = s_rows;
  if (rows <= 0) return;  // uniform: past the block's count, nothing is sent and no flag is published
  const int64_t r0 = (int64_t)c * a.chunk_rows;
  if (!combine)
    for (int i = threadIdx.x; i < rows; i += kA2aThreads) s_tok[i] = a.lists[(int64_t)b * a.T_r + r0 + i];
  const bool paced = a.ticks_per_row > 0.0 && link != a.rank;
  const uint64_t release = paced ? (uint64_t)((double)(s_before + r0 + rows) * a.ticks_per_row) : 0;
  if (threadIdx.x == 0 && paced) {
    // start about one copy time before the release (at the ~20 GB/s one
    // workgroup streams: 200 bytes per 10 ns tick); the wait is finite
    const uint64_t lead = (uint64_t)rows * (uint64_t)a.row_bytes / 200u + 100u;
    if (release > lead)
      while (clock_ticks() < s_t0 + release - lead) __builtin_amdgcn_s_sleep(4);
  }
  __syncthreads();

  const uint32_t block_bytes = (uint32_t)(a.T_r * a.row_bytes);
  const char* src = static_cast<const char*>(a.src.p[link]) + (combine ? (int64_t)l * a.T_r * a.row_bytes : 0);
  char* dst = a.dst + (int64_t)b * a.T_r * a.row_bytes;
  const __amdgpu_buffer_rsrc_t rs = a2a_rsrc(src, block_bytes), rd = a2a_rsrc(dst, block_bytes);
  const uint32_t upr = (uint32_t)(a.row_bytes >> 4);
  const uint32_t total = (uint32_t)rows * upr;
  for (uint32_t u0 = threadIdx.x; u0 < total; u0 += kA2aThreads * kA2aUnroll) {
    u32x4 v[kA2aUnroll];
    uint32_t dof[kA2aUnroll];
#pragma unroll
    for (int u = 0; u < kA2aUnroll; ++u) {
      const uint32_t unit = u0 + (uint32_t)u * kA2aThreads;
      const uint32_t row = unit / upr, col = unit - row * upr;
      const bool in = unit < total;
      const uint32_t srow = combine ? (uint32_t)r0 + row : (uint32_t)s_tok[in ? row : 0];
      const uint32_t sof = in ? srow * (uint32_t)a.row_bytes + col * 16u : kOob;
      dof[u] = in ? ((uint32_t)r0 + row) * (uint32_t)a.row_bytes + col * 16u : kOob;
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, sof, 0, kCpolNt);
    }
    // every load in flight before the first store
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kA2aUnroll; ++u) __builtin_amdgcn_raw_buffer_store_b128(v[u], rd, dof[u], 0, kCpolSc1);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    if (paced)
      while (clock_ticks() < s_t0 + release) __builtin_amdgcn_s_sleep(4);  // finite
    if (link != a.withhold) flag_publish_coherent(a.flags + item, a.epoch);
  }
}

// Dispatch sender with its own scan (the dispatch is one launch; up to 64
// local experts, else the scan kernel runs first and a2a_send sends): the
// workgroup of chunk c of block b = l * W + p reads source p's routing table
// once (kScanSub x 256 tokens per pass, the ids of a pass loaded before any
// is used) and derives, for p's tokens and this rank's local experts,
//   the block's count (tokens that picked expert l),
//   the rows link p carries before the block (tokens that picked each of the
//     local experts before l, a token counted once per expert),
//   the tokens at positions [c * chunk_rows, +chunk_rows) of the block's
//     ascending list, which it writes to recv_token and copies;
// chunk 0 also stores the block's count packet.  Then it sends like a2a_send.
__device__ __forceinline__ void a2a_dispatch_send(const A2aArgs& a, int item) {
  __shared__ int32_t s_tok[kA2aMaxChunkRows];
  __shared__ int wsum[kScanSub][kA2aThreads / 64];
  __shared__ int wbefore[kA2aThreads / 64];
  __shared__ uint64_t s_t0;
  const int b = item / a.n_chunks, c = item % a.n_chunks;
  const int link = b % a.W, l = b / a.W;
  const int ebase = a.rank * a.E_l;
  const int32_t* tab = static_cast<const int32_t*>(a.table.p[link]);
  const int k = a.k;
  const bool vec = (k == 4 || k == 8) && ((reinterpret_cast<uintptr_t>(tab) & 15u) == 0);
  const __amdgpu_buffer_rsrc_t rt = a2a_rsrc(tab, (uint32_t)(a.T_r * k * 4));
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t r0 = (int64_t)c * a.chunk_rows;
  if (threadIdx.x == 0) s_t0 = clock_ticks();
  int running = 0, before_mine = 0;
  for (int64_t t0 = 0; t0 < a.T_r; t0 += kA2aThreads * kScanSub) {
    uint64_t m[kScanSub];  // local experts each of the thread's tokens picked (bit d: expert ebase + d)
#pragma unroll
    for (int i = 0; i < kScanSub; ++i) m[i] = 0;
    auto add = [&](int i, int v) {
      const int d = v - ebase;
      if (d >= 0 && d < a.E_l) m[i] |= 1ull << d;
    };
    if (vec) {
      int4 v[kScanSub][2];
#pragma unroll
      for (int i = 0; i < kScanSub; ++i) {
        const int64_t t = t0 + i * kA2aThreads + threadIdx.x;
        v[i][0] = ids4(rt, t < a.T_r ? (uint32_t)(t * k * 4) : kOob);
        v[i][1] = ids4(rt, t < a.T_r && k == 8 ? (uint32_t)(t * k * 4 + 16) : kOob);
      }
#pragma unroll
      for (int i = 0; i < kScanSub; ++i)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          add(i, v[i][q].x); add(i, v[i][q].y); add(i, v[i][q].z); add(i, v[i][q].w);
        }
    } else {
#pragma unroll
      for (int i = 0; i < kScanSub; ++i) {
        const int64_t t = t0 + i * kA2aThreads + threadIdx.x;
        if (t < a.T_r)
          for (int j = 0; j < k; ++j) add(i, tab[t * k + j]);
      }
    }
    const uint64_t below = l > 0 ? (~0ull >> (64 - l)) : 0ull;  // local experts before l
    bool hit[kScanSub];
    int pre[kScanSub];
#pragma unroll
    for (int i = 0; i < kScanSub; ++i) {
      hit[i] = ((m[i] >> l) & 1ull) != 0;
      before_mine += __popcll(m[i] & below);
      const uint64_t bal = __ballot(hit[i]);
      pre[i] = __popcll(bal & ((1ull << lane) - 1ull));
      if (lane == 0) wsum[i][wave] = __popcll(bal);
    }
    __syncthreads();
    int base = running;
#pragma unroll
    for (int i = 0; i < kScanSub; ++i) {
      int off = base, tot = 0;
      for (int w = 0; w < kA2aThreads / 64; ++w) {
        if (w < wave) off += wsum[i][w];
        tot += wsum[i][w];
      }
      const int pos = off + pre[i];
      if (hit[i] && pos >= r0 && pos < r0 + a.chunk_rows) {
        const int32_t t = (int32_t)(t0 + i * kA2aThreads + threadIdx.x);
        s_tok[pos - r0] = t;
        a.lists[(int64_t)b * a.T_r + pos] = t;
      }
      base += tot;
    }
    running = base;
    __syncthreads();  // wsum is rewritten by the next pass
  }
  // rows of the link's earlier blocks: the sum of every thread's count
  for (int sh = 32; sh > 0; sh >>= 1) before_mine += __shfl_xor(before_mine, sh);
  if (lane == 0) wbefore[wave] = before_mine;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < kA2aThreads / 64; ++w) before += wbefore[w];
  const int count = running;  // uniform
  if (c == 0 && threadIdx.x == 0)
    __hip_atomic_store(a.count_sig + b, ((uint64_t)a.epoch << 32) | (uint32_t)count, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  const int64_t rest = count - r0;
  const int rows = rest < a.chunk_rows ? (int)rest : a.chunk_rows;
  if (rows <= 0) return;  // uniform: past the block's count, nothing is sent and no flag is published
  const bool paced = a.ticks_per_row > 0.0 && link != a.rank;
  const uint64_t release = paced ? (uint64_t)((double)(before + r0 + rows) * a.ticks_per_row) : 0;
  if (threadIdx.x == 0 && paced) {
    const uint64_t lead = (uint64_t)rows * (uint64_t)a.row_bytes / 200u + 100u;
    if (release > lead)
      while (clock_ticks() < s_t0 + release - lead) __builtin_amdgcn_s_sleep(4);  // finite
  }
  __syncthreads();
  const uint32_t block_bytes = (uint32_t)(a.T_r * a.row_bytes);
  const __amdgpu_buffer_rsrc_t rs = a2a_rsrc(a.src.p[link], block_bytes);
  const __amdgpu_buffer_rsrc_t rd = a2a_rsrc(a.dst + (int64_t)b * a.T_r * a.row_bytes, block_bytes);
  const uint32_t upr = (uint32_t)(a.row_bytes >> 4);
  const uint32_t total = (uint32_t)rows * upr;
  for (uint32_t u0 = threadIdx.x; u0 < total; u0 += kA2aThreads * kA2aUnroll) {
    u32x4 v[kA2aUnroll];
    uint32_t dof[kA2aUnroll];
#pragma unroll
    for (int u = 0; u < kA2aUnroll; ++u) {
      const uint32_t unit = u0 + (uint32_t)u * kA2aThreads;
      const uint32_t row = unit / upr, col = unit - row * upr;
      const bool in = unit < total;
      const uint32_t srow = (uint32_t)s_tok[in ? row : 0];
      const uint32_t sof = in ? srow * (uint32_t)a.row_bytes + col * 16u : kOob;
      dof[u] = in ? ((uint32_t)r0 + row) * (uint32_t)a.row_bytes + col * 16u : kOob;
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, sof, 0, kCpolNt);
    }
    __builtin_amdgcn_sched_barrier(0);  // every load in flight before the first store
#pragma unroll
    for (int u = 0; u < kA2aUnroll; ++u) __builtin_amdgcn_raw_buffer_store_b128(v[u], rd, dof[u], 0, kCpolSc1);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    if (paced)
      while (clock_ticks() < s_t0 + release) __builtin_amdgcn_s_sleep(4);  // finite
    if (link != a.withhold) flag_publish_coherent(a.flags + item, a.epoch);
  }
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Combine receiver: one wave per token (wave g takes tokens g, g + G, ...).
// Lane j < k holds pick j (expert, slot, gate) and polls the flag of the
// chunk holding its row; once every pick's flag is set (and after the
// acquire), the wave sums gate * row over the picks in pick order in fp32,
// kRecvPicks rows in flight at a time, and stores the token's fp32 row.
// Picks of ids outside [0, E) add nothing (their loads read zero).
__device__ __forceinline__ void a2a_receive(const A2aArgs& a, int wave_id, int n_waves) {
  const int lane = threadIdx.x & 63;
  const int k = a.k;
  const int32_t* tab = static_cast<const int32_t*>(a.table.p[0]);
  const uint32_t row_bytes = (uint32_t)a.row_bytes;
  const uint32_t upr = row_bytes >> 4;  // 16-byte units (8 bf16) per row
  const int64_t out_row_bytes = a.row_bytes * 2;  // fp32 output: 4 bytes per element
  for (int64_t t = wave_id; t < a.T_r; t += n_waves) {
    int e = -1, s = 0;
    float g = 0.f;
    bool valid = false;
    if (lane < k) {
      e = tab[t * k + lane];
      valid = e >= 0 && e < a.E;
      s = valid ? a.lists[t * k + lane] : 0;
      g = valid ? a.gate[t * k + lane] : 0.f;
    }
    const int64_t f = valid ? (int64_t)e * a.n_chunks + s / a.chunk_rows : -1;
    const uint64_t w0 = clock_ticks();
    bool mine = !valid;
    uint32_t seen = 0;
    while (true) {
      if (!mine) {
        seen = flag_peek(a.flags + f);
        mine = flag_is_set(seen, a.epoch);
      }
      if (__all(mine)) break;
      if (clock_ticks() - w0 > a.timeout_ticks) {
        if (!mine) report_timeout(a.status, f, seen, a.epoch);
        return;  // the wave stops; the call reports the timeout
      }
      __builtin_amdgcn_s_sleep(1);
    }
    acquire_agent();
    const __amdgpu_buffer_rsrc_t ro = a2a_rsrc(a.out + t * (a.row_bytes >> 1), (uint32_t)out_row_bytes);
    for (uint32_t p0 = 0; p0 < upr; p0 += 64 * kRecvUnits) {
      float acc[kRecvUnits][8];
#pragma unroll
      for (int m = 0; m < kRecvUnits; ++m)
#pragma unroll
        for (int x = 0; x < 8; ++x) acc[m][x] = 0.f;
      for (int j0 = 0; j0 < k; j0 += kRecvPicks) {
        u32x4 v[kRecvPicks][kRecvUnits];
        float gj[kRecvPicks];
#pragma unroll
        for (int jj = 0; jj < kRecvPicks; ++jj) {
          const int j = j0 + jj;  // uniform; lanes >= k hold no pick, so j >= k reads as invalid
          const int ej = __shfl(e, j & 63), sj = __shfl(s, j & 63);
          const bool vj = j < k && __shfl((int)valid, j & 63) != 0;
          gj[jj] = vj ? __shfl(g, j & 63) : 0.f;
          const char* row = a.dst + ((int64_t)(vj ? ej : 0) * a.T_r + (vj ? sj : 0)) * a.row_bytes;
          const __amdgpu_buffer_rsrc_t rr = a2a_rsrc(row, vj ? row_bytes : 0u);
#pragma unroll
          for (int m = 0; m < kRecvUnits; ++m) {
            const uint32_t unit = p0 + (uint32_t)(m * 64 + lane);
            v[jj][m] = __builtin_amdgcn_raw_buffer_load_b128(rr, unit < upr ? unit * 16u : kOob, 0, 0);
          }
        }
#pragma unroll
        for (int jj = 0; jj < kRecvPicks; ++jj)
#pragma unroll
          for (int m = 0; m < kRecvUnits; ++m) {
            const u32x4 w = v[jj][m];
            acc[m][0] = fmaf(gj[jj], bf16_lo(w.x), acc[m][0]);
            acc[m][1] = fmaf(gj[jj], bf16_hi(w.x), acc[m][1]);
            acc[m][2] = fmaf(gj[jj], bf16_lo(w.y), acc[m][2]);
            acc[m][3] = fmaf(gj[jj], bf16_hi(w.y), acc[m][3]);
            acc[m][4] = fmaf(gj[jj], bf16_lo(w.z), acc[m][4]);
            acc[m][5] = fmaf(gj[jj], bf16_hi(w.z), acc[m][5]);
            acc[m][6] = fmaf(gj[jj], bf16_lo(w.w), acc[m][6]);
            acc[m][7] = fmaf(gj[jj], bf16_hi(w.w), acc[m][7]);
          }
      }
#pragma unroll
      for (int m = 0; m < kRecvUnits; ++m) {
        const uint32_t unit = p0 + (uint32_t)(m * 64 + lane);
        const uint32_t o = unit < upr ? unit * 32u : kOob;
        const f32x4_t lo = {acc[m][0], acc[m][1], acc[m][2], acc[m][3]};
        const f32x4_t hi = {acc[m][4], acc[m][5], acc[m][6], acc[m][7]};
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, lo), ro, o, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, hi), ro, o == kOob ? kOob : o + 16u, 0, 0);
      }
    }
  }
}

// One launch: workgroups [0, n_send) are the senders (one per chunk), the
// rest (combine only) the receiver.  The receiver's workgroups come after
// every sender's in the grid, so by the time one of them runs, every sender
// has been dispatched and runs to its end: each wait can end.
__global__ void __launch_bounds__(kA2aThreads) a2a_kernel(A2aArgs a) {
  if ((int)blockIdx.x < a.n_send) {
    if (a.mode == 0 && a.fused_scan) a2a_dispatch_send(a, blockIdx.x);
    else a2a_send(a, blockIdx.x);
  } else {
    const int per = kA2aThreads / 64;
    a2a_receive(a, ((int)blockIdx.x - a.n_send) * per + (int)(threadIdx.x >> 6), ((int)gridDim.x - a.n_send) * per);
  }
}

}  // namespace

hipError_t launch_a2a_scan(const A2aArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(a2a_scan_kernel, dim3(a.E), dim3(kA2aThreads), 0, stream, a);
  return hipGetLastError();
}

// `done`, when given, is recorded by the launch itself at the kernel's end (no
// separate marker on the stream).
hipError_t launch_a2a(const A2aArgs& a, int recv_grid, hipStream_t stream, hipEvent_t done) {
  hipExtLaunchKernelGGL(a2a_kernel, dim3(a.n_send + recv_grid), dim3(kA2aThreads), 0, stream, nullptr, done, 0, a);
  return hipGetLastError();
}

}  // namespace sgt
