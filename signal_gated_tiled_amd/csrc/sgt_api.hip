// Host runtime of libsgt: context, validation, epochs, the producer schedule
// and the stream choreography of each call (declared in include/sgt.h).
//
// Streams (paper summary, "Method": communication and computation are
// launched on different streams so they run concurrently):
//   caller's stream  -- consumer kernel (and everything in serial mode)
//   ctx->prod        -- producer kernel; forked from and joined back into the
//                       caller's stream with events, so calls stay ordered.
#include <hip/hip_runtime.h>
#include <hsa/hsa.h>
#include <hsa/hsa_ext_amd.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "sgt.h"
#include "common.hpp"
#include "ring.hpp"
#include "sched.hpp"
#include "alltoall.hpp"

namespace sgt {
hipError_t launch_ag_producer(uint32_t* flags, const ProdItem* items, int n_items,
                              int64_t tile_bytes, uint32_t epoch, int withhold_peer, uint64_t* trace_release, int grid,
                              hipStream_t stream, uint32_t* started = nullptr, uint64_t* trace_issue = nullptr,
                              uint32_t seg_rows = 0, uint32_t seg_bytes = 0, uint32_t row_stride = 0,
                              const RelItem* rel = nullptr, int n_rel = 0, const uint32_t* marks = nullptr,
                              uint64_t timeout_ticks = 0, uint32_t* status = nullptr, uint32_t* finished = nullptr);
hipError_t launch_ll_allgather(const ProdItem* items, int n_prod, int n_recv, int n_prod_blocks, int grid,
                               int64_t chunk_bytes, uint32_t epoch, int withhold_peer, uint64_t lead, int rank,
                               uint64_t timeout_ticks, uint32_t* status, uint64_t* trace, hipStream_t stream);
hipError_t launch_ring_allreduce(const RingArgs& a, int grid, hipStream_t stream);
hipError_t launch_ag_allgather(uint32_t* flags, const ProdItem* items, int n_prod, int n_recv, int n_prod_blocks,
                               int grid, int64_t tile_bytes, uint32_t epoch, int withhold_peer,
                               uint64_t timeout_ticks, uint32_t* status, uint64_t* trace, hipStream_t stream);
hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t stream);
hipError_t launch_rs_prepare(uint32_t* pflags, int64_t n, uint32_t v, uint32_t* counter, hipStream_t stream);
hipError_t launch_ag_consumer(const AgArgs& a, int in_dtype, int grid, hipStream_t stream, hipEvent_t done);
int ag_panel_rows(int in_dtype);
int ag_panel_cols(int in_dtype);
hipError_t launch_gemm_rs(const RsArgs& a, int grid, hipStream_t stream, hipEvent_t done = nullptr);
int rs_gemm_tile();
int moe_tokens_per_group(int64_t T, int k);
hipError_t launch_moe_route(const float* logits, int64_t T, int E, int k, int tile_rows, const MoeTables& tb,
                            int32_t* expert_off, int32_t* row_token, int32_t* topk_ids, hipStream_t stream);
hipError_t launch_moe_rs(const MoeRsArgs& a, int grid, hipStream_t stream, hipEvent_t done = nullptr);
hipError_t launch_moe_consumer(const MoeArgs& a, int b_layout, int out_dtype, int tile_rows, int tile_waves, int grid,
                               hipStream_t stream, hipEvent_t done);
hipError_t launch_a2a_scan(const A2aArgs& a, hipStream_t stream);
hipError_t launch_a2a(const A2aArgs& a, int recv_grid, hipStream_t stream, hipEvent_t done = nullptr);
inline int kBMrs() { return rs_gemm_tile(); }
constexpr int kBNmoe() { return 256; }  // column tile of the tile core
}  // namespace sgt

using namespace sgt;

namespace {

thread_local std::string g_last_error;

sgt_status fail(sgt_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

#define HIP_TRY(expr)                                                                            \
  do {                                                                                           \
    hipError_t e_ = (expr);                                                                      \
    if (e_ != hipSuccess) return fail(SGT_EHIP, "%s: %s (%s:%d)", #expr, hipGetErrorString(e_), \
                                      __FILE__, __LINE__);                                       \
  } while (0)

constexpr int kSlots = 4;                 // producer schedule tables in flight
// Counter words of a context: [0] GEMM+RS reduction claims, [32] AllGather
// producer workgroups started (cumulative), [64 + 16 x] claim counter of XCD x
// for the AllGather consumer (cleared by a fill kernel before each launch).
constexpr int kCounterWords = 512;
constexpr int kAgStartedWord = 32, kAgDoneWord = 48, kAgClaimWord = 64;  // claim sets: 64.. and 192..
constexpr int kRingDoneWord = 56;  // the ring AllReduce producer's finished count
constexpr int kRsDoneWord = 60;    // the paced ReduceScatter peers' producer's finished count
constexpr int kSdmaMaxUnits = 4096;       // copy-engine copies per call
constexpr int64_t kSdmaUnitBytes = 4 << 20;  // bytes per copy-engine copy (whole-row signal tiles grouped up to this)
constexpr int64_t kItemsCap = 1 << 18;    // signal tiles per call
constexpr int64_t kMoeMaxTokens = 1 << 20;  // tokens of one MoE AllGather call
constexpr double kTicksPerUs = 100.0;     // constant GPU clock: 100 MHz

}  // namespace

struct sgt_ctx {
  int device = 0;
  int n_cu = 0;
  hipStream_t prod = nullptr;
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
  uint32_t epoch = 0;
  uint32_t* d_status = nullptr;  // 4 words
  uint32_t* d_counters = nullptr;  // work-claim counters, zeroed before each launch that uses them
  uint32_t ag_prod_started = 0;    // AllGather producer workgroups launched so far (cumulative)
  uint32_t ag_prod_done = 0;       // of those, the ones that count themselves finished (cumulative)
  uint32_t ring_prod_done = 0;     // ring AllReduce producer workgroups finished (cumulative)
  uint32_t rs_prod_done = 0;       // paced ReduceScatter producer workgroups finished (cumulative)
  int ag_claim_parity = 0;         // which of the two AllGather claim-counter sets the next consumer uses
  ProdItem* h_items[kSlots] = {};
  ProdItem* d_items[kSlots] = {};
  uint32_t* d_moe = nullptr;       // MoE: tile count (word 0), producer started (12) and finished (16) counts,
                                   // per-XCD claim counters (words 64 + 16 x), counts[2][256] by call parity
                                   // (words 256..767)
  int moe_parity = 0;
  uint32_t moe_prod_started = 0;   // producer workgroups launched by overlapped MoE calls (cumulative)
  uint32_t moe_prod_done = 0;      // of those, the ones that count themselves finished (cumulative)
  MoeTile* d_moe_order = nullptr;  // MoE row tiles in the XCD-partitioned work lists; grow on demand
  int64_t moe_cap = 0;
  uint32_t* d_moe_masks = nullptr; // MoE token bitmasks; grow on demand
  int64_t moe_masks_cap = 0;
  // MoE combine side: inverse routing table, group row tiles, counters (tile
  // count, claim, per-column done counts); grow on demand
  int32_t* d_mrs_rowof = nullptr;
  int64_t mrs_rowof_cap = 0;
  MoeTile* d_mrs_tiles = nullptr;
  int64_t mrs_tiles_cap = 0;
  uint32_t* d_mrs_ctr = nullptr;
  int64_t mrs_ctr_cap = 0;
  int32_t* d_a2a_counts = nullptr;  // AllToAll: rows of each (link, expert) block, kA2aMaxE entries
  hipEvent_t slot_ev[kSlots] = {};
  bool slot_used[kSlots] = {};
  std::vector<ProdItem> slot_items[kSlots];  // what d_items[slot] holds since its last upload
  std::vector<ProdItem> build;               // host scratch for building a schedule (grows only)
  int slot = 0;
  // Copy-engine producer (SGT_PROD_SDMA), set up on its first use: the HSA
  // agent of this device and its copy engines, a mark word per copy unit
  // (device memory, written by the engines), and per call slot a gate signal
  // (opened by a host function when the caller's stream reaches the call), the
  // epoch word the mark copies read (pinned host memory), the copies'
  // completion signals and the releaser's item table.
  bool sdma_ready = false;
  hsa_agent_t sdma_agent{};
  std::vector<uint32_t> sdma_engines;     // engine id bits (hsa_amd_sdma_engine_id_t)
  uint32_t* d_marks = nullptr;            // kSdmaMaxUnits words
  uint32_t* h_sdma_epoch = nullptr;       // kSlots words, pinned
  hsa_signal_t sdma_gate[kSlots] = {};
  std::vector<hsa_signal_t> sdma_sig[kSlots];  // 2 per unit: data copy, mark copy
  int sdma_used[kSlots] = {};             // signals of the slot's last call
  RelItem* h_rel[kSlots] = {};
  RelItem* d_rel[kSlots] = {};
  int64_t rel_cap = 0;
  hipEvent_t sdma_ev[kSlots] = {};
  bool sdma_ev_used[kSlots] = {};
  int sdma_slot = 0;
  bool sdma_hsa = false;                  // hsa_init taken (released by sgt_ctx_destroy)
  hipEvent_t ev_done = nullptr;           // recorded at the end of each call's work
  bool ev_done_used = false;
  std::mutex mu;
};

namespace {

struct DeviceGuard {
  int prev = -1;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != dev) (void)hipSetDevice(dev);
  }
  ~DeviceGuard() {
    if (prev >= 0) (void)hipSetDevice(prev);
  }
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_bytes(int dtype) { return dtype == SGT_BF16 ? 2 : 4; }

uint64_t timeout_ticks(const sgt_opts& o) {
  const double ms = o.timeout_ms > 0 ? o.timeout_ms : 2000.0;
  return (uint64_t)(ms * 1000.0 * kTicksPerUs);
}

// SplitMix64 (Steele, Lea and Flood, 2014): seeded arrival orders and jitter.
uint64_t splitmix64(uint64_t& s) {
  uint64_t z = (s += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Default rows per AllGather signal tile: about 512 KiB per tile (so a link
// delivers one every few microseconds), a divisor of the shard's rows, and no
// more than the consumer panel.
int64_t default_flag_rows(int64_t rows_per_shard, int64_t K, int esz, int panel) {
  int64_t target = std::max<int64_t>(1, (512 * 1024) / std::max<int64_t>(1, K * esz));
  target = std::min<int64_t>(target, panel);
  for (int64_t fr = std::min(target, rows_per_shard); fr > 1; --fr)
    if (rows_per_shard % fr == 0) return fr;
  return 1;
}

sgt_status check_opts(const sgt_opts* o, int W, bool sdma_ok = false) {
  if (!o) return fail(SGT_EINVAL, "opts is NULL");
  if (o->rank < 0 || o->rank >= W) return fail(SGT_EINVAL, "rank %d outside [0, %d)", o->rank, W);
  if (o->in_dtype != SGT_F32 && o->in_dtype != SGT_BF16) return fail(SGT_EINVAL, "in_dtype %d", o->in_dtype);
  if (o->out_dtype != SGT_F32 && o->out_dtype != SGT_BF16) return fail(SGT_EINVAL, "out_dtype %d", o->out_dtype);
  if (o->b_layout != SGT_KN && o->b_layout != SGT_NK) return fail(SGT_EINVAL, "b_layout %d", o->b_layout);
  if (o->producer < SGT_PROD_CU || o->producer > SGT_PROD_SDMA) return fail(SGT_EINVAL, "producer %d", o->producer);
  if (o->sdma_peers < 0) return fail(SGT_EINVAL, "sdma_peers %d", o->sdma_peers);
  if (o->producer == SGT_PROD_SDMA && !sdma_ok)
    return fail(SGT_EUNSUPPORTED, "the copy-engine producer (SGT_PROD_SDMA) applies to sgt_ag_gemm");
  if (o->order != SGT_ORDER_MESH && o->order != SGT_ORDER_SHARD) return fail(SGT_EINVAL, "order %d", o->order);
  if (o->flag_rows < 0 || o->producer_cus < 0 || o->consumer_cus < 0) return fail(SGT_EINVAL, "negative count");
  if (!(o->peer_gbps >= 0) || !(o->jitter_us >= 0) || !(o->timeout_ms >= 0))
    return fail(SGT_EINVAL, "negative or NaN rate/jitter/timeout");
  if (o->rs_tile < 0) return fail(SGT_EINVAL, "rs_tile %d", o->rs_tile);
  if (o->arrival_order < 0 || o->arrival_order > 2) return fail(SGT_EINVAL, "arrival_order %d", o->arrival_order);
  if (o->tile_waves != 0 && o->tile_waves != 4 && o->tile_waves != 8)
    return fail(SGT_EINVAL, "tile_waves %d (0, 4 or 8)", o->tile_waves);
  if (o->tile_rows != 0 && o->tile_rows != 128 && o->tile_rows != 256)
    return fail(SGT_EINVAL, "tile_rows %d (0, 128 or 256)", o->tile_rows);
  if (o->k_chunks < 0 || o->k_chunks > 64) return fail(SGT_EINVAL, "k_chunks %d outside [0, 64]", o->k_chunks);
  return SGT_OK;
}

struct AgPlan {
  int64_t rows_per_shard, flag_rows, n_flags, tiles_per_shard;
  int panel_rows, panel_cols, tiles_m, tiles_n;
  int n_kc = 0, kc_cols = 0;  // K-chunked signal tiles (opts.k_chunks): chunks per panel and their width
};

sgt_status plan_ag(int W, int64_t M, int64_t K, int64_t N, const sgt_opts& o, AgPlan* p) {
  if (W < 1 || W > kMaxW) return fail(SGT_EINVAL, "W = %d outside [1, %d]", W, kMaxW);
  if (M < 0 || N < 0 || K < 1) return fail(SGT_EINVAL, "bad shape M=%lld K=%lld N=%lld", (long long)M,
                                           (long long)K, (long long)N);
  if (M % W) return fail(SGT_EINVAL, "M = %lld is not a multiple of W = %d", (long long)M, W);
  if (o.in_dtype == SGT_BF16 && (K % 8 || N % 8))
    return fail(SGT_EINVAL, "bf16 needs K %% 8 == 0 and N %% 8 == 0 (K=%lld N=%lld)", (long long)K, (long long)N);
  const int esz = elem_bytes(o.in_dtype);
  p->rows_per_shard = M / W;
  p->panel_rows = ag_panel_rows(o.in_dtype);
  p->panel_cols = ag_panel_cols(o.in_dtype);
  if (o.k_chunks > 0 && o.flag_rows != 0 && o.flag_rows != p->panel_rows)
    return fail(SGT_EINVAL, "flag_rows %d with k_chunks: a signal tile is one %d-row panel (pass 0)", o.flag_rows,
                p->panel_rows);
  if (o.flag_rows > 0) {
    p->flag_rows = o.flag_rows;
  } else {
    p->flag_rows = p->rows_per_shard > 0 ? default_flag_rows(p->rows_per_shard, K, esz, p->panel_rows) : 1;
  }
  if (p->rows_per_shard % p->flag_rows)
    return fail(SGT_EINVAL, "rows per shard %lld not a multiple of flag_rows %lld", (long long)p->rows_per_shard,
                (long long)p->flag_rows);
  p->n_flags = M / p->flag_rows;
  if (o.k_chunks > 0) {
    // signal tiles of one consumer panel x one column chunk of K
    if (o.in_dtype != SGT_BF16) return fail(SGT_EUNSUPPORTED, "k_chunks needs bf16 inputs");
    if (K % (128 * (int64_t)o.k_chunks))
      return fail(SGT_EINVAL, "K = %lld is not a multiple of 128 x k_chunks (%d)", (long long)K, o.k_chunks);
    if (p->rows_per_shard % p->panel_rows)
      return fail(SGT_EUNSUPPORTED, "k_chunks needs shards of whole %d-row panels", p->panel_rows);
    p->flag_rows = p->panel_rows;
    p->n_kc = o.k_chunks;
    p->kc_cols = (int)(K / o.k_chunks);
    p->n_flags = M / p->panel_rows * o.k_chunks;
  }
  if (p->n_flags > kItemsCap) return fail(SGT_EINVAL, "%lld signal tiles exceed %lld", (long long)p->n_flags,
                                          (long long)kItemsCap);
  p->tiles_per_shard = p->rows_per_shard / p->flag_rows * (p->n_kc > 0 ? p->n_kc : 1);
  if (p->flag_rows * K * esz >= ((int64_t)1 << 31)) return fail(SGT_EUNSUPPORTED, "signal tile of 2 GiB or more");
  const int64_t tm = (M + p->panel_rows - 1) / p->panel_rows, tn = (N + p->panel_cols - 1) / p->panel_cols;
  if (tm * tn > (int64_t)1 << 30) return fail(SGT_EINVAL, "too many tiles");
  p->tiles_m = (int)tm;
  p->tiles_n = (int)tn;
  // 32-bit buffer offsets inside a tile and across K x N
  if ((int64_t)p->panel_rows * K * esz >= ((int64_t)1 << 31) || (int64_t)p->panel_rows * N * 4 >= ((int64_t)1 << 31))
    return fail(SGT_EUNSUPPORTED, "K or N too large for 32-bit tile offsets");
  // B stored K x N is addressed as one buffer: its size must stay below the
  // out-of-range offset 2^31 so masked lanes always read zero.
  if (o.in_dtype == SGT_BF16 && o.b_layout == SGT_KN && K * N * 2 >= ((int64_t)1 << 31))
    return fail(SGT_EUNSUPPORTED, "K x N too large for 32-bit offsets");
  return SGT_OK;
}

// Producer work list: every remote tile at the time its link would deliver it,
// then the local signal tiles (released as soon as copied).  Each peer's link carries
// one tile every tile_bytes / peer_gbps; the tiles of a peer go in order, or
// in a seeded order per peer, or (arrival_order 2) all remote tiles follow one
// seeded order at the aggregate rate of the W - 1 links.  Each release is then
// delayed by U[0, jitter].
double jitter_ticks(const sgt_opts& o, uint64_t& s) {
  if (o.jitter_us <= 0) return 0.0;
  return o.jitter_us * kTicksPerUs * (double)(splitmix64(s) >> 11) * (1.0 / 9007199254740992.0);
}

void shuffle(std::vector<int64_t>& v, uint64_t& s) {
  for (int64_t i = (int64_t)v.size() - 1; i > 0; --i) {
    const int64_t j = (int64_t)(splitmix64(s) % (uint64_t)(i + 1));
    std::swap(v[(size_t)i], v[(size_t)j]);
  }
}

// local_first: the local shard's tiles go first (released at once), for a
// consumer that reads every row from the gathered buffer; otherwise they go
// last.  ranks (optional): ranks[tile] = the tile's position in the list.
ProdItem sched_item(int64_t tile, int peer, double release) {
  ProdItem it{};
  it.flag0 = (uint32_t)tile;
  it.nflags = 1;
  it.peer = (uint16_t)peer;
  it.release = (uint64_t)release;
  return it;
}

// The k-th signal tile a link delivers, in link order.  Whole-row signal tiles
// go in order.  K-chunked ones go two panels at a time, chunk-major within the
// pair (panel 0 chunk 0, panel 1 chunk 0, panel 0 chunk 1, ...): two panels'
// tiles can start together, and each panel's chunks land at half the link
// rate, near the rate at which a tile computes them, so a panel's tiles spend
// less time waiting on its last chunks than when it arrives in one burst.
int64_t interleaved_chunk(const AgPlan& p, int64_t k) {
  if (p.n_kc <= 0) return k;
  const int64_t per_pair = 2 * (int64_t)p.n_kc, panels = p.tiles_per_shard / p.n_kc;
  const int64_t j0 = 2 * (k / per_pair), within = k % per_pair;
  const int64_t np = panels - j0 < 2 ? panels - j0 : 2;  // the last panel of an odd count goes alone
  return (j0 + within % np) * p.n_kc + within / np;
}

int build_schedule(const AgPlan& p, int W, int rank, int64_t K, int esz, const sgt_opts& o,
                   const void* const* shards, void* gathered, ProdItem* items, bool local_first = false) {
  // a K-chunked signal tile is one panel's rows x one column chunk
  const double tile_bytes = (double)p.flag_rows * (double)(p.n_kc > 0 ? p.kc_cols : K) * esz;
  const double ticks_per_tile = o.peer_gbps > 0 ? tile_bytes / (o.peer_gbps * 1e3) * kTicksPerUs : 0.0;
  const int64_t tps = p.tiles_per_shard;
  int n = 0;
  if (local_first)
    for (int64_t t = 0; t < tps; ++t) items[n++] = sched_item(rank * tps + t, rank, 0.0);
  const int first_remote = n;
  uint64_t s = o.arrival_seed * 0x100000001B3ull + 0x5851F42D4C957F2Dull;
  if (o.arrival_order == 2 && W > 1) {
    std::vector<int64_t> all;
    for (int d = 1; d < W; ++d)
      for (int64_t t = 0; t < tps; ++t) all.push_back(((rank + d) % W) * tps + t);
    shuffle(all, s);
    const double per = ticks_per_tile / (double)(W - 1);
    for (size_t g = 0; g < all.size(); ++g) {
      const double rel = (double)(g + 1) * per + jitter_ticks(o, s);
      items[n++] = sched_item(all[g], (int)(all[g] / tps), rel);
    }
  } else if (W > 1) {
    // each link delivers its tiles in order (or a seeded order per link), all
    // links concurrently; items with equal release times (unthrottled links)
    // keep the order the consumer takes panels in: round-robin over the peers
    // for the mesh order, peer by peer for the shard order
    std::vector<std::vector<int64_t>> order((size_t)W - 1, std::vector<int64_t>((size_t)tps));
    for (int d = 1; d < W; ++d) {
      std::vector<int64_t>& od = order[(size_t)d - 1];
      for (int64_t t = 0; t < tps; ++t) od[(size_t)t] = interleaved_chunk(p, t);
      if (o.arrival_order == 1) shuffle(od, s);
    }
    const bool mesh = o.order == SGT_ORDER_MESH;
    for (int64_t outer = 0; outer < (mesh ? tps : (int64_t)W - 1); ++outer)
      for (int64_t inner = 0; inner < (mesh ? (int64_t)W - 1 : tps); ++inner) {
        const int d = 1 + (int)(mesh ? inner : outer);
        const int64_t k = mesh ? outer : inner;
        const int peer = (rank + d) % W;
        const double rel = (double)(k + 1) * ticks_per_tile + jitter_ticks(o, s);
        items[n++] = sched_item(peer * tps + order[(size_t)d - 1][(size_t)k], peer, rel);
      }
  }
  std::stable_sort(items + first_remote, items + n,
                   [](const ProdItem& a, const ProdItem& b) { return a.release < b.release; });
  // The AllGather consumer reads the local shard from the shard itself, so its
  // copy into the gathered buffer goes last, off the critical path.
  if (!local_first)
    for (int64_t t = 0; t < tps; ++t) items[n++] = sched_item(rank * tps + t, rank, 0.0);
  for (int i = 0; i < n; ++i) {
    const int64_t tile = items[i].flag0, local_tile = tile - (int64_t)items[i].peer * tps;
    if (p.n_kc > 0) {
      // panel j of the shard, column chunk q: rows [j * panel, +panel), columns [q * kc, +kc)
      const int64_t j = local_tile / p.n_kc, q = local_tile % p.n_kc;
      const int64_t src_el = j * p.flag_rows * K + q * p.kc_cols;
      const int64_t dst_el = ((int64_t)items[i].peer * p.rows_per_shard + j * p.flag_rows) * K + q * p.kc_cols;
      items[i].src = static_cast<const char*>(shards[items[i].peer]) + src_el * esz;
      items[i].dst = static_cast<char*>(gathered) + dst_el * esz;
    } else {
      items[i].src = static_cast<const char*>(shards[items[i].peer]) + local_tile * (int64_t)tile_bytes;
      items[i].dst = static_cast<char*>(gathered) + tile * (int64_t)tile_bytes;
    }
  }
  return n;
}

int default_producer_wgs(const sgt_opts& o, int n_cu) {
  if (o.producer_cus > 0) return o.producer_cus;
  return std::max(8, n_cu / 8);
}

// Workgroups a persistent consumer may keep beside a producer kernel of pwg
// workgroups.  Dispatch spreads each kernel's workgroups round-robin over the
// XCDs, and within an XCD over its groups of CUs, and a consumer workgroup
// fills a CU (its LDS allows one).  The producer's share is therefore rounded
// up to a multiple of n_cu / 8 CUs (4 per XCD on 256 CUs): with an uneven
// split (say 228 consumers beside 28 producers) one group of CUs can end up
// fully held by consumers waiting on flags, and a producer workgroup sent
// there never starts.
int consumer_beside(const sgt_ctx* ctx, int pwg) {
  const int unit = std::max(8, ctx->n_cu / 8);
  const int reserve = (pwg + unit - 1) / unit * unit;
  return std::max(1, ctx->n_cu - reserve);
}

sgt_status next_slot(sgt_ctx* ctx, int* slot) {
  const int s = ctx->slot;
  ctx->slot = (ctx->slot + 1) % kSlots;
  if (ctx->slot_used[s]) HIP_TRY(hipEventSynchronize(ctx->slot_ev[s]));
  *slot = s;
  return SGT_OK;
}

// Upload a schedule into a slot's device table, unless the table already
// holds exactly these items (a repeated call with the same arguments).  The
// slot's previous upload is complete: next_slot has waited for the event
// recorded after the last kernel that read the slot, which ran after it.
sgt_status upload_items(sgt_ctx* ctx, int slot, const ProdItem* items, int n, hipStream_t stream) {
  std::vector<ProdItem>& held = ctx->slot_items[slot];
  if (n <= 0) return SGT_OK;
  if ((int)held.size() == n && std::memcmp(held.data(), items, (size_t)n * sizeof(ProdItem)) == 0) return SGT_OK;
  HIP_TRY(hipMemcpyAsync(ctx->d_items[slot], items, (size_t)n * sizeof(ProdItem), hipMemcpyHostToDevice, stream));
  held.assign(items, items + n);
  return SGT_OK;
}

// Host scratch of at least n items for building a schedule.
ProdItem* build_buffer(sgt_ctx* ctx, int64_t n) {
  if ((int64_t)ctx->build.size() < n) ctx->build.resize((size_t)n);
  return ctx->build.data();
}

// Make `items` resident in a slot's device table and return the slot.  A
// slot that already holds exactly these items (a repeated call with the same
// arguments) is reused as it is: kernels only read the tables, so no upload
// and no wait are needed.  Otherwise the next slot is taken (waiting for its
// last reader), and the items go through its pinned staging buffer on
// `stream`.  The caller records slot_ev[slot] after the kernel that reads it.
sgt_status stage_items(sgt_ctx* ctx, const ProdItem* items, int n, hipStream_t stream, int* slot_out) {
  const size_t bytes = (size_t)std::max(n, 0) * sizeof(ProdItem);
  for (int s = 0; s < kSlots; ++s) {
    const std::vector<ProdItem>& held = ctx->slot_items[s];
    if (n > 0 && (int)held.size() == n && std::memcmp(held.data(), items, bytes) == 0) {
      *slot_out = s;
      return SGT_OK;
    }
  }
  int s;
  sgt_status st = next_slot(ctx, &s);
  if (st != SGT_OK) return st;
  ctx->slot_items[s].clear();
  if (n > 0) {
    std::memcpy(ctx->h_items[s], items, bytes);
    HIP_TRY(hipMemcpyAsync(ctx->d_items[s], ctx->h_items[s], bytes, hipMemcpyHostToDevice, stream));
    ctx->slot_items[s].assign(items, items + n);
  }
  *slot_out = s;
  return SGT_OK;
}

// Record the caller's optional event (before / after the consumer launch).
sgt_status mark(const sgt_opts& o, int which, hipStream_t stream) {
  if (o.consumer_events[which])
    HIP_TRY(hipEventRecord(static_cast<hipEvent_t>(o.consumer_events[which]), stream));
  return SGT_OK;
}

sgt_status sdma_drain_all(sgt_ctx* c);

// Wait for the context's own work -- its producer stream, the end of its last
// call on the caller's stream, and any copy-engine copies still in flight --
// and return the device status (SGT_ETIMEDOUT after an expired wait, then
// cleared).  The caller holds the context's lock.
sgt_status sync_locked(sgt_ctx* c) {
  DeviceGuard g(c->device);
  HIP_TRY(hipStreamSynchronize(c->prod));
  if (c->ev_done_used) HIP_TRY(hipEventSynchronize(c->ev_done));
  sgt_status s = sdma_drain_all(c);
  if (s != SGT_OK) return s;
  uint32_t st[4] = {0, 0, 0, 0};
  HIP_TRY(hipMemcpy(st, c->d_status, sizeof st, hipMemcpyDeviceToHost));
  if (st[0] == kStatusTimeout) {
    HIP_TRY(hipMemset(c->d_status, 0, sizeof st));
    if (st[1] == 0xFFFFFFFFu)
      return fail(SGT_ETIMEDOUT, "waiting for the producer to finish timed out: count %u, expected %u", st[2], st[3]);
    return fail(SGT_ETIMEDOUT, "wait on flag %u timed out: saw %u, expected %u", st[1], st[2], st[3]);
  }
  return SGT_OK;
}

// End of a call that launched work on `stream`: remember where the call's work
// ends (sgt_sync waits for it; done_recorded: the call's last kernel launch
// already records ev_done at its end), and in blocking mode wait and report.
sgt_status finish(sgt_ctx* ctx, const sgt_opts& o, hipStream_t stream, bool done_recorded = false);

// The event a call's last kernel launch records at its end in place of
// finish()'s marker: ev_done when that kernel ends the call's work on the
// caller's stream (`last`) and the caller does not time it with events of its
// own (whose end marker then follows it); else none.
hipEvent_t end_event(sgt_ctx* ctx, const sgt_opts& o, bool last) {
  return last && !o.consumer_events[1] ? ctx->ev_done : nullptr;
}

sgt_status finish(sgt_ctx* ctx, const sgt_opts& o, hipStream_t stream, bool done_recorded) {
  if (!done_recorded) HIP_TRY(hipEventRecord(ctx->ev_done, stream));
  ctx->ev_done_used = true;
  if (!o.blocking) return SGT_OK;
  HIP_TRY(hipStreamSynchronize(stream));
  return sync_locked(ctx);
}

// ---- copy-engine producer (SGT_PROD_SDMA) ----

struct AgentMatch {
  unsigned domain, bus, device;
  hsa_agent_t agent;
  bool found;
};

hsa_status_t match_agent(hsa_agent_t a, void* data) {
  AgentMatch* m = static_cast<AgentMatch*>(data);
  hsa_device_type_t t;
  if (hsa_agent_get_info(a, HSA_AGENT_INFO_DEVICE, &t) != HSA_STATUS_SUCCESS || t != HSA_DEVICE_TYPE_GPU)
    return HSA_STATUS_SUCCESS;
  uint32_t bdf = 0, dom = 0;
  if (hsa_agent_get_info(a, (hsa_agent_info_t)HSA_AMD_AGENT_INFO_BDFID, &bdf) != HSA_STATUS_SUCCESS ||
      hsa_agent_get_info(a, (hsa_agent_info_t)HSA_AMD_AGENT_INFO_DOMAIN, &dom) != HSA_STATUS_SUCCESS)
    return HSA_STATUS_SUCCESS;
  if (dom == m->domain && ((bdf >> 8) & 0xFFu) == m->bus && ((bdf >> 3) & 0x1Fu) == m->device) {
    m->agent = a;
    m->found = true;
    return HSA_STATUS_INFO_BREAK;
  }
  return HSA_STATUS_SUCCESS;
}

// Wait (on the host, bounded) until every completion signal of an SDMA slot's
// last call reads 0: its copies are done and their signals may be reused.
sgt_status sdma_slot_drain(sgt_ctx* c, int slot) {
  const int n = 2 * c->sdma_used[slot];
  for (int i = 0; i < n; ++i) {
    hsa_signal_t sg = c->sdma_sig[slot][(size_t)i];
    int64_t left_us = 10 * 1000 * 1000;
    while (hsa_signal_load_scacquire(sg) != 0) {
      if (left_us <= 0) return fail(SGT_EHIP, "copy-engine copies of an earlier call did not complete");
      hsa_signal_wait_scacquire(sg, HSA_SIGNAL_CONDITION_EQ, 0, 1000000, HSA_WAIT_STATE_BLOCKED);
      left_us -= 1000;
    }
  }
  c->sdma_used[slot] = 0;
  return SGT_OK;
}

sgt_status sdma_drain_all(sgt_ctx* c) {
  if (!c->sdma_ready) return SGT_OK;
  for (int s = 0; s < kSlots; ++s) {
    if (c->sdma_ev_used[s]) HIP_TRY(hipEventSynchronize(c->sdma_ev[s]));
    sgt_status st = sdma_slot_drain(c, s);
    if (st != SGT_OK) return st;
  }
  return SGT_OK;
}

// First use of the copy-engine producer on a context: the HSA agent of the
// context's device (matched by PCI location), its available copy engines, the
// mark words, the pinned epoch words and the slots' gate signals and events.
sgt_status sdma_setup(sgt_ctx* c) {
  if (c->sdma_ready) return SGT_OK;
  if (hsa_init() != HSA_STATUS_SUCCESS) return fail(SGT_EHIP, "hsa_init failed");
  c->sdma_hsa = true;
  char pci[64] = {0};
  HIP_TRY(hipDeviceGetPCIBusId(pci, (int)sizeof pci, c->device));
  AgentMatch m{};
  unsigned fn = 0;
  if (std::sscanf(pci, "%x:%x:%x.%x", &m.domain, &m.bus, &m.device, &fn) != 4)
    return fail(SGT_EHIP, "unexpected PCI bus id '%s'", pci);
  hsa_iterate_agents(match_agent, &m);
  if (!m.found) return fail(SGT_EUNSUPPORTED, "no HSA agent for device %d (%s)", c->device, pci);
  // The device's copy engines for copies within its memory.  Some runtime
  // versions answer this query only for copies between a GPU and the host:
  // then the engines of that direction are used, less the first two (which
  // carry the host's transfers) when others exist.
  uint32_t mask = 0;
  hsa_status_t hs = hsa_amd_memory_copy_engine_status(m.agent, m.agent, &mask);
  if (hs != HSA_STATUS_SUCCESS || mask == 0) {
    hsa_agent_t cpu{};
    hsa_iterate_agents(
        [](hsa_agent_t a, void* d) -> hsa_status_t {
          hsa_device_type_t t;
          if (hsa_agent_get_info(a, HSA_AGENT_INFO_DEVICE, &t) == HSA_STATUS_SUCCESS && t == HSA_DEVICE_TYPE_CPU) {
            *static_cast<hsa_agent_t*>(d) = a;
            return HSA_STATUS_INFO_BREAK;
          }
          return HSA_STATUS_SUCCESS;
        },
        &cpu);
    mask = 0;
    hs = cpu.handle ? hsa_amd_memory_copy_engine_status(m.agent, cpu, &mask) : HSA_STATUS_ERROR_INVALID_AGENT;
    if (hs == HSA_STATUS_SUCCESS && (mask & ~3u)) mask &= ~3u;
  }
  if (hs != HSA_STATUS_SUCCESS || mask == 0)
    return fail(SGT_EUNSUPPORTED, "no copy engine available on device %d (%s, status %d, mask 0x%x)", c->device, pci,
                (int)hs, mask);
  c->sdma_agent = m.agent;
  c->sdma_engines.clear();
  for (int b = 0; b < 32; ++b)
    if (mask & (1u << b)) c->sdma_engines.push_back(1u << b);
  HIP_TRY(hipMalloc(&c->d_marks, kSdmaMaxUnits * sizeof(uint32_t)));
  HIP_TRY(hipMemset(c->d_marks, 0, kSdmaMaxUnits * sizeof(uint32_t)));
  HIP_TRY(hipHostMalloc(&c->h_sdma_epoch, kSlots * 16 * sizeof(uint32_t), hipHostMallocDefault));
  for (int s = 0; s < kSlots; ++s) {
    if (hsa_signal_create(0, 0, nullptr, &c->sdma_gate[s]) != HSA_STATUS_SUCCESS)
      return fail(SGT_ENOMEM, "hsa_signal_create");
    HIP_TRY(hipEventCreateWithFlags(&c->sdma_ev[s], hipEventDisableTiming));
  }
  HIP_TRY(hipDeviceSynchronize());
  c->sdma_ready = true;
  return SGT_OK;
}

// Runs on the runtime's host thread when the producer stream reaches the call:
// the copy engines may start (their copies wait on this gate).
void open_gate(void* gate) { hsa_signal_store_screlease(*static_cast<hsa_signal_t*>(gate), 0); }

// The copy-engine producer of one AllGather+GEMM call (SGT_PROD_SDMA), up to
// and including its producer-stream launch; the caller launches the consumer
// beside it and joins.  items: the call's schedule (release order).  Items of
// the local shard and of the first n_sd remote peers in mesh order (rank+1,
// rank+2, ...) go to the copy engines: each copy unit (a whole 256-row panel
// with K-chunked signal tiles, else up to kSdmaUnitBytes of consecutive signal
// tiles of one peer) is one engine copy, gated on the call's host-function gate
// (so no copy starts before the caller's stream reaches the call) and followed
// on the same engine by a 4-byte copy of the epoch into the unit's mark word.
// The other items go to *cu_wgs CU producer workgroups; one more workgroup of
// the same launch releases the copy-engine items.
sgt_status ag_sdma_launch(sgt_ctx* ctx, const sgt_opts& o, const AgPlan& p, int W, int64_t K, int esz,
                          const void* const* shards, void* gathered, uint32_t* flags, const ProdItem* items,
                          int n_items, int64_t tile_bytes, uint32_t seg_rows, uint32_t seg_bytes,
                          uint32_t row_stride, uint64_t* trace_rel, uint32_t e, hipStream_t stream, int* cu_wgs,
                          uint32_t* started) {
  sgt_status st = sdma_setup(ctx);
  if (st != SGT_OK) return st;
  const int n_sd = o.sdma_peers > 0 ? std::min(o.sdma_peers, W - 1) : W - 1;
  const int64_t tps = p.tiles_per_shard;
  // copy units: with K-chunked signal tiles a unit is a panel of one peer, else
  // a run of upu consecutive signal tiles of one peer
  const int64_t upu = p.n_kc > 0 ? p.n_kc : std::max<int64_t>(1, kSdmaUnitBytes / tile_bytes);
  const int64_t units_per_shard = (tps + upu - 1) / upu;
  std::vector<int> unit_of((size_t)(W * units_per_shard), -1);
  struct Unit { const char* src; char* dst; int64_t bytes; };
  std::vector<Unit> units;
  std::vector<RelItem> rel;
  std::vector<ProdItem> cu;
  rel.reserve((size_t)n_items);
  for (int i = 0; i < n_items; ++i) {
    const ProdItem& it = items[i];
    const int d = ((int)it.peer - o.rank + W) % W;  // 0: the local shard
    if (d > n_sd) {
      cu.push_back(it);
      continue;
    }
    const int64_t local_tile = (int64_t)it.flag0 - (int64_t)it.peer * tps;
    const int64_t u = local_tile / upu;
    int& id = unit_of[(size_t)(it.peer * units_per_shard + u)];
    if (id < 0) {
      if ((int)units.size() >= kSdmaMaxUnits)
        return fail(SGT_EUNSUPPORTED, "more than %d copy-engine copies in one call", kSdmaMaxUnits);
      id = (int)units.size();
      // the unit's rows: panel u (K-chunked) or signal tiles [u upu, +upu) of the shard
      const int64_t row0 = p.n_kc > 0 ? u * p.flag_rows : u * upu * p.flag_rows;
      const int64_t rows = p.n_kc > 0 ? p.flag_rows : std::min(upu, tps - u * upu) * p.flag_rows;
      const int64_t row_bytes = K * esz;
      units.push_back(Unit{static_cast<const char*>(shards[it.peer]) + row0 * row_bytes,
                           static_cast<char*>(gathered) + ((int64_t)it.peer * p.rows_per_shard + row0) * row_bytes,
                           rows * row_bytes});
    }
    rel.push_back(RelItem{it.release, it.flag0, it.nflags, (uint32_t)id, it.peer});
  }
  const int n_units = (int)units.size(), n_rel = (int)rel.size(), n_cu = (int)cu.size();
  // this call's slot: its previous call's copies must be done before its signals are reused
  const int ss = ctx->sdma_slot;
  ctx->sdma_slot = (ss + 1) % kSlots;
  if (ctx->sdma_ev_used[ss]) HIP_TRY(hipEventSynchronize(ctx->sdma_ev[ss]));
  if ((st = sdma_slot_drain(ctx, ss)) != SGT_OK) return st;
  std::vector<hsa_signal_t>& sig = ctx->sdma_sig[ss];
  while ((int)sig.size() < 2 * n_units) {
    hsa_signal_t sg;
    if (hsa_signal_create(0, 0, nullptr, &sg) != HSA_STATUS_SUCCESS) return fail(SGT_ENOMEM, "hsa_signal_create");
    sig.push_back(sg);
  }
  if (n_rel > ctx->rel_cap) {
    // grow every slot's releaser table (no call of this context is in flight after the drain)
    if ((st = sdma_drain_all(ctx)) != SGT_OK) return st;
    HIP_TRY(hipStreamSynchronize(ctx->prod));
    const int64_t cap = std::max<int64_t>(n_rel, 4096);
    for (int s2 = 0; s2 < kSlots; ++s2) {
      if (ctx->h_rel[s2]) (void)hipHostFree(ctx->h_rel[s2]);
      if (ctx->d_rel[s2]) (void)hipFree(ctx->d_rel[s2]);
      ctx->h_rel[s2] = nullptr;
      ctx->d_rel[s2] = nullptr;
    }
    ctx->rel_cap = 0;
    for (int s2 = 0; s2 < kSlots; ++s2) {
      HIP_TRY(hipHostMalloc(&ctx->h_rel[s2], cap * sizeof(RelItem), hipHostMallocDefault));
      HIP_TRY(hipMalloc(&ctx->d_rel[s2], cap * sizeof(RelItem)));
    }
    ctx->rel_cap = cap;
  }
  // the copies, gated; each followed by its mark copy (the pinned epoch word of this slot)
  uint32_t* ep = ctx->h_sdma_epoch + 16 * ss;
  *ep = e;
  hsa_signal_store_relaxed(ctx->sdma_gate[ss], 1);
  const int n_eng = (int)ctx->sdma_engines.size();
  for (int u = 0; u < n_units; ++u) {
    hsa_signal_store_relaxed(sig[(size_t)(2 * u)], 1);
    hsa_signal_store_relaxed(sig[(size_t)(2 * u + 1)], 1);
  }
  ctx->sdma_used[ss] = n_units;
  for (int u = 0; u < n_units; ++u) {
    const hsa_amd_sdma_engine_id_t eng = (hsa_amd_sdma_engine_id_t)ctx->sdma_engines[(size_t)(u % n_eng)];
    hsa_status_t h1 = hsa_amd_memory_async_copy_on_engine(units[(size_t)u].dst, ctx->sdma_agent, units[(size_t)u].src,
                                                          ctx->sdma_agent, (size_t)units[(size_t)u].bytes, 1,
                                                          &ctx->sdma_gate[ss], sig[(size_t)(2 * u)], eng, true);
    hsa_status_t h2 = h1 == HSA_STATUS_SUCCESS
                          ? hsa_amd_memory_async_copy_on_engine(ctx->d_marks + u, ctx->sdma_agent, ep,
                                                                ctx->sdma_agent, sizeof(uint32_t), 1,
                                                                &sig[(size_t)(2 * u)], sig[(size_t)(2 * u + 1)], eng,
                                                                true)
                          : h1;
    if (h2 != HSA_STATUS_SUCCESS) {
      // nothing of this call has reached the stream yet: let the copies already
      // queued run once the stream's earlier work is done, then report
      for (int v = u; v < n_units; ++v) {
        hsa_signal_store_relaxed(sig[(size_t)(2 * v)], 0);
        hsa_signal_store_relaxed(sig[(size_t)(2 * v + 1)], 0);
      }
      (void)hipStreamSynchronize(stream);
      hsa_signal_store_screlease(ctx->sdma_gate[ss], 0);
      return fail(SGT_EHIP, "copy-engine copy %d of %d could not be queued (HSA status %d)", u, n_units, (int)h2);
    }
  }
  // producer stream: fork, open the gate when the stream gets there, then the
  // CU producer workgroups (if any) and the releaser in one launch
  HIP_TRY(hipEventRecord(ctx->ev_fork, stream));
  HIP_TRY(hipStreamWaitEvent(ctx->prod, ctx->ev_fork, 0));
  HIP_TRY(hipLaunchHostFunc(ctx->prod, open_gate, &ctx->sdma_gate[ss]));
  std::memcpy(ctx->h_rel[ss], rel.data(), (size_t)n_rel * sizeof(RelItem));
  HIP_TRY(hipMemcpyAsync(ctx->d_rel[ss], ctx->h_rel[ss], (size_t)n_rel * sizeof(RelItem), hipMemcpyHostToDevice,
                         ctx->prod));
  int slot = -1;
  if (n_cu > 0 && (st = stage_items(ctx, cu.data(), n_cu, ctx->prod, &slot)) != SGT_OK) return st;
  // the releaser is one more workgroup of the same launch: the CU share takes one fewer, so the two
  // together hold the CUs a CU producer alone would
  const int pwg = n_cu > 0 ? std::max(1, std::min(default_producer_wgs(o, ctx->n_cu) - 1, n_cu)) : 0;
  HIP_TRY(launch_ag_producer(flags, slot >= 0 ? ctx->d_items[slot] : nullptr, n_cu, tile_bytes, e, o.withhold_peer,
                             trace_rel, pwg, ctx->prod, started, nullptr, seg_rows, seg_bytes, row_stride,
                             ctx->d_rel[ss], n_rel, ctx->d_marks, timeout_ticks(o), ctx->d_status));
  if (slot >= 0) {
    HIP_TRY(hipEventRecord(ctx->slot_ev[slot], ctx->prod));
    ctx->slot_used[slot] = true;
  }
  HIP_TRY(hipEventRecord(ctx->sdma_ev[ss], ctx->prod));
  ctx->sdma_ev_used[ss] = true;
  *cu_wgs = pwg + (n_rel > 0 ? 1 : 0);
  return SGT_OK;
}

}  // namespace

// Reduction items per ReduceScatter signal tile: row bands of kRedBandRows
// rows (the whole tile when it is shorter).
constexpr int kRedBandRows = 32;
int rs_red_split(int rs_tile) { return rs_tile > kRedBandRows ? rs_tile / kRedBandRows : 1; }

extern "C" {

const char* sgt_version(void) { return "sgt 0.1 gfx950"; }

const char* sgt_status_str(int st) {
  switch (st) {
    case SGT_OK: return "SGT_OK";
    case SGT_EINVAL: return "SGT_EINVAL";
    case SGT_EUNSUPPORTED: return "SGT_EUNSUPPORTED";
    case SGT_ETIMEDOUT: return "SGT_ETIMEDOUT";
    case SGT_EHIP: return "SGT_EHIP";
    case SGT_ENOMEM: return "SGT_ENOMEM";
    default: return "SGT_UNKNOWN";
  }
}

const char* sgt_last_error(void) { return g_last_error.c_str(); }

size_t sgt_opts_size(void) { return sizeof(sgt_opts); }

void sgt_opts_init(sgt_opts* o) {
  if (!o) return;
  std::memset(o, 0, sizeof *o);
  o->in_dtype = SGT_BF16;
  o->out_dtype = SGT_F32;
  o->b_layout = SGT_KN;
  o->producer = SGT_PROD_CU;
  o->order = SGT_ORDER_MESH;
  o->timeout_ms = 2000.0;
  o->withhold_peer = -1;
}

sgt_status sgt_ctx_create(sgt_ctx** out, int device) {
  if (!out) return fail(SGT_EINVAL, "out is NULL");
  *out = nullptr;
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || device < 0 || device >= n)
    return fail(SGT_EINVAL, "device %d not present (%d devices)", device, n);
  DeviceGuard g(device);
  sgt_ctx* c = new (std::nothrow) sgt_ctx();
  if (!c) return fail(SGT_ENOMEM, "context");
  c->device = device;
  hipDeviceProp_t prop;
  sgt_status st = SGT_OK;
  auto chk = [&](hipError_t e, const char* what) {
    if (e != hipSuccess && st == SGT_OK) st = fail(SGT_EHIP, "%s: %s", what, hipGetErrorString(e));
  };
  chk(hipGetDeviceProperties(&prop, device), "hipGetDeviceProperties");
  if (st == SGT_OK) c->n_cu = prop.multiProcessorCount;
  chk(hipStreamCreateWithFlags(&c->prod, hipStreamNonBlocking), "hipStreamCreate");
  chk(hipEventCreateWithFlags(&c->ev_fork, hipEventDisableTiming), "hipEventCreate");
  chk(hipEventCreateWithFlags(&c->ev_join, hipEventDisableTiming), "hipEventCreate");
  chk(hipEventCreateWithFlags(&c->ev_done, hipEventDisableTiming), "hipEventCreate");
  chk(hipMalloc(&c->d_status, 4 * sizeof(uint32_t)), "hipMalloc(status)");
  chk(hipMalloc(&c->d_counters, kCounterWords * sizeof(uint32_t)), "hipMalloc(counters)");
  if (st == SGT_OK) chk(hipMemset(c->d_counters, 0, kCounterWords * sizeof(uint32_t)), "hipMemset(counters)");
  chk(hipMalloc(&c->d_moe, 1024 * sizeof(uint32_t)), "hipMalloc(moe)");
  if (st == SGT_OK) chk(hipMemset(c->d_moe, 0, 1024 * sizeof(uint32_t)), "hipMemset(moe)");
  chk(hipMalloc(&c->d_a2a_counts, kA2aMaxE * sizeof(int32_t)), "hipMalloc(a2a counts)");
  if (st == SGT_OK) chk(hipMemset(c->d_status, 0, 4 * sizeof(uint32_t)), "hipMemset");
  for (int s = 0; s < kSlots && st == SGT_OK; ++s) {
    chk(hipHostMalloc(&c->h_items[s], kItemsCap * sizeof(ProdItem), hipHostMallocDefault), "hipHostMalloc");
    chk(hipMalloc(&c->d_items[s], kItemsCap * sizeof(ProdItem)), "hipMalloc(items)");
    chk(hipEventCreateWithFlags(&c->slot_ev[s], hipEventDisableTiming), "hipEventCreate");
  }
  if (st != SGT_OK) {
    std::string keep = g_last_error;
    sgt_ctx_destroy(c);
    g_last_error = keep;
    return st;
  }
  *out = c;
  return SGT_OK;
}

sgt_status sgt_ctx_destroy(sgt_ctx* c) {
  if (!c) return SGT_OK;
  DeviceGuard g(c->device);
  if (c->prod) (void)hipStreamSynchronize(c->prod);
  (void)hipDeviceSynchronize();
  if (c->sdma_ready) {
    (void)sdma_drain_all(c);
    for (int s = 0; s < kSlots; ++s) {
      for (hsa_signal_t sg : c->sdma_sig[s]) hsa_signal_destroy(sg);
      c->sdma_sig[s].clear();
      if (c->sdma_gate[s].handle) hsa_signal_destroy(c->sdma_gate[s]);
      if (c->sdma_ev[s]) (void)hipEventDestroy(c->sdma_ev[s]);
      if (c->h_rel[s]) (void)hipHostFree(c->h_rel[s]);
      if (c->d_rel[s]) (void)hipFree(c->d_rel[s]);
    }
    if (c->d_marks) (void)hipFree(c->d_marks);
    if (c->h_sdma_epoch) (void)hipHostFree(c->h_sdma_epoch);
  }
  if (c->sdma_hsa) (void)hsa_shut_down();
  if (c->ev_done) (void)hipEventDestroy(c->ev_done);
  for (int s = 0; s < kSlots; ++s) {
    if (c->h_items[s]) (void)hipHostFree(c->h_items[s]);
    if (c->d_items[s]) (void)hipFree(c->d_items[s]);
    if (c->slot_ev[s]) (void)hipEventDestroy(c->slot_ev[s]);
  }
  if (c->d_status) (void)hipFree(c->d_status);
  if (c->d_counters) (void)hipFree(c->d_counters);
  if (c->d_moe) (void)hipFree(c->d_moe);
  if (c->d_moe_order) (void)hipFree(c->d_moe_order);
  if (c->d_moe_masks) (void)hipFree(c->d_moe_masks);
  if (c->d_mrs_rowof) (void)hipFree(c->d_mrs_rowof);
  if (c->d_mrs_tiles) (void)hipFree(c->d_mrs_tiles);
  if (c->d_mrs_ctr) (void)hipFree(c->d_mrs_ctr);
  if (c->d_a2a_counts) (void)hipFree(c->d_a2a_counts);
  if (c->ev_fork) (void)hipEventDestroy(c->ev_fork);
  if (c->ev_join) (void)hipEventDestroy(c->ev_join);
  if (c->prod) (void)hipStreamDestroy(c->prod);
  delete c;
  return SGT_OK;
}

sgt_status sgt_sync(sgt_ctx* c) {
  if (!c) return fail(SGT_EINVAL, "ctx is NULL");
  std::lock_guard<std::mutex> lock(c->mu);
  return sync_locked(c);
}

int64_t sgt_ag_flag_count(int W, int64_t M, int64_t K, const sgt_opts* opts) {
  sgt_opts o;
  if (opts) o = *opts; else sgt_opts_init(&o);
  AgPlan p;
  sgt_status st = plan_ag(W, M, K, o.in_dtype == SGT_BF16 ? 8 : 1, o, &p);
  return st == SGT_OK ? p.n_flags : (int64_t)st;
}

int32_t sgt_ag_panel_rows(int W, int64_t M, int64_t K, int64_t N, const sgt_opts* opts) {
  (void)W; (void)M; (void)K; (void)N;
  sgt_opts o;
  if (opts) o = *opts; else sgt_opts_init(&o);
  return ag_panel_rows(o.in_dtype);
}

int64_t sgt_panel_order(int W, int rank, int64_t M, int32_t panel_rows, int order, int32_t* out, int64_t cap) {
  if (W < 1 || W > kMaxW || rank < 0 || rank >= W || M < 0 || M % W || panel_rows < 1 || !out ||
      (order != SGT_ORDER_MESH && order != SGT_ORDER_SHARD))
    return fail(SGT_EINVAL, "bad panel-order arguments");
  const int64_t tiles_m = (M + panel_rows - 1) / panel_rows;
  if (tiles_m > cap) return fail(SGT_EINVAL, "cap %lld < %lld panels", (long long)cap, (long long)tiles_m);
  for (int64_t i = 0; i < tiles_m; ++i) out[i] = (int32_t)panel_at(i, tiles_m, M / W, panel_rows, W, rank, order);
  return tiles_m;
}

int64_t sgt_trace_words(int W, int64_t M, int64_t K, int64_t N, const sgt_opts* opts) {
  sgt_opts o;
  if (opts) o = *opts; else sgt_opts_init(&o);
  AgPlan p;
  sgt_status st = plan_ag(W, M, K, N, o, &p);
  if (st != SGT_OK) return st;
  return (int64_t)p.tiles_m * p.tiles_n * 4 + p.n_flags;
}

sgt_status sgt_ag_gemm(sgt_ctx* ctx, const void* const* A_shards, const void* B, void* A_gathered, void* C,
                       uint32_t* flags, int W, int64_t M, int64_t K, int64_t N, const sgt_opts* opts, void* stream_) {
  if (!ctx) return fail(SGT_EINVAL, "ctx is NULL");
  sgt_status st = check_opts(opts, W < 1 ? 1 : W, true);
  if (st != SGT_OK) return st;
  const sgt_opts& o = *opts;
  AgPlan p;
  if ((st = plan_ag(W, M, K, N, o, &p)) != SGT_OK) return st;
  if (!A_shards && M > 0) return fail(SGT_EINVAL, "A_shards is NULL");
  if (M > 0) {
    for (int q = 0; q < W; ++q)
      if (!A_shards[q] || !aligned16(A_shards[q])) return fail(SGT_EINVAL, "A_shards[%d] NULL or not 16-byte aligned", q);
    if (!A_gathered || !flags || !aligned16(A_gathered) || !aligned16(flags))
      return fail(SGT_EINVAL, "A_gathered or flags NULL or not 16-byte aligned");
    if (N > 0 && (!B || !C || !aligned16(B) || !aligned16(C)))
      return fail(SGT_EINVAL, "B or C NULL or not 16-byte aligned");
  }
  std::lock_guard<std::mutex> lock(ctx->mu);
  DeviceGuard g(ctx->device);
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  const uint32_t e = ++ctx->epoch;
  if (M == 0) return SGT_OK;
  const int esz = elem_bytes(o.in_dtype);

  AgArgs a{};
  a.A = A_gathered; a.A_local = A_shards[o.rank]; a.B = B; a.C = C; a.flags = flags; a.status = ctx->d_status;
  a.trace = o.trace;
  a.M = M; a.N = N; a.K = K; a.rows_per_shard = p.rows_per_shard; a.flag_rows = (int32_t)p.flag_rows;
  a.n_kc = p.n_kc; a.kc_cols = p.kc_cols;
  a.W = W; a.rank = o.rank; a.order = o.order; a.tiles_m = p.tiles_m; a.tiles_n = p.tiles_n;
  a.b_layout = o.b_layout; a.out_dtype = o.out_dtype; a.epoch = e; a.timeout_ticks = timeout_ticks(o);
  a.tile_waves = o.tile_waves ? o.tile_waves : 8;
  const int total_tiles = p.tiles_m * p.tiles_n;
  uint32_t* started = ctx->d_counters + kAgStartedWord;
  // bf16 tiles are claimed dynamically, XCD by XCD in the order the static
  // schedule of a `base`-workgroup grid gives them (a grid that is not a
  // multiple of the XCD count keeps the static schedule).  The claim counters
  // come in two sets used by alternate consumer launches: each launch claims
  // from one set (zeroed by the launch before it, or at context creation) and
  // zeroes the other at its start, so no clearing launch is needed.
  auto claim_setup = [&](int base, int late) -> sgt_status {
    if (o.in_dtype != SGT_BF16 || base % kXcds || N <= 0) return SGT_OK;
    const int set = ctx->ag_claim_parity, words = kXcds * kXcdClaimStride;
    a.xcd_claim = ctx->d_counters + kAgClaimWord + set * words;
    a.xcd_claim_next = ctx->d_counters + kAgClaimWord + (1 - set) * words;
    a.base_grid = base;
    a.late_blocks = late;
    a.started = started;
    a.started_all = ctx->ag_prod_started;
    return SGT_OK;
  };
  // the consumer launch; a launch that claims from a counter set hands the
  // other set to the next one
  // bound: the consumer ends the call's work on this stream, and its launch
  // records ev_done itself (finish then records nothing more), unless the
  // caller times the consumer with events of its own
  bool bound = false;
  auto launch_consumer = [&](int grid, bool last) -> sgt_status {
    if ((st = mark(o, 0, stream)) != SGT_OK) return st;
    bound = last && !o.consumer_events[1];
    HIP_TRY(launch_ag_consumer(a, o.in_dtype, grid, stream, bound ? ctx->ev_done : nullptr));
    if (a.xcd_claim) ctx->ag_claim_parity ^= 1;
    return mark(o, 1, stream);
  };

  if (o.producer == SGT_PROD_PRESET) {
    HIP_TRY(launch_fill_u32(flags, p.n_flags, e, stream));
    const int grid = std::min(total_tiles, o.consumer_cus > 0 ? o.consumer_cus
                                            : (o.in_dtype == SGT_BF16 ? ctx->n_cu : 4 * ctx->n_cu));
    if ((st = claim_setup(grid, 0)) != SGT_OK) return st;
    if (N > 0 && (st = launch_consumer(grid, true)) != SGT_OK) return st;
    return finish(ctx, o, stream, bound);
  }

  int slot;
  ProdItem* items = build_buffer(ctx, p.n_flags);
  const int n_items = build_schedule(p, W, o.rank, K, esz, o, A_shards, A_gathered, items);
  const int pwg = std::min(default_producer_wgs(o, ctx->n_cu), n_items);
  uint64_t* trace_rel = o.trace ? o.trace + (int64_t)total_tiles * 4 : nullptr;
  const int64_t tile_bytes = p.flag_rows * (p.n_kc > 0 ? p.kc_cols : K) * esz;
  // K-chunked signal tiles are column blocks: panel rows of kc_cols elements, K apart
  const uint32_t seg_rows = p.n_kc > 0 ? (uint32_t)p.flag_rows : 0u;
  const uint32_t seg_bytes = (uint32_t)(p.kc_cols * esz), row_stride = (uint32_t)(K * esz);

  if (o.producer == SGT_PROD_SERIAL) {
    if ((st = stage_items(ctx, items, n_items, stream, &slot)) != SGT_OK) return st;
    HIP_TRY(launch_ag_producer(flags, ctx->d_items[slot], n_items, tile_bytes, e, o.withhold_peer,
                               trace_rel, pwg, stream, nullptr, nullptr, seg_rows, seg_bytes, row_stride));
    HIP_TRY(hipEventRecord(ctx->slot_ev[slot], stream));
    ctx->slot_used[slot] = true;
    const int grid = std::min(total_tiles, o.consumer_cus > 0 ? o.consumer_cus
                                            : (o.in_dtype == SGT_BF16 ? ctx->n_cu : 4 * ctx->n_cu));
    if ((st = claim_setup(grid, 0)) != SGT_OK) return st;
    if (N > 0 && (st = launch_consumer(grid, true)) != SGT_OK) return st;
    return finish(ctx, o, stream, bound);
  }

  // Overlapped: the producer runs on its own stream.  The consumer keeps one
  // workgroup per CU (its LDS use allows no more) on all but the producer's
  // share of CUs, so both kernels are resident at once and no wait can starve.
  int prod_wgs = pwg;
  uint32_t* gpu_join = nullptr;
  if (o.producer == SGT_PROD_SDMA) {
    if ((st = ag_sdma_launch(ctx, o, p, W, K, esz, A_shards, A_gathered, flags, items, n_items, tile_bytes, seg_rows,
                             seg_bytes, row_stride, trace_rel, e, stream, &prod_wgs, started)) != SGT_OK)
      return st;
  } else {
    HIP_TRY(hipEventRecord(ctx->ev_fork, stream));
    HIP_TRY(hipStreamWaitEvent(ctx->prod, ctx->ev_fork, 0));
    if ((st = stage_items(ctx, items, n_items, ctx->prod, &slot)) != SGT_OK) return st;
    // the bf16 consumer joins the producer itself: its workgroups wait, before
    // they exit, until every producer workgroup has counted itself finished
    if (o.in_dtype == SGT_BF16 && N > 0) gpu_join = ctx->d_counters + kAgDoneWord;
    HIP_TRY(launch_ag_producer(flags, ctx->d_items[slot], n_items, tile_bytes, e, o.withhold_peer,
                               trace_rel, pwg, ctx->prod, started, nullptr, seg_rows, seg_bytes, row_stride, nullptr,
                               0, nullptr, 0, nullptr, gpu_join));
    if (gpu_join) {  // counted once the launch has gone in
      ctx->ag_prod_done += (uint32_t)pwg;
      a.prod_done = gpu_join;
      a.prod_done_all = ctx->ag_prod_done;
    }
    HIP_TRY(hipEventRecord(ctx->slot_ev[slot], ctx->prod));
    ctx->slot_used[slot] = true;
  }
  ctx->ag_prod_started += (uint32_t)prod_wgs;
  int grid;
  if (o.in_dtype == SGT_BF16) {
    // The consumer keeps consumer_beside() workgroups that never yield (an
    // equal share of every XCD beside the producer's).  With no caller count
    // it launches one workgroup per CU: the others wait in the dispatcher for
    // the producer's CUs and, once there, run only if the whole producer is
    // already running (else they exit and leave the CUs to it), then claim
    // tiles like the rest.
    const int keep = consumer_beside(ctx, prod_wgs);
    if (o.consumer_cus > 0) {
      grid = std::min(std::min(o.consumer_cus, keep), total_tiles);
      if ((st = claim_setup(grid, 0)) != SGT_OK) return st;
    } else {
      grid = std::min(ctx->n_cu, total_tiles);
      if ((st = claim_setup(std::min(keep, grid), std::max(0, grid - keep))) != SGT_OK) return st;
      if (!a.xcd_claim) grid = std::min(grid, keep);   // a static schedule keeps off the producer's CUs
    }
  } else {  // fp32 tiles: at most one workgroup per CU beside the producer's share, so even at one resident
            // workgroup per CU the waiting consumers leave every XCD the CUs the producer needs
    const int keep = consumer_beside(ctx, prod_wgs);
    grid = o.consumer_cus > 0 ? std::min(o.consumer_cus, keep) : keep;
    grid = std::min(grid, total_tiles);
  }
  if (N > 0 && (st = launch_consumer(grid, gpu_join != nullptr)) != SGT_OK) return st;
  if (!gpu_join) {
    HIP_TRY(hipEventRecord(ctx->ev_join, ctx->prod));
    HIP_TRY(hipStreamWaitEvent(stream, ctx->ev_join, 0));
  }
  return finish(ctx, o, stream, bound);
}

int64_t sgt_rs_trace_words(int W, int64_t M, int64_t N, const sgt_opts* opts) {
  int64_t ng;
  if (sgt_rs_flag_count(W, M, N, opts, &ng, nullptr) != SGT_OK) return -1;
  const int rt = opts && opts->rs_tile > 0 ? opts->rs_tile : 128;
  const int bm = rs_gemm_tile();
  const int64_t br = M / W, tn = (N + bm - 1) / bm;
  const int64_t n_gemm = (int64_t)W * ((br + bm - 1) / bm) * tn;
  const int64_t n_red = (br / rt) * ((N + rt - 1) / rt) * rs_red_split(rt);
  return 3 * (n_gemm + n_red);
}

sgt_status sgt_rs_flag_count(int W, int64_t M, int64_t N, const sgt_opts* opts, int64_t* gflags_n,
                             int64_t* pflags_n) {
  if (W < 1 || W > kMaxW || M < 0 || N < 0 || M % W) return fail(SGT_EINVAL, "bad GEMM+RS shape");
  const int rt = opts && opts->rs_tile > 0 ? opts->rs_tile : 128;
  if (rt < 16 || (rs_gemm_tile() % rt) || ((M / W) % rt))
    return fail(SGT_EINVAL, "rs_tile %d must be >= 16 and divide %d and the block rows %lld", rt, rs_gemm_tile(),
                (long long)(M / W));
  const int64_t tn = (N + rt - 1) / rt;
  if (gflags_n) *gflags_n = (M / rt) * tn;
  if (pflags_n) *pflags_n = (int64_t)W * ((M / W) / rt) * tn;
  return SGT_OK;
}

}  // extern "C"

namespace {

// Paced peers of a ReduceScatter: peer p's block (bands of rs_tile rows, band_bytes
// each, rs_tm bands) is copied from peer_blocks[p] into inbox[p] by the producer,
// each band no earlier than link p would deliver it (in order or shuffled, plus
// jitter), and the band's rs_tn peer flags are published.  The peers' flags
// start unset and `counter` (the reduction claim counter) restarts at zero.
// Serial mode: the producer runs first on the caller's stream.  Otherwise it
// runs on the context's producer stream, forked from the caller's; the caller
// launches its consumer and then joins with join_paced_peers.  *pwg_out: the
// producer's workgroups.
sgt_status launch_paced_peers(sgt_ctx* ctx, const sgt_opts& o, uint32_t* pflags, const float* const* peer_blocks,
                              const float* const* inbox, int W, int rs_tm, int rs_tn, int64_t band_bytes, uint32_t e,
                              uint32_t* counter, hipStream_t stream, int* pwg_out, RsArgs* join) {
  int slot;
  sgt_status st;
  const int64_t bands = rs_tm, block_tiles = (int64_t)rs_tm * rs_tn;
  ProdItem* items = build_buffer(ctx, (int64_t)(W - 1) * bands);
  const double ticks_per_band = o.peer_gbps > 0 ? (double)band_bytes / (o.peer_gbps * 1e3) * kTicksPerUs : 0.0;
  uint64_t seed = o.arrival_seed * 0x100000001B3ull + 0x5851F42D4C957F2Dull;
  int n = 0;
  std::vector<int64_t> order((size_t)bands);
  for (int d = 1; d < W; ++d) {
    const int peer = (o.rank + d) % W;
    for (int64_t j = 0; j < bands; ++j) order[(size_t)j] = j;
    if (o.arrival_order != 0) shuffle(order, seed);
    for (int64_t q = 0; q < bands; ++q) {
      const int64_t j = order[(size_t)q];
      ProdItem it = sched_item(peer * block_tiles + j * rs_tn, peer, (double)(q + 1) * ticks_per_band +
                                                                      jitter_ticks(o, seed));
      it.nflags = (uint16_t)rs_tn;
      it.src = reinterpret_cast<const char*>(peer_blocks[peer]) + j * band_bytes;
      it.dst = reinterpret_cast<char*>(const_cast<float*>(inbox[peer])) + j * band_bytes;
      items[n++] = it;
    }
  }
  std::stable_sort(items, items + n, [](const ProdItem& x, const ProdItem& y) { return x.release < y.release; });
  const int pwg = std::min(default_producer_wgs(o, ctx->n_cu), std::max(n, 1));
  *pwg_out = pwg;
  HIP_TRY(launch_rs_prepare(pflags, 0, e, counter, stream));  // counter only: peers' flags come on arrival
  if (o.producer == SGT_PROD_SERIAL) {
    if ((st = stage_items(ctx, items, n, stream, &slot)) != SGT_OK) return st;
    HIP_TRY(launch_ag_producer(pflags, ctx->d_items[slot], n, band_bytes, e, o.withhold_peer, nullptr, pwg, stream));
    HIP_TRY(hipEventRecord(ctx->slot_ev[slot], stream));
    ctx->slot_used[slot] = true;
    return SGT_OK;
  }
  HIP_TRY(hipEventRecord(ctx->ev_fork, stream));
  HIP_TRY(hipStreamWaitEvent(ctx->prod, ctx->ev_fork, 0));
  if ((st = stage_items(ctx, items, n, ctx->prod, &slot)) != SGT_OK) return st;
  // The consumer kernel joins the producer on the GPU: each producer workgroup
  // counts itself finished, and the consumer's workgroups wait for the call's
  // total before they exit (join_paced_peers is then not needed).
  uint32_t* done = n > 0 ? ctx->d_counters + kRsDoneWord : nullptr;
  HIP_TRY(launch_ag_producer(pflags, ctx->d_items[slot], n, band_bytes, e, o.withhold_peer, nullptr, pwg, ctx->prod,
                             nullptr, nullptr, 0, 0, 0, nullptr, 0, nullptr, 0, nullptr, done));
  if (done) {  // counted once the launch has gone in
    ctx->rs_prod_done += (uint32_t)pwg;
    join->prod_done = done;
    join->prod_done_all = ctx->rs_prod_done;
  }
  HIP_TRY(hipEventRecord(ctx->slot_ev[slot], ctx->prod));
  ctx->slot_used[slot] = true;
  return SGT_OK;
}

// The caller's stream waits for the producer forked by launch_paced_peers
// (when the consumer kernel does not join it on the GPU).
sgt_status join_paced_peers(sgt_ctx* ctx, hipStream_t stream) {
  HIP_TRY(hipEventRecord(ctx->ev_join, ctx->prod));
  HIP_TRY(hipStreamWaitEvent(stream, ctx->ev_join, 0));
  return SGT_OK;
}

// Validation and kernel arguments of a GEMM + ReduceScatter call, shared by
// the context entry points and the static-scratch one.  peer_blocks != NULL:
// paced peers.  caller_flags: gflags / pflags are the caller's (else they live
// in the library's scratch and are filled in by the caller of this function).
// Fills every field of *a except the epoch, the status word, the claim
// counter and the flags; *np = peer flag words.
sgt_status rs_plan(const void* A_local, const void* B, const float* const* reduce_from,
                   const float* const* peer_blocks, float* partial_out, float* C_shard, const uint32_t* gflags,
                   const uint32_t* pflags, bool caller_flags, int W, int64_t M, int64_t K, int64_t N,
                   const sgt_opts* opts, RsArgs* a, int64_t* ng_out, int64_t* np_out) {
  sgt_status st = check_opts(opts, W < 1 ? 1 : W);
  if (st != SGT_OK) return st;
  const sgt_opts& o = *opts;
  const bool paced = peer_blocks != nullptr;
  a->prod_done = nullptr;  // set by a paced overlapped call once its producer is launched
  a->prod_done_all = 0;
  if (o.in_dtype != SGT_BF16) return fail(SGT_EUNSUPPORTED, "GEMM+RS takes bf16 inputs");
  if (o.out_dtype != SGT_F32) return fail(SGT_EUNSUPPORTED, "GEMM+RS partials are fp32");
  if (!paced && o.producer == SGT_PROD_CU && o.peer_gbps > 0)
    return fail(SGT_EUNSUPPORTED, "sgt_gemm_rs takes resident peers; paced arrival is sgt_gemm_rs_paced");
  if (paced && o.producer == SGT_PROD_PRESET)
    return fail(SGT_EINVAL, "sgt_gemm_rs_paced needs a producer mode (CU or serial); resident peers: sgt_gemm_rs");
  if (W < 1 || W > kMaxW) return fail(SGT_EINVAL, "W = %d outside [1, %d]", W, kMaxW);
  if (M < 0 || N < 0 || K < 1 || M % W) return fail(SGT_EINVAL, "bad shape M=%lld K=%lld N=%lld W=%d",
                                                    (long long)M, (long long)K, (long long)N, W);
  if (K % 8 || N % 8) return fail(SGT_EINVAL, "bf16 needs K %% 8 == 0 and N %% 8 == 0");
  int64_t ng = 0, np = 0;
  if ((st = sgt_rs_flag_count(W, M, N, opts, &ng, &np)) != SGT_OK) return st;
  const int rt = o.rs_tile > 0 ? o.rs_tile : 128;
  const int64_t br = M / W;
  if ((int64_t)kBMrs() * K * 2 >= ((int64_t)1 << 31) || (int64_t)kBMrs() * N * 4 >= ((int64_t)1 << 31) ||
      (o.b_layout == SGT_KN && K * N * 2 >= ((int64_t)1 << 31)))
    return fail(SGT_EUNSUPPORTED, "K or N too large for 32-bit tile offsets");
  const int64_t band_bytes = (int64_t)rt * N * 4;
  const int64_t rs_tn = (N + rt - 1) / rt;
  if (paced && (band_bytes >= ((int64_t)1 << 31) || rs_tn > 65535 || (int64_t)(W - 1) * (br / rt) > kItemsCap))
    return fail(SGT_EUNSUPPORTED, "bands too large or too many for the producer");
  if (M > 0 && N > 0) {
    if (!A_local || !B || !partial_out || !C_shard || !reduce_from || (caller_flags && (!gflags || !pflags)))
      return fail(SGT_EINVAL, "NULL pointer argument");
    if (!aligned16(A_local) || !aligned16(B) || !aligned16(partial_out) || !aligned16(C_shard) ||
        (caller_flags && (!aligned16(gflags) || !aligned16(pflags))))
      return fail(SGT_EINVAL, "pointers must be 16-byte aligned");
    for (int p = 0; p < W; ++p) {
      if (p == o.rank) continue;
      if (!reduce_from[p] || !aligned16(reduce_from[p]))
        return fail(SGT_EINVAL, "%s[%d] NULL or not 16-byte aligned", paced ? "inbox" : "partials", p);
      if (paced && (!peer_blocks[p] || !aligned16(peer_blocks[p])))
        return fail(SGT_EINVAL, "peer_blocks[%d] NULL or not 16-byte aligned", p);
    }
  }
  *a = RsArgs{};
  a->A = A_local; a->B = B; a->P = partial_out; a->C_shard = C_shard;
  for (int p = 0; p < W; ++p) a->partials.p[p] = (p == o.rank) ? nullptr : reduce_from[p];
  a->trace = o.trace;
  a->M = M; a->N = N; a->K = K; a->block_rows = br; a->W = W; a->rank = o.rank;
  const int bm = rs_gemm_tile();
  a->tiles_n = (int)((N + bm - 1) / bm);
  a->tiles_m = (int)(W * ((br + bm - 1) / bm));
  a->rs_tile = rt; a->rs_tm = (int)(br / rt); a->rs_tn = (int)rs_tn;
  a->b_layout = o.b_layout;
  a->n_gemm_tiles = a->tiles_m * a->tiles_n;
  a->red_split = rs_red_split(rt);
  a->n_red_items = a->rs_tm * a->rs_tn * a->red_split;
  a->timeout_ticks = timeout_ticks(o);
  a->tile_waves = o.tile_waves ? o.tile_waves : 8;
  *ng_out = ng;
  *np_out = np;
  return SGT_OK;
}

// GEMM + ReduceScatter, shared by the resident and the paced entry points.
// reduce_from[p]: what the reduction sums for peer p.  peer_blocks == NULL:
// the peers' data is resident and their flags are preset.  Otherwise the
// producer copies peer_blocks[p] into reduce_from[p] in bands of rs_tile rows,
// each band released (its tiles' peer flags) when peer p's link would deliver it.
sgt_status gemm_rs_impl(sgt_ctx* ctx, const void* A_local, const void* B, const float* const* reduce_from,
                        const float* const* peer_blocks, float* partial_out, float* C_shard, uint32_t* gflags,
                        uint32_t* pflags, int W, int64_t M, int64_t K, int64_t N, const sgt_opts* opts,
                        void* stream_) {
  if (!ctx) return fail(SGT_EINVAL, "ctx is NULL");
  const bool paced = peer_blocks != nullptr;
  RsArgs a;
  int64_t ng = 0, np = 0;
  sgt_status st = rs_plan(A_local, B, reduce_from, peer_blocks, partial_out, C_shard, gflags, pflags, true, W, M, K,
                          N, opts, &a, &ng, &np);
  if (st != SGT_OK) return st;
  const sgt_opts& o = *opts;
  const int64_t band_bytes = (int64_t)a.rs_tile * N * 4;
  std::lock_guard<std::mutex> lock(ctx->mu);
  DeviceGuard g(ctx->device);
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  const uint32_t e = ++ctx->epoch;
  if (M == 0 || N == 0) return SGT_OK;
  a.gflags = gflags; a.pflags = pflags; a.status = ctx->d_status;
  a.epoch = e;
  a.red_counter = ctx->d_counters;
  const int total = a.n_gemm_tiles + a.n_red_items;

  if (!paced) {
    // Peers' partials are resident: their flags are set before the kernel
    // starts, and the reduction-claim counter restarts (a fill kernel, not a memset).
    HIP_TRY(launch_rs_prepare(pflags, np, e, ctx->d_counters, stream));
    // at most one workgroup per CU, so every workgroup is resident: a reduction
    // item waits on GEMM tiles statically assigned to other workgroups
    const int grid = std::min(total, o.consumer_cus > 0 ? std::min(o.consumer_cus, ctx->n_cu) : ctx->n_cu);
    if ((st = mark(o, 0, stream)) != SGT_OK) return st;
    HIP_TRY(launch_gemm_rs(a, grid, stream, end_event(ctx, o, true)));
    if ((st = mark(o, 1, stream)) != SGT_OK) return st;
    return finish(ctx, o, stream, end_event(ctx, o, true) != nullptr);
  }

  // Paced peers: the producer, on its own stream (or first on the caller's in
  // serial mode), copies the peers' bands into the inbox and releases their flags.
  int pwg = 0;
  if ((st = launch_paced_peers(ctx, o, pflags, peer_blocks, reduce_from, W, a.rs_tm, a.rs_tn, band_bytes, e,
                               ctx->d_counters, stream, &pwg, &a)) != SGT_OK)
    return st;
  if (o.producer == SGT_PROD_SERIAL) {
    const int grid = std::min(total, o.consumer_cus > 0 ? std::min(o.consumer_cus, ctx->n_cu) : ctx->n_cu);
    if ((st = mark(o, 0, stream)) != SGT_OK) return st;
    HIP_TRY(launch_gemm_rs(a, grid, stream, end_event(ctx, o, true)));
    if ((st = mark(o, 1, stream)) != SGT_OK) return st;
    return finish(ctx, o, stream, end_event(ctx, o, true) != nullptr);
  }
  // Overlapped: the GEMM+RS kernel on the CUs the producer leaves (one
  // workgroup per CU), so the reduction's waits cannot starve it.
  const int grid = std::min(total, std::min(o.consumer_cus > 0 ? o.consumer_cus : ctx->n_cu, consumer_beside(ctx, pwg)));
  if ((st = mark(o, 0, stream)) != SGT_OK) return st;
  HIP_TRY(launch_gemm_rs(a, grid, stream, end_event(ctx, o, a.prod_done != nullptr)));
  if ((st = mark(o, 1, stream)) != SGT_OK) return st;
  if (!a.prod_done && (st = join_paced_peers(ctx, stream)) != SGT_OK) return st;
  return finish(ctx, o, stream, end_event(ctx, o, a.prod_done != nullptr) != nullptr);
}

}  // namespace

extern "C" {

sgt_status sgt_gemm_rs(sgt_ctx* ctx, const void* A_local, const void* B, const float* const* partials,
                       float* partial_out, float* C_shard, uint32_t* gflags, uint32_t* pflags, int W, int64_t M,
                       int64_t K, int64_t N, const sgt_opts* opts, void* stream) {
  return gemm_rs_impl(ctx, A_local, B, partials, nullptr, partial_out, C_shard, gflags, pflags, W, M, K, N, opts,
                      stream);
}

sgt_status sgt_gemm_rs_paced(sgt_ctx* ctx, const void* A_local, const void* B, const float* const* peer_blocks,
                             float* const* inbox, float* partial_out, float* C_shard, uint32_t* gflags,
                             uint32_t* pflags, int W, int64_t M, int64_t K, int64_t N, const sgt_opts* opts,
                             void* stream) {
  if (!peer_blocks || !inbox) return fail(SGT_EINVAL, "peer_blocks or inbox is NULL");
  return gemm_rs_impl(ctx, A_local, B, inbox, peer_blocks, partial_out, C_shard, gflags, pflags, W, M, K, N, opts,
                      stream);
}

}  // extern "C"

// ---- GEMM + ReduceScatter with no allocation: the library's static scratch ----
//
// For callers that cannot allocate device memory (code under stream capture,
// tight serving loops): the status word, the reduction's claim counter and
// every signal flag of the call live in `scratch`, a file-scope device array
// of 64 KiB that each GPU holds until the process ends.  Its device
// address is taken once per device with hipGetSymbolAddress (the array's name
// in host code is not a device address) and only that address is used.
namespace {

constexpr int kScratchWords = 16384;                  // 64 KiB
constexpr int kScratchHead = 64;                      // status (4 words), claim counter, padding
constexpr int kScratchFlagWords = kScratchWords - kScratchHead;
constexpr int kMaxDevices = 64;

__device__ __align__(256) uint32_t scratch[kScratchWords];

struct StaticDev {
  uint32_t* ptr = nullptr;  // device address of this device's copy of scratch
  int n_cu = 0;
  uint32_t epoch = 0;       // flags in scratch hold earlier epochs of this device's calls
};
StaticDev g_static[kMaxDevices];
std::mutex g_static_mu;

}  // namespace

extern "C" {

int64_t sgt_gemm_rs_static_scratch_bytes(void) { return (int64_t)kScratchWords * 4; }

sgt_status sgt_gemm_rs_static(const void* A_local, const void* B, const float* const* partials, float* partial_out,
                              float* C_shard, int W, int64_t M, int64_t K, int64_t N, const sgt_opts* opts,
                              void* stream_) {
  RsArgs a;
  int64_t ng = 0, np = 0;
  sgt_status st = rs_plan(A_local, B, partials, nullptr, partial_out, C_shard, nullptr, nullptr, false, W, M, K, N,
                          opts, &a, &ng, &np);
  if (st != SGT_OK) return st;
  const sgt_opts& o = *opts;
  if (o.producer != SGT_PROD_PRESET && o.producer != SGT_PROD_CU)
    return fail(SGT_EINVAL, "sgt_gemm_rs_static takes resident peers (producer CU or preset)");
  if (o.trace) return fail(SGT_EUNSUPPORTED, "sgt_gemm_rs_static records no trace");
  if (ng + np > kScratchFlagWords)
    return fail(SGT_EINVAL, "%lld signal flags (%lld GEMM + %lld peer) exceed the %d words of static scratch",
                (long long)(ng + np), (long long)ng, (long long)np, kScratchFlagWords);
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(SGT_EUNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  std::lock_guard<std::mutex> lock(g_static_mu);
  StaticDev& sd = g_static[dev];
  if (!sd.ptr) {
    // once per device, with that device current: its copy of the array
    void* p = nullptr;
    HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return fail(SGT_EHIP, "hipGetSymbolAddress(scratch) returned NULL");
    int n_cu = 0;
    HIP_TRY(hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev));
    sd.ptr = static_cast<uint32_t*>(p);
    sd.n_cu = n_cu > 0 ? n_cu : 1;
  }
  if (M == 0 || N == 0) return SGT_OK;
  uint32_t* flags = sd.ptr + kScratchHead;
  if (++sd.epoch >= 0x40000000u) {
    // before any flag could alias a later epoch: clear them (a fill kernel) and restart
    HIP_TRY(launch_fill_u32(flags, kScratchFlagWords, 0u, stream));
    sd.epoch = 1;
  }
  uint32_t* pflags = flags + ng;
  a.gflags = flags;
  a.pflags = pflags;
  a.status = sd.ptr;
  a.red_counter = sd.ptr + 4;
  a.epoch = sd.epoch;
  // the resident peers' flags take the epoch and the claim counter restarts (one fill kernel, no memset)
  HIP_TRY(launch_rs_prepare(pflags, np, a.epoch, a.red_counter, stream));
  const int grid = std::min(a.n_gemm_tiles + a.n_red_items,
                            o.consumer_cus > 0 ? std::min(o.consumer_cus, sd.n_cu) : sd.n_cu);
  if ((st = mark(o, 0, stream)) != SGT_OK) return st;
  HIP_TRY(launch_gemm_rs(a, grid, stream));
  if ((st = mark(o, 1, stream)) != SGT_OK) return st;
  if (!o.blocking) return SGT_OK;
  HIP_TRY(hipStreamSynchronize(stream));
  uint32_t s4[4] = {0, 0, 0, 0};
  HIP_TRY(hipMemcpy(s4, sd.ptr, sizeof s4, hipMemcpyDeviceToHost));
  if (s4[0] == kStatusTimeout) {
    static const uint32_t zero4[4] = {0, 0, 0, 0};
    HIP_TRY(hipMemcpy(sd.ptr, zero4, sizeof zero4, hipMemcpyHostToDevice));
    return fail(SGT_ETIMEDOUT, "wait on flag %u timed out: saw %u, expected %u", s4[1], s4[2], s4[3]);
  }
  return SGT_OK;
}

static int moe_tile_rows(const sgt_opts& o) { return o.tile_rows > 0 ? o.tile_rows : 256; }

// Upper bound of the grouped row tiles of a routing: sum over experts of
// ceil(n_e / rows) <= T * topk / rows + E.
static int64_t moe_max_tiles(int64_t T, int E, int topk, int rows) { return T * topk / rows + E; }

int64_t sgt_moe_trace_words(int W, int64_t T, int64_t H, int64_t I, int E, int topk, const sgt_opts* opts) {
  sgt_opts o;
  if (opts) o = *opts; else sgt_opts_init(&o);
  AgPlan p;
  sgt_status st = plan_ag(W, T, H, I, o, &p);
  if (st != SGT_OK) return st;
  if (E < 1 || topk < 1 || topk > E) return fail(SGT_EINVAL, "bad E / topk");
  if (o.tile_rows != 0 && o.tile_rows != 128 && o.tile_rows != 256) return fail(SGT_EINVAL, "tile_rows");
  return moe_max_tiles(T, E, topk, moe_tile_rows(o)) * p.tiles_n * 4 + p.n_flags;
}

sgt_status sgt_moe_ag_gemm(sgt_ctx* ctx, const void* const* X_shards, const void* W_experts, const float* logits,
                           void* X_gathered, void* Y, int32_t* expert_off, int32_t* row_token, int32_t* topk_ids,
                           uint32_t* shard_flags, int W, int64_t T, int64_t H, int64_t I, int E, int topk,
                           const sgt_opts* opts, void* stream_) {
  if (!ctx) return fail(SGT_EINVAL, "ctx is NULL");
  sgt_status st = check_opts(opts, W < 1 ? 1 : W);
  if (st != SGT_OK) return st;
  const sgt_opts& o = *opts;
  if (o.in_dtype != SGT_BF16) return fail(SGT_EUNSUPPORTED, "MoE takes bf16 tokens and weights");
  if (o.k_chunks) return fail(SGT_EUNSUPPORTED, "k_chunks applies to sgt_ag_gemm");
  if (E < 1 || E > 256 || topk < 1 || topk > E) return fail(SGT_EINVAL, "need 1 <= topk <= E <= 256 (E=%d topk=%d)", E, topk);
  if (T < 0 || H < 1 || I < 0) return fail(SGT_EINVAL, "bad shape T=%lld H=%lld I=%lld", (long long)T, (long long)H,
                                           (long long)I);
  const int rows = moe_tile_rows(o);
  if (T > kMoeMaxTokens) return fail(SGT_EUNSUPPORTED, "T = %lld tokens exceeds %lld", (long long)T,
                                     (long long)kMoeMaxTokens);
  AgPlan p;
  if ((st = plan_ag(W, T, H, I, o, &p)) != SGT_OK) return st;
  const int64_t lim = (int64_t)1 << 31;
  if (T * H * 2 >= lim || (int64_t)256 * H * 2 >= lim || (int64_t)256 * I * 4 >= lim ||
      (o.b_layout == SGT_KN && H * I * 2 >= lim))
    return fail(SGT_EUNSUPPORTED, "T x H or one expert's H x I too large for 32-bit offsets");
  if (moe_max_tiles(T, E, topk, rows) * p.tiles_n >= lim) return fail(SGT_EUNSUPPORTED, "too many grouped tiles");
  if (T > 0) {
    // W_experts and Y are read / written only when I > 0
    if (!X_shards || !logits || !X_gathered || !expert_off || !row_token || !topk_ids || !shard_flags ||
        (I > 0 && (!Y || !W_experts)))
      return fail(SGT_EINVAL, "NULL pointer argument");
    for (int q = 0; q < W; ++q)
      if (!X_shards[q] || !aligned16(X_shards[q])) return fail(SGT_EINVAL, "X_shards[%d] NULL or not 16-byte aligned", q);
    if (!aligned16(X_gathered) || !aligned16(shard_flags) || (I > 0 && (!aligned16(Y) || !aligned16(W_experts))) ||
        (reinterpret_cast<uintptr_t>(logits) & 3u) || (reinterpret_cast<uintptr_t>(expert_off) & 3u) ||
        (reinterpret_cast<uintptr_t>(row_token) & 3u) || (reinterpret_cast<uintptr_t>(topk_ids) & 3u))
      return fail(SGT_EINVAL, "pointer not aligned (16 bytes for matrices and flags, 4 for tables)");
  } else if (!expert_off) {
    return fail(SGT_EINVAL, "expert_off is NULL");
  }
  std::lock_guard<std::mutex> lock(ctx->mu);
  DeviceGuard g(ctx->device);
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  const uint32_t e = ++ctx->epoch;
  if (T == 0) {  // no tokens: every group is empty
    HIP_TRY(launch_fill_u32(reinterpret_cast<uint32_t*>(expert_off), E + 1, 0u, stream));
    return finish(ctx, o, stream);
  }

  // Routing tables: grow (after draining the device) when a larger routing needs more.
  const int64_t max_tiles = moe_max_tiles(T, E, topk, rows);
  const int tpg = moe_tokens_per_group(T, topk);
  const int64_t n_groups = (T + tpg - 1) / tpg;
  const int64_t mask_words = (int64_t)((E + 31) / 32) * T;
  if (ctx->moe_cap < max_tiles || ctx->moe_masks_cap < mask_words) {
    HIP_TRY(hipDeviceSynchronize());
    if (ctx->moe_cap < max_tiles) {
      if (ctx->d_moe_order) (void)hipFree(ctx->d_moe_order);
      ctx->d_moe_order = nullptr;
      ctx->moe_cap = 0;
      const int64_t cap = std::max<int64_t>(max_tiles, 1024);
      HIP_TRY(hipMalloc(&ctx->d_moe_order, cap * sizeof(MoeTile)));
      ctx->moe_cap = cap;
    }
    if (ctx->moe_masks_cap < mask_words) {
      if (ctx->d_moe_masks) (void)hipFree(ctx->d_moe_masks);
      ctx->d_moe_masks = nullptr;
      ctx->moe_masks_cap = 0;
      const int64_t cap = std::max<int64_t>(mask_words, 1 << 16);
      HIP_TRY(hipMalloc(&ctx->d_moe_masks, cap * sizeof(uint32_t)));
      ctx->moe_masks_cap = cap;
    }
  }
  MoeTables tb{};
  tb.masks = ctx->d_moe_masks;
  tb.counts = ctx->d_moe + 256 + 256 * ctx->moe_parity;
  tb.counts_next = ctx->d_moe + 256 + 256 * (1 - ctx->moe_parity);
  tb.n_groups = (int32_t)n_groups;
  tb.tokens_per_group = tpg;
  tb.n_tiles = ctx->d_moe;
  tb.tiles_cap = (uint32_t)ctx->moe_cap;
  tb.xcd_claim = ctx->d_moe + 64;  // kXcds counters at words 64, 80, ..., 176
  tb.order = ctx->d_moe_order;

  const int esz = 2;
  MoeArgs a{};
  a.X = static_cast<const uint16_t*>(X_gathered);
  a.We = static_cast<const uint16_t*>(W_experts);
  a.Y = Y; a.row_token = row_token; a.expert_off = expert_off; a.order = tb.order; a.n_tiles = tb.n_tiles;
  a.tiles_cap = tb.tiles_cap;
  a.xcd_claim = tb.xcd_claim; a.flags = shard_flags; a.status = ctx->d_status; a.trace = o.trace;
  a.T = T; a.H = H; a.I = I; a.rows = T * topk; a.E = E; a.flag_rows = (int32_t)p.flag_rows; a.tiles_n = p.tiles_n;
  a.epoch = e; a.timeout_ticks = timeout_ticks(o);
  const int64_t n_items_max = max_tiles * p.tiles_n;
  uint64_t* trace_rel = o.trace ? o.trace + n_items_max * 4 : nullptr;
  const int64_t tile_bytes = p.flag_rows * H * esz;

  // Routing and the grouped consumer, on the caller's stream.  keep > 0: an
  // overlapped call, where only `keep` workgroups of the launched grid may wait
  // for the producer; the others (the last launched - keep) yield unless every
  // producer workgroup already runs.  The split is taken on the grid actually
  // launched, so a grid of keep workgroups or fewer never yields.
  const bool done_bound = I > 0 && !o.consumer_events[1];
  auto route_and_compute = [&](int grid, int keep) -> sgt_status {
    HIP_TRY(launch_moe_route(logits, T, E, topk, rows, tb, expert_off, row_token, topk_ids, stream));
    ctx->moe_parity ^= 1;  // this call's top-k cleared the other counts buffer for the next call
    if (I > 0) {
      const int launched = (int)std::max<int64_t>(1, std::min<int64_t>(grid, n_items_max));
      a.late_blocks = keep > 0 ? std::max(0, launched - keep) : 0;
      sgt_status s2;
      if ((s2 = mark(o, 0, stream)) != SGT_OK) return s2;
      // the launch records ev_done at the consumer's end, the end of the call's
      // work on this stream (finish records nothing more), unless the caller
      // times the consumer with events of its own (then its end marker follows)
      HIP_TRY(launch_moe_consumer(a, o.b_layout, o.out_dtype, rows, o.tile_waves ? o.tile_waves : 8, launched,
                                  stream, done_bound ? ctx->ev_done : nullptr));
      if ((s2 = mark(o, 1, stream)) != SGT_OK) return s2;
    }
    return SGT_OK;
  };

  if (o.producer == SGT_PROD_PRESET) {
    // X_gathered already holds every shard: all flags take the epoch.
    HIP_TRY(launch_fill_u32(shard_flags, p.n_flags, e, stream));
    if ((st = route_and_compute(o.consumer_cus > 0 ? std::min(o.consumer_cus, ctx->n_cu) : ctx->n_cu, 0)) != SGT_OK)
      return st;
    return finish(ctx, o, stream, done_bound);
  }

  int slot;
  if ((st = next_slot(ctx, &slot)) != SGT_OK) return st;
  const int n_items = build_schedule(p, W, o.rank, H, esz, o, X_shards, X_gathered, ctx->h_items[slot], true);
  const int pwg = std::min(default_producer_wgs(o, ctx->n_cu), n_items);
  // The producer's schedule is copied on the stream that runs the producer.
  if (o.producer == SGT_PROD_SERIAL) {
    if ((st = upload_items(ctx, slot, ctx->h_items[slot], n_items, stream)) != SGT_OK) return st;
    HIP_TRY(launch_ag_producer(shard_flags, ctx->d_items[slot], n_items, tile_bytes, e, o.withhold_peer,
                               trace_rel, pwg, stream));
    if ((st = route_and_compute(o.consumer_cus > 0 ? std::min(o.consumer_cus, ctx->n_cu) : ctx->n_cu, 0)) != SGT_OK)
      return st;
    HIP_TRY(hipEventRecord(ctx->slot_ev[slot], stream));
    ctx->slot_used[slot] = true;
    return finish(ctx, o, stream, done_bound);
  }

  // Overlapped: producer on its own stream and CUs; routing, then the grouped
  // consumer on the remaining CUs (one workgroup per CU).
  HIP_TRY(hipEventRecord(ctx->ev_fork, stream));
  HIP_TRY(hipStreamWaitEvent(ctx->prod, ctx->ev_fork, 0));
  if ((st = upload_items(ctx, slot, ctx->h_items[slot], n_items, ctx->prod)) != SGT_OK) return st;
  // The grouped consumer joins the producer itself (its workgroups wait, before
  // they exit, until every producer workgroup has counted itself finished);
  // with no consumer launched (I == 0) the stream waits for the producer instead.
  uint32_t* gpu_join = I > 0 ? ctx->d_moe + 16 : nullptr;
  HIP_TRY(launch_ag_producer(shard_flags, ctx->d_items[slot], n_items, tile_bytes, e, o.withhold_peer,
                             trace_rel, pwg, ctx->prod, ctx->d_moe + 12, nullptr, 0, 0, 0, nullptr, 0, nullptr, 0,
                             nullptr, gpu_join));
  if (gpu_join) {  // counted once the launch has gone in
    ctx->moe_prod_done += (uint32_t)pwg;
    a.prod_done = gpu_join;
    a.prod_done_all = ctx->moe_prod_done;
  }
  // the slot's schedule is read only on the producer's stream (its upload and
  // the producer), so its reuse waits on that stream, and the caller's stream
  // carries no extra marker between one call's consumer and the next call
  HIP_TRY(hipEventRecord(ctx->slot_ev[slot], ctx->prod));
  ctx->slot_used[slot] = true;
  HIP_TRY(hipEventRecord(ctx->ev_join, ctx->prod));
  // The consumer takes the whole chip: its last pwg workgroups land on the
  // producer's CUs as the producer finishes (they claim work dynamically, so
  // arriving late only means fewer items).  Each of those checks once, without
  // waiting, that every producer workgroup is running; if not (the producer is
  // not fully dispatched), it exits, so it can never keep the producer off the
  // chip.  A count that never matches (a failed earlier call) only makes them exit.
  ctx->moe_prod_started += (uint32_t)pwg;
  a.started = ctx->d_moe + 12;
  a.started_all = ctx->moe_prod_started;
  // (the workgroups that never yield are consumer_beside(pwg), the CUs left
  // beside the producer's share rounded up as for the other overlapped calls,
  // so they are spread evenly over the XCDs; a caller's count is capped there)
  const int keep = consumer_beside(ctx, pwg);
  if ((st = route_and_compute(o.consumer_cus > 0 ? std::min(o.consumer_cus, keep) : ctx->n_cu, keep)) != SGT_OK)
    return st;
  if (!gpu_join) HIP_TRY(hipStreamWaitEvent(stream, ctx->ev_join, 0));
  return finish(ctx, o, stream, done_bound);
}


}  // extern "C"

namespace {

// MoE GEMM + ReduceScatter, shared by the resident and the paced entry points
// (partials: what the reduction sums for each peer; peer_blocks == NULL: they
// are resident and their flags preset, else the producer copies peer_blocks[p]
// into partials[p] band by band at the link rate).
sgt_status moe_gemm_rs_impl(sgt_ctx* ctx, const void* Hg, const void* W2, const float* gate, const int32_t* topk_ids,
                            const int32_t* expert_off, const int32_t* row_token, const float* const* partials,
                            const float* const* peer_blocks, void* Y, float* partial_out, float* C_shard,
                            uint32_t* gflags, uint32_t* pflags, int W, int64_t T, int topk, int64_t I, int64_t H,
                            int E, const sgt_opts* opts, void* stream_) {
  if (!ctx) return fail(SGT_EINVAL, "ctx is NULL");
  sgt_status st = check_opts(opts, W < 1 ? 1 : W);
  if (st != SGT_OK) return st;
  const sgt_opts& o = *opts;
  if (o.in_dtype != SGT_BF16) return fail(SGT_EUNSUPPORTED, "MoE takes bf16 rows and weights");
  // out_dtype is Y's: fp32, or bf16 (RNE) to halve its traffic; P and C_shard are fp32 either way
  const bool y_bf16 = o.out_dtype == SGT_BF16;
  const bool paced = peer_blocks != nullptr;
  if (!paced && o.peer_gbps > 0)
    return fail(SGT_EUNSUPPORTED, "sgt_moe_gemm_rs takes resident peers; paced arrival is sgt_moe_gemm_rs_paced");
  if (paced && o.producer == SGT_PROD_PRESET)
    return fail(SGT_EINVAL, "sgt_moe_gemm_rs_paced needs a producer mode (CU or serial)");
  if (o.rs_tile != 0 && o.rs_tile != 128) return fail(SGT_EINVAL, "rs_tile %d (the combine tile is 128)", o.rs_tile);
  if (o.tile_waves != 0 && o.tile_waves != 8) return fail(SGT_EUNSUPPORTED, "tile_waves %d (8 only)", o.tile_waves);
  if (W < 1 || W > kMaxW) return fail(SGT_EINVAL, "W = %d outside [1, %d]", W, kMaxW);
  if (E < 1 || E > 256 || topk < 1 || topk > E) return fail(SGT_EINVAL, "need 1 <= topk <= E <= 256 (E=%d topk=%d)", E, topk);
  if (T < 1 || I < 8 || H < 8 || I % 8 || H % 8 || T % W || (T / W) % 128)
    return fail(SGT_EINVAL, "bad shape T=%lld I=%lld H=%lld W=%d (I, H multiples of 8; T/W a multiple of 128)",
                (long long)T, (long long)I, (long long)H, W);
  const int64_t rows = T * topk;
  const int64_t lim = (int64_t)1 << 31;
  if (rows * H * 4 >= lim || T * H * 4 >= lim || (int64_t)256 * I * 2 >= lim || (int64_t)256 * H * 4 >= lim ||
      (o.b_layout == SGT_KN && I * H * 2 >= lim))
    return fail(SGT_EUNSUPPORTED, "rows x H or one expert's I x H too large for 32-bit offsets");
  if (!Hg || !W2 || !gate || !topk_ids || !expert_off || !row_token || !Y || !partial_out || !C_shard || !gflags ||
      !pflags || !partials)
    return fail(SGT_EINVAL, "NULL pointer argument");
  if (!aligned16(Hg) || !aligned16(W2) || !aligned16(Y) || !aligned16(partial_out) || !aligned16(C_shard) ||
      !aligned16(gflags) || !aligned16(pflags) || (reinterpret_cast<uintptr_t>(gate) & 3u) ||
      (reinterpret_cast<uintptr_t>(topk_ids) & 3u) || (reinterpret_cast<uintptr_t>(expert_off) & 3u) ||
      (reinterpret_cast<uintptr_t>(row_token) & 3u))
    return fail(SGT_EINVAL, "pointer not aligned (16 bytes for matrices and flags, 4 for tables)");
  for (int p = 0; p < W; ++p) {
    if (p == o.rank) continue;
    if (!partials[p] || !aligned16(partials[p]))
      return fail(SGT_EINVAL, "%s[%d] NULL or not 16-byte aligned", paced ? "inbox" : "partials", p);
    if (paced && (!peer_blocks[p] || !aligned16(peer_blocks[p])))
      return fail(SGT_EINVAL, "peer_blocks[%d] NULL or not 16-byte aligned", p);
  }
  const int64_t band_bytes = (int64_t)128 * H * 4;
  if (paced && ((int64_t)(W - 1) * ((T / W) / 128) > kItemsCap || (H + 127) / 128 > 65535))
    return fail(SGT_EUNSUPPORTED, "too many bands for the producer");
  int64_t ng = 0, np = 0;
  sgt_opts o128 = o;
  o128.rs_tile = 128;
  if ((st = sgt_rs_flag_count(W, T, H, &o128, &ng, &np)) != SGT_OK) return st;

  std::lock_guard<std::mutex> lock(ctx->mu);
  DeviceGuard g(ctx->device);
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  const int64_t tiles_n = (H + kBNmoe() - 1) / kBNmoe();
  const int64_t max_tiles = (rows + 255) / 256 + E;
  if (ctx->mrs_rowof_cap < rows || ctx->mrs_tiles_cap < max_tiles || ctx->mrs_ctr_cap < tiles_n + 4) {
    // grow the tables after draining the device (no call of this context is in flight then)
    HIP_TRY(hipDeviceSynchronize());
    if (ctx->mrs_rowof_cap < rows) {
      if (ctx->d_mrs_rowof) (void)hipFree(ctx->d_mrs_rowof);
      ctx->d_mrs_rowof = nullptr;
      ctx->mrs_rowof_cap = 0;
      const int64_t cap = std::max<int64_t>(rows, 1 << 16);
      HIP_TRY(hipMalloc(&ctx->d_mrs_rowof, cap * sizeof(int32_t)));
      HIP_TRY(hipMemset(ctx->d_mrs_rowof, 0, cap * sizeof(int32_t)));
      ctx->mrs_rowof_cap = cap;
    }
    if (ctx->mrs_tiles_cap < max_tiles) {
      if (ctx->d_mrs_tiles) (void)hipFree(ctx->d_mrs_tiles);
      ctx->d_mrs_tiles = nullptr;
      ctx->mrs_tiles_cap = 0;
      const int64_t cap = std::max<int64_t>(max_tiles, 1024);
      HIP_TRY(hipMalloc(&ctx->d_mrs_tiles, cap * sizeof(MoeTile)));
      ctx->mrs_tiles_cap = cap;
    }
    if (ctx->mrs_ctr_cap < tiles_n + 4) {
      if (ctx->d_mrs_ctr) (void)hipFree(ctx->d_mrs_ctr);
      ctx->d_mrs_ctr = nullptr;
      ctx->mrs_ctr_cap = 0;
      const int64_t cap = std::max<int64_t>(tiles_n + 4, 256);
      HIP_TRY(hipMalloc(&ctx->d_mrs_ctr, cap * sizeof(uint32_t)));
      HIP_TRY(hipMemset(ctx->d_mrs_ctr, 0, cap * sizeof(uint32_t)));
      ctx->mrs_ctr_cap = cap;
    }
  }
  const uint32_t e = ++ctx->epoch;

  RsArgs rs{};
  rs.P = partial_out; rs.C_shard = C_shard;
  for (int p = 0; p < W; ++p) rs.partials.p[p] = (p == o.rank) ? nullptr : partials[p];
  rs.gflags = gflags; rs.pflags = pflags; rs.status = ctx->d_status; rs.trace = nullptr;
  rs.M = T; rs.N = H; rs.K = I; rs.block_rows = T / W; rs.W = W; rs.rank = o.rank;
  rs.rs_tile = 128; rs.rs_tm = (int)((T / W) / 128); rs.rs_tn = (int)((H + 127) / 128);
  rs.red_split = rs_red_split(rs.rs_tile);
  rs.n_red_items = rs.rs_tm * rs.rs_tn * rs.red_split;
  rs.epoch = e; rs.timeout_ticks = timeout_ticks(o);
  rs.red_counter = ctx->d_mrs_ctr + 1;

  MoeRsArgs a{};
  a.Hg = static_cast<const uint16_t*>(Hg);
  a.W2 = static_cast<const uint16_t*>(W2);
  a.Y = Y; a.y_bf16 = y_bf16 ? 1 : 0;
  a.gate = gate; a.topk_ids = topk_ids; a.expert_off = expert_off; a.row_token = row_token;
  a.row_of = ctx->d_mrs_rowof; a.tiles = ctx->d_mrs_tiles;
  a.n_row_tiles = ctx->d_mrs_ctr; a.claim = ctx->d_mrs_ctr + 1; a.col_done = ctx->d_mrs_ctr + 4;
  a.T = T; a.I = I; a.H = H; a.rows = rows; a.E = E; a.k = topk; a.tiles_n = (int32_t)tiles_n;
  a.tiles_cap = (int32_t)ctx->mrs_tiles_cap; a.b_layout = o.b_layout;
  a.rs = rs;

  if (!paced) {
    // the peers' partials are resident: their flags take the epoch before the kernel
    HIP_TRY(launch_rs_prepare(pflags, np, e, a.claim, stream));
    const int grid = o.consumer_cus > 0 ? std::min(o.consumer_cus, ctx->n_cu) : ctx->n_cu;
    if ((st = mark(o, 0, stream)) != SGT_OK) return st;
    HIP_TRY(launch_moe_rs(a, grid, stream, end_event(ctx, o, true)));
    if ((st = mark(o, 1, stream)) != SGT_OK) return st;
    return finish(ctx, o, stream, end_event(ctx, o, true) != nullptr);
  }
  int pwg = 0;
  if ((st = launch_paced_peers(ctx, o, pflags, peer_blocks, partials, W, rs.rs_tm, rs.rs_tn, band_bytes, e, a.claim,
                               stream, &pwg, &a.rs)) != SGT_OK)
    return st;
  const bool serial = o.producer == SGT_PROD_SERIAL;
  const int avail = serial ? ctx->n_cu : consumer_beside(ctx, pwg);
  const int grid = o.consumer_cus > 0 ? std::min(o.consumer_cus, avail) : avail;
  if ((st = mark(o, 0, stream)) != SGT_OK) return st;
  const bool last = serial || a.rs.prod_done != nullptr;  // the kernel ends the call's work on this stream
  HIP_TRY(launch_moe_rs(a, grid, stream, end_event(ctx, o, last)));
  if ((st = mark(o, 1, stream)) != SGT_OK) return st;
  if (!serial && !a.rs.prod_done && (st = join_paced_peers(ctx, stream)) != SGT_OK) return st;
  return finish(ctx, o, stream, end_event(ctx, o, last) != nullptr);
}

}  // namespace

extern "C" {

sgt_status sgt_moe_gemm_rs(sgt_ctx* ctx, const void* Hg, const void* W2, const float* gate, const int32_t* topk_ids,
                           const int32_t* expert_off, const int32_t* row_token, const float* const* partials,
                           void* Y, float* partial_out, float* C_shard, uint32_t* gflags, uint32_t* pflags, int W,
                           int64_t T, int topk, int64_t I, int64_t H, int E, const sgt_opts* opts, void* stream) {
  return moe_gemm_rs_impl(ctx, Hg, W2, gate, topk_ids, expert_off, row_token, partials, nullptr, Y, partial_out,
                          C_shard, gflags, pflags, W, T, topk, I, H, E, opts, stream);
}

sgt_status sgt_moe_gemm_rs_paced(sgt_ctx* ctx, const void* Hg, const void* W2, const float* gate,
                                 const int32_t* topk_ids, const int32_t* expert_off, const int32_t* row_token,
                                 const float* const* peer_blocks, float* const* inbox, void* Y, float* partial_out,
                                 float* C_shard, uint32_t* gflags, uint32_t* pflags, int W, int64_t T, int topk,
                                 int64_t I, int64_t H, int E, const sgt_opts* opts, void* stream) {
  if (!peer_blocks || !inbox) return fail(SGT_EINVAL, "NULL peer_blocks or inbox");
  return moe_gemm_rs_impl(ctx, Hg, W2, gate, topk_ids, expert_off, row_token, inbox, peer_blocks, Y, partial_out,
                          C_shard, gflags, pflags, W, T, topk, I, H, E, opts, stream);
}

}  // extern "C"

namespace {

// Stand-alone AllGather, flag-based (ll_buf == NULL) or low-latency (LL).
// Chunks are the signal tiles of the AllGather+GEMM plan (flag_rows rows).
// Flag-based: the producer copies each chunk into the gathered buffer and
// releases its flag; the receiving side waits on the flags in arrival order.
// LL: the producer writes each remote chunk as packets into ll_buf (chunk c at
// byte 2 * c * chunk_bytes); the receiver spins on the packets and unpacks
// them into the gathered buffer, and copies the local shard itself.
sgt_status allgather_impl(sgt_ctx* ctx, const void* const* shards, void* gathered, uint32_t* flags, void* ll_buf,
                          bool ll, int W, int64_t M, int64_t K, const sgt_opts* opts, void* stream_) {
  if (!ctx) return fail(SGT_EINVAL, "ctx is NULL");
  sgt_status st = check_opts(opts, W < 1 ? 1 : W);
  if (st != SGT_OK) return st;
  const sgt_opts& o = *opts;
  if (o.producer == SGT_PROD_PRESET) return fail(SGT_EINVAL, "an AllGather needs a producer mode (CU or serial)");
  if (o.k_chunks) return fail(SGT_EUNSUPPORTED, "k_chunks applies to sgt_ag_gemm");
  AgPlan p;
  if ((st = plan_ag(W, M, K, 0, o, &p)) != SGT_OK) return st;
  const int esz = elem_bytes(o.in_dtype);
  const int64_t chunk = p.flag_rows * K * esz;
  if (chunk % 16) return fail(SGT_EINVAL, "a chunk (flag_rows x K elements = %lld bytes) must be a multiple of 16",
                              (long long)chunk);
  if (ll && 2 * chunk >= ((int64_t)1 << 31)) return fail(SGT_EUNSUPPORTED, "LL chunk of 1 GiB or more");
  if (2 * p.n_flags > kItemsCap)
    return fail(SGT_EUNSUPPORTED, "%lld chunks exceed the schedule table", (long long)p.n_flags);
  if (M > 0) {
    if (!shards) return fail(SGT_EINVAL, "shards is NULL");
    for (int q = 0; q < W; ++q)
      if (!shards[q] || !aligned16(shards[q])) return fail(SGT_EINVAL, "shards[%d] NULL or not 16-byte aligned", q);
    if (!gathered || !aligned16(gathered)) return fail(SGT_EINVAL, "gathered NULL or not 16-byte aligned");
    if (!ll && (!flags || !aligned16(flags))) return fail(SGT_EINVAL, "flags NULL or not 16-byte aligned");
    if (ll && (!ll_buf || !aligned16(ll_buf))) return fail(SGT_EINVAL, "ll_buf NULL or not 16-byte aligned");
  }
  std::lock_guard<std::mutex> lock(ctx->mu);
  DeviceGuard g(ctx->device);
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  const uint32_t e = ++ctx->epoch;
  if (M == 0) return SGT_OK;

  // One schedule table: the producer's items, then the receiver's.
  int slot;
  // The receiver's list is built in the upper half of a host buffer, the
  // producer's derived from it at the start, and the receiver's then moved
  // down behind it.
  ProdItem* tab = build_buffer(ctx, 2 * p.n_flags);
  ProdItem* recv = tab + p.n_flags;
  const int n = build_schedule(p, W, o.rank, K, esz, o, shards, gathered, recv, /*local_first=*/true);
  int n_prod = 0;
  for (int i = 0; i < n; ++i) {
    // LL: the peers write the remote chunks' packets, and the receiver reads
    // the packets (the local shard it copies itself); flag-based: the
    // producer copies every chunk and the receiver waits on each flag
    if (ll && (int)recv[i].peer == o.rank) continue;
    tab[n_prod] = recv[i];
    if (ll) {
      tab[n_prod].dst = static_cast<char*>(ll_buf) + (int64_t)recv[i].flag0 * 2 * chunk;
      recv[i].src = tab[n_prod].dst;
    }
    ++n_prod;
  }
  if (tab + n_prod != recv) std::memmove(tab + n_prod, recv, (size_t)n * sizeof(ProdItem));
  const int pwg = std::min(default_producer_wgs(o, ctx->n_cu), std::max(n_prod, 1));
  const int rgrid = std::min(n, o.consumer_cus > 0 ? o.consumer_cus : default_producer_wgs(o, ctx->n_cu));
  const uint64_t to = timeout_ticks(o);
  if ((st = stage_items(ctx, tab, n_prod + n, stream, &slot)) != SGT_OK) return st;
  const ProdItem* d = ctx->d_items[slot];
  // LL: start a chunk's writes about one write time before its release (at
  // about 24 GB/s per workgroup: 240 bytes per 10 ns tick)
  const uint64_t lead = (uint64_t)(2 * chunk / 240) + 100;
  auto launch = [&](int n_pb, int grid) -> hipError_t {
    return ll ? launch_ll_allgather(d, n_prod, n, n_pb, grid, chunk, e, o.withhold_peer, lead, o.rank, to,
                                    ctx->d_status, o.trace, stream)
              : launch_ag_allgather(flags, d, n_prod, n, n_pb, grid, chunk, e, o.withhold_peer, to, ctx->d_status,
                                    o.trace, stream);
  };
  if (o.producer == SGT_PROD_SERIAL) {
    // the peers' part first, then the receiver, one launch each
    if (n_prod > 0) HIP_TRY(launch(pwg, pwg));
    if ((st = mark(o, 0, stream)) != SGT_OK) return st;
    HIP_TRY(launch(0, rgrid));
    if ((st = mark(o, 1, stream)) != SGT_OK) return st;
  } else {
    // one launch: the peers' workgroups and the receiver's side by side (a
    // small grid, so all of it is resident at once and every wait can end)
    const int n_pb = n_prod > 0 ? pwg : 0;
    if ((st = mark(o, 0, stream)) != SGT_OK) return st;
    HIP_TRY(launch(n_pb, n_pb + rgrid));
    if ((st = mark(o, 1, stream)) != SGT_OK) return st;
  }
  HIP_TRY(hipEventRecord(ctx->slot_ev[slot], stream));
  ctx->slot_used[slot] = true;
  return finish(ctx, o, stream);
}

}  // namespace

extern "C" {

int64_t sgt_ll_buffer_bytes(int W, int64_t M, int64_t K, const sgt_opts* opts) {
  if (!opts || check_opts(opts, W < 1 ? 1 : W) != SGT_OK) return -1;
  AgPlan p;
  if (plan_ag(W, M, K, 0, *opts, &p) != SGT_OK) return -1;
  return 2 * M * K * elem_bytes(opts->in_dtype);
}

sgt_status sgt_allgather(sgt_ctx* ctx, const void* const* shards, void* gathered, uint32_t* flags, int W, int64_t M,
                         int64_t K, const sgt_opts* opts, void* stream) {
  return allgather_impl(ctx, shards, gathered, flags, nullptr, false, W, M, K, opts, stream);
}

sgt_status sgt_ll_allgather(sgt_ctx* ctx, const void* const* shards, void* ll_buf, void* gathered, int W, int64_t M,
                            int64_t K, const sgt_opts* opts, void* stream) {
  return allgather_impl(ctx, shards, gathered, nullptr, ll_buf, true, W, M, K, opts, stream);
}

}  // extern "C"


namespace {

constexpr int64_t kRingTileMax = 16384;  // elements (64 KiB of fp32)

// Tile of a ring chunk of C elements: the largest multiple of 4 dividing C,
// at most kRingTileMax (C itself when C is smaller).
int64_t ring_tile(int64_t C) {
  if (C <= kRingTileMax) return C;
  for (int64_t t = kRingTileMax; t >= 4; t -= 4)
    if (C % t == 0) return t;
  return 4;
}

sgt_status ring_plan(int W, int64_t N, int64_t* C, int64_t* tile, int64_t* T) {
  if (W < 1 || W > kMaxW) return fail(SGT_EINVAL, "W = %d outside [1, %d]", W, kMaxW);
  if (N < 0 || N % W) return fail(SGT_EINVAL, "N = %lld is not a non-negative multiple of W = %d", (long long)N, W);
  *C = N / W;
  if (*C % 4) return fail(SGT_EINVAL, "a chunk (N / W = %lld elements) must be a multiple of 4", (long long)*C);
  if (*C * 4 >= ((int64_t)1 << 31)) return fail(SGT_EUNSUPPORTED, "chunk of 2 GiB or more");
  *tile = *C > 0 ? ring_tile(*C) : 4;
  *T = *C > 0 ? *C / *tile : 0;
  if (*T * (2 * (int64_t)W - 1) > kItemsCap) return fail(SGT_EUNSUPPORTED, "%lld ring tiles exceed the schedule table",
                                                          (long long)(*T * (2 * (int64_t)W - 1)));
  return SGT_OK;
}

}  // namespace

extern "C" {

int64_t sgt_ring_flag_count(int W, int64_t N, int64_t* tile_elems) {
  int64_t C, tile, T;
  if (ring_plan(W, N, &C, &tile, &T) != SGT_OK) return -1;
  if (tile_elems) *tile_elems = tile;
  return 4 * (int64_t)(W - 1) * T;
}

sgt_status sgt_ring_allreduce(sgt_ctx* ctx, const float* x, const float* left_msgs, float* inbox, float* outbox,
                              float* out, uint32_t* flags, int W, int64_t N, const sgt_opts* opts, void* stream_) {
  if (!ctx) return fail(SGT_EINVAL, "ctx is NULL");
  sgt_status st = check_opts(opts, W < 1 ? 1 : W);
  if (st != SGT_OK) return st;
  const sgt_opts& o = *opts;
  if (o.in_dtype != SGT_F32 || o.out_dtype != SGT_F32) return fail(SGT_EUNSUPPORTED, "the ring AllReduce is fp32");
  int64_t C, tile, T;
  if ((st = ring_plan(W, N, &C, &tile, &T)) != SGT_OK) return st;
  const bool resident = o.producer == SGT_PROD_PRESET;
  if (N > 0) {
    if (!x || !out || !aligned16(x) || !aligned16(out)) return fail(SGT_EINVAL, "x or out NULL or not 16-byte aligned");
    if (W > 1) {
      if (!inbox || !outbox || !flags || !aligned16(inbox) || !aligned16(outbox) || !aligned16(flags))
        return fail(SGT_EINVAL, "inbox, outbox or flags NULL or not 16-byte aligned");
      if (!resident && (!left_msgs || !aligned16(left_msgs)))
        return fail(SGT_EINVAL, "left_msgs NULL or not 16-byte aligned (needed unless the producer is preset)");
    }
  }
  std::lock_guard<std::mutex> lock(ctx->mu);
  DeviceGuard g(ctx->device);
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  const uint32_t e = ++ctx->epoch;
  if (N == 0) return SGT_OK;

  const int64_t n_msg = 2 * (int64_t)(W - 1);
  RingArgs a{};
  a.x = x; a.inbox = inbox; a.outbox = outbox; a.out = out;
  a.in_flags = flags; a.out_flags = flags ? flags + n_msg * T : nullptr;
  a.status = ctx->d_status; a.trace = o.trace;
  a.C = C; a.W = W; a.rank = o.rank; a.T = (int32_t)T; a.tile = (int32_t)tile;
  a.epoch = e; a.timeout_ticks = timeout_ticks(o);
  const int64_t n_items = T * (2 * (int64_t)W - 1);

  if (W == 1 || resident) {
    // the left neighbour's messages are already in the inbox
    if (W > 1) HIP_TRY(launch_fill_u32(flags, n_msg * T, e, stream));
    const int grid = (int)std::min<int64_t>(n_items, o.consumer_cus > 0 ? o.consumer_cus : ctx->n_cu);
    if ((st = mark(o, 0, stream)) != SGT_OK) return st;
    HIP_TRY(launch_ring_allreduce(a, grid, stream));
    if ((st = mark(o, 1, stream)) != SGT_OK) return st;
    return finish(ctx, o, stream);
  }

  // The left neighbour's link delivers its messages in order, one tile every
  // tile_bytes / peer_gbps (plus jitter), into the inbox, each with its flag.
  ProdItem* items = build_buffer(ctx, n_msg * T);
  const double tile_bytes = (double)tile * 4.0;
  const double ticks_per_tile = o.peer_gbps > 0 ? tile_bytes / (o.peer_gbps * 1e3) * kTicksPerUs : 0.0;
  uint64_t seed = o.arrival_seed * 0x100000001B3ull + 0x5851F42D4C957F2Dull;
  const int left = (o.rank + W - 1) % W;
  const int n = (int)(n_msg * T);
  for (int i = 0; i < n; ++i) {
    ProdItem it = sched_item(i, left, (double)(i + 1) * ticks_per_tile + jitter_ticks(o, seed));
    it.src = reinterpret_cast<const char*>(left_msgs) + (int64_t)i * tile * 4;
    it.dst = reinterpret_cast<char*>(inbox) + (int64_t)i * tile * 4;
    items[i] = it;
  }
  std::stable_sort(items, items + n, [](const ProdItem& p, const ProdItem& q) { return p.release < q.release; });
  const int pwg = std::min(default_producer_wgs(o, ctx->n_cu), n);
  int slot;
  if (o.producer == SGT_PROD_SERIAL) {
    if ((st = stage_items(ctx, items, n, stream, &slot)) != SGT_OK) return st;
    HIP_TRY(launch_ag_producer(flags, ctx->d_items[slot], n, (int64_t)tile * 4, e, o.withhold_peer, nullptr, pwg,
                               stream));
    HIP_TRY(hipEventRecord(ctx->slot_ev[slot], stream));
    ctx->slot_used[slot] = true;
    const int grid = (int)std::min<int64_t>(n_items, o.consumer_cus > 0 ? o.consumer_cus : ctx->n_cu);
    if ((st = mark(o, 0, stream)) != SGT_OK) return st;
    HIP_TRY(launch_ring_allreduce(a, grid, stream));
    if ((st = mark(o, 1, stream)) != SGT_OK) return st;
    return finish(ctx, o, stream);
  }
  HIP_TRY(hipEventRecord(ctx->ev_fork, stream));
  HIP_TRY(hipStreamWaitEvent(ctx->prod, ctx->ev_fork, 0));
  if ((st = stage_items(ctx, items, n, ctx->prod, &slot)) != SGT_OK) return st;
  // The ring kernel joins the producer on the GPU: each producer workgroup
  // counts itself finished and every ring workgroup waits for the call's total
  // before it exits, so no event wait sits on the caller's stream.
  uint32_t* done = n > 0 && pwg > 0 ? ctx->d_counters + kRingDoneWord : nullptr;
  HIP_TRY(launch_ag_producer(flags, ctx->d_items[slot], n, (int64_t)tile * 4, e, o.withhold_peer, nullptr, pwg,
                             ctx->prod, nullptr, nullptr, 0, 0, 0, nullptr, 0, nullptr, 0, nullptr, done));
  if (done) {  // counted once the launch has gone in
    ctx->ring_prod_done += (uint32_t)pwg;
    a.prod_done = done;
    a.prod_done_all = ctx->ring_prod_done;
  }
  HIP_TRY(hipEventRecord(ctx->slot_ev[slot], ctx->prod));
  ctx->slot_used[slot] = true;
  // the ring's workgroups take the CUs the producer leaves, so every wait can end
  const int grid = (int)std::min<int64_t>(n_items, std::min(o.consumer_cus > 0 ? o.consumer_cus : ctx->n_cu,
                                                            consumer_beside(ctx, pwg)));
  if ((st = mark(o, 0, stream)) != SGT_OK) return st;
  HIP_TRY(launch_ring_allreduce(a, grid, stream));
  if ((st = mark(o, 1, stream)) != SGT_OK) return st;
  if (!done) {
    HIP_TRY(hipEventRecord(ctx->ev_join, ctx->prod));
    HIP_TRY(hipStreamWaitEvent(stream, ctx->ev_join, 0));
  }
  return finish(ctx, o, stream);
}

}  // extern "C"


namespace {

constexpr int kA2aDefaultChunkRows = 32;

bool aligned_to(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Shape checks shared by the AllToAll calls; chunk rows and chunks per block.
sgt_status a2a_plan(int W, int64_t T_r, int E, int k, const sgt_opts& o, int* cr, int64_t* nch) {
  if (W < 1 || W > kMaxW) return fail(SGT_EINVAL, "W = %d outside [1, %d]", W, kMaxW);
  if (E < 1 || E > kA2aMaxE || E % W) return fail(SGT_EINVAL, "E = %d: must be a multiple of W = %d in [1, %d]", E, W,
                                                  kA2aMaxE);
  if (k < 1 || k > 64) return fail(SGT_EINVAL, "k = %d outside [1, 64]", k);
  if (T_r < 0) return fail(SGT_EINVAL, "negative token count");
  if (T_r * k * 4 >= ((int64_t)1 << 31)) return fail(SGT_EUNSUPPORTED, "a routing table of 2 GiB or more");
  *cr = o.flag_rows > 0 ? o.flag_rows : kA2aDefaultChunkRows;
  if (*cr > kA2aMaxChunkRows) return fail(SGT_EINVAL, "chunk rows %d above %d", *cr, kA2aMaxChunkRows);
  *nch = (T_r + *cr - 1) / *cr;
  if ((int64_t)E * *nch > ((int64_t)1 << 30)) return fail(SGT_EUNSUPPORTED, "%lld chunks", (long long)(E * *nch));
  return SGT_OK;
}

sgt_status a2a_rows_ok(int64_t T_r, int64_t H, int esz) {
  if (H < 0) return fail(SGT_EINVAL, "negative H");
  if ((H * esz) % 16) return fail(SGT_EINVAL, "a row (H = %lld elements) must be a multiple of 16 bytes", (long long)H);
  if (T_r * H * esz >= ((int64_t)1 << 31)) return fail(SGT_EUNSUPPORTED, "a block of T_r rows is 2 GiB or more");
  return SGT_OK;
}

A2aArgs a2a_args(sgt_ctx* ctx, const sgt_opts& o, int W, int64_t T_r, int64_t row_bytes, int E, int k, int cr,
                 int64_t nch, int mode, uint32_t* flags, uint32_t e) {
  A2aArgs a{};
  a.counts = ctx->d_a2a_counts;
  a.flags = flags;
  a.status = ctx->d_status;
  a.T_r = T_r; a.row_bytes = row_bytes;
  a.W = W; a.E = E; a.E_l = E / W; a.k = k; a.rank = o.rank; a.chunk_rows = cr; a.n_chunks = (int32_t)nch;
  a.mode = mode;
  a.n_send = (int32_t)(E * nch);
  a.withhold = o.withhold_peer;
  a.epoch = e;
  // 100 MHz ticks per row on a link of peer_gbps GB/s (= peer_gbps * 1e3 bytes per microsecond)
  a.ticks_per_row = o.peer_gbps > 0 ? (double)row_bytes / (o.peer_gbps * 1e3) * kTicksPerUs : 0.0;
  a.timeout_ticks = timeout_ticks(o);
  return a;
}

// The slowest link's last release (all of a link's blocks full) must come
// within the call's time budget, so no sender workgroup waits longer than it.
sgt_status a2a_pacing_ok(const A2aArgs& a) {
  const double last = (double)a.E_l * (double)a.T_r * a.ticks_per_row;
  if (last > (double)a.timeout_ticks)
    return fail(SGT_EINVAL, "links of %.3g GB/s need up to %.0f us, beyond the %.0f us timeout",
                a.ticks_per_row > 0 ? (double)a.row_bytes / a.ticks_per_row * kTicksPerUs / 1e3 : 0.0,
                last / kTicksPerUs, (double)a.timeout_ticks / kTicksPerUs);
  return SGT_OK;
}

}  // namespace

extern "C" {

int64_t sgt_a2a_flag_count(int W, int64_t T_r, int E, const sgt_opts* opts) {
  if (!opts || check_opts(opts, W < 1 ? 1 : W) != SGT_OK) return -1;
  int cr;
  int64_t nch;
  if (a2a_plan(W, T_r, E, 1, *opts, &cr, &nch) != SGT_OK) return -1;
  return (int64_t)E * nch;
}

sgt_status sgt_a2a_dispatch(sgt_ctx* ctx, const void* const* X, const int32_t* const* topk, void* recv,
                            int32_t* recv_token, uint64_t* recv_count, uint32_t* flags, int W, int64_t T_r, int64_t H,
                            int E, int k, const sgt_opts* opts, void* stream_) {
  if (!ctx) return fail(SGT_EINVAL, "ctx is NULL");
  sgt_status st = check_opts(opts, W < 1 ? 1 : W);
  if (st != SGT_OK) return st;
  const sgt_opts& o = *opts;
  if (o.producer == SGT_PROD_PRESET) return fail(SGT_EINVAL, "a dispatch needs a producer mode (CU or serial)");
  int cr;
  int64_t nch;
  if ((st = a2a_plan(W, T_r, E, k, o, &cr, &nch)) != SGT_OK) return st;
  const int esz = elem_bytes(o.in_dtype);
  if ((st = a2a_rows_ok(T_r, H, esz)) != SGT_OK) return st;
  if (!recv_count || !aligned_to(recv_count, 8)) return fail(SGT_EINVAL, "recv_count NULL or misaligned");
  if (T_r > 0) {
    if (!topk) return fail(SGT_EINVAL, "topk is NULL");
    for (int p = 0; p < W; ++p)
      if (!topk[p] || !aligned_to(topk[p], 4)) return fail(SGT_EINVAL, "topk[%d] NULL or misaligned", p);
    if (!X) return fail(SGT_EINVAL, "X is NULL");
    for (int p = 0; p < W; ++p)
      if (!X[p] || !aligned16(X[p])) return fail(SGT_EINVAL, "X[%d] NULL or not 16-byte aligned", p);
    if (!recv || !aligned16(recv)) return fail(SGT_EINVAL, "recv NULL or not 16-byte aligned");
    if (!recv_token || !aligned_to(recv_token, 4)) return fail(SGT_EINVAL, "recv_token NULL or misaligned");
    if (!flags || !aligned_to(flags, 4)) return fail(SGT_EINVAL, "flags NULL or misaligned");
  }
  std::lock_guard<std::mutex> lock(ctx->mu);
  DeviceGuard g(ctx->device);
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  A2aArgs a = a2a_args(ctx, o, W, T_r, H * esz, E, k, cr, nch, 0, flags, 0);
  if ((st = a2a_pacing_ok(a)) != SGT_OK) return st;  // rejected before the epoch advances
  const uint32_t e = ++ctx->epoch;
  a.epoch = e;
  for (int p = 0; p < W; ++p) {
    a.src.p[p] = X ? X[p] : nullptr;
    a.table.p[p] = topk ? topk[p] : nullptr;  // not read when T_r = 0
  }
  a.dst = static_cast<char*>(recv);
  a.lists = recv_token;
  a.count_sig = recv_count;
  // up to 64 local experts each sender scans its source's table itself (one launch); beyond, a scan
  // kernel writes the token lists and counts first (it also stores the count packets of T_r = 0)
  a.fused_scan = (a.E_l <= kA2aMaxFusedLocal && a.n_send > 0) ? 1 : 0;
  if ((st = mark(o, 0, stream)) != SGT_OK) return st;
  if (!a.fused_scan) HIP_TRY(launch_a2a_scan(a, stream));
  hipEvent_t done = end_event(ctx, o, a.n_send > 0);  // the senders' launch ends the call's work
  if (a.n_send > 0) HIP_TRY(launch_a2a(a, 0, stream, done));
  if ((st = mark(o, 1, stream)) != SGT_OK) return st;
  return finish(ctx, o, stream, done != nullptr);
}

sgt_status sgt_a2a_combine(sgt_ctx* ctx, const void* const* back, const int32_t* topk, const float* gate, void* cbuf,
                           int32_t* slot_of, float* out, uint32_t* flags, int W, int64_t T_r, int64_t H, int E, int k,
                           const sgt_opts* opts, void* stream_) {
  if (!ctx) return fail(SGT_EINVAL, "ctx is NULL");
  sgt_status st = check_opts(opts, W < 1 ? 1 : W);
  if (st != SGT_OK) return st;
  const sgt_opts& o = *opts;
  if (o.in_dtype != SGT_BF16 || o.out_dtype != SGT_F32)
    return fail(SGT_EUNSUPPORTED, "the combine takes bf16 expert outputs and writes fp32");
  int cr;
  int64_t nch;
  if ((st = a2a_plan(W, T_r, E, k, o, &cr, &nch)) != SGT_OK) return st;
  if ((st = a2a_rows_ok(T_r, H, 2)) != SGT_OK) return st;
  const bool preset = o.producer == SGT_PROD_PRESET;
  if (T_r > 0) {
    if (!topk || !gate || !slot_of || !aligned_to(topk, 4) || !aligned_to(gate, 4) || !aligned_to(slot_of, 4))
      return fail(SGT_EINVAL, "topk, gate or slot_of NULL or misaligned");
    if (!preset) {
      if (!back) return fail(SGT_EINVAL, "back is NULL");
      for (int q = 0; q < W; ++q)
        if (!back[q] || !aligned16(back[q])) return fail(SGT_EINVAL, "back[%d] NULL or not 16-byte aligned", q);
    }
    if (!cbuf || !out || !aligned16(cbuf) || !aligned16(out)) return fail(SGT_EINVAL, "cbuf or out NULL or misaligned");
    if (!flags || !aligned_to(flags, 4)) return fail(SGT_EINVAL, "flags NULL or misaligned");
  }
  std::lock_guard<std::mutex> lock(ctx->mu);
  DeviceGuard g(ctx->device);
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  A2aArgs a = a2a_args(ctx, o, W, T_r, H * 2, E, k, cr, nch, 1, flags, 0);
  if ((st = a2a_pacing_ok(a)) != SGT_OK) return st;  // rejected before the epoch advances
  const uint32_t e = ++ctx->epoch;
  a.epoch = e;
  if (T_r == 0) return finish(ctx, o, stream);
  for (int q = 0; q < W; ++q) a.src.p[q] = back && !preset ? back[q] : nullptr;
  a.table.p[0] = topk;
  a.dst = static_cast<char*>(cbuf);
  a.lists = slot_of;
  a.gate = gate;
  a.out = out;
  const int rgrid = (int)std::max<int64_t>(1, o.consumer_cus > 0 ? o.consumer_cus
                                                                 : std::min<int64_t>((T_r + 3) / 4, ctx->n_cu / 2));
  if ((st = mark(o, 0, stream)) != SGT_OK) return st;
  HIP_TRY(launch_a2a_scan(a, stream));
  hipEvent_t done = end_event(ctx, o, true);  // the receiver's launch (the last) ends the call's work
  if (preset) {
    // the expert outputs are already in cbuf: every chunk flag set, then the receiver alone
    HIP_TRY(launch_fill_u32(flags, E * nch, e, stream));
    A2aArgs r = a;
    r.n_send = 0;
    HIP_TRY(launch_a2a(r, rgrid, stream, done));
  } else if (o.producer == SGT_PROD_SERIAL) {
    HIP_TRY(launch_a2a(a, 0, stream));
    A2aArgs r = a;
    r.n_send = 0;
    HIP_TRY(launch_a2a(r, rgrid, stream, done));
  } else {
    HIP_TRY(launch_a2a(a, rgrid, stream, done));
  }
  if ((st = mark(o, 1, stream)) != SGT_OK) return st;
  return finish(ctx, o, stream, done != nullptr);
}

}  // extern "C"
