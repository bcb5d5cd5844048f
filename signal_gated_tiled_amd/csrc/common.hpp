// Internal types shared by the host runtime and the kernels of libsgt.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sgt {

constexpr int kMaxW = 64;
constexpr int kXcds = 8;             // XCDs of the device; workgroup b of a grid runs on XCD b % kXcds
constexpr int kXcdClaimStride = 16;  // words between per-XCD claim counters

// Device status word written by a kernel whose bounded wait expired.
// status[0] = code (0 ok, 3 timeout), [1] = flag index, [2] = value seen, [3] = value expected.
constexpr uint32_t kStatusTimeout = 3;

struct PtrTable {
  const void* p[kMaxW];
};

// One producer work item: copy tile_bytes from `src` (in peer `peer`'s
// buffer) to `dst`, then release flags [flag0, flag0 + nflags) no earlier than
// `release` clock ticks after the producer workgroup started.  An AllGather
// signal tile releases its one flag; a GEMM+ReduceScatter band of a peer's
// partial block releases the flags of every tile in the band.
struct ProdItem {
  const char* src;
  char* dst;
  uint64_t release;
  uint32_t flag0;
  uint16_t nflags;
  uint16_t peer;
};

// One release of the copy-engine producer: once the copy engine has written
// the bytes of copy unit `mark` (marks[mark] holds the call's epoch), and no
// earlier than `release` ticks after the releaser started, flags [flag0,
// flag0 + nflags) take the epoch.  Items are in release order.
struct RelItem {
  uint64_t release;
  uint32_t flag0;
  uint32_t nflags;
  uint32_t mark;
  uint32_t peer;
};

// Arguments of the AllGather consumer (both the bf16 MFMA and fp32 kernels).
struct AgArgs {
  const void* A;          // gathered M x K
  const void* A_local;    // this rank's shard: rows [rank * rows_per_shard, +rows_per_shard) of A
  const void* B;          // K x N or N x K
  void* C;                // M x N
  const uint32_t* flags;  // one per signal tile
  uint32_t* status;
  uint64_t* trace;        // optional: 4 words per consumer tile
  int64_t M, N, K;
  int64_t rows_per_shard;
  int32_t flag_rows;
  int32_t n_kc, kc_cols;  // K-chunked signal tiles: n_kc chunks of kc_cols columns per panel (0: whole rows)
  int32_t W, rank, order;
  int32_t tiles_m, tiles_n;
  int32_t b_layout, out_dtype;
  uint32_t epoch;
  int32_t tile_waves;     // 4 or 8 wave64s per bf16 workgroup
  uint64_t timeout_ticks;
  // bf16 tiles claimed dynamically (xcd_claim != null): the tiles the static
  // schedule of a base_grid-workgroup grid gives XCD x are claimed in that
  // order from counter xcd_claim[x * kXcdClaimStride], then the other XCDs'
  // lists; the last late_blocks workgroups run only if every producer
  // workgroup already runs (*started == started_all), else they exit at once.
  uint32_t* xcd_claim;
  uint32_t* xcd_claim_next;   // the other counter set: zeroed by workgroup 0 at the start, for the next launch
  int32_t base_grid;
  int32_t late_blocks;
  const uint32_t* started;
  uint32_t started_all;
  // overlapped call (prod_done != null): before it exits, each workgroup that
  // took work waits until the producer workgroups finished so far (cumulative)
  // reach prod_done_all, so the caller's stream is ordered after the whole
  // AllGather without a cross-stream event wait
  const uint32_t* prod_done;
  uint32_t prod_done_all;
};

// Arguments of the GEMM+ReduceScatter kernel.
struct RsArgs {
  const void* A;            // A_local M x K
  const void* B;            // K x N or N x K
  float* P;                 // partial_out M x N fp32
  float* C_shard;           // (M/W) x N
  PtrTable partials;        // W pointers, (M/W) x N fp32
  uint32_t* gflags;         // per rs_tile^2 tile of P
  const uint32_t* pflags;   // W x tiles of one block
  uint32_t* status;
  uint64_t* trace;          // optional: {start, end, workgroup} per work item
  uint32_t* red_counter;    // next reduction item to claim; zeroed before the launch
  int64_t M, N, K;
  int64_t block_rows;       // M / W
  int32_t W, rank;
  int32_t tiles_m, tiles_n; // GEMM tiles
  int32_t rs_tile;          // signal tile edge
  int32_t rs_tm, rs_tn;     // signal tiles of one block (rows, cols)
  int32_t b_layout;
  int32_t n_gemm_tiles, n_red_items;
  int32_t red_split;        // reduction items per signal tile: row bands of rs_tile / red_split rows
  uint32_t epoch;
  int32_t tile_waves;
  uint64_t timeout_ticks;
  const uint32_t* prod_done;  // paced peers: the producer's finished count to wait for before exit, or null
  uint32_t prod_done_all;
};

// One grouped row tile: rows [r0, r0 + rows) of expert e's group (rows at
// most the tile height; the tile ends at the group's end or earlier).
struct MoeTile {
  int32_t expert;
  int32_t r0;       // first row (index into the grouped rows of Y)
  int32_t rows;
};

// MoE GEMM + ReduceScatter (the combine side).  `rs` carries the
// ReduceScatter part exactly as the dense GEMM+ReduceScatter uses it (P is
// the combined partial, M = T tokens, N = H).
struct MoeRsArgs {
  const uint16_t* Hg;        // rows x I bf16, grouped rows
  const uint16_t* W2;        // E x I x H (KN) or E x H x I (NK) bf16
  void* Y;                   // rows x H fp32 (or bf16): each grouped row times its expert's weight
  const float* gate;         // T x k
  const int32_t* topk_ids;   // T x k
  const int32_t* expert_off; // E + 1
  const int32_t* row_token;  // rows
  int32_t* row_of;           // T x k: grouped row of pick (t, j) (prologue)
  MoeTile* tiles;            // 256-row tiles of the expert groups (prologue)
  uint32_t* n_row_tiles;     // (prologue)
  uint32_t* col_done;        // per 256-column GEMM tile: row tiles stored (cleared by the prologue)
  uint32_t* claim;           // combine / reduction claim counter (cleared by the prologue)
  int64_t T, I, H, rows;
  int32_t E, k, tiles_n, tiles_cap;
  int32_t b_layout;
  int32_t y_bf16;            // Y stored as bf16 (RNE) instead of fp32
  RsArgs rs;
};

// XCD-partitioned work lists of the MoE grouped consumer.  The row tiles, in
// expert-major order, are cut into chunks of kMoeXcdGroup consecutive tiles;
// chunk c goes to the list of XCD c % kXcds (the XCD that runs workgroups
// b with b % kXcds == c % kXcds), in order.  So every XCD gets an even share of
// the list, and the tiles it runs together (the column tiles of one row tile,
// neighbouring row tiles of one expert) share operands in its L2.
constexpr uint32_t kMoeXcdGroup = 4;

// Row tiles in XCD x's list, for n tiles in total.
__host__ __device__ inline uint32_t xcd_list_len(uint32_t n, int x) {
  const uint32_t G = kMoeXcdGroup, nf = n / G, r = n % G;
  uint32_t len = G * (nf / kXcds + ((uint32_t)x < nf % kXcds ? 1u : 0u));
  if (r && nf % kXcds == (uint32_t)x) len += r;
  return len;
}

// First entry of XCD x's list.
__host__ __device__ inline uint32_t xcd_list_start(uint32_t n, int x) {
  uint32_t s = 0;
  for (int y = 0; y < x; ++y) s += xcd_list_len(n, y);
  return s;
}

// Entry of the partitioned list that holds the row tile at sorted position p.
__host__ __device__ inline uint32_t xcd_list_pos(uint32_t p, uint32_t n) {
  const uint32_t G = kMoeXcdGroup, c = p / G;
  const int x = (int)(c % kXcds);
  return xcd_list_start(n, x) + (c / kXcds) * G + p % G;
}

// Routing and work-list tables of one MoE call (device memory owned by the context).
struct MoeTables {
  uint32_t* masks;        // ceil(E / 32) x T: bit e % 32 of word e / 32 set when token t chose e
  uint32_t* counts;       // E: tokens routed to each expert (zero on entry: cleared by the previous call)
  uint32_t* counts_next;  // E: the next call's counts, cleared by this call's top-k kernel
  int32_t n_groups;       // workgroups of the top-k kernel (tokens_per_group tokens each, the last ragged)
  int32_t tokens_per_group;
  uint32_t* n_tiles;      // 1: number of grouped row tiles
  uint32_t tiles_cap;     // entries of order
  uint32_t* xcd_claim;    // kXcds counters, kXcdClaimStride words apart: next item of each XCD's list
  MoeTile* order;         // the row tiles, expert-major, in the XCD-partitioned lists (xcd_list_pos)
};

// Arguments of the MoE grouped consumer.
struct MoeArgs {
  const uint16_t* X;          // gathered tokens, T x H bf16
  const uint16_t* We;         // experts' weights, E x H x I (KN) or E x I x H (NK)
  void* Y;                    // grouped rows x I
  const int32_t* row_token;   // token of each grouped row
  const int32_t* expert_off;  // E + 1
  const MoeTile* order;
  const uint32_t* n_tiles;
  uint32_t tiles_cap;         // entries of `order`
  uint32_t* xcd_claim;        // per-XCD claim counters (MoeTables::xcd_claim)
  const uint32_t* flags;      // one per signal tile of X
  uint32_t* status;
  uint64_t* trace;            // optional: 4 words per work item in claim order
  int64_t T, H, I;
  int64_t rows;               // T * topk: rows of Y and row_token
  const uint32_t* started;    // producer workgroups started so far (cumulative over calls), or null
  uint32_t started_all;       // its value once every producer workgroup of this call runs
  int32_t late_blocks;        // the last late_blocks workgroups run only when started == started_all
  const uint32_t* prod_done;  // as in AgArgs: the producer's finished count to wait for before exit, or null
  uint32_t prod_done_all;
  int32_t E, flag_rows, tiles_n;
  uint32_t epoch;
  uint64_t timeout_ticks;
};

}  // namespace sgt
