// Consumer tile scheduling shared by the host query (sgt_panel_order) and the
// persistent kernels, so the order the tests check is the order the kernels run.
//
// Panel = consumer M-tile of `bm` rows.  Two orders:
//  * SGT_ORDER_SHARD: the threadblock swizzle of the Triton-distributed
//    semantics page ("Threadblock swizzle"): the m-tile index is shifted by the
//    first m-tile of the local shard modulo the number of m-tiles, so a rank
//    starts on data it already holds and then walks whole shards in rank order.
//  * SGT_ORDER_MESH: the AMD full-mesh variant of the paper summary ("Method":
//    on a full mesh every rank gathers from all peers at once): after the local
//    shard, panel j of shards rank+1, rank+2, ..., rank+W-1, then panel j+1, ...
//    so the consumer follows the order in which concurrent links deliver.
//    Needs whole panels per shard; otherwise it falls back to the shard order.
#pragma once

#include <stdint.h>

namespace sgt {

__host__ __device__ inline int64_t panel_at(int64_t i, int64_t tiles_m, int64_t rows_per_shard, int64_t bm, int W,
                                            int rank, int order) {
  if (order == 0 && W > 1 && rows_per_shard % bm == 0) {
    const int64_t pps = rows_per_shard / bm;
    if (i < pps) return (int64_t)rank * pps + i;
    const int64_t j = i - pps;
    const int64_t peer = 1 + j % (W - 1), pj = j / (W - 1);
    return ((rank + peer) % W) * pps + pj;
  }
  const int64_t first = ((int64_t)rank * rows_per_shard) / bm;
  return (i + first) % tiles_m;
}

// Tile t of the consumer's sequence: panels are taken in groups of four (in
// panel order) and, inside a group, column tile by column tile, so the 32 or
// so consecutive tiles one XCD runs in a round share 4 A panels and about 8
// column tiles of B in its L2 (instead of 2 panels and every column tile).
constexpr int kPanelGroup = 4;

__host__ __device__ inline void tile_at(int64_t t, int64_t tiles_m, int64_t tiles_n, int64_t* seq_m, int64_t* pn) {
  const int64_t grp = t / (kPanelGroup * tiles_n);
  const int64_t gm = tiles_m - grp * kPanelGroup < kPanelGroup ? tiles_m - grp * kPanelGroup : kPanelGroup;
  const int64_t idx = t - grp * kPanelGroup * tiles_n;
  *pn = idx / gm;
  *seq_m = grp * kPanelGroup + idx % gm;
}

// Dynamic claiming in the static schedule's XCD order: with a grid of G
// workgroups (G % 8 == 0), XCD x runs, round after round, the G / 8
// consecutive tiles [r G + x G / 8, r G + (x + 1) G / 8).  xcd_seq_tile gives
// the i-th of them (or -1 past the last of `total` tiles).
__host__ __device__ inline int64_t xcd_seq_tile(int x, int64_t i, int64_t G, int64_t total) {
  const int64_t per = G / 8;
  const int64_t t = (i / per) * G + (int64_t)x * per + i % per;
  return t < total ? t : -1;
}

// Workgroup b of a persistent grid of G workgroups is dispatched to XCD b % 8.
// Renumber so that the workgroups sharing an XCD take consecutive tiles of each
// round (tiles sharing an A panel then hit the same XCD-private L2).
__host__ __device__ inline int xcd_remap(int b, int G) {
  if (G % 8) return b;
  return (b % 8) * (G / 8) + b / 8;
}

}  // namespace sgt
