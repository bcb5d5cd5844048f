// Arguments of the expert-parallel AllToAll kernels (one rank's share),
// shared by the host runtime and the kernels.
#pragma once

#include <stdint.h>

#include "common.hpp"

namespace sgt {

constexpr int kA2aMaxE = 4096;        // experts (size of the context's count table)
constexpr int kA2aMaxChunkRows = 1024;
constexpr int kA2aMaxFusedLocal = 64;  // local experts a dispatch sender's own scan covers (one 64-bit mask)

// Block b of a call is one (link, expert) pair: the rows one link carries for
// one expert.  Dispatch: b = l * W + p (local expert l, source rank p; the
// link is p).  Combine: b = e = q * E_l + l (expert e of owner q; the link is
// q).  Chunk c of block b covers rows [c * chunk_rows, ...) of the block and
// has flag b * n_chunks + c.
struct A2aArgs {
  PtrTable src;           // dispatch: X[p] (T_r rows); combine: back[q] (E_l x T_r rows)
  PtrTable table;         // dispatch: topk of source p (T_r x k); combine: [0] = this rank's topk
  char* dst;              // dispatch: recv (E_l x W x T_r rows); combine: cbuf (E x T_r rows)
  int32_t* lists;         // dispatch: recv_token (E_l x W x T_r); combine: slot_of (T_r x k)
  uint64_t* count_sig;    // dispatch: E_l x W packets (epoch << 32 | count); combine: null
  int32_t* counts;        // E: rows of each block (context table, written by the scan)
  uint32_t* flags;        // E x n_chunks
  const float* gate;      // combine: T_r x k
  float* out;             // combine: T_r x H
  uint32_t* status;
  int64_t T_r, row_bytes;
  int32_t W, E, E_l, k, rank, chunk_rows, n_chunks, mode;  // mode 0 dispatch, 1 combine
  int32_t n_send;         // sender workgroups: E x n_chunks
  int32_t withhold;       // link whose chunk flags are never published (-1: none); a test hook
  int32_t fused_scan;     // dispatch senders scan their source's table themselves (E_l <= 64)
  uint32_t epoch;
  double ticks_per_row;   // link pacing in 100 MHz ticks per row (0: unthrottled)
  uint64_t timeout_ticks;
};

}  // namespace sgt
