// Arguments of the ring AllReduce kernel (one rank's share), shared by the
// host runtime and the kernel.
#pragma once

#include <stdint.h>

namespace sgt {

struct RingArgs {
  const float* x;            // N
  const float* inbox;        // 2(W-1) x C: the left neighbour's messages land here
  float* outbox;             // 2(W-1) x C: this rank's messages to its right neighbour
  float* out;                // N: the sum
  const uint32_t* in_flags;  // 2(W-1) x T
  uint32_t* out_flags;       // 2(W-1) x T
  uint32_t* status;
  uint64_t* trace;           // optional: {wait start, seen, end} per item
  int64_t C;                 // elements per chunk (N / W)
  int32_t W, rank, T, tile;  // T tiles of `tile` elements (a multiple of 4) per chunk
  uint32_t epoch;
  uint64_t timeout_ticks;
  const uint32_t* prod_done;  // the producer's finished count to wait for before exit (overlapped), or null
  uint32_t prod_done_all;
};

}  // namespace sgt
