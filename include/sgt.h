/*
 * sgt.h -- C ABI of libsgt, the signal-gated tiled AllGather+GEMM and
 * GEMM+ReduceScatter library for AMD Instinct MI355X (gfx950).
 *
 * The operations follow the Triton-distributed pages:
 *   - "Triton-distributed semantics" (triton-distributed-ascend docs), sections
 *     "Producer-consumer model", "Signal-based synchronization", "AllGather + GEMM
 *     overlap", "GEMM + ReduceScatter overlap", "Threadblock swizzle",
 *     "Token-based data dependency", "Best practices";
 *   - the Triton-distributed paper summary (hyper.ai, arXiv 2504.19442), section
 *     "Method": copy-engine/producer AllGather, push-mode intra-node ReduceScatter,
 *     the AMD full-mesh swizzle and resource partitioning, AMD persistent kernels.
 *
 * One GPU holds one rank's share of a tensor-parallel layer.  The W peers'
 * shards ("symmetric memory" on the pages) are device buffers on that same GPU;
 * a producer moves them tile by tile into the gathered buffer at a simulated
 * per-peer link rate and sets one flag per tile; a persistent HIP consumer
 * waits on each tile's flag before reading it.
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers owned by the caller; arrays of
 *     pointers (A_shards, partials, X_shards) are HOST arrays of W device
 *     pointers.  Matrices are row-major and densely packed.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream) unless opts->blocking is set.  The library allocates no device
 *     memory per call: it owns only a few streams, events, a device status
 *     word and small schedule tables created with the context (the MoE calls'
 *     tables grow on demand).
 *   - Arguments are validated before anything is launched; a bad argument
 *     returns SGT_EINVAL (or SGT_EUNSUPPORTED) and launches nothing.
 *     sgt_last_error() then describes the problem.
 *   - Flags: uint32 words zeroed once by the caller before first use.  Each
 *     call takes the next epoch e of its context (1, 2, ...); a flag is "set"
 *     for this call when (int32_t)(flag - e) >= 0.  On return every flag the
 *     call owns equals e, so flags are reused across calls without a reset.
 *     Buffers shared by two contexts would need distinct epochs: use one
 *     context per buffer set.
 *   - Every wait inside a kernel is bounded by opts->timeout_ms; on expiry the
 *     kernel records {SGT_ETIMEDOUT, flag index, value seen, value expected} in
 *     the context's device status word and exits.  The error is returned by
 *     sgt_sync() or by a blocking call.  No call can hang the GPU.
 *   - Two calls that overlap in time on one context (different streams) are
 *     not supported; calls on one stream are ordered.
 */
#ifndef SGT_H_
#define SGT_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define SGT_API __attribute__((visibility("default")))
#else
#define SGT_API
#endif

typedef enum sgt_status {
  SGT_OK = 0,
  SGT_EINVAL = -1,        /* bad argument (shape, pointer, alignment, option) */
  SGT_EUNSUPPORTED = -2,  /* valid request the library does not implement     */
  SGT_ETIMEDOUT = -3,     /* a kernel's bounded wait on a flag expired         */
  SGT_EHIP = -4,          /* a HIP runtime call failed                          */
  SGT_ENOMEM = -5         /* context creation could not allocate               */
} sgt_status;

enum sgt_dtype { SGT_F32 = 0, SGT_BF16 = 1 };

/* Storage of the K x N right-hand matrix: row-major K x N, or row-major N x K
 * (the same matrix transposed, as a Linear layer stores its weight). */
enum sgt_layout { SGT_KN = 0, SGT_NK = 1 };

/* Who moves the peer data and sets the flags. */
enum sgt_producer {
  SGT_PROD_CU = 0,      /* producer kernel on a second stream, paced per peer        */
  SGT_PROD_PRESET = 1,  /* data already resident: flags are set up front, then the
                           consumer runs (the "GEMM alone" baseline)                */
  SGT_PROD_SERIAL = 2,  /* producer, then consumer, on one stream (debug: barrier
                           semantics instead of fine-grained signals)               */
  SGT_PROD_SDMA = 3     /* sgt_ag_gemm: the copy engines move the data, off the
                           compute units (paper summary, "Method": intra-node
                           AllGather by copy engines, communication and compute on
                           separate resources); a one-workgroup releaser publishes
                           each flag once its copy has landed and its link time has
                           come.  opts->sdma_peers > 0 sends only that many remote
                           peers (rank+1, rank+2, ...) through the copy engines and
                           the others through producer_cus CU workgroups           */
};

/* Consumer order over the row panels of the gathered matrix. */
enum sgt_order {
  SGT_ORDER_MESH = 0,   /* local shard first, then the peers' panels round-robin, as
                           every peer of a full mesh sends at once                   */
  SGT_ORDER_SHARD = 1   /* pid_m shifted by rank * tiles_per_pe: local shard first,
                           then whole shards in rank order                            */
};

typedef struct sgt_opts {
  int32_t rank;          /* this GPU's rank, 0 <= rank < W                                     */
  int32_t in_dtype;      /* SGT_BF16 (MFMA path) or SGT_F32 (FMA path)                         */
  int32_t out_dtype;     /* SGT_F32 (default) or SGT_BF16 (round to nearest even)              */
  int32_t b_layout;      /* SGT_KN or SGT_NK                                                    */
  int32_t producer;      /* enum sgt_producer                                                   */
  int32_t order;         /* enum sgt_order                                                      */
  int32_t flag_rows;     /* rows per AllGather signal tile; 0 = library default                 */
  int32_t producer_cus;  /* workgroups of the producer kernel; 0 = library default              */
  int32_t consumer_cus;  /* workgroups of the persistent consumer; 0 = one per CU.  Beside an
                            overlapped producer at most the CUs less the producer's share (its
                            workgroup count rounded up to a multiple of CUs / 8, an equal share
                            of every XCD) run unconditionally, and a caller's count is capped
                            there, so the producer can always start; with no caller count the
                            bf16 AllGather and MoE consumers launch one per CU and run the rest
                            only if every producer workgroup is already running              */
  int32_t blocking;      /* nonzero: synchronize and return the device status                   */
  double peer_gbps;      /* simulated link rate per peer in GB/s; 0 = unthrottled               */
  double jitter_us;      /* each remote tile's release is delayed by U[0, jitter_us]            */
  double timeout_ms;     /* bound on every wait; 0 = 2000 ms                                    */
  uint64_t arrival_seed; /* seed of the arrival order (if shuffled) and of the jitter           */
  int32_t withhold_peer; /* test hook: this peer's tiles are copied but never signalled (-1 off)*/
  int32_t rs_tile;       /* GEMM+RS signal tile edge (rows = cols); 0 = 128                     */
  int32_t arrival_order; /* 0: each peer sends its tiles in order; 1: a seeded order per peer;
                            2: one seeded order over all remote tiles                             */
  int32_t tile_waves;    /* bf16 consumer workgroup: 4 or 8 wave64s per tile; 0 = 8             */
  int32_t tile_rows;     /* MoE grouped tile height: 128 or 256 rows; 0 = 256 (AllGather and
                            GEMM+RS tiles are 256 x 256)                                          */
  int32_t k_chunks;      /* sgt_ag_gemm, bf16: 0 = signal tiles of flag_rows rows x all K; n (1..64) =
                            signal tiles of one 256-row consumer panel x one of n equal column
                            chunks of K (K a multiple of 128 n), so a tile whose panel is still
                            arriving computes it chunk by chunk (same bits)                      */
  int32_t sdma_peers;    /* SGT_PROD_SDMA: remote peers moved by the copy engines; 0 = all      */
  uint64_t* trace;       /* optional device buffer, see sgt_trace_words(); NULL = off           */
  void* consumer_events[2]; /* optional hipEvent_t pair recorded on the consumer's stream right
                               before and after the consumer kernel launch (NULL = off)            */
} sgt_opts;

typedef struct sgt_ctx sgt_ctx;

/* Library version string, e.g. "sgt 0.1 gfx950". */
SGT_API const char* sgt_version(void);

/* Short name of a status code. */
SGT_API const char* sgt_status_str(int status);

/* Detail of the last error on the calling thread ("" if none). */
SGT_API const char* sgt_last_error(void);

/* sizeof(sgt_opts) as this library was built (for bindings that mirror the struct). */
SGT_API size_t sgt_opts_size(void);

/* Fill *o with defaults: rank 0, bf16 in, fp32 out, K x N, CU producer, mesh
 * order, unthrottled, no jitter, 2000 ms timeout, no trace. */
SGT_API void sgt_opts_init(sgt_opts* o);

/* Create a context on HIP device `device` (streams, events, status word,
 * schedule tables).  Returns SGT_EINVAL for a bad device, SGT_EHIP/SGT_ENOMEM on
 * runtime failure.  The context must be destroyed by sgt_ctx_destroy. */
SGT_API sgt_status sgt_ctx_create(sgt_ctx** out, int device);

/* Wait for all of the context's work and free it.  NULL is accepted. */
SGT_API sgt_status sgt_ctx_destroy(sgt_ctx* ctx);

/* Wait for the context's outstanding work and return the device status
 * (SGT_ETIMEDOUT after an expired wait; the status is then cleared). */
SGT_API sgt_status sgt_sync(sgt_ctx* ctx);

/* Number of AllGather flags sgt_ag_gemm uses for these arguments (the size of
 * its `flags` array), or a negative status for invalid arguments. */
SGT_API int64_t sgt_ag_flag_count(int W, int64_t M, int64_t K, const sgt_opts* opts);

/* Rows per consumer panel (the M tile) sgt_ag_gemm uses for these arguments. */
SGT_API int32_t sgt_ag_panel_rows(int W, int64_t M, int64_t K, int64_t N, const sgt_opts* opts);

/* The order in which the persistent consumer takes the row panels: writes
 * ceil(M / panel_rows) panel indices to out (host memory).  Source: the
 * semantics page's "Threadblock swizzle" and the paper summary's AMD full-mesh
 * swizzle ("Method").  Returns the count or a negative status. */
SGT_API int64_t sgt_panel_order(int W, int rank, int64_t M, int32_t panel_rows, int order, int32_t* out, int64_t cap);

/*
 * AllGather + GEMM (semantics page, "AllGather + GEMM overlap"; paper summary,
 * "Method"):
 *     A_gathered = rows of A_shards[0], A_shards[1], ..., A_shards[W-1]
 *     C          = A_gathered * B          (C is M x N, fp32 or bf16)
 * A_shards[p]: (M/W) x K device buffer of rank p (in_dtype); A_shards[rank] is
 *     the local shard.  Shard p lands at rows [p*M/W, (p+1)*M/W) of A_gathered.
 * B: K x N (SGT_KN) or N x K (SGT_NK), in_dtype.
 * A_gathered: M x K, written by the producer (read-only for SGT_PROD_PRESET,
 *     where it must already hold the gathered rows).
 * flags: sgt_ag_flag_count() uint32 words, one per signal tile of flag_rows
 *     rows x K; zeroed once by the caller.  With opts->k_chunks = n > 0 (bf16)
 *     a signal tile is one 256-row consumer panel x one of n column chunks of
 *     K, flag pm * n + q for panel pm and chunk q; a tile whose panel has not
 *     fully arrived computes the chunks in order as they land (8-wave tiles
 *     with B stored N x K; the other tile shapes wait for the whole panel).
 *     The results are the same bits as with whole-row signal tiles.
 * Requirements: 1 <= W <= 64, M % W == 0, (M/W) % flag_rows == 0, K, N >= 1;
 *     bf16: K % 8 == 0 and N % 8 == 0; all pointers 16-byte aligned.  With
 *     k_chunks = n: K % (128 n) == 0, (M/W) % 256 == 0 and flag_rows 0 (or 256).
 * M = 0 or N = 0 is a no-op that still advances the epoch.
 */
SGT_API sgt_status sgt_ag_gemm(sgt_ctx* ctx, const void* const* A_shards, const void* B, void* A_gathered, void* C,
                       uint32_t* flags, int W, int64_t M, int64_t K, int64_t N, const sgt_opts* opts, void* stream);

/*
 * GEMM + ReduceScatter (semantics page, "GEMM + ReduceScatter overlap"; paper
 * summary, "Method": intra-node ReduceScatter in push mode, reduction running
 * alongside and synchronized by signals):
 *     P           = A_local * B              (M x N, fp32)
 *     partial_out = P  (row block p is this rank's push to rank p; block rank is kept)
 *     C_shard     = P[block rank] + sum over p != rank, ascending, of partials[p]
 * The GEMM releases gflags[t] = e after storing each rs_tile x rs_tile tile t
 * of P; the reduction of a tile of the local block waits for gflags of that
 * tile and for pflags[p * tiles_per_block + t] of every peer p, then sums in
 * fp32 (local block first, then peers by ascending rank).
 * A_local: M x K (in_dtype); B: K x N or N x K (in_dtype).
 * partials: host array of W device pointers to (M/W) x N fp32 buffers that peer
 *     p pushed for this rank; partials[rank] is not read (may be NULL).
 * partial_out: M x N fp32.  C_shard: (M/W) x N fp32.
 * gflags: ceil(M/rs_tile) * ceil(N/rs_tile) words; pflags: W * (tiles of one
 *     block) words.  The peers' partials are resident: their flags are set by
 *     the library before the reduction may read (for paced arrival see
 *     sgt_gemm_rs_paced; here opts->peer_gbps > 0 is SGT_EUNSUPPORTED).
 * Requirements: as sgt_ag_gemm, and (M/W) % rs_tile == 0.
 */
SGT_API sgt_status sgt_gemm_rs(sgt_ctx* ctx, const void* A_local, const void* B, const float* const* partials,
                       float* partial_out, float* C_shard, uint32_t* gflags, uint32_t* pflags, int W, int64_t M,
                       int64_t K, int64_t N, const sgt_opts* opts, void* stream);

/*
 * GEMM + ReduceScatter with the peers' blocks arriving over simulated links
 * (semantics page, "GEMM + ReduceScatter overlap": the reduction of a tile
 * waits for the signals of every contribution to it; paper summary, "Method":
 * ReduceScatter in push mode).  Same results as sgt_gemm_rs with
 * partials = peer_blocks, but the peers' data is not resident: the producer
 * copies each peer's block peer_blocks[p] (its push for this rank, in its
 * memory) into this rank's receive buffer inbox[p], in bands of rs_tile rows,
 * and releases the peer flags of a band's rs_tile x rs_tile tiles no earlier
 * than the time link p would deliver the band at opts->peer_gbps (0 =
 * unthrottled), in order or seeded order (opts->arrival_order != 0), plus
 * U[0, opts->jitter_us].  The reduction sums inbox[p] as tiles arrive.
 * peer_blocks, inbox: host arrays of W device pointers to (M/W) x N fp32
 *     (16-byte aligned); entry [rank] is not read.  On return inbox[p] holds
 *     peer_blocks[p] bit for bit.  Other arguments as sgt_gemm_rs.
 * Modes: SGT_PROD_CU (overlapped: the producer on its own stream and CUs) or
 *     SGT_PROD_SERIAL; SGT_PROD_PRESET is SGT_EINVAL (use sgt_gemm_rs).
 * Requirements: as sgt_gemm_rs, and rs_tile * N * 4 < 2^31.
 */
SGT_API sgt_status sgt_gemm_rs_paced(sgt_ctx* ctx, const void* A_local, const void* B, const float* const* peer_blocks,
                                     float* const* inbox, float* partial_out, float* C_shard, uint32_t* gflags,
                                     uint32_t* pflags, int W, int64_t M, int64_t K, int64_t N, const sgt_opts* opts,
                                     void* stream);

/*
 * sgt_gemm_rs without any allocation, for callers that cannot allocate device
 * memory (code under stream capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same operation, arguments, kernels and results as
 * sgt_gemm_rs with resident peers (producer SGT_PROD_CU or SGT_PROD_PRESET,
 * peer_gbps 0), but there is no context and no flag array: the status word,
 * the reduction's claim counter and every GEMM and peer flag live in the
 * library's static scratch, a device array of sgt_gemm_rs_static_scratch_bytes()
 * (64 KiB) that each GPU the library runs on holds until the process ends.
 * The call runs on the calling thread's current device; the first call on a
 * device looks up that device's copy of the array (no allocation), and the
 * call itself launches two kernels and calls no hipMalloc, hipFree or other
 * allocating routine.  Epochs are kept per device by the library.
 * Limits: a call needing more than the scratch's flag words (GEMM flags
 * ceil(M/rs_tile) * ceil(N/rs_tile) plus peer flags W * (M/W/rs_tile) *
 * ceil(N/rs_tile), at most 16320) returns SGT_EINVAL and launches nothing;
 * opts->trace must be NULL (SGT_EUNSUPPORTED).
 * Sharing: every call on a GPU uses that GPU's one array and leaves its
 * contents for the next call (the counter is cleared by the call's first
 * kernel; flags carry the epoch).  Calls on one stream are ordered; calls that
 * overlap in time on one GPU (other streams, other threads) race and are not
 * supported.  Errors: SGT_EINVAL / SGT_EUNSUPPORTED before any launch; with
 * opts->blocking the call synchronizes `stream` and returns SGT_ETIMEDOUT if a
 * bounded wait expired (in this call or an earlier non-blocking one), clearing
 * the status.
 */
SGT_API sgt_status sgt_gemm_rs_static(const void* A_local, const void* B, const float* const* partials,
                                      float* partial_out, float* C_shard, int W, int64_t M, int64_t K, int64_t N,
                                      const sgt_opts* opts, void* stream);

/* Bytes of the static scratch sgt_gemm_rs_static uses on each device (64 KiB). */
SGT_API int64_t sgt_gemm_rs_static_scratch_bytes(void);

/* Flag counts for sgt_gemm_rs: *gflags_n and *pflags_n (either may be NULL). */
SGT_API sgt_status sgt_rs_flag_count(int W, int64_t M, int64_t N, const sgt_opts* opts, int64_t* gflags_n, int64_t* pflags_n);

/*
 * MoE AllGather + grouped GEMM (paper summary, "Experiments": MoE routing
 * operations; DITRON article, "three-level tiling": device-level tiles whose
 * size depends on how many tokens each expert receives):
 *     X_gathered = rows of X_shards[0..W-1]                  (T x H bf16)
 *     route      = top-k experts per token by descending logit (ties: lower id)
 *     rows of Y  = (expert, token) pairs grouped by expert ascending, tokens
 *                  ascending inside a group; expert_off[e] is the first row of e
 *     Y[row]     = X_gathered[row_token[row]] * W_e          (fp32 or bf16)
 * Routing runs on the GPU; the shards arrive through the producer in signal
 * tiles of opts->flag_rows tokens (default: about 512 KiB per tile), the local
 * shard first; each grouped tile (expert, opts->tile_rows rows of its group,
 * 256 columns)
 * waits for exactly the signal tiles holding its rows' tokens.  Tiles are
 * claimed in the order their rows can arrive.
 * X_shards: host array of W device pointers, (T/W) x H bf16, 16-byte aligned.
 * W_experts: E x H x I (SGT_KN) or E x I x H (SGT_NK) bf16.  logits: T x E fp32
 *     (NaN logits are not supported: the selection stays k distinct experts,
 *     in an unspecified order).
 * Outputs (caller-owned device memory): X_gathered T x H; Y (T*topk) x I in
 *     opts->out_dtype; expert_off E+1 int32; row_token T*topk int32;
 *     topk_ids T x topk int32 (in selection order).
 * shard_flags: sgt_ag_flag_count(W, T, H, opts) words, zeroed once; later
 *     calls reuse them through the context's epoch.
 * Modes (opts->producer): SGT_PROD_CU overlapped; SGT_PROD_SERIAL gather then
 *     compute; SGT_PROD_PRESET X_gathered already holds every shard.
 * Requirements: opts->in_dtype SGT_BF16; T % W == 0, T <= 2^20;
 *     1 <= topk <= E <= 256; H % 8 == 0, I % 8 == 0; T*H*2 < 2^31 and, for
 *     SGT_KN, H*I*2 < 2^31.  The context keeps the routing work list (grown on
 *     demand, after draining the device); calls sharing a context must be
 *     ordered on one stream.  Errors: SGT_EINVAL / SGT_EUNSUPPORTED before any
 *     launch; a wait past opts->timeout_ms surfaces as SGT_ETIMEDOUT from
 *     sgt_sync (or this call when opts->blocking).
 */
SGT_API sgt_status sgt_moe_ag_gemm(sgt_ctx* ctx, const void* const* X_shards, const void* W_experts, const float* logits,
                           void* X_gathered, void* Y, int32_t* expert_off, int32_t* row_token, int32_t* topk_ids,
                           uint32_t* shard_flags, int W, int64_t T, int64_t H, int64_t I, int E, int topk,
                           const sgt_opts* opts, void* stream);

/*
 * MoE GEMM + ReduceScatter: the combine side of an MoE layer (paper summary,
 * "Experiments": MoE ReduceScatter among the measured kernels; semantics
 * page, "GEMM + ReduceScatter overlap": the GEMM signals output tiles and the
 * reduction waits for exactly the tiles it reads).  One GPU's share: this
 * rank's slice of the intermediate width of every expert.
 *   Y[r]   = Hg[r] * W2[e(r)]                    (fp32 accumulation; e(r) = the expert of grouped row r)
 *   P[t]   = sum_j gate[t][j] * Y[row(t, j)]     (j ascending; row(t, j) = the row of group
 *                                                 topk_ids[t][j] that holds token t)
 *   C_shard = P[rank block] + sum_{p != rank} partials[p]   (p ascending)
 * Hg: (T * topk) x I bf16, rows in the grouped order of the routing tables
 *     (expert_off, row_token, topk_ids as sgt_moe_ag_gemm writes them).
 * W2: E x I x H (SGT_KN) or E x H x I (SGT_NK) bf16.  gate: T x topk fp32.
 * partials: host array of W device pointers to (T/W) x H fp32 (entry [rank]
 *     not read): the peers' combined partials for this rank's tokens, resident.
 * Y: (T * topk) x H, out: fp32, or bf16 (round to nearest even) when
 *     opts->out_dtype = SGT_BF16, which halves the bytes Y is written and read
 *     back with (the combine then sums the rounded rows; P and C_shard stay
 *     fp32).  partial_out: T x H fp32, out (P; block p is this rank's push to
 *     rank p).  C_shard: (T/W) x H fp32, out.
 * gflags / pflags: as sgt_gemm_rs with M = T, N = H and rs_tile 128
 *     (sgt_rs_flag_count); pflags are set by the library (resident peers).
 * Requirements: bf16 in, Y fp32 or bf16, 1 <= topk <= E <= 256, I and H multiples of
 *     8, T/W a multiple of 128, rows x H x 4 < 2^31, peer_gbps = 0 (paced peers:
 *     sgt_moe_gemm_rs_paced; here it is SGT_EUNSUPPORTED), tile_waves
 *     0 or 8, rs_tile 0 or 128; 16-byte aligned matrices and flags, 4-byte
 *     aligned tables.  Routing tables that disagree with each other are not
 *     detected (the result is then undefined, but every access stays in bounds).
 * Context tables grow on demand (after draining the device); calls sharing a
 * context must be ordered on one stream.  Errors: SGT_EINVAL / SGT_EUNSUPPORTED
 * before any launch; SGT_ETIMEDOUT from a bounded wait (blocking or sgt_sync).
 */
SGT_API sgt_status sgt_moe_gemm_rs(sgt_ctx* ctx, const void* Hg, const void* W2, const float* gate,
                                   const int32_t* topk_ids, const int32_t* expert_off, const int32_t* row_token,
                                   const float* const* partials, void* Y, float* partial_out, float* C_shard,
                                   uint32_t* gflags, uint32_t* pflags, int W, int64_t T, int topk, int64_t I,
                                   int64_t H, int E, const sgt_opts* opts, void* stream);

/*
 * sgt_moe_gemm_rs with the peers' partials arriving over simulated links (as
 * sgt_gemm_rs_paced does for the dense ReduceScatter): peer p's block
 * peer_blocks[p] ((T/W) x H fp32, in its memory) is copied into this rank's
 * inbox[p] in bands of 128 rows, each band released (its peer flags) no
 * earlier than link p would deliver it at opts->peer_gbps (0 = unthrottled), in
 * order or seeded order, plus U[0, opts->jitter_us]; the reduction sums the
 * inboxes.  On return inbox[p] holds peer_blocks[p] bit for bit.
 * Modes: SGT_PROD_CU (overlapped; the combine kernel on the CUs the producer
 * leaves) or SGT_PROD_SERIAL; SGT_PROD_PRESET is SGT_EINVAL.  Other arguments,
 * requirements and errors as sgt_moe_gemm_rs.
 */
SGT_API sgt_status sgt_moe_gemm_rs_paced(sgt_ctx* ctx, const void* Hg, const void* W2, const float* gate,
                                         const int32_t* topk_ids, const int32_t* expert_off, const int32_t* row_token,
                                         const float* const* peer_blocks, float* const* inbox, void* Y,
                                         float* partial_out, float* C_shard, uint32_t* gflags, uint32_t* pflags,
                                         int W, int64_t T, int topk, int64_t I, int64_t H, int E,
                                         const sgt_opts* opts, void* stream);

/* Words of the optional trace buffer of an sgt_moe_ag_gemm call: 4 x uint64
 * {wait start, flags seen, tile end, workgroup} per work item, indexed by the
 * item's place in the consumer's work list (room for the largest possible
 * routing), then 1 x uint64 release time per signal tile.  Times are the
 * 100 MHz constant GPU clock; the last word holds the workgroup in bits 0..15
 * and the item's engine-clock cycles (from its wait start to its end) in bits
 * 16..63. */
SGT_API int64_t sgt_moe_trace_words(int W, int64_t T, int64_t H, int64_t I, int E, int topk, const sgt_opts* opts);

/*
 * Stand-alone AllGather, flag-based (Triton-distributed semantics page,
 * "Producer-consumer model", "Signal-based synchronization"; paper summary,
 * "Method": intra-node AllGather by a producer, pull mode).
 *   gathered (M x K) = the W row shards shards[0..W-1] ((M/W) x K each) stacked
 *   in rank order, moved in chunks of flag_rows rows (the signal tiles of the
 *   AllGather+GEMM plan, sgt_ag_flag_count with N = 0); after each chunk the
 *   producer releases its flag (as sgt_ag_gemm, same pacing options: peer_gbps,
 *   jitter_us, arrival_seed, arrival_order, withhold_peer; the local shard
 *   first, unpaced).  The receiving side waits for every flag in arrival order
 *   (producer_cus / consumer_cus workgroups; 0 = max(8, CUs / 8)).  SGT_PROD_CU
 *   runs both in one launch (the producer's workgroups beside the receiver's);
 *   SGT_PROD_SERIAL runs the producer's launch, then the receiver's.
 * Element size from opts->in_dtype (SGT_BF16: 2 bytes, SGT_F32: 4).  A chunk
 * (flag_rows x K elements) must be a multiple of 16 bytes, and at most 2^17
 * chunks.  SGT_PROD_PRESET is SGT_EINVAL.  opts->trace (optional, 2 words per chunk):
 * {tick the producer began the chunk, tick the receiver saw its flag}.
 * Errors as sgt_ag_gemm; a withheld peer gives SGT_ETIMEDOUT with the flag index.
 */
SGT_API sgt_status sgt_allgather(sgt_ctx* ctx, const void* const* shards, void* gathered, uint32_t* flags, int W,
                                 int64_t M, int64_t K, const sgt_opts* opts, void* stream);

/*
 * Low-latency (LL) AllGather (paper summary, "Method": for short messages the
 * AllGather stores data and flag together in 8-byte blocks and spins on them,
 * saving the signal operation of every transfer).
 *   LL packet: an aligned 8-byte word, payload dword first (bits 0..31), the
 *   call's epoch second (bits 32..63).  ll_buf (sgt_ll_buffer_bytes() bytes,
 *   16-byte aligned, zeroed once before first use like flags) receives peer
 *   p's shard as packets: chunk c (flag_rows rows, c over the gathered rows)
 *   at byte offset 2 * c * chunk_bytes, payload dword i of the chunk in word i.
 *   The producer (simulated peers) writes the remote chunks' packets, paced at
 *   opts->peer_gbps per peer counted on the packets (twice the payload); the
 *   receiver polls the packets until each holds the epoch and unpacks them
 *   into gathered, and copies the local shard; no flag is stored or read.
 *   On return gathered is as for sgt_allgather and every remote chunk's packets
 *   hold {payload, epoch}; the local shard's slot is untouched.
 * Options, modes, requirements and trace as sgt_allgather (2 * chunk < 2^31).
 * A withheld peer gives SGT_ETIMEDOUT; its "flag index" is then the index of
 * the first missing 8-byte packet in ll_buf.
 */
SGT_API sgt_status sgt_ll_allgather(sgt_ctx* ctx, const void* const* shards, void* ll_buf, void* gathered, int W,
                                    int64_t M, int64_t K, const sgt_opts* opts, void* stream);

/* Bytes of the LL receive buffer of an sgt_ll_allgather call (2 * M * K *
 * element size), or -1 for an invalid shape or options. */
SGT_API int64_t sgt_ll_buffer_bytes(int W, int64_t M, int64_t K, const sgt_opts* opts);

/*
 * One rank's share of a signal-gated ring AllReduce (Triton-distributed
 * semantics page, "Example: ring AllReduce with overlap": a ReduceScatter
 * phase and an AllGather phase of W-1 steps each, every tile synchronized on
 * its own, no barrier between steps).
 *   out (N fp32) = the elementwise sum over the W ranks' vectors.  This rank
 *   (opts->rank = r) holds x (N fp32), cut into W chunks of C = N / W
 *   elements (chunk c = [c*C, (c+1)*C)) and each chunk into T tiles
 *   (sgt_ring_flag_count).  It receives from rank r-1 and sends to r+1 (mod W).
 *   ReduceScatter step s = 0 .. W-2: it sends chunk r-s and receives chunk
 *   r-s-1, to which it adds its own x; after the last step it holds the full
 *   sum of chunk r+1.  AllGather step s = 0 .. W-2: it sends chunk r+1-s (the
 *   chunk it just finished, then what it received the step before) and
 *   receives the full chunk r-s.  Message k (k = s in the ReduceScatter,
 *   W-1+s in the AllGather) is C floats.
 *   inbox (2(W-1) x C): message k from the left neighbour lands at inbox + k*C;
 *   outbox (2(W-1) x C): this rank's message k to its right neighbour (the
 *   neighbour's inbox on a real ring), written tile by tile with device-scope
 *   stores.  flags (4(W-1)T uint32, zeroed once): the first 2(W-1)T are the
 *   arrival flags of the inbox tiles (message k, tile j at k*T + j), the rest
 *   this rank's notifications for its outbox tiles, same order.
 *   left_msgs (2(W-1) x C): the left neighbour's messages in its memory.  With
 *   SGT_PROD_CU (overlapped) or SGT_PROD_SERIAL the library's producer copies
 *   them into the inbox tile by tile as that link would deliver them (one link,
 *   messages in order, a tile every tile_bytes / opts->peer_gbps, plus
 *   U[0, opts->jitter_us]) and sets each arrival flag; with SGT_PROD_PRESET the
 *   inbox already holds them (left_msgs may be NULL) and the arrival flags are
 *   set before the kernel.  Every tile of this rank's work waits only on its
 *   own arrival flag.  W = 1: out = x.
 * Requirements: fp32 (in_dtype = out_dtype = SGT_F32), N a multiple of W, C a
 * multiple of 4, C*4 < 2^31; 16-byte aligned buffers.  opts->trace (optional):
 * 3 x uint64 {wait start, flag seen, end} per item, T*(2W-1) items: the T
 * tiles of the first send, then message k's tiles, k ascending.
 * Errors: SGT_EINVAL / SGT_EUNSUPPORTED before any launch; SGT_ETIMEDOUT from a
 * bounded wait (a withheld left neighbour, opts->withhold_peer = r-1).
 */
SGT_API sgt_status sgt_ring_allreduce(sgt_ctx* ctx, const float* x, const float* left_msgs, float* inbox,
                                      float* outbox, float* out, uint32_t* flags, int W, int64_t N,
                                      const sgt_opts* opts, void* stream);

/* Flag words of an sgt_ring_allreduce call (4(W-1)T), or -1 for an invalid
 * shape; *tile_elems (optional) receives the tile: the largest multiple of 4
 * dividing C that is at most 16384 elements (C itself when C is smaller). */
SGT_API int64_t sgt_ring_flag_count(int W, int64_t N, int64_t* tile_elems);

/*
 * Expert-parallel AllToAll, one rank's share (paper summary, "Experiments":
 * AllToAll dispatch and combine of expert parallelism, measured against
 * DeepEP; complete guide, §4.2: low-latency AllToAll for expert parallelism).
 * E experts in contiguous blocks of E_l = E / W per rank (expert e lives on
 * rank e / E_l).  Each of the W ranks holds T_r tokens of H elements and its
 * routing topk (T_r x k int32 expert ids; ids outside [0, E) select nothing).
 * This rank is opts->rank = r.  Blocks travel in chunks of opts->flag_rows
 * rows (0 = 32, at most 1024); n_chunks = ceil(T_r / chunk rows).  On one GPU
 * the other ranks' sending is simulated by sender workgroups in the same
 * launch, each publishing its chunk's flag no earlier than its link (one per
 * peer at opts->peer_gbps, all concurrent, blocks in expert order; the local
 * rank's own blocks unthrottled; 0 = unthrottled) would deliver it.
 *
 * sgt_a2a_dispatch: rank r receives, for its local expert l (global e =
 * r*E_l + l) and each source p, the rows of p's tokens that picked e, in
 * ascending token order:
 *   X[p] (T_r x H, bf16 or fp32 per opts->in_dtype; rows copied as bits);
 *   topk[p] (T_r x k int32);
 *   recv (E_l x W x T_r x H): block (l, p) at rows (l*W + p)*T_r, slot i =
 *     X[p][token i]; slots past the count are not written;
 *   recv_token (E_l x W x T_r int32): token i of block (l, p); entries past the
 *     count are not written;
 *   recv_count (E_l x W uint64): packet (epoch << 32) | count, stored with
 *     device scope (a receiver polls it until it holds the call's epoch, then
 *     waits on the block's first ceil(count / chunk rows) chunk flags);
 *   flags (sgt_a2a_flag_count words, zeroed once): chunk c of block b = l*W + p
 *     at b*n_chunks + c, set to the call's epoch once its rows have landed
 *     (chunks past the count are not written).
 *   opts->producer: SGT_PROD_CU (default) or SGT_PROD_SERIAL (the same launch).
 *
 * sgt_a2a_combine: the expert outputs come back to rank r in the same slot
 * order, and token t's output is out[t] = sum over picks j of gate[t, j] *
 * (row slot(t, j) of expert topk[t, j]), fp32, picks in order, where
 * slot(t, j) = the number of r's tokens before t that picked that expert:
 *   back[q] (E_l x T_r x H bf16): owner q's outputs for r's tokens, expert
 *     q*E_l + l at rows l*T_r, slot i for r's i-th token routed to it (only
 *     the first count rows are read);
 *   topk (T_r x k int32), gate (T_r x k fp32): this rank's routing;
 *   cbuf (E x T_r x H bf16): the receive slots, expert e at rows e*T_r;
 *   slot_of (T_r x k int32, written): slot(t, j), -1 for ids outside [0, E);
 *   out (T_r x H fp32, written);
 *   flags (sgt_a2a_flag_count words, zeroed once): chunk c of expert e at
 *     e*n_chunks + c.  Each token waits only on the chunks holding its rows.
 *   opts->producer: SGT_PROD_CU (senders and receiver in one launch),
 *   SGT_PROD_SERIAL (senders, then the receiver), SGT_PROD_PRESET (cbuf already
 *   holds the rows, back may be NULL: flags set, then the receiver alone).
 *   opts->consumer_cus: receiver workgroups (4 tokens at a time each; 0 =
 *   min(ceil(T_r / 4), CUs / 2)).  in_dtype must be SGT_BF16, out_dtype SGT_F32.
 *
 * Requirements: 1 <= W <= 64, E a multiple of W with E <= 4096, 1 <= k <= 64,
 * rows of a multiple of 16 bytes, T_r*H*elem < 2^31; X, back, recv, cbuf, out
 * 16-byte aligned.  Ownership: every buffer is the caller's device memory; the
 * context keeps a table of E per-block row counts between the scan kernel and
 * the senders (the combine, and a dispatch with more than 64 local experts; up
 * to 64, a dispatch is one launch whose senders scan the routing themselves),
 * so calls sharing a context must be ordered on one stream.  Errors: SGT_EINVAL / SGT_EUNSUPPORTED before any launch;
 * SGT_ETIMEDOUT when a combine wait expires (a withheld link,
 * opts->withhold_peer = q, whose chunks are copied but never flagged).
 */
SGT_API sgt_status sgt_a2a_dispatch(sgt_ctx* ctx, const void* const* X, const int32_t* const* topk, void* recv,
                                    int32_t* recv_token, uint64_t* recv_count, uint32_t* flags, int W, int64_t T_r,
                                    int64_t H, int E, int k, const sgt_opts* opts, void* stream);
SGT_API sgt_status sgt_a2a_combine(sgt_ctx* ctx, const void* const* back, const int32_t* topk, const float* gate,
                                   void* cbuf, int32_t* slot_of, float* out, uint32_t* flags, int W, int64_t T_r,
                                   int64_t H, int E, int k, const sgt_opts* opts, void* stream);

/* Flag words of an AllToAll call (E * ceil(T_r / chunk rows)), or -1 for an
 * invalid shape. */
SGT_API int64_t sgt_a2a_flag_count(int W, int64_t T_r, int E, const sgt_opts* opts);

/* Words of the optional trace buffer for an AllGather call: per consumer tile
 * 4 x uint64 {wait start, flag seen, tile end, workgroup}; then per signal tile
 * 1 x uint64 release time.  Times are the 100 MHz constant GPU clock.  The bf16
 * consumer puts the workgroup in bits 0..15 of the last word and the tile's
 * engine-clock cycles (s_memtime, from the tile's start to its end, waits
 * included) in bits 16..63, so cycles / duration is the engine clock.
 * (A GEMM+ReduceScatter call's trace is sized by sgt_rs_trace_words.) */
SGT_API int64_t sgt_trace_words(int W, int64_t M, int64_t K, int64_t N, const sgt_opts* opts);

/* Words of the optional trace buffer for a GEMM+ReduceScatter call (M x N
 * output, W row blocks, opts->rs_tile), or -1 for an invalid shape: 3 x uint64
 * {start, end, workgroup} per work item, first the GEMM tiles ((W *
 * ceil(M/W/256)) * ceil(N/256), local block first), then the reduction items:
 * each signal tile of the local block (tile-row-major) cut into row bands of
 * 32 rows (the whole tile when rs_tile <= 32), band-minor. */
SGT_API int64_t sgt_rs_trace_words(int W, int64_t M, int64_t N, const sgt_opts* opts);

#ifdef __cplusplus
}
#endif

#endif /* SGT_H_ */
