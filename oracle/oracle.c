/*
 * CPU oracle for the signal-gated tiled AllGather+GEMM, GEMM+ReduceScatter and
 * MoE AllGather-grouped-GEMM.  TEST INFRASTRUCTURE ONLY: it may be used by the
 * test suite, the smoke check and the benchmark's CPU-baseline leg, never by
 * the product path.  It shares no code, header or table with the HIP library.
 *
 * What it computes (sources: the Triton-distributed semantics page, sections
 * "AllGather + GEMM overlap" and "GEMM + ReduceScatter overlap"; the
 * Triton-distributed paper summary, section "Method"):
 *
 *   AllGather+GEMM   A_full = the W row shards stacked in shard order, then
 *                    C = A_full * B.
 *   GEMM+RS          P = A_local * B; rank r keeps row block r and adds the
 *                    other ranks' partial blocks: C_shard = P[r] + sum_p partial[p].
 *   MoE AG-GEMM      each gathered token is routed to its top-k experts and
 *                    multiplied by each expert's weight.
 *   MoE GEMM+RS      each grouped row times its expert's weight, the rows of a
 *                    token summed with its gate weights, then the ReduceScatter
 *                    of GEMM+RS over token blocks.
 *
 * Both results have a plain definition, so the oracle is that definition,
 * written out: loops in double precision, each output element summed in
 * ascending k.  Products of two bf16 or two fp32 values are exact in double
 * (8+8 or 24+24 significand bits), so the only rounding is the fp64 sum.
 *
 * The protocol emulator at the end runs the same computation through host
 * threads that imitate the producer/consumer signal protocol (copy a tile,
 * release-store its flag; wait on the flag with acquire, then compute), with
 * seeded arrival orders and delays.  Its result must be bit-identical to the
 * plain computation for every order and delay.
 */
#define _GNU_SOURCE
#include <stdatomic.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <pthread.h>
#include <time.h>
#include <sched.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1 };
enum { ORC_KN = 0, ORC_NK = 1 };

/* bf16 -> double: the 16 stored bits are the top half of an IEEE binary32. */
static double bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double elem(const void* p, int dtype, int64_t idx) {
  if (dtype == ORC_BF16) return bf16_to_double(((const uint16_t*)p)[idx]);
  return (double)((const float*)p)[idx];
}

static size_t elem_size(int dtype) { return dtype == ORC_BF16 ? 2 : 4; }

/* B(k, j) of the logical K x N matrix, stored K x N ("kn") or N x K ("nk"). */
static double b_at(const void* B, int dtype, int layout, int64_t K, int64_t N, int64_t k, int64_t j) {
  return layout == ORC_KN ? elem(B, dtype, k * N + j) : elem(B, dtype, j * K + k);
}

int orc_version(void) { return 1; }

int orc_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* AllGather of row shards: shard p lands at rows [p*rows, (p+1)*rows). */
void orc_allgather(const void* const* shards, int W, int64_t rows_per_shard, int64_t row_bytes, void* out) {
  for (int p = 0; p < W; ++p)
    memcpy((char*)out + (size_t)p * rows_per_shard * row_bytes, shards[p], (size_t)(rows_per_shard * row_bytes));
}

/* Low-latency packets (paper summary, "Method": for short messages data and
 * flag share one 8-byte block): word i = the payload's 4-byte word i in the
 * low half and the flag value (the call's epoch) in the high half. */
void orc_ll_pack(const uint32_t* payload, int64_t n_words, uint32_t epoch, uint64_t* out) {
  for (int64_t i = 0; i < n_words; ++i) out[i] = ((uint64_t)epoch << 32) | (uint64_t)payload[i];
}

/* One output row: c[j] = sum_{k ascending} a[k] * B(k, j), all in double. */
static void gemm_row(const void* a_row, int a_dt, const void* B, int b_dt, int b_layout, int64_t K, int64_t N,
                     double* c) {
  for (int64_t j = 0; j < N; ++j) c[j] = 0.0;
  if (b_layout == ORC_KN) {
    for (int64_t k = 0; k < K; ++k) {
      double a = elem(a_row, a_dt, k);
      for (int64_t j = 0; j < N; ++j) c[j] += a * b_at(B, b_dt, ORC_KN, K, N, k, j);
    }
  } else {
    for (int64_t j = 0; j < N; ++j) {
      double s = 0.0;
      for (int64_t k = 0; k < K; ++k) s += elem(a_row, a_dt, k) * b_at(B, b_dt, ORC_NK, K, N, k, j);
      c[j] = s;
    }
  }
}

/*
 * C[r][:] = A[rows[r]][:] * B for r < nrows (rows == NULL: all M rows, in order).
 * A is M x K row-major; C is nrows x N doubles.  Threads split the rows.
 */
void orc_gemm_rows(const void* A, int a_dt, const void* B, int b_dt, int b_layout, int64_t M, int64_t K, int64_t N,
                   const int64_t* rows, int64_t nrows, double* C, int nthreads) {
  if (rows == NULL) nrows = M;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
  for (int64_t r = 0; r < nrows; ++r) {
    int64_t i = rows ? rows[r] : r;
    gemm_row((const char*)A + (size_t)i * K * elem_size(a_dt), a_dt, B, b_dt, b_layout, K, N, C + (size_t)r * N);
  }
  (void)nthreads;
}

/*
 * GEMM+ReduceScatter for rank `rank` of W: rows i of its block (block_rows = M/W),
 *   C_shard[i][j] = P[rank*block_rows + i][j] + sum_{p != rank, ascending p} partials[p][i][j]
 * with P = A_local * B in double.  partials[p] are (M/W) x N fp32; partials[rank] is not read.
 * rows == NULL: every row of the block.
 */
void orc_gemm_rs(const void* A, int a_dt, const void* B, int b_dt, int b_layout, int64_t M, int64_t K, int64_t N,
                 const float* const* partials, int W, int rank, const int64_t* rows, int64_t nrows, double* C_shard,
                 int nthreads) {
  int64_t mb = M / W;
  if (rows == NULL) nrows = mb;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
  for (int64_t r = 0; r < nrows; ++r) {
    int64_t i = rows ? rows[r] : r;
    double* c = C_shard + (size_t)r * N;
    gemm_row((const char*)A + (size_t)(rank * mb + i) * K * elem_size(a_dt), a_dt, B, b_dt, b_layout, K, N, c);
    for (int p = 0; p < W; ++p) {
      if (p == rank) continue;
      for (int64_t j = 0; j < N; ++j) c[j] += (double)partials[p][i * N + j];
    }
  }
  (void)nthreads;
}

/*
 * MoE routing: for each token, its top-k experts by descending logit, ties to the
 * lower expert id (selection by k passes of arg-max over the experts not yet taken).
 * Rows are then grouped by expert (ascending) and, inside a group, by token (ascending):
 *   expert_off[e] .. expert_off[e+1]-1 are the rows of expert e,
 *   row_token[row] is the token of that row.
 * topk_ids: T x k (in selection order).  Returns 0, or -1 if k > E.
 */
int orc_moe_route(const float* logits, int64_t T, int E, int k, int32_t* topk_ids, int32_t* expert_off,
                  int32_t* row_token) {
  if (k > E || k <= 0) return -1;
  char* taken = (char*)calloc((size_t)E, 1);
  for (int64_t t = 0; t < T; ++t) {
    memset(taken, 0, (size_t)E);
    const float* l = logits + (size_t)t * E;
    for (int s = 0; s < k; ++s) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || l[e] > l[best]) best = e; /* strict '>' keeps the lower id on ties */
      }
      taken[best] = 1;
      topk_ids[t * k + s] = best;
    }
  }
  free(taken);
  int32_t row = 0;
  for (int e = 0; e < E; ++e) {
    expert_off[e] = row;
    for (int64_t t = 0; t < T; ++t)
      for (int s = 0; s < k; ++s)
        if (topk_ids[t * k + s] == e) row_token[row++] = (int32_t)t;
  }
  expert_off[E] = row;
  return 0;
}

/*
 * Grouped expert GEMM over routed rows: Y[row][:] = X_full[row_token[row]][:] * W_e
 * for e the expert owning the row.  X_full T x H bf16, W_experts E x H x I ("kn") or
 * E x I x H ("nk") bf16.  rows == NULL: all expert_off[E] rows.
 */
void orc_moe_gemm_rows(const uint16_t* X_full, const uint16_t* W_experts, int w_layout, int64_t H, int64_t I, int E,
                       const int32_t* expert_off, const int32_t* row_token, const int64_t* rows, int64_t nrows,
                       double* Y, int nthreads) {
  if (rows == NULL) nrows = expert_off[E];
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
  for (int64_t r = 0; r < nrows; ++r) {
    int64_t row = rows ? rows[r] : r;
    int e = 0;
    while (e + 1 <= E && expert_off[e + 1] <= row) ++e;
    const uint16_t* x = X_full + (size_t)row_token[row] * H;
    const uint16_t* w = W_experts + (size_t)e * H * I;
    gemm_row(x, ORC_BF16, w, ORC_BF16, w_layout, H, I, Y + (size_t)r * I);
  }
  (void)nthreads;
}

/*
 * MoE GEMM + ReduceScatter, the combine side of an MoE layer (paper summary,
 * "Experiments": MoE ReduceScatter; semantics page, "GEMM + ReduceScatter
 * overlap"), as its plain definition.  Grouped rows Hg (rows x I bf16, in the
 * expert-grouped order of the routing tables) times the owning expert's W2
 * (E x I x H "kn" or E x H x I "nk" bf16), combined per token with its gate
 * weights in pick order:
 *   P[t][n] = sum_j gate[t][j] * sum_i Hg[row(t, j)][i] * W2[e(t, j)][i][n]
 * with e(t, j) = topk_ids[t][j] and row(t, j) the row of group e(t, j) that
 * holds token t; rank r's block then adds the other ranks' partial blocks:
 *   C[t - r T/W][n] = P[t][n] + sum_{p != r} partial_p[t - r T/W][n].
 * tokens: the tokens to compute (NULL: all T).  P_out: ntok x H (may be NULL);
 * C_out: ntok x H for tokens of block `rank` (may be NULL; -3 if a token is
 * outside the block).  Returns -2 when a pick has no row in its group.
 */
int orc_moe_gemm_rs(const uint16_t* Hg, const uint16_t* W2, int w_layout, int64_t T, int k, int64_t I, int64_t H,
                    int E, const int32_t* topk_ids, const float* gate, const int32_t* expert_off,
                    const int32_t* row_token, const float* const* partials, int W, int rank, const int64_t* tokens,
                    int64_t ntok, double* P_out, double* C_out, int nthreads) {
  if (tokens == NULL) ntok = T;
  const int64_t blk = T / W, b0 = (int64_t)rank * blk;
  int bad = 0;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(| : bad)
#endif
  for (int64_t i = 0; i < ntok; ++i) {
    const int64_t t = tokens ? tokens[i] : i;
    double* acc = (double*)calloc((size_t)H, sizeof(double));
    double* y = (double*)malloc((size_t)H * sizeof(double));
    for (int j = 0; j < k && !bad; ++j) {
      const int e = topk_ids[t * k + j];
      int64_t row = -1;
      for (int64_t r = expert_off[e]; r < expert_off[e + 1]; ++r)
        if (row_token[r] == t) { row = r; break; }
      if (row < 0) { bad |= 2; break; }
      gemm_row(Hg + (size_t)row * I, ORC_BF16, W2 + (size_t)e * I * H, ORC_BF16, w_layout, I, H, y);
      const double g = (double)gate[t * k + j];
      for (int64_t n = 0; n < H; ++n) acc[n] += g * y[n];
    }
    if (P_out)
      for (int64_t n = 0; n < H; ++n) P_out[i * H + n] = acc[n];
    if (C_out) {
      if (t < b0 || t >= b0 + blk) {
        bad |= 4;
      } else {
        for (int p = 0; p < W; ++p) {
          if (p == rank) continue;
          const float* part = partials[p] + (size_t)(t - b0) * H;
          for (int64_t n = 0; n < H; ++n) acc[n] += (double)part[n];
        }
        for (int64_t n = 0; n < H; ++n) C_out[i * H + n] = acc[n];
      }
    }
    free(acc);
    free(y);
  }
  (void)nthreads;
  return (bad & 2) ? -2 : (bad & 4) ? -3 : 0;
}

/* ------------------------------------------------------------------------- */
/* Protocol emulator                                                          */
/* ------------------------------------------------------------------------- */

/* SplitMix64 (Steele, Lea and Flood, OOPSLA 2014) drives arrival orders and delays. */
static uint64_t splitmix64(uint64_t* s) {
  uint64_t z = (*s += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static void sleep_us(double us) {
  if (us <= 0) return;
  struct timespec ts;
  ts.tv_sec = (time_t)(us / 1e6);
  ts.tv_nsec = (long)((us - (double)ts.tv_sec * 1e6) * 1e3);
  nanosleep(&ts, NULL);
}

typedef struct {
  /* problem */
  const void* const* shards;
  int W, rank, a_dt, b_dt, b_layout;
  int64_t M, K, N, rows_per_shard, flag_rows, panel_rows;
  const void* B;
  /* shared state */
  void* A_gathered;
  _Atomic uint32_t* flags;
  uint32_t epoch;
  double* C;
  /* arrival model */
  uint64_t seed;
  double max_delay_us;
  int global_perm;     /* 1: one seeded order over all remote tiles, one producer thread */
  int order;           /* consumer panel order: 0 = shard-major swizzle, 1 = peers interleaved */
  int n_consumers;
  int skip_wait;       /* deliberately broken consumer (for tests that the checks have teeth) */
} proto_t;

typedef struct {
  proto_t* P;
  int id;
} worker_t;

static void copy_tile(proto_t* P, int64_t tile) {
  size_t rb = (size_t)P->K * elem_size(P->a_dt);
  int64_t row0 = tile * P->flag_rows;
  int64_t p = row0 / P->rows_per_shard, local_row = row0 % P->rows_per_shard;
  memcpy((char*)P->A_gathered + (size_t)row0 * rb, (const char*)P->shards[p] + (size_t)local_row * rb,
         (size_t)P->flag_rows * rb);
  atomic_store_explicit(&P->flags[tile], P->epoch, memory_order_release);
}

/* Producer for one shard (id = shard), or for all remote tiles (global_perm). */
static void* producer_main(void* arg) {
  worker_t* w = (worker_t*)arg;
  proto_t* P = w->P;
  int64_t tiles_per_shard = P->rows_per_shard / P->flag_rows;
  int64_t n = P->global_perm ? tiles_per_shard * (P->W - 1) : tiles_per_shard;
  int64_t* order = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n ? n : 1));
  int64_t c = 0;
  for (int p = 0; p < P->W; ++p) {
    if (P->global_perm ? p == P->rank : p != w->id) continue;
    for (int64_t t = 0; t < tiles_per_shard; ++t) order[c++] = p * tiles_per_shard + t;
  }
  int local = !P->global_perm && w->id == P->rank;
  uint64_t s = P->seed * 0x100000001B3ull + (uint64_t)w->id + 1;
  if (!local && P->seed) /* Fisher-Yates */
    for (int64_t i = n - 1; i > 0; --i) {
      int64_t j = (int64_t)(splitmix64(&s) % (uint64_t)(i + 1));
      int64_t t = order[i]; order[i] = order[j]; order[j] = t;
    }
  for (int64_t i = 0; i < n; ++i) {
    if (!local && P->max_delay_us > 0)
      sleep_us(P->max_delay_us * (double)(splitmix64(&s) >> 11) * (1.0 / 9007199254740992.0));
    copy_tile(P, order[i]);
  }
  free(order);
  return NULL;
}

/* Consumer panel list.  Panel q covers rows [q*panel_rows, ...).
 * order 0: start at the local shard and walk shards in rank order,
 *          pid_m = (i + rank * panels_per_shard) % panels (the pages' threadblock swizzle);
 * order 1: local shard first, then the other shards' panels interleaved
 *          (panel j of shard rank+1, rank+2, ..., then panel j+1 ...). */
static int64_t panel_at(const proto_t* P, int64_t i) {
  int64_t pps = P->rows_per_shard / P->panel_rows, panels = P->M / P->panel_rows;
  if (P->order == 0 || i < pps) return (i + P->rank * pps) % panels;
  int64_t j = i - pps;
  int64_t peer = 1 + j % (P->W - 1), pj = j / (P->W - 1);
  return ((P->rank + peer) % P->W) * pps + pj;
}

/* The consumer panel order, exported for the fixture tests. */
int orc_panel_order(int W, int rank, int64_t rows_per_shard, int64_t panel_rows, int order, int64_t* out) {
  if (W <= 0 || rank < 0 || rank >= W || panel_rows <= 0 || rows_per_shard % panel_rows) return -1;
  proto_t P;
  memset(&P, 0, sizeof P);
  P.W = W; P.rank = rank; P.rows_per_shard = rows_per_shard; P.panel_rows = panel_rows;
  P.M = rows_per_shard * W; P.order = order;
  for (int64_t i = 0; i < P.M / panel_rows; ++i) out[i] = panel_at(&P, i);
  return 0;
}

static void* consumer_main(void* arg) {
  worker_t* w = (worker_t*)arg;
  proto_t* P = w->P;
  int64_t panels = P->M / P->panel_rows;
  size_t rb = (size_t)P->K * elem_size(P->a_dt);
  for (int64_t i = w->id; i < panels; i += P->n_consumers) {
    int64_t q = panel_at(P, i);
    int64_t r0 = q * P->panel_rows, r1 = r0 + P->panel_rows;
    if (!P->skip_wait)
      for (int64_t f = r0 / P->flag_rows; f <= (r1 - 1) / P->flag_rows; ++f)
        while (atomic_load_explicit(&P->flags[f], memory_order_acquire) != P->epoch) sched_yield();
    for (int64_t r = r0; r < r1; ++r)
      gemm_row((const char*)P->A_gathered + (size_t)r * rb, P->a_dt, P->B, P->b_dt, P->b_layout, P->K, P->N,
               P->C + (size_t)r * P->N);
  }
  return NULL;
}

/*
 * Runs AllGather+GEMM through the signal protocol with host threads.
 * A_gathered must be pre-filled by the caller (poison); flags are local.
 * Returns 0, or -1 on bad arguments.
 */
int orc_ag_gemm_protocol(const void* const* shards, int W, int rank, int a_dt, const void* B, int b_dt, int b_layout,
                         int64_t M, int64_t K, int64_t N, int64_t flag_rows, int64_t panel_rows, uint64_t seed,
                         double max_delay_us, int global_perm, int order, int n_consumers, int skip_wait,
                         void* A_gathered, double* C) {
  if (W <= 0 || M % W || rank < 0 || rank >= W) return -1;
  int64_t rows = M / W;
  if (flag_rows <= 0 || rows % flag_rows || panel_rows <= 0 || rows % panel_rows || n_consumers <= 0) return -1;
  proto_t P = {shards, W, rank, a_dt, b_dt, b_layout, M, K, N, rows, flag_rows, panel_rows, B, A_gathered, NULL,
               1u, C, seed, max_delay_us, global_perm, order, n_consumers, skip_wait};
  int64_t ntiles = M / flag_rows;
  P.flags = (_Atomic uint32_t*)calloc((size_t)ntiles, sizeof(uint32_t));
  int nprod = global_perm ? 2 : W;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)(nprod + n_consumers));
  worker_t* wk = (worker_t*)malloc(sizeof(worker_t) * (size_t)(nprod + n_consumers));
  /* consumers start first, so that early reads would see poison if the waits were wrong */
  for (int c = 0; c < n_consumers; ++c) {
    wk[nprod + c].P = &P; wk[nprod + c].id = c;
    pthread_create(&th[nprod + c], NULL, consumer_main, &wk[nprod + c]);
  }
  if (global_perm) {
    /* the local shard by its own thread (a per-shard view of the same state),
       every remote tile in one seeded order by a second thread */
    proto_t Pl = P;
    Pl.global_perm = 0;
    worker_t wl = {&Pl, rank};
    wk[0].P = &P; wk[0].id = 0;
    pthread_create(&th[0], NULL, producer_main, &wl);
    pthread_create(&th[1], NULL, producer_main, &wk[0]);
    pthread_join(th[0], NULL);
    pthread_join(th[1], NULL);
  } else {
    for (int p = 0; p < W; ++p) {
      wk[p].P = &P; wk[p].id = p;
      pthread_create(&th[p], NULL, producer_main, &wk[p]);
    }
    for (int p = 0; p < W; ++p) pthread_join(th[p], NULL);
  }
  for (int c = 0; c < n_consumers; ++c) pthread_join(th[nprod + c], NULL);
  free((void*)P.flags);
  free(th);
  free(wk);
  return 0;
}
