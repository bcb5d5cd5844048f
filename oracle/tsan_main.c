/*
 * Test infrastructure: drives the oracle's protocol emulator (orc_ag_gemm_protocol: producer threads
 * that copy signal tiles and release-store their flags, consumer threads that acquire-wait on the flags
 * of a panel before reading it; Triton-distributed semantics page, "Producer-consumer model" and
 * "Signal-based synchronization") under ThreadSanitizer.  Built by tests/test_oracle_tsan.py with
 * gcc -fsanitize=thread as one translation unit with oracle.c (OpenMP off).
 *
 * Usage: tsan_main [skip]   -- "skip" runs the emulator with its consumers' waits removed (a planted
 * race, which the sanitizer must report).  Exit status 0 when every run gives the plain oracle's C.
 */
#include "oracle.c"

#include <math.h>
#include <stdio.h>

static uint64_t rng = 88172645463325252ull;
static float urand(void) {
  rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
  return (float)((double)(rng >> 11) * (1.0 / 9007199254740992.0) * 2.0 - 1.0);
}

int main(int argc, char** argv) {
  const int skip = argc > 1 && strcmp(argv[1], "skip") == 0;
  const int W = 4;
  const int64_t rows = 32, K = 24, N = 20, M = rows * W;
  float* shard[4];
  for (int p = 0; p < W; ++p) {
    shard[p] = (float*)malloc(sizeof(float) * (size_t)(rows * K));
    for (int64_t i = 0; i < rows * K; ++i) shard[p][i] = urand();
  }
  float* B = (float*)malloc(sizeof(float) * (size_t)(K * N));
  for (int64_t i = 0; i < K * N; ++i) B[i] = urand();
  float* A_full = (float*)malloc(sizeof(float) * (size_t)(M * K));
  orc_allgather((const void* const*)shard, W, rows, K * 4, A_full);
  double* C_ref = (double*)malloc(sizeof(double) * (size_t)(M * N));
  orc_gemm_rows(A_full, ORC_F32, B, ORC_F32, ORC_KN, M, K, N, NULL, 0, C_ref, 1);
  float* A_g = (float*)malloc(sizeof(float) * (size_t)(M * K));
  double* C = (double*)malloc(sizeof(double) * (size_t)(M * N));
  int bad = 0, runs = 0;
  for (int rank = 0; rank < W; rank += 3)
    for (int global = 0; global < 2; ++global)
      for (int order = 0; order < 2; ++order)
        for (uint64_t seed = 0; seed < 3; ++seed) {
          for (int64_t i = 0; i < M * K; ++i) A_g[i] = NAN;
          if (orc_ag_gemm_protocol((const void* const*)shard, W, rank, ORC_F32, B, ORC_F32, ORC_KN, M, K, N, 8, 16,
                                   seed, seed ? 30.0 : 0.0, global, order, 3, skip, A_g, C) != 0)
            return 2;
          ++runs;
          if (memcmp(A_g, A_full, sizeof(float) * (size_t)(M * K)) != 0 ||
              memcmp(C, C_ref, sizeof(double) * (size_t)(M * N)) != 0)
            ++bad;
        }
  printf("%d runs, %d differ from the plain oracle\n", runs, bad);
  return bad ? 1 : 0;
}
