// bf16 x bf16 -> fp32 tile GEMM on CDNA4 matrix cores, shared by the
// AllGather, GEMM+ReduceScatter and MoE consumers.
//
// One workgroup computes a 256 x 256 fp32 tile C[m0:m0+256, n0:n0+256] =
// A[rows, :] * B[:, n0:n0+256] with v_mfma_f32_32x32x16_bf16.  Two shapes of
// workgroup, chosen by the template parameter kW (wave64s per workgroup):
//   kW = 4: 2 x 2 waves of 128 x 128 (4 x 4 MFMA blocks, 256 accumulators per
//           lane): one wave per SIMD.
//   kW = 8: 4 x 2 waves of 64 x 128 (2 x 4 MFMA blocks, 128 accumulators): two
//           waves per SIMD, so one wave's LDS waits and barrier skew are
//           covered by the other's matrix-core work (a pure MFMA loop reaches
//           ~11% more throughput with two waves per SIMD than with one).
//
// K loop: BK = 64, two LDS stages of 64 KiB, one barrier per K step.  Operands
// whose k index is contiguous in memory (A, and B stored N x K) go straight
// from HBM to LDS with buffer_load_dwordx4 ... lds (no register staging),
// issued between the MFMAs of the current step's first substep; B stored
// K x N is loaded to registers in blocks of 8 n x (8 or 4) k, transposed
// there and written to LDS, so LDS always holds [row][k].  The next step's
// loads are in flight while the current step's MFMAs run.  A kernel that
// gives the K loop all 160 KiB of LDS can run the 8-wave tile with both
// operands k-contiguous on a ring of five one-operand slots instead, which
// loads A two steps ahead (gemm_tile_range_r5).
//
// LDS layout of a stage, both operands: [256 rows][64 k] bf16 = 128 bytes per
// row = 8 chunks of 16 bytes; chunk c of row r is stored at chunk
// c ^ (r & 7) ^ ((r >> 3) & 3).  The MFMA operand reads (8 consecutive rows,
// one chunk) hit distinct banks, and since the swizzle only uses row bits 0..4
// the reads of different 32-row MFMA blocks differ by a constant (an
// immediate offset).  The DMA writes whole 1 KiB runs; the K x N loader's
// transposed writes see at most a 2-way conflict.
//
// Tails: 32-bit buffer offsets from a per-tile base; rows past the end of the
// matrix fall outside the buffer's record range and read as zero, and chunks
// past K (or columns past N) get an out-of-range offset.  The hardware range
// check covers the VGPR offset only, so every offset is passed there.
// K % 8 == 0 and N % 8 == 0 are required (whole 16-byte chunks).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sgt {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kStageBytes = kBM * kBK * 2;          // one operand, one stage: 32 KiB
constexpr uint32_t kOOB = 0x80000000u;              // buffer offset that reads 0 / drops a store
constexpr int kRsrcWord3 = 0x00020000;              // raw buffer, 32-bit data format (gfx9)

// kR: rows of the tile (256, or 128 for the short tiles of ragged groups);
// the tile is always 256 columns wide.
template <int kW, int kR = kBM>
struct Tile {
  static_assert(kW == 4 || kW == 8, "4 or 8 waves");
  static_assert(kR == 256 || kR == 128, "256 or 128 rows");
  static constexpr int kThreads = 64 * kW;
  static constexpr int kWaveRows = kR / (kW / 2);   // 128, 64 or 32 rows per wave
  static constexpr int kMI = kWaveRows / 32;        // 32-row MFMA blocks per wave
  static constexpr int kDmaLoads = kBM / kW / 8;    // 1 KiB DMA loads per wave per 256-row operand and stage
};

__device__ __forceinline__ int lds_swz(int row, int chunk) {
  return row * 128 + ((chunk ^ (row & 7) ^ ((row >> 3) & 3)) << 4);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint64_t bytes) {
  const uint32_t n = bytes > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, kRsrcWord3);
}

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

template <int kW, int kR = kBM>
struct MfmaAcc {
  f32x16_t v[Tile<kW, kR>::kMI][4];
};

template <int kW, int kR>
__device__ __forceinline__ void acc_zero(MfmaAcc<kW, kR>& acc) {
#pragma unroll
  for (int i = 0; i < Tile<kW, kR>::kMI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc.v[i][j][r] = 0.f;
}

// A k-contiguous operand tile (A, or B stored N x K) seen by the DMA loader:
// a buffer resource whose record range ends after the last valid row (later
// rows read as zero).  Lane l of wave w fills, with its load i, LDS row
// r = (kRows / kW) w + 8 i + l / 8 at physical chunk l % 8, i.e. logical chunk
// (l % 8) ^ swz(r) = (l % 8) ^ (l / 8) ^ (i % 4).  row_off[i] is the byte
// offset of that row (rows `ld` elements apart, or gathered rows for MoE;
// kOOB for a row that does not exist); all offsets are 32-bit.
struct KRows {
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t row_off[8];  // entries [0, kRows / kW / 8) are used
  uint32_t chunk[4];   // this lane's logical chunk byte offset for i % 4
};

// Logical chunk of this lane's load i: its LDS row r has r % 8 = lane / 8
// and (r / 8) % 4 = (w L + i) % 4 for L = kRows / kW / 8 loads per wave (just
// i % 4 when L is a multiple of 4).
template <int kW, int kRows = kBM>
__device__ __forceinline__ void krows_chunks(KRows& kr) {
  constexpr int L = kRows / kW / 8;
  const int lane = threadIdx.x & 63, w = wave_id();
#pragma unroll
  for (int q = 0; q < 4; ++q) kr.chunk[q] = (uint32_t)((((lane & 7) ^ (lane >> 3) ^ ((w * L + q) & 3)) & 7) * 16);
}

// LDS row filled by this lane's load i of an operand of kRows rows.
template <int kW, int kRows = kBM>
__device__ __forceinline__ int dma_row(int i) {
  return (kRows / kW) * wave_id() + 8 * i + ((threadIdx.x & 63) >> 3);
}

// Strided rows: row r at element offset r * ld from base; rows >= rows_valid are zero.
template <int kW, int kRows = kBM>
__device__ __forceinline__ KRows krows_strided(const uint16_t* base, int64_t rows_valid, int64_t ld) {
  KRows kr;
  const int64_t rows = rows_valid < kRows ? rows_valid : kRows;
  kr.rsrc = make_rsrc(base, rows > 0 ? (uint64_t)rows * (uint64_t)ld * 2u : 0u);
#pragma unroll
  for (int i = 0; i < kRows / kW / 8; ++i) kr.row_off[i] = (uint32_t)(dma_row<kW, kRows>(i) * ld * 2);
  krows_chunks<kW, kRows>(kr);
  return kr;
}

// Issue the DMA of K step [k0, k0 + 64) of a k-contiguous operand of kRows
// rows into `stage`.  Chunks at or past K (including whole steps past the end)
// read as zero.
template <int kW, int kRows = kBM>
__device__ __forceinline__ void dma_stage(const KRows& kr, uint8_t* stage, int64_t k0, int64_t K) {
  constexpr int L = kRows / kW / 8;
  const int w = wave_id();
  const uint32_t kbyte = (uint32_t)(k0 * 2);
  const int64_t rem = (K - k0) * 2;                  // valid bytes of this step's rows
  const uint32_t lim = rem <= 0 ? 0u : (rem >= 128 ? 128u : (uint32_t)rem);
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const uint32_t c = kr.chunk[i & 3];
    // kOOB + (k0 + c) stays >= 2^31, past every record range
    const uint32_t off = c < lim ? kr.row_off[i] + kbyte + c : kOOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(kr.rsrc, (lds_ptr_t)(stage + (w * L + i) * 1024), 16, off, 0, 0, 0);
  }
}

// B stored K x N: registers, transpose, LDS.  Thread t handles columns
// n0 + 8 (t % 32) .. + 7 and, of the K step's 8 groups of 8 rows, group
// (t / 32) % 8; with 512 threads each thread takes half of the group's rows.
template <int kW>
struct KNLoader {
  static constexpr int kRows = kW == 4 ? 8 : 4;   // rows per thread
  __amdgpu_buffer_rsrc_t rsrc;  // whole of B
  uint32_t lane_off;            // byte offset of this thread's first row at k0 = 0, or kOOB
  int64_t row_bytes;            // N * 2
  u32x4_t gb[kRows];

  __device__ __forceinline__ void init(const uint16_t* B, int64_t K, int64_t N, int64_t n0) {
    rsrc = make_rsrc(B, (uint64_t)K * (uint64_t)N * 2u);
    const int t = threadIdx.x, ng = t & 31, kg = (t >> 5) & 7, h = t >> 8;
    row_bytes = N * 2;
    lane_off = (n0 + 8 * ng < N) ? (uint32_t)((8 * kg + kRows * h) * row_bytes + (n0 + 8 * ng) * 2) : kOOB;
  }
  __device__ __forceinline__ void load(int64_t k0) {
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
      // the range check ignores soffset, so the whole offset goes in voffset
      const uint32_t off = lane_off == kOOB ? kOOB : lane_off + (uint32_t)((k0 + i) * row_bytes);
      gb[i] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0);
    }
  }
  // gb[i] holds B[k0 + 8kg + kRows h + i][n0 + 8ng + 0..7] (two bf16 per dword).
  // Column j of the block, k ascending, goes to LDS row 8 ng + j, chunk kg
  // (bytes 8 h .. 8 h + 8 of the chunk when a thread holds 4 rows).
  __device__ __forceinline__ void store(uint8_t* sB) const {
    const int t = threadIdx.x, ng = t & 31, kg = (t >> 5) & 7, h = t >> 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t col[kRows / 2];
#pragma unroll
      for (int q = 0; q < kRows / 2; ++q) {
        const uint32_t lo = gb[2 * q][j >> 1], hi = gb[2 * q + 1][j >> 1];
        col[q] = (j & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
      }
      uint8_t* dst = sB + lds_swz(8 * ng + j, kg);
      if constexpr (kRows == 8)
        *reinterpret_cast<u32x4_t*>(dst) = u32x4_t{col[0], col[1], col[2], col[3]};
      else
        *reinterpret_cast<u32x2_t*>(dst + 8 * h) = u32x2_t{col[0], col[1]};
    }
  }
};

__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <int kW, int kR>
__device__ __forceinline__ void read_frags(const uint8_t* sA, const uint8_t* sB, int kk,
                                           bf16x8_t (&a)[Tile<kW, kR>::kMI], bf16x8_t (&b)[4]) {
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, chunk = 2 * kk + (lane >> 5);
#pragma unroll
  for (int i = 0; i < Tile<kW, kR>::kMI; ++i)
    a[i] = *reinterpret_cast<const bf16x8_t*>(sA + lds_swz(wm * Tile<kW, kR>::kWaveRows + i * 32 + lr, chunk));
#pragma unroll
  for (int j = 0; j < 4; ++j)
    b[j] = *reinterpret_cast<const bf16x8_t*>(sB + lds_swz(wn * 128 + j * 32 + lr, chunk));
}

// The DMA loads of one K step of the k-contiguous operands (A, then B when it
// is stored N x K), issued one at a time from inside the MFMA stream: load j
// is A's load j for j < kLA, else B's load j - kLA.
template <int kW, int kR, bool kBNK>
struct StepDma {
  static constexpr int kLA = kR / kW / 8, kLB = kBNK ? kBM / kW / 8 : 0, kN = kLA + kLB;
  const KRows* ka;
  const KRows* kb;
  uint8_t* sA;
  uint8_t* sB;
  uint32_t kbyte, lim;
  __device__ __forceinline__ StepDma(const KRows& a, const KRows& b, uint8_t* stA, uint8_t* stB, int64_t k0,
                                     int64_t K)
      : ka(&a), kb(&b), sA(stA), sB(stB), kbyte((uint32_t)(k0 * 2)) {
    const int64_t rem = (K - k0) * 2;  // valid bytes of this step's rows
    lim = rem <= 0 ? 0u : (rem >= 128 ? 128u : (uint32_t)rem);
  }
  template <int L>
  __device__ __forceinline__ void one(const KRows& kr, uint8_t* stage, int i) const {
    const uint32_t c = kr.chunk[i & 3];
    // kOOB + (k0 + c) stays >= 2^31, past every record range
    const uint32_t off = c < lim ? kr.row_off[i] + kbyte + c : kOOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(kr.rsrc, (lds_ptr_t)(stage + (wave_id() * L + i) * 1024), 16, off, 0,
                                             0, 0);
  }
  __device__ __forceinline__ void issue(int j) const {
    if (j < kLA) one<kLA>(*ka, sA, j);
    else if constexpr (kLB > 0) one<kLB>(*kb, sB, j - kLA);
  }
};

// Substeps over which a K step's DMA loads are spread.  Issued in one burst
// by all waves right after the barrier, the loads (1 KiB each, 64 KiB per step
// and CU) back each wave's in-order issue up behind the CU's load path while
// the matrix cores idle; interleaved with the first substep's MFMAs they drain
// under matrix-core work and still have three substeps of MFMA time to land
// before the end-of-step wait.  Spreading them further (2 or 4 substeps)
// measured slower: the last loads then land after the wait begins.
constexpr int kDmaSubsteps = 1;

// The MFMAs of one wave on one LDS stage, software-pipelined over the four
// k-substeps: the fragment reads of substep kk + 1 are interleaved with the
// MFMAs of substep kk (1 MFMA, 1 LDS read), so LDS latency and transfer hide
// under matrix-core work and only the first substep's reads are exposed; the
// next K step's DMA loads are interleaved with the MFMAs of the first
// kDmaSubsteps substeps.  The scheduling barriers keep the compiler from
// undoing that order and from hoisting the caller's DMA wait and barrier above
// the MFMAs (they touch no memory, so it otherwise would).
template <int kW, int kR, int KK, class Dma>
__device__ __forceinline__ void mfma_substep(const uint8_t* sA, const uint8_t* sB,
                                             bf16x8_t (&a)[2][Tile<kW, kR>::kMI], bf16x8_t (&b)[2][4],
                                             MfmaAcc<kW, kR>& acc, const Dma& dma) {
  constexpr int MI = Tile<kW, kR>::kMI;
  constexpr int NM = 4 * MI;                                    // MFMAs
  constexpr int cur = KK & 1;
  constexpr int R = KK < 3 ? MI + 4 : 0;                        // reads of the next substep
  constexpr int J0 = KK < kDmaSubsteps ? KK * Dma::kN / kDmaSubsteps : 0;
  constexpr int J1 = KK < kDmaSubsteps ? (KK + 1) * Dma::kN / kDmaSubsteps : 0;
  constexpr int V = J1 - J0;                                    // DMA loads
  if constexpr (KK < 3) read_frags<kW, kR>(sA, sB, KK + 1, a[cur ^ 1], b[cur ^ 1]);
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc.v[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[cur][i], b[cur][j], acc.v[i][j], 0, 0, 0);
#pragma unroll
  for (int j = J0; j < J1; ++j) dma.issue(j);
  // order: after MFMA m comes one read (while reads remain) and the DMA
  // loads whose even share of the NM slots ends there (V may exceed NM)
  static_assert(NM >= 4 && V >= 0 && R >= 0, "substep shape");
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, KK);        // 1 MFMA
    if (m < R) __builtin_amdgcn_sched_group_barrier(0x100, 1, KK);  // 1 LDS read
    const int nv = (m + 1) * V / NM - m * V / NM;
#pragma unroll
    for (int q = 0; q < nv; ++q) __builtin_amdgcn_sched_group_barrier(0x060, 1, KK);  // 1 DMA load
  }
  if constexpr (R > NM) __builtin_amdgcn_sched_group_barrier(0x100, R - NM, KK);
  // one scheduling region per substep
  __builtin_amdgcn_sched_barrier(0);
}

template <int kW, int kR, class Dma>
__device__ __forceinline__ void mfma_stage(const uint8_t* sA, const uint8_t* sB, MfmaAcc<kW, kR>& acc,
                                           const Dma& dma) {
  bf16x8_t a[2][Tile<kW, kR>::kMI], b[2][4];
  read_frags<kW, kR>(sA, sB, 0, a[0], b[0]);
  __builtin_amdgcn_sched_barrier(0);
  // A wave in its MFMA phase takes issue priority over the other wave of its
  // SIMD (which is then typically issuing loads or waiting at the barrier).
  __builtin_amdgcn_s_setprio(1);
  mfma_substep<kW, kR, 0>(sA, sB, a, b, acc, dma);
  mfma_substep<kW, kR, 1>(sA, sB, a, b, acc, dma);
  mfma_substep<kW, kR, 2>(sA, sB, a, b, acc, dma);
  mfma_substep<kW, kR, 3>(sA, sB, a, b, acc, dma);
  __builtin_amdgcn_s_setprio(0);
  __builtin_amdgcn_sched_barrier(0);
}

// Full K loop for one kR x 256 tile.  A is k-contiguous (DMA); B is N x K
// (kBNK, DMA) or K x N (register transpose).  The two stages are distinct LDS
// objects and the loop is unrolled by two, so the compiler can see that a DMA
// into one stage never aliases the MFMA reads of the other and does not wait
// for it.  The loop body has no branches: the K-step count is rounded up to
// even and the loads of steps past K use out-of-range offsets, so they fill
// the stage with zeros (which add nothing) without touching memory; a
// conditional MFMA block would split the accumulators' live ranges and force
// copies.  The caller must have passed a barrier since the previous use.
// K steps [k_begin, k_end) of the tile, accumulated into acc (k_begin a
// multiple of 2 kBK; a range of an even number of steps, except the last of
// K, keeps the step sequence of one whole-K call, so the accumulation order,
// and the bits, are the same however K is cut).  Operand loads stop at k_end:
// columns of A past it are neither read nor needed.
// The stages are LDS arrays of the caller (sA* at least kR x kBK bf16, sB*
// kStageBytes): a kernel that runs tiles of two heights passes the same four
// arrays to both, so they share one allocation.  Everything here is inlined,
// so the compiler still sees four distinct objects.
template <int kW, bool kBNK, int kR>
__device__ __forceinline__ void gemm_tile_range_lds(const KRows& ka, const KRows& kb_nk, const uint16_t* B_kn,
                                                    int64_t N, int64_t n0, int64_t K, int64_t k_begin, int64_t k_end,
                                                    MfmaAcc<kW, kR>& acc, uint8_t* sA0, uint8_t* sB0, uint8_t* sA1,
                                                    uint8_t* sB1) {
  const int64_t nk2 = ((k_end - k_begin + kBK - 1) / kBK + 1) & ~int64_t(1);
  KNLoader<kW> kn;
  if constexpr (!kBNK) {
    kn.init(B_kn, K, N, n0);
    kn.load(k_begin);
  }
  dma_stage<kW, kR>(ka, sA0, k_begin, k_end);
  if constexpr (kBNK) dma_stage<kW>(kb_nk, sB0, k_begin, k_end);
  else kn.store(sB0);
  wait_dma();
  __syncthreads();
  for (int64_t kt = 0; kt < nk2; kt += 2) {
    const int64_t k1 = k_begin + (kt + 1) * kBK, k2 = k_begin + (kt + 2) * kBK;
    // stage 0 computes while stage 1 fills
    if constexpr (!kBNK) kn.load(k1);
    mfma_stage<kW, kR>(sA0, sB0, acc, StepDma<kW, kR, kBNK>(ka, kb_nk, sA1, sB1, k1, k_end));
    if constexpr (!kBNK) kn.store(sB1);
    wait_dma();
    __syncthreads();
    // stage 1 computes while stage 0 fills (past the end: zeros, unused)
    if constexpr (!kBNK) kn.load(k2);
    mfma_stage<kW, kR>(sA1, sB1, acc, StepDma<kW, kR, kBNK>(ka, kb_nk, sA0, sB0, k2, k_end));
    if constexpr (!kBNK) kn.store(sB0);
    wait_dma();
    __syncthreads();
  }
}

// ---- five-slot ring: the 8-wave tile with both operands by DMA ----
// LDS holds five 32 KiB slots, each one operand's K step in the step loop's
// layout.  One operand leads: the slots take lead_0 follow_0 lead_1 follow_1
// ... (item i in slot i % 5), so while step s reads both operands of step s
// the loads of follow_{s+1} and lead_{s+2} are in flight: the lead operand is
// loaded two steps ahead and the other one.  Each step's loads are still
// interleaved with the first substep's MFMAs, and each step ends with one
// barrier.  The lead goes to the operand whose loads miss the L2 and the MALL
// more (measured per kernel: the gathered rows of the AllGather consumer).
__device__ __forceinline__ void bar_raw() { asm volatile("s_barrier" ::: "memory"); }

// At most N (0, 2, 4) of this wave's vector memory operations in flight.  The
// compiler's own wait counting sees this builtin (it does not see an asm
// wait), so it knows which loads are in when the next step reads their slots.
// Encoding (gfx9): vmcnt in bits 3:0, expcnt (bits 6:4) and lgkmcnt (11:8) at
// their maxima.
template <int N>
__device__ __forceinline__ void wait_vm_ring() {
  static_assert(N == 0 || N == 2 || N == 4, "loads left in flight");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// Loads per wave of one operand's K step (8 waves): 8 rows each.
template <int kRows>
constexpr int ring_loads() {
  return kRows / 8 / 8;
}

// A ring step's loads: this wave's loads of the follow operand for step s + 1,
// then its loads of the lead operand for step s + 2.
template <int kR, bool kLeadA>
struct StepDmaR5 {
  static constexpr int kLA = ring_loads<kR>(), kLB = ring_loads<kBM>();
  static constexpr int kLF = kLeadA ? kLB : kLA, kN = kLA + kLB;  // follow loads go first
  const KRows* ka;
  const KRows* kb;
  uint8_t* sA;
  uint8_t* sB;
  uint32_t kbA, limA, kbB, limB;
  static __device__ __forceinline__ uint32_t lim_of(int64_t k0, int64_t K) {
    const int64_t rem = (K - k0) * 2;  // valid bytes of the step's rows
    return rem <= 0 ? 0u : (rem >= 128 ? 128u : (uint32_t)rem);
  }
  __device__ __forceinline__ StepDmaR5(const KRows& a, const KRows& b, uint8_t* stA, uint8_t* stB, int64_t kA,
                                       int64_t kB, int64_t K)
      : ka(&a), kb(&b), sA(stA), sB(stB), kbA((uint32_t)(kA * 2)), limA(lim_of(kA, K)), kbB((uint32_t)(kB * 2)),
        limB(lim_of(kB, K)) {}
  template <int L>
  __device__ __forceinline__ void one(const KRows& kr, uint8_t* stage, int i, uint32_t kbyte, uint32_t lim) const {
    const uint32_t c = kr.chunk[i & 3];
    // kOOB + (k0 + c) stays >= 2^31, past every record range
    const uint32_t off = c < lim ? kr.row_off[i] + kbyte + c : kOOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(kr.rsrc, (lds_ptr_t)(stage + (wave_id() * L + i) * 1024), 16, off, 0,
                                             0, 0);
  }
  __device__ __forceinline__ void issue(int j) const {
    if constexpr (kLeadA) {
      if (j < kLB) one<kLB>(*kb, sB, j, kbB, limB);
      else one<kLA>(*ka, sA, j - kLB, kbA, limA);
    } else {
      if (j < kLA) one<kLA>(*ka, sA, j, kbA, limA);
      else one<kLB>(*kb, sB, j - kLA, kbB, limB);
    }
  }
};

// Step s of the ring: read the lead operand of step s from slot RL and the
// follow operand from RF; load follow_{s+1} into WF and lead_{s+2} into WL (the
// slots step s - 1 read, free since its barrier); then wait until at most this
// step's lead loads (the last issued) are in flight, so both operands of step
// s + 1 are in, and pass the barrier.  False after the range's last step.
template <int kR, bool kLeadA, int RL, int RF, int WF, int WL>
__device__ __forceinline__ bool r5_step(uint8_t* const (&slot)[5], const KRows& ka, const KRows& kb, int64_t k_begin,
                                        int64_t k_end, int64_t& s, int64_t nk2, MfmaAcc<8, kR>& acc) {
  using D = StepDmaR5<kR, kLeadA>;
  const int64_t kF = k_begin + (s + 1) * kBK, kL = k_begin + (s + 2) * kBK;
  uint8_t* const rA = kLeadA ? slot[RL] : slot[RF];
  uint8_t* const rB = kLeadA ? slot[RF] : slot[RL];
  if constexpr (kLeadA) mfma_stage<8, kR>(rA, rB, acc, D(ka, kb, slot[WL], slot[WF], kL, kF, k_end));
  else mfma_stage<8, kR>(rA, rB, acc, D(ka, kb, slot[WF], slot[WL], kF, kL, k_end));
  wait_vm_ring<kLeadA ? D::kLA : D::kLB>();
  bar_raw();
  return ++s < nk2;
}

// K steps [k_begin, k_end) of a kR x 256 tile on the ring (A and B stored
// N x K, KRows in the step loop's 8-wave layout), accumulated into acc.  The
// step count is rounded up to even and the steps past K load zeros, as in the
// step loop, so the MFMAs and their order, and the bits, are the same.  The
// slots are 32 KiB LDS arrays of the caller, who must have passed a barrier
// since their previous use; the first loads go to slots 0-2, the first step's
// to 3 and 4.  On return no load is in flight and every wave has passed a
// barrier after its last read.  Item i = 2 s (lead) or 2 s + 1 (follow) of
// step s sits in slot i % 5, so the slots repeat every five steps (the loop
// body).
template <int kR, bool kLeadA>
__device__ __forceinline__ void gemm_tile_range_r5(const KRows& ka, const KRows& kb, int64_t k_begin, int64_t k_end,
                                                   MfmaAcc<8, kR>& acc, uint8_t* s0, uint8_t* s1, uint8_t* s2,
                                                   uint8_t* s3, uint8_t* s4) {
  using D = StepDmaR5<kR, kLeadA>;
  uint8_t* const slot[5] = {s0, s1, s2, s3, s4};
  const int64_t nk2 = ((k_end - k_begin + kBK - 1) / kBK + 1) & ~int64_t(1);
  auto dma_lead = [&](uint8_t* st, int64_t k0) {
    if constexpr (kLeadA) dma_stage<8, kR>(ka, st, k0, k_end);
    else dma_stage<8>(kb, st, k0, k_end);
  };
  auto dma_follow = [&](uint8_t* st, int64_t k0) {
    if constexpr (kLeadA) dma_stage<8>(kb, st, k0, k_end);
    else dma_stage<8, kR>(ka, st, k0, k_end);
  };
  dma_lead(s0, k_begin);
  dma_follow(s1, k_begin);
  dma_lead(s2, k_begin + kBK);
  // All three in before the loop.  Leaving lead_1 in flight here (it lands soon
  // after follow_0) makes the compiler's wait counting, which cannot tell
  // these loads from the loop's own at the loop head, wait for every load at
  // the head of each five-step body instead.
  wait_vm_ring<0>();
  bar_raw();
  int64_t s = 0;
  while (r5_step<kR, kLeadA, 0, 1, 3, 4>(slot, ka, kb, k_begin, k_end, s, nk2, acc) &&
         r5_step<kR, kLeadA, 2, 3, 0, 1>(slot, ka, kb, k_begin, k_end, s, nk2, acc) &&
         r5_step<kR, kLeadA, 4, 0, 2, 3>(slot, ka, kb, k_begin, k_end, s, nk2, acc) &&
         r5_step<kR, kLeadA, 1, 2, 4, 0>(slot, ka, kb, k_begin, k_end, s, nk2, acc) &&
         r5_step<kR, kLeadA, 3, 4, 1, 2>(slot, ka, kb, k_begin, k_end, s, nk2, acc)) {
  }
  // the loads issued by the last steps (zeros past k_end) land before the slots are used again
  wait_dma();
  bar_raw();
}

template <int kW, bool kBNK, int kR = kBM>
__device__ __forceinline__ void gemm_tile_range(const KRows& ka, const KRows& kb_nk, const uint16_t* B_kn, int64_t N,
                                                int64_t n0, int64_t K, int64_t k_begin, int64_t k_end,
                                                MfmaAcc<kW, kR>& acc) {
  __shared__ __attribute__((aligned(1024))) uint8_t sA0[kR * kBK * 2];
  __shared__ __attribute__((aligned(1024))) uint8_t sB0[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sA1[kR * kBK * 2];
  __shared__ __attribute__((aligned(1024))) uint8_t sB1[kStageBytes];
  gemm_tile_range_lds<kW, kBNK, kR>(ka, kb_nk, B_kn, N, n0, K, k_begin, k_end, acc, sA0, sB0, sA1, sB1);
}

template <int kW, bool kBNK, int kR = kBM>
__device__ __forceinline__ void gemm_tile(const KRows& ka, const KRows& kb_nk, const uint16_t* B_kn, int64_t N,
                                          int64_t n0, int64_t K, MfmaAcc<kW, kR>& acc) {
  acc_zero<kW, kR>(acc);
  gemm_tile_range<kW, kBNK, kR>(ka, kb_nk, B_kn, N, n0, K, 0, K, acc);
}

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Store the tile to a row-major M x N output (ldc = N) at (m0, n0); elements
// outside the matrix are dropped.  kOutBf16: round to bf16, else fp32.  kCpol:
// cache policy of the stores (16 = sc1, device scope, for tiles that other
// workgroups read back in the same kernel).
// Accumulator (i, j, r) of a lane is tile row wm * rows_per_wave + 32 i +
// 8 (r / 4) + 4 (lane / 32) + r % 4, column 128 wn + 32 j + lane % 32: the
// 32 x 32 MFMA result puts column lane % 32 in a lane and those rows in its
// 16 registers.
template <int kW, bool kOutBf16, int kCpol = 0, int kR = kBM>
__device__ __forceinline__ void store_tile(void* C, int64_t M, int64_t N, int64_t m0, int64_t n0,
                                           const MfmaAcc<kW, kR>& acc) {
  const int esz = kOutBf16 ? 2 : 4;
  const uint8_t* base = static_cast<const uint8_t*>(C) + (m0 * N + n0) * esz;
  // Record range: from the tile origin to the end of its last valid row (at most
  // 256 rows, < 2^31 bytes), so an offset of kOOB or more is always dropped.
  const int64_t rows = M - m0 < kR ? M - m0 : kR;
  const int64_t valid = rows * N - n0;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, valid > 0 ? (uint64_t)valid * esz : 0u);
  const int lane = threadIdx.x & 63, w = wave_id();
  const int lr = lane & 31, lk = lane >> 5;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int col = (w & 1) * 128 + j * 32 + lr;
    const uint32_t voff = (n0 + col < N) ? (uint32_t)((4 * lk * N + col) * esz) : kOOB;
#pragma unroll
    for (int i = 0; i < Tile<kW, kR>::kMI; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = (w >> 1) * Tile<kW, kR>::kWaveRows + i * 32 + 8 * (r >> 2) + (r & 3);  // + 4 lk in voff
        // kOOB + (row offset < 2^31) stays out of range: no select needed
        const uint32_t off = voff + (uint32_t)(row * N * esz);
        if constexpr (kOutBf16)
          __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_rne(acc.v[i][j][r]), rs, off, 0, kCpol);
        else
          // the builtin's data operand is an integer: pass the float's bits, not its value
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc.v[i][j][r]), rs, off, 0, kCpol);
      }
    // bound live ranges: one column of MFMA blocks at a time
    __builtin_amdgcn_sched_barrier(0);
  }
}

}  // namespace sgt
