// Shared tile pipeline of the MFMA kernels (tiled forward and tiled backward): a 256 x 256
// output tile of bf16 x bf16 -> fp32 products with K = 64 per step.
//
//   * 256 threads = 4 wavefronts, one per SIMD; wavefront (wm, wn) owns rows 128 wm .. +128
//     and columns 128 wn .. +128 of the tile: 4 x 4 accumulators of
//     v_mfma_f32_32x32x16_bf16 (256 fp32 per lane, in the accumulation registers).
//   * Both operands are K-major ("A[M][K] times B[N][K]^T").  A 256-row panel of A and a
//     256-row tile of B go from global memory straight into LDS (global_load_lds_dwordx4,
//     no registers) through a ring of two 64 KB stages; every staged row of a step is one
//     whole 128-byte line.  Each lane picks its global source so that the 16-byte chunks
//     land XOR-swizzled by row (conflict-free ds_read_b128).
//   * Stage map: A half at [0, 64 KB), B half at [64 KB, 128 KB).
//   * kloop8 / Acc8: the same product with 512 threads = 8 wavefronts, two per SIMD.
//     Wavefront w owns rows 64 (w % 4) .. +64 and columns 128 (w / 4) .. +128 of the tile:
//     2 x 4 accumulators (128 fp32 per lane).  The two groups of four wavefronts (w / 4 =
//     0, 1) take turns: while one group issues the MFMAs of a step, the other reads its
//     fragments of the next step from LDS and issues the ring's DMA, and the two swap at a
//     workgroup barrier; the MFMA phase runs at raised wave priority.
#pragma once

#include "lrq_internal.h"

namespace lrq {
namespace tile {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 64;
constexpr int kRowBytes = BK * 2;            // one staged row: 64 bf16 = 128 bytes
constexpr int kTileBytes = BM * kRowBytes;   // 32 KB per operand per stage
constexpr int kSlices = BK / 16;             // 16-wide MFMA K slices per step
constexpr int kStageA = 0;                   // 2 x [256][64] bf16
constexpr int kStageB = 2 * kTileBytes;      // 2 x [256][64] bf16
constexpr int kRingBytes = 4 * kTileBytes;   // 128 KB
constexpr int kLdsMax = 160 * 1024;

// XOR pattern of the 16-byte chunks of staged row `row`.  Any 16 consecutive rows read at
// one logical chunk hit 16 distinct 16-byte bank groups of a 256-byte window
// (ds_read_b128 serves 16 lanes per cycle from 64 banks), and any 8 consecutive rows hit 8
// distinct groups of a 128-byte window.
__device__ __forceinline__ int chunk_xor(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// byte offset of logical 16-byte chunk `chunk` (0..7) of row `row` in a [rows][64] bf16 tile
__device__ __forceinline__ int swz(int row, int chunk) { return row * kRowBytes + ((chunk ^ chunk_xor(row)) << 4); }

__device__ __forceinline__ float lo_bf16(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// 16 bytes per lane from global memory into LDS at byte address lds + 16 * lane (lds is
// wave-uniform).  Written as inline assembly on purpose: the compiler then neither counts
// these loads nor makes every later LDS read wait for all of them; the stage ring waits
// for exactly the stage it needs (wait_barrier).  Loads the compiler does not know about
// can only make its own vmcnt waits longer, never too short.  The destination goes in M0
// (the compiler sets it); M0 needs one wait state after it is written.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(lds) : "memory");
}

// The same with a wave-uniform base address in scalar registers and a 32-bit byte offset per
// lane: per-lane state of one VGPR per distinct row instead of a 64-bit pointer.
__device__ __forceinline__ void dma16s(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds) : "memory");
}

// LDS byte address of a pointer into a __shared__ array (the low half of its flat address).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

// s_waitcnt vmcnt(N) lgkmcnt(0), then a workgroup barrier; the empty asm statements keep
// the compiler from moving LDS accesses across it.
template <int N>
__device__ __forceinline__ void wait_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Barrier once this wave's LDS reads have completed (its DMA may stay in flight).
__device__ __forceinline__ void barrier_lds() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ void barrier_all() { wait_barrier<0>(); }

// Keeps the compiler's scheduler from moving instructions across this point.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// ss += sum of squares of the 8 bf16 values of a fragment (products exact, fp32 sums)
__device__ __forceinline__ void sumsq8(const bf16x8& x, float& ss) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const bf16x2 v = {x[2 * e], x[2 * e + 1]};
    ss = __builtin_amdgcn_fdot2_f32_bf16(v, v, ss, false);
  }
}

// Per-wave state of one tile.
struct Acc {
  floatx16 acc[4][4];
  float ss[4];  // sums of squares (halves) of A rows 32 i + lane % 32 of the wave pair
};

// Fragments of one 16-wide K slice: rows of the A panel and of the B tile.
struct Frags {
  bf16x8 a[4], b[4];
};

__device__ __forceinline__ void read_frags(Frags& f, const unsigned char* xs, const unsigned char* ws, int kk, int wm,
                                           int wn, int l32, int h32) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    f.a[i] = *reinterpret_cast<const bf16x8*>(xs + swz(wm * 128 + i * 32 + l32, kk * 2 + h32));
#pragma unroll
  for (int j = 0; j < 4; ++j)
    f.b[j] = *reinterpret_cast<const bf16x8*>(ws + swz(wn * 128 + j * 32 + l32, kk * 2 + h32));
}

// The four MFMAs of row block i of one slice.
__device__ __forceinline__ void mfma_row(Acc& ta, const Frags& f, int i) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    ta.acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], ta.acc[i][j], 0, 0, 0);
}

// Sums of squares of the wave's four A row blocks of one slice (both waves of a pair
// gather the same sums; selecting half of the blocks per wave costs more than it saves).
__device__ __forceinline__ void slice_stats(Acc& ta, const Frags& f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) sumsq8(f.a[i], ta.ss[i]);
}

// Per-lane DMA sources.  Instruction c (0..7) of wave w fills rows R = 64 w + 8 c + lane / 8
// of a stage; the lane's 16 bytes land in physical chunk lane % 8, which holds logical
// chunk (lane % 8) ^ chunk_xor(R) = (lane % 8) ^ (lane / 8) ^ (c & 1).
// Two forms of the A sources: Src holds the eight row pointers; SrcC forms a row's address
// where its load is issued, from one base pointer and the lane's first row.  Eight 64-bit
// pointers live through a whole K loop are what the register allocator spills in a kernel
// with a heavy epilogue, and every reload of a spilled pointer in the loop makes the wave
// wait for all of its loads in flight (the stage ring drains); the compact form avoids that
// at the price of a few VALU instructions per load, and can push spills elsewhere instead,
// so each kernel takes the form it measures faster with.
struct Src {
  const uint16_t* a[8];  // A row per instruction; rows past the panel's end re-read its last row
  const uint16_t* b[2];  // B row 64 w + lane / 8 of column tile 0, for even / odd c
  int64_t ldb;           // row stride of B (elements)
};
struct SrcC {
  const uint16_t* a_even;  // A + the lane's logical chunk of even instructions
  int64_t lda;             // row stride of A (elements)
  int row_first;           // panel row of instruction 0 for this lane
  int row_last;            // rows past the panel's end re-read this one (never stored)
  int a_odd;               // element offset of the odd instructions' chunk (+8 or -8)
  const uint16_t* b[2];
  int64_t ldb;
};

// The lane's first row as a value the compiler cannot treat as loop-invariant (so it does
// not hoist the eight addresses out of the loop).
__device__ __forceinline__ int opaque_row(int r) {
  asm volatile("" : "+v"(r));
  return r;
}
// A wave-uniform value the compiler cannot see through: addresses formed from it stay where
// they are written instead of being formed once at kernel entry and spilled.
__device__ __forceinline__ int opaque_s(int v) {
  asm volatile("" : "+s"(v));
  return v;
}
// A row of instruction c; `rf` from issue_row(s), taken once per group of loads
__device__ __forceinline__ int issue_row(const Src&) { return 0; }
__device__ __forceinline__ const uint16_t* src_a(const Src& s, int c, int) { return s.a[c]; }
__device__ __forceinline__ int issue_row(const SrcC& s) { return opaque_row(s.row_first); }
__device__ __forceinline__ const uint16_t* src_a(const SrcC& s, int c, int rf) {
  const int row = min(rf + 8 * c, s.row_last);
  return s.a_even + static_cast<int64_t>(row) * s.lda + ((c & 1) ? s.a_odd : 0);
}

// Sources for the A panel rows [row0, row0 + 256) of A (stride lda; rows >= rows_valid
// re-read row rows_valid - 1, whose results are never stored) and the B rows (stride ldb).
__device__ __forceinline__ Src make_src(const uint16_t* A, int64_t lda, int64_t row0, int64_t rows_valid,
                                        const uint16_t* B, int64_t ldb, int wave, int lane) {
  Src s;
  const int pc = lane & 7;
  const int rsub = lane >> 3;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int R = 64 * wave + 8 * c + rsub;
    const int64_t row = min(row0 + R, rows_valid - 1);
    s.a[c] = A + row * lda + (pc ^ chunk_xor(R)) * 8;
  }
  // chunk_xor(64 w + 8 c + rsub) = rsub ^ (c & 1)
  s.b[0] = B + static_cast<int64_t>(64 * wave + rsub) * ldb + (pc ^ rsub) * 8;
  s.b[1] = B + static_cast<int64_t>(64 * wave + rsub) * ldb + (pc ^ rsub ^ 1) * 8;
  s.ldb = ldb;
  return s;
}

// The same sources in the compact form (row indices fit in 32 bits: the library limits T).
__device__ __forceinline__ SrcC make_src_c(const uint16_t* A, int64_t lda, int64_t row0, int64_t rows_valid,
                                           const uint16_t* B, int64_t ldb, int wave, int lane) {
  SrcC s;
  const int pc = lane & 7;
  const int rsub = lane >> 3;
  s.a_even = A + (pc ^ rsub) * 8;
  s.a_odd = ((pc ^ rsub ^ 1) - (pc ^ rsub)) * 8;
  s.lda = lda;
  s.row_first = static_cast<int>(row0) + 64 * wave + rsub;
  s.row_last = static_cast<int>(rows_valid - 1);
  // chunk_xor(64 w + 8 c + rsub) = rsub ^ (c & 1)
  s.b[0] = B + static_cast<int64_t>(64 * wave + rsub) * ldb + (pc ^ rsub) * 8;
  s.b[1] = B + static_cast<int64_t>(64 * wave + rsub) * ldb + (pc ^ rsub ^ 1) * 8;
  s.ldb = ldb;
  return s;
}

// One tile's K-loop over nk steps: acc = A_panel B_tile^T, B_tile = B rows [col0, col0 + 256);
// with STATS also the A rows' sums of squares.
//
//   prologue: DMA stages 0 and 1; wait for stage 0; read slice (0, 0)
//   step ks:  read (ks, 1) | MFMA (ks, 0) | read (ks, 2) | MFMA (ks, 1) | read (ks, 3) |
//             MFMA (ks, 2) | wait for stage ks + 1, barrier | MFMA (ks, 3) with the 16 DMA
//             instructions of stage ks + 2 (into buffer ks % 2) spread between its rows
//             and the read of (ks + 1, 0)
// After the barrier of step ks every wave holds the rest of stage ks in registers, so that
// buffer is free.  Spreading the DMA keeps the wave from stalling on a full address queue
// while the matrix core waits.  sched_fence() pins the interleaving.
// Options, for kernels whose register allocation does better with them:
//   kOpqPrologue: form the prologue's addresses where they are used (see below);
//   kXorReads: form each slice's LDS read addresses from one per-lane offset per operand:
//     slice kk's 16-byte chunk is slice 0's XOR 2 kk (the swizzle is an XOR of the row's
//     bits), so the byte offset is slice 0's XOR (kk << 5), with kk << 5 opaque so the four
//     offsets are not formed ahead and kept (or spilled) for the whole loop.
constexpr int kOpqPrologue = 1, kXorReads = 2;
template <bool STATS, int OPT = kOpqPrologue, typename S>
__device__ __forceinline__ void kloop(unsigned char* smem, Acc& ta, const S& src, int64_t col0, int nk, int wave,
                                      int lane) {
  constexpr int kLoads = 16;  // DMA instructions per stage and wave
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, h32 = lane >> 5;
  const int64_t d = src.ldb;
  const uint32_t sbase = lds_addr(smem);
  const uint16_t* w0 = src.b[0] + col0 * d;
  const uint16_t* w1 = src.b[1] + col0 * d;

  auto issue_x = [&](int ks, int c0) {
    const uint32_t xs = sbase + kStageA + (ks & 1) * kTileBytes + wave * 8192;
    const int rf = issue_row(src);
#pragma unroll
    for (int c = c0; c < c0 + 4; ++c) dma16(src_a(src, c, rf) + ks * BK, xs + c * 1024);
  };
  auto issue_w = [&](int ks, int c0) {
    const uint32_t ws = sbase + kStageB + (ks & 1) * kTileBytes + wave * 8192;
#pragma unroll
    for (int c = c0; c < c0 + 4; ++c)
      dma16(((c & 1) ? w1 : w0) + static_cast<int64_t>(8 * c) * d + ks * BK, ws + c * 1024);
  };
  // instructions c0, c0 + 1 of the x / W' loads of step ks
  auto issue_x2 = [&](int ks, int c0) {
    const uint32_t xs = sbase + kStageA + (ks & 1) * kTileBytes + wave * 8192;
    const int rf = issue_row(src);
    dma16(src_a(src, c0, rf) + ks * BK, xs + c0 * 1024);
    dma16(src_a(src, c0 + 1, rf) + ks * BK, xs + (c0 + 1) * 1024);
  };
  auto issue_w2 = [&](int ks, int c0) {
    const uint32_t ws = sbase + kStageB + (ks & 1) * kTileBytes + wave * 8192;
    dma16(w0 + static_cast<int64_t>(8 * c0) * d + ks * BK, ws + c0 * 1024);
    dma16(w1 + static_cast<int64_t>(8 * (c0 + 1)) * d + ks * BK, ws + (c0 + 1) * 1024);
  };
  auto sx = [&](int ks) { return smem + kStageA + (ks & 1) * kTileBytes; };
  auto sw = [&](int ks) { return smem + kStageB + (ks & 1) * kTileBytes; };
  const int ra0 = swz(wm * 128 + l32, h32), rb0 = swz(wn * 128 + l32, h32);
  auto rd = [&](Frags& f, const unsigned char* xs, const unsigned char* ws, int kk) {
    if constexpr ((OPT & kXorReads) != 0) {
      const int m = opaque_s(kk << 5);
      const unsigned char* xa = xs + (ra0 ^ m);
      const unsigned char* wb = ws + (rb0 ^ m);
#pragma unroll
      for (int i = 0; i < 4; ++i) f.a[i] = *reinterpret_cast<const bf16x8*>(xa + i * 32 * kRowBytes);
#pragma unroll
      for (int j = 0; j < 4; ++j) f.b[j] = *reinterpret_cast<const bf16x8*>(wb + j * 32 * kRowBytes);
    } else {
      read_frags(f, xs, ws, kk, wm, wn, l32, h32);
    }
  };

  // The prologue's step index is opaque: with constant steps the compiler forms these
  // addresses (and the first fragment reads') at kernel entry, spills them over the
  // epilogue, and reloads each one right before its load, which makes every load wait for
  // all loads in flight.
  const int k0 = (OPT & kOpqPrologue) ? opaque_s(0) : 0;
  issue_x(k0, 0);
  issue_x(k0, 4);
  issue_w(k0, 0);
  issue_w(k0, 4);
  if (nk > 1) {
    issue_x(k0 + 1, 0);
    issue_x(k0 + 1, 4);
    issue_w(k0 + 1, 0);
    issue_w(k0 + 1, 4);
    wait_barrier<kLoads>();
  } else {
    wait_barrier<0>();
  }
  // slices 0..2 of step ks: MFMAs on (fa, fb, fa) with the next slice read ahead
  auto first3 = [&](int ks, Frags& fa, Frags& fb) {
    const unsigned char* xs = sx(ks);
    const unsigned char* ws = sw(ks);
    sched_fence();
    rd(fb, xs, ws, 1);
    sched_fence();
#pragma unroll
    for (int i = 0; i < 4; ++i) mfma_row(ta, fa, i);
    if (STATS) slice_stats(ta, fa);
    sched_fence();
    rd(fa, xs, ws, 2);
    sched_fence();
#pragma unroll
    for (int i = 0; i < 4; ++i) mfma_row(ta, fb, i);
    if (STATS) slice_stats(ta, fb);
    sched_fence();
    rd(fb, xs, ws, 3);
    sched_fence();
#pragma unroll
    for (int i = 0; i < 4; ++i) mfma_row(ta, fa, i);
    if (STATS) slice_stats(ta, fa);
    sched_fence();
  };

  Frags fa, fb;
  rd(fa, sx(k0), sw(k0), 0);
  // all steps but the last (the last has no barrier, DMA or read-ahead; peeling it keeps
  // every accumulator update out of conditional code)
  for (int ks = 0; ks + 1 < nk; ++ks) {
    first3(ks, fa, fb);
    wait_barrier<0>();  // stage ks + 1 landed (nothing later is in flight)
    const bool more = ks + 2 < nk;
    sched_fence();
    mfma_row(ta, fb, 0);
    sched_fence();
    if (more) {
      issue_x2(ks + 2, 0);
      issue_w2(ks + 2, 0);
    }
    sched_fence();
    mfma_row(ta, fb, 1);
    sched_fence();
    if (more) {
      issue_x2(ks + 2, 2);
      issue_w2(ks + 2, 2);
    }
    sched_fence();
    mfma_row(ta, fb, 2);
    sched_fence();
    if (more) {
      issue_x2(ks + 2, 4);
      issue_w2(ks + 2, 4);
    }
    sched_fence();
    rd(fa, sx(ks + 1), sw(ks + 1), 0);
    sched_fence();
    mfma_row(ta, fb, 3);
    sched_fence();
    if (more) {
      issue_x2(ks + 2, 6);
      issue_w2(ks + 2, 6);
    }
    if (STATS) slice_stats(ta, fb);
  }
  first3(nk - 1, fa, fb);
#pragma unroll
  for (int i = 0; i < 4; ++i) mfma_row(ta, fb, i);
  if (STATS) slice_stats(ta, fb);
  sched_fence();
  barrier_all();  // every wave is done with the stage ring
}

// ------------------------------------------------------------------ 8-wavefront products
constexpr int kThreads8 = 512;

// Per-wave accumulators of one tile: rows 64 wm + 32 i + (lane layout), columns
// 128 wn + 32 j + l32.
struct Acc8 {
  floatx16 acc[2][4];
};

// Per-lane DMA sources of the 8-wavefront pipeline.  Instruction c (0..3) of wave w fills
// rows R = 32 w + 8 c + lane / 8 of the A and the B half of a stage (logical chunk
// (lane % 8) ^ chunk_xor(R) = (lane % 8) ^ (lane / 8) ^ (c & 1) lands in physical chunk
// lane % 8).  Addresses are a wave-uniform base (scalar registers, formed per load) plus a
// 32-bit byte offset per lane: six VGPRs of state instead of eight 64-bit pointers, which the
// register allocator spilled -- and each reload of a spilled pointer in the K loop waited for
// every load in flight.  The library's limits (K < 2^19 columns, 256-row panels) keep every
// offset below 2^32.
struct Src8 {
  const char* a_base;  // A + row0 * lda, bytes
  uint32_t a_off[4];   // (min(row0 + R, rows_valid - 1) - row0) * lda * 2 + 16 * chunk
  const char* b_base;  // B + 32 w * ldb, bytes (column tile 0)
  uint32_t b_off[2];   // (lane / 8) * ldb * 2 + 16 * chunk, even / odd instructions
  int64_t ldb;
  // K steps >= nk1 read B from a second matrix `tail` (row stride ld_tail) at K offset
  // 64 (ks - nk1); its lane offsets are formed in those steps only
  const uint16_t* tail;
  int64_t ld_tail;
  int nk1;
};

// B = [B1 | B2]: K steps [0, nk1) from B1 (stride ldb), the rest from B2 (stride ld2).
__device__ __forceinline__ Src8 make_src8(const uint16_t* A, int64_t lda, int64_t row0, int64_t rows_valid,
                                          const uint16_t* B, int64_t ldb, int nk1, const uint16_t* B2,
                                          int64_t ld2, int wave, int lane) {
  Src8 s;
  const int pc = lane & 7, rsub = lane >> 3;
  s.a_base = reinterpret_cast<const char*>(A + row0 * lda);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int R = 32 * wave + 8 * c + rsub;
    const int64_t row = min(row0 + R, rows_valid - 1) - row0;
    s.a_off[c] = static_cast<uint32_t>(row * lda * 2 + (pc ^ chunk_xor(R)) * 16);
  }
  s.b_base = reinterpret_cast<const char*>(B + static_cast<int64_t>(32 * wave) * ldb);
  s.b_off[0] = static_cast<uint32_t>(rsub * ldb * 2 + (pc ^ rsub) * 16);
  s.b_off[1] = static_cast<uint32_t>(rsub * ldb * 2 + (pc ^ rsub ^ 1) * 16);
  s.ldb = ldb;
  s.tail = B2;
  s.ld_tail = ld2;
  s.nk1 = nk1;
  return s;
}

// workgroup barrier that the compiler's scheduler does not move instructions across
__device__ __forceinline__ void fenced_barrier() {
  sched_fence();
  __builtin_amdgcn_s_barrier();
  sched_fence();
}

// kloop with 8 wavefronts: acc = A_panel B_tile^T, B_tile = B rows [col0, col0 + 256) (B as
// set up by make_src8: two matrices side by side along K).
// Called by all 8 wavefronts; leaves the stage ring free.
//
// Step ks is two intervals between workgroup barriers.  Group 0 reads the fragments of
// stage ks (all four 16-wide slices) in interval 2 ks and multiplies in 2 ks + 1; group 1
// is one interval behind.  The DMA of stage ks + 1 goes out in interval 2 ks (group 0 at
// the start of its read phase, group 1 at the start of its MFMA phase for step ks - 1),
// into the buffer of stage ks - 1, which both groups finished reading in interval 2 ks - 1;
// every wave waits for its own part of stage ks + 1 at the end of interval 2 ks + 1, so
// the stage is complete when group 0 reads it in interval 2 ks + 2.
__device__ __forceinline__ void kloop8(unsigned char* smem, Acc8& ta, const Src8& src, int64_t col0, int nk, int wave,
                                      int lane) {
  const int g = wave >> 2;
  const int wm = wave & 3, wn = g;
  const int l32 = lane & 31, h32 = lane >> 5;
  const uint32_t sbase = lds_addr(smem);
  const int64_t boff = col0 * src.ldb;

  auto issue = [&](int ks) {
    const uint32_t xa = sbase + kStageA + (ks & 1) * kTileBytes + wave * 4096;
    const uint32_t xb = sbase + kStageB + (ks & 1) * kTileBytes + wave * 4096;
    const char* ab = src.a_base + static_cast<int64_t>(ks) * BK * 2;
    if (ks < src.nk1) {
      const char* bb = src.b_base + (boff + static_cast<int64_t>(ks) * BK) * 2;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        dma16s(ab, src.a_off[c], xa + c * 1024);
        dma16s(bb + static_cast<int64_t>(8 * c) * src.ldb * 2, src.b_off[c & 1], xb + c * 1024);
      }
    } else {
      const int64_t kt = static_cast<int64_t>(ks - src.nk1) * BK;
      const int rsub = lane >> 3, pc = lane & 7;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const char* tb = reinterpret_cast<const char*>(src.tail + (col0 + 32 * wave + 8 * c) * src.ld_tail + kt);
        const uint32_t toff = static_cast<uint32_t>(rsub * src.ld_tail * 2 + (pc ^ rsub ^ (c & 1)) * 16);
        dma16s(ab, src.a_off[c], xa + c * 1024);
        dma16s(tb, toff, xb + c * 1024);
      }
    }
  };
  bf16x8 fa[kSlices][2], fb[kSlices][4];
  auto read = [&](int ks) {
    const unsigned char* xs = smem + kStageA + (ks & 1) * kTileBytes;
    const unsigned char* ws = smem + kStageB + (ks & 1) * kTileBytes;
#pragma unroll
    for (int s = 0; s < kSlices; ++s) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
        fa[s][i] = *reinterpret_cast<const bf16x8*>(xs + swz(wm * 64 + i * 32 + l32, s * 2 + h32));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        fb[s][j] = *reinterpret_cast<const bf16x8*>(ws + swz(wn * 128 + j * 32 + l32, s * 2 + h32));
    }
  };
  auto multiply = [&]() {
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int s = 0; s < kSlices; ++s) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          ta.acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[s][i], fb[s][j], ta.acc[i][j], 0, 0, 0);
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // s_waitcnt encodings: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8
  constexpr int kLgkm0 = 15 | (3 << 14) | (7 << 4) | (0 << 8);
  constexpr int kVm0Lgkm0 = 0 | (0 << 14) | (7 << 4) | (0 << 8);
  constexpr int kVm0 = 0 | (0 << 14) | (7 << 4) | (15 << 8);

  issue(0);
  wait_barrier<0>();
  if (g == 1) {
    if (nk > 1) issue(1);
    fenced_barrier();
  }
  for (int ks = 0; ks < nk; ++ks) {
    sched_fence();
    if (g == 0 && ks + 1 < nk) issue(ks + 1);
    sched_fence();
    read(ks);
    sched_fence();
    if (g == 1)
      __builtin_amdgcn_s_waitcnt(kVm0Lgkm0);
    else
      __builtin_amdgcn_s_waitcnt(kLgkm0);
    fenced_barrier();
    if (g == 1 && ks + 2 < nk) issue(ks + 2);
    sched_fence();
    multiply();
    sched_fence();
    if (g == 0) __builtin_amdgcn_s_waitcnt(kVm0);
    fenced_barrier();
  }
  if (g == 0) fenced_barrier();
  barrier_all();  // every wave is done with the stage ring
}

// Rows of a small B operand (up to 32 RB rows, K-major, stride ldr) for rankpass:
// instruction q (0 .. RB - 1) of wave w fills rows R = 8 RB w + 8 q + lane / 8 of
// [32 RB][64]; rows >= nrows re-read row nrows - 1.
struct RankSrc {
  const uint16_t* r[2];
};

__device__ __forceinline__ RankSrc make_rank_src(const uint16_t* Bs, int64_t ldr, int nrows, int rb, int wave,
                                                 int lane) {
  RankSrc s;
  const int pc = lane & 7;
  const int rsub = lane >> 3;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int R = 8 * rb * wave + 8 * q + rsub;
    s.r[q] = Bs + static_cast<int64_t>(min(R, nrows - 1)) * ldr + (pc ^ chunk_xor(R)) * 8;
  }
  return s;
}

// Skinny product of the 256-row A panel with up to 32 RB rows of a small K-major operand:
// u = A_panel Bs^T over nk steps of 64 (A through the A half of the stage ring, Bs rows
// through the B half).  RB == 1: wave (wm, wn) gets columns 0..31 of row blocks 2 wn + i
// (i = 0, 1) of its 128 rows in u[i]; RB == 2: columns 32 wn .. +32 of row blocks i
// (i = 0..3).  Lane layout of u[i] is that of a 32x32 MFMA accumulator.  Leaves the stage
// ring free (barrier at the end).
//   step ks: DMA stage ks + 1 | wait for stage ks, barrier | MFMAs | barrier (reads done)
template <int RB, typename S>
__device__ __forceinline__ void rankpass(unsigned char* smem, const S& src, const RankSrc& rs, int nk, int wave,
                                         int lane, floatx16 (&u)[RB == 2 ? 4 : 2]) {
  constexpr int kLoads = 8 + RB;       // DMA instructions per stage and wave
  constexpr int NB = RB == 2 ? 4 : 2;  // row blocks per wave
  constexpr int kRStage = RB * 32 * kRowBytes;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, h32 = lane >> 5;
  const uint32_t sbase = lds_addr(smem);

  auto issue = [&](int ks) {
    const uint32_t as = sbase + kStageA + (ks & 1) * kTileBytes + wave * 8192;
    const int rf = issue_row(src);
#pragma unroll
    for (int c = 0; c < 8; ++c) dma16(src_a(src, c, rf) + ks * BK, as + c * 1024);
    const uint32_t rsl = sbase + kStageB + (ks & 1) * kRStage + wave * RB * 1024;
#pragma unroll
    for (int q = 0; q < RB; ++q) dma16(rs.r[q] + ks * BK, rsl + q * 1024);
  };

#pragma unroll
  for (int i = 0; i < NB; ++i) u[i] = floatx16{};
  issue(0);
  for (int ks = 0; ks < nk; ++ks) {
    if (ks + 1 < nk) {
      issue(ks + 1);
      wait_barrier<kLoads>();  // stage ks landed
    } else {
      wait_barrier<0>();
    }
    const unsigned char* as = smem + kStageA + (ks & 1) * kTileBytes;
    const unsigned char* rsl = smem + kStageB + (ks & 1) * kRStage;
#pragma unroll
    for (int kk = 0; kk < kSlices; ++kk) {
      const bf16x8 lf = *reinterpret_cast<const bf16x8*>(rsl + swz((RB == 2 ? wn * 32 : 0) + l32, kk * 2 + h32));
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int rb = RB == 2 ? i : 2 * wn + i;
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(as + swz(wm * 128 + rb * 32 + l32, kk * 2 + h32));
        u[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, lf, u[i], 0, 0, 0);
      }
    }
    barrier_lds();  // every wave is done with stage ks before the DMA of step ks + 2
  }
}

// Row (within the 256-row tile) and column of element v of u[i] of rankpass for this lane.
template <int RB>
__device__ __forceinline__ int rank_row(int i, int v, int wm, int wn, int h32) {
  const int rb = RB == 2 ? i : 2 * wn + i;
  return wm * 128 + rb * 32 + (v >> 2) * 8 + h32 * 4 + (v & 3);
}
template <int RB>
__device__ __forceinline__ int rank_col(int wn, int l32) {
  return (RB == 2 ? wn * 32 : 0) + l32;
}

}  // namespace tile
}  // namespace lrq
