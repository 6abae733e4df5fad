// MFMA tile family of the forward: bf16 operands, fp32 accumulation, head_dim 128.
//
//   out = RoPE( inv_t * ( W' x + s B (A' x) ) + b ),   W' = W diag(gamma), A' = A diag(gamma)
//
// which equals RoPE(W h + b + s B (A h)) with h = x * inv * gamma, inv = 1/rms(x): the
// norm weight scales the K dimension of both products, so it is folded into the weights
// (one bandwidth-bound pass per call, W' = bf16(W * gamma) into the workspace), and the row
// scale inv commutes with both products, so it is applied to the fp32 accumulators in the
// epilogue.  x enters the MFMAs exactly as given; sum(x^2) of the rows is gathered from the
// same LDS tiles.  Neither h nor U = A h is written to memory.
//
// Work decomposition (gfx950: 64-wide wavefronts, 160 KB LDS, one workgroup per CU)
//   * Output tile 256 tokens x 256 columns (two heads), 256 threads = 4 wavefronts, one
//     per SIMD.  Wavefront (wm, wn) owns tokens 128 wm .. +128 of the tile and the whole
//     head wn: 4 x 4 accumulators of v_mfma_f32_32x32x16_bf16 (256 fp32 per lane, held in
//     the accumulation registers).  The rotate-half partners (i, i + 64) of a head are in
//     the same lane and accumulator index, so RoPE needs no data exchange.
//   * K-loop: 64-wide steps over d, two LDS stages of 64 KB (x and W' tiles).  The tiles go
//     from global memory straight into LDS (global_load_lds_dwordx4, no registers); every
//     tile row of a step is one whole 128-byte line.  Each lane picks its global source so
//     that the 16-byte chunks land XOR-swizzled by row (conflict-free ds_read_b128).  The
//     loads of stage ks + 1 run while stage ks is multiplied; fragment reads run one
//     16-wide slice ahead of the MFMAs that use them; one barrier per step.
//   * One workgroup processes one token tile against a run of consecutive column tiles.
//     Before the first tile of the run that needs target t's adapter, a short K pass over
//     the x tile and the rows of A'_t computes U_t = x A'_t^T and keeps bf16(s U_t) in LDS
//     for the rest of the run; the rank-r up projection is an extra K segment of MFMAs
//     (K = r rounded up to 16) before the epilogue of every tile of that target.
//   * Workgroup ids are remapped so that the runs of one token tile share an XCD (and its
//     L2) when the grid is a multiple of the XCD count.
//   * Epilogue: row sums of squares -> inv, bias, RoPE on q and k heads (angle pos * omega_i
//     reduced in double precision to a fraction of a turn, then the hardware sin / cos),
//     bf16 store.
#include <algorithm>

#include "lrq_internal.h"

namespace lrq {
namespace {

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
constexpr int kLdsMax = 160 * 1024;

// LDS map for RB blocks of 32 LoRA ranks.  The stage ring holds two steps of x and W'.
// The U pass stages the rows of A'_t in the W' half (it does not read W').  The rows' inv
// and positions live in registers (two per lane, for the wave pair's 128 rows).
template <int RB>
struct Lay {
  static constexpr int X = 0;                          // 2 x [256][64] bf16, x
  static constexpr int W = 2 * kTileBytes;             // 2 x [256][64] bf16, W'
  static constexpr int L = W;                          // 2 x [32 RB][64] bf16, A'_t rows (U pass)
  static constexpr int kLStage = RB * 32 * kRowBytes;
  static constexpr int U = 4 * kTileBytes;             // [256][32 RB] bf16, bf16(s U)
  static constexpr int kUStride = RB * 32;
  static constexpr int TMP = X;                        // float [256]: row sums, once per run
  static constexpr int kBytes = U + BM * kUStride * 2;
  static_assert(kBytes <= kLdsMax, "LDS budget");
  static_assert(2 * kLStage <= 2 * kTileBytes, "A' stages fit in the W' half");
};

struct TiledArgs {
  const uint16_t* x;
  const uint16_t* wg;     // W' = bf16(W * gamma) [N][d] (workspace)
  const uint16_t* ag[3];  // A'_t = bf16(A_t * gamma) [r][d] (workspace)
  const uint16_t* bias;  // nullptr without bias
  const uint16_t* b[3];
  const int32_t* pos;
  uint16_t* out;
  int64_t T;
  int d, N, Hq, Hkv, col_k, col_v, r;
  float scale, eps;
  double log2_theta;
  uint32_t targets;
  int n_nt;        // column tiles
  int run;         // column tiles per workgroup
  int runs_per_m;  // workgroups per token tile
  int items;       // grid size
  int remap;       // XCD-aware id remap on/off
};

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
struct TileAcc {
  floatx16 acc[4][4];
  float ss[4];  // sum(x^2) halves of rows 32 i + lane % 32 of the wave pair
};

// Fragments of one 16-wide K slice: x rows (A operand) and W' rows (B operand).
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
__device__ __forceinline__ void mfma_row(TileAcc& ta, const Frags& f, int i) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    ta.acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], ta.acc[i][j], 0, 0, 0);
}

// Row sums of squares of the wave's four row blocks of one slice (both waves of a pair
// gather the same sums; selecting half of the blocks per wave costs more than it saves).
__device__ __forceinline__ void slice_stats(TileAcc& ta, const Frags& f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) sumsq8(f.a[i], ta.ss[i]);
}

// Per-lane DMA sources.  Instruction c (0..7) of wave w fills rows R = 64 w + 8 c + lane / 8
// of a stage; the lane's 16 bytes land in physical chunk lane % 8, which holds logical
// chunk (lane % 8) ^ chunk_xor(R) = (lane % 8) ^ (lane / 8) ^ (c & 1).
struct DmaSrc {
  const uint16_t* x[8];  // per instruction; rows past T re-read row T - 1 (never stored)
  const uint16_t* w[2];  // W' row 64 w + lane / 8 of column tile 0, for even / odd c
};

// One tile's K-loop: acc = x W'_tile^T over all of d; with STATS also the rows' sums of
// squares.
//
//   prologue: DMA stages 0 and 1; wait for stage 0; read slice (0, 0)
//   step ks:  read (ks, 1) | MFMA (ks, 0) | read (ks, 2) | MFMA (ks, 1) | read (ks, 3) |
//             MFMA (ks, 2) | wait for stage ks + 1, barrier | MFMA (ks, 3) with the 16 DMA
//             instructions of stage ks + 2 (into buffer ks % 2) spread between its rows
//             and the read of (ks + 1, 0)
// After the barrier of step ks every wave holds the rest of stage ks in registers, so that
// buffer is free.  Spreading the DMA keeps the wave from stalling on a full address queue
// while the matrix core waits.  sched_fence() pins the interleaving.
template <int RB, bool STATS>
__device__ __forceinline__ void kloop(const TiledArgs& p, unsigned char* smem, TileAcc& ta, const DmaSrc& src,
                                      int64_t col0, int wave, int lane) {
  using L = Lay<RB>;
  constexpr int kLoads = 16;  // DMA instructions per stage and wave
  const int nk = p.d / BK;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, h32 = lane >> 5;
  const int64_t d = p.d;
  const uint32_t sbase = lds_addr(smem);
  const uint16_t* w0 = src.w[0] + col0 * d;
  const uint16_t* w1 = src.w[1] + col0 * d;

  auto issue_x = [&](int ks, int c0) {
    const uint32_t xs = sbase + L::X + (ks & 1) * kTileBytes + wave * 8192;
#pragma unroll
    for (int c = c0; c < c0 + 4; ++c) dma16(src.x[c] + ks * BK, xs + c * 1024);
  };
  auto issue_w = [&](int ks, int c0) {
    const uint32_t ws = sbase + L::W + (ks & 1) * kTileBytes + wave * 8192;
#pragma unroll
    for (int c = c0; c < c0 + 4; ++c)
      dma16(((c & 1) ? w1 : w0) + static_cast<int64_t>(8 * c) * d + ks * BK, ws + c * 1024);
  };
  // instructions c0, c0 + 1 of the x / W' loads of step ks
  auto issue_x2 = [&](int ks, int c0) {
    const uint32_t xs = sbase + L::X + (ks & 1) * kTileBytes + wave * 8192;
    dma16(src.x[c0] + ks * BK, xs + c0 * 1024);
    dma16(src.x[c0 + 1] + ks * BK, xs + (c0 + 1) * 1024);
  };
  auto issue_w2 = [&](int ks, int c0) {
    const uint32_t ws = sbase + L::W + (ks & 1) * kTileBytes + wave * 8192;
    dma16(w0 + static_cast<int64_t>(8 * c0) * d + ks * BK, ws + c0 * 1024);
    dma16(w1 + static_cast<int64_t>(8 * (c0 + 1)) * d + ks * BK, ws + (c0 + 1) * 1024);
  };
  auto sx = [&](int ks) { return smem + L::X + (ks & 1) * kTileBytes; };
  auto sw = [&](int ks) { return smem + L::W + (ks & 1) * kTileBytes; };

  issue_x(0, 0);
  issue_x(0, 4);
  issue_w(0, 0);
  issue_w(0, 4);
  if (nk > 1) {
    issue_x(1, 0);
    issue_x(1, 4);
    issue_w(1, 0);
    issue_w(1, 4);
    wait_barrier<kLoads>();
  } else {
    wait_barrier<0>();
  }
  // slices 0..2 of step ks: MFMAs on (fa, fb, fa) with the next slice read ahead
  auto first3 = [&](int ks, Frags& fa, Frags& fb) {
    const unsigned char* xs = sx(ks);
    const unsigned char* ws = sw(ks);
    sched_fence();
    read_frags(fb, xs, ws, 1, wm, wn, l32, h32);
    sched_fence();
#pragma unroll
    for (int i = 0; i < 4; ++i) mfma_row(ta, fa, i);
    if (STATS) slice_stats(ta, fa);
    sched_fence();
    read_frags(fa, xs, ws, 2, wm, wn, l32, h32);
    sched_fence();
#pragma unroll
    for (int i = 0; i < 4; ++i) mfma_row(ta, fb, i);
    if (STATS) slice_stats(ta, fb);
    sched_fence();
    read_frags(fb, xs, ws, 3, wm, wn, l32, h32);
    sched_fence();
#pragma unroll
    for (int i = 0; i < 4; ++i) mfma_row(ta, fa, i);
    if (STATS) slice_stats(ta, fa);
    sched_fence();
  };

  Frags fa, fb;
  read_frags(fa, sx(0), sw(0), 0, wm, wn, l32, h32);
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
    read_frags(fa, sx(ks + 1), sw(ks + 1), 0, wm, wn, l32, h32);
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

// A'_t rows staged for the U pass: instruction q (0 .. RB - 1) of wave w fills rows
// R = 8 RB w + 8 q + lane / 8 of [32 RB][64]; rows >= r re-read row r - 1 (those ranks are
// stored as 0).
struct LSrc {
  const uint16_t* l[2];
};

// LoRA down projection of the token tile, U = x A'_t^T (256 rows x 32 RB ranks), as its own
// K pass over d (x tiles and A'_t rows only); it runs before the first column tile of a run
// that needs target t and writes bf16(s U) to LDS (ranks >= r as 0).  RB == 1: wave
// (wm, wn) computes ranks 0..31 of row blocks 2 wn, 2 wn + 1 of its 128 rows; RB == 2:
// ranks 32 wn .. +32 of all four.
//   step ks: DMA stage ks + 1 | wait for stage ks, barrier | MFMAs | barrier (reads done)
template <int RB>
__device__ __forceinline__ void upass(const TiledArgs& p, unsigned char* smem, const DmaSrc& src, const LSrc& ls_src,
                                      int wave, int lane) {
  using L = Lay<RB>;
  constexpr int kLoads = 8 + RB;       // DMA instructions per stage and wave
  constexpr int NB = RB == 2 ? 4 : 2;  // row blocks per wave
  const int nk = p.d / BK;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, h32 = lane >> 5;
  const uint32_t sbase = lds_addr(smem);

  auto issue = [&](int ks) {
    const uint32_t xs = sbase + L::X + (ks & 1) * kTileBytes + wave * 8192;
#pragma unroll
    for (int c = 0; c < 8; ++c) dma16(src.x[c] + ks * BK, xs + c * 1024);
    const uint32_t ls = sbase + L::L + (ks & 1) * L::kLStage + wave * RB * 1024;
#pragma unroll
    for (int q = 0; q < RB; ++q) dma16(ls_src.l[q] + ks * BK, ls + q * 1024);
  };

  floatx16 u[NB];
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
    const unsigned char* xs = smem + L::X + (ks & 1) * kTileBytes;
    const unsigned char* ls = smem + L::L + (ks & 1) * L::kLStage;
#pragma unroll
    for (int kk = 0; kk < kSlices; ++kk) {
      const bf16x8 lf = *reinterpret_cast<const bf16x8*>(ls + swz((RB == 2 ? wn * 32 : 0) + l32, kk * 2 + h32));
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int rb = RB == 2 ? i : 2 * wn + i;
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(xs + swz(wm * 128 + rb * 32 + l32, kk * 2 + h32));
        u[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, lf, u[i], 0, 0, 0);
      }
    }
    barrier_lds();  // every wave is done with stage ks before the DMA of step ks + 2
  }
  uint16_t* s_u = reinterpret_cast<uint16_t*>(smem + L::U);
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int rb = RB == 2 ? i : 2 * wn + i;
    const int rank = (RB == 2 ? wn * 32 : 0) + l32;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = wm * 128 + rb * 32 + (v >> 2) * 8 + h32 * 4 + (v & 3);
      s_u[row * L::kUStride + rank] = rank < p.r ? f32_to_bf16_bits(p.scale * u[i][v]) : uint16_t{0};
    }
  }
  barrier_all();
}

// Row data of one wave's part of the output tile in the epilogue.  inv / pos of the wave
// pair's row q * 64 + l are held by lane l in inv[q] / pos[q]; out points at the lane's
// first row, consecutive rows `stride` elements apart.
struct EpiRows {
  float inv[2];
  int pos[2];
  uint16_t* out;
  int64_t stride;
  int64_t rows_left;  // rows of this lane's block still below T
  int h32;
};

// y = acc * inv + bias, rotate-half on the pairs (j, j + 2) when ROT (turns per position
// om0 / om1 for the lane's two frequencies), bf16 store; rows at or past T are skipped
// unless FULL.  Lane rows: i * 32 + (v / 4) * 8 + v % 4 past the lane's first row.
template <bool ROT, bool FULL>
__device__ __forceinline__ void store_tile(const floatx16 (&acc)[4][4], const EpiRows& er, const float (&bias)[4],
                                           double om0, double om1) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int ro = i * 32 + (v >> 2) * 8 + (v & 3);
      const int src_lane = (i & 1) * 32 + (v >> 2) * 8 + er.h32 * 4 + (v & 3);
      const float inv = __shfl(er.inv[i >> 1], src_lane);
      float y0 = fmaf(acc[i][0][v], inv, bias[0]);
      float y1 = fmaf(acc[i][1][v], inv, bias[1]);
      float y2 = fmaf(acc[i][2][v], inv, bias[2]);
      float y3 = fmaf(acc[i][3][v], inv, bias[3]);
      if (ROT) {
        const double pos = static_cast<double>(__shfl(er.pos[i >> 1], src_lane));
        const double t0 = pos * om0, t1 = pos * om1;
        const float f0 = static_cast<float>(t0 - rint(t0));
        const float f1 = static_cast<float>(t1 - rint(t1));
        const float s0 = __builtin_amdgcn_sinf(f0), c0 = __builtin_amdgcn_cosf(f0);
        const float s1 = __builtin_amdgcn_sinf(f1), c1 = __builtin_amdgcn_cosf(f1);
        const float r0 = y0 * c0 - y2 * s0, r2 = y2 * c0 + y0 * s0;
        const float r1 = y1 * c1 - y3 * s1, r3 = y3 * c1 + y1 * s1;
        y0 = r0; y1 = r1; y2 = r2; y3 = r3;
      }
      if (FULL || ro < er.rows_left) {
        uint16_t* o = er.out + ro * er.stride;
        o[0] = f32_to_bf16_bits(y0);
        o[32] = f32_to_bf16_bits(y1);
        o[64] = f32_to_bf16_bits(y2);
        o[96] = f32_to_bf16_bits(y3);
      }
    }
  }
}

template <int RB>
__global__ __launch_bounds__(kThreads, 1) void fwd_tiled_kernel(TiledArgs p) {
  using L = Lay<RB>;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[L::kBytes];
  float* s_tmp = reinterpret_cast<float*>(smem + L::TMP);
  uint16_t* s_u = reinterpret_cast<uint16_t*>(smem + L::U);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, h32 = lane >> 5;

  int item = blockIdx.x;
  if (p.remap) item = (blockIdx.x & 7) * (p.items >> 3) + (blockIdx.x >> 3);
  const int mt = item / p.runs_per_m;
  const int run = item - mt * p.runs_per_m;
  const int nt0 = run * p.run;
  const int nt1 = min(nt0 + p.run, p.n_nt);
  const int64_t row0 = static_cast<int64_t>(mt) * BM;
  const int64_t T = p.T;
  const int64_t d = p.d;

  DmaSrc src;
  const int pc = lane & 7;
  const int rsub = lane >> 3;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int R = 64 * wave + 8 * c + rsub;
    const int64_t row = min(row0 + R, T - 1);
    src.x[c] = p.x + row * d + (pc ^ chunk_xor(R)) * 8;
  }
  // W' row R = 64 w + 8 c + rsub of the column tile; chunk_xor(R) = rsub ^ (c & 1)
  src.w[0] = p.wg + static_cast<int64_t>(64 * wave + rsub) * d + (pc ^ rsub) * 8;
  src.w[1] = p.wg + static_cast<int64_t>(64 * wave + rsub) * d + (pc ^ rsub ^ 1) * 8;

  int u_target = -1;
  float inv_reg[2] = {0.f, 0.f};  // rows 64 q + lane of the wave pair
  int pos_reg[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) pos_reg[q] = p.pos[min(row0 + wm * 128 + q * 64 + lane, T - 1)];

  for (int nt = nt0; nt < nt1; ++nt) {
    const int head0 = 2 * nt;
    const int t = head0 < p.Hq ? 0 : (head0 < p.Hq + p.Hkv ? 1 : 2);
    const bool lora = RB > 0 && ((p.targets >> t) & 1u);
    const bool need_u = lora && u_target != t;
    const int64_t col0 = static_cast<int64_t>(nt) * BN;

    if (RB > 0 && need_u) {
      LSrc ls;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int R = 8 * RB * wave + 8 * q + rsub;
        ls.l[q] = p.ag[t] + static_cast<int64_t>(min(R, p.r - 1)) * d + (pc ^ chunk_xor(R)) * 8;
      }
      upass<RB>(p, smem, src, ls, wave, lane);
      u_target = t;
    }

    TileAcc ta;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) ta.acc[i][j] = floatx16{};
#pragma unroll
    for (int i = 0; i < 4; ++i) ta.ss[i] = 0.f;

    if (nt == nt0) {
      kloop<RB, true>(p, smem, ta, src, col0, wave, lane);
      // rows' inv, once per run: the wave pair's row sums meet in the idle x half
      const float inv_d = 1.0f / static_cast<float>(p.d);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float s = ta.ss[i] + __shfl_xor(ta.ss[i], 32);
        if (h32 == 0 && wn == 0) s_tmp[wm * 128 + i * 32 + l32] = 1.0f / sqrtf(s * inv_d + p.eps);
      }
      barrier_all();
#pragma unroll
      for (int q = 0; q < 2; ++q) inv_reg[q] = s_tmp[wm * 128 + q * 64 + lane];
      barrier_all();
    } else {
      kloop<RB, false>(p, smem, ta, src, col0, wave, lane);
    }

    // ---- LoRA up projection: acc += bf16(s U) B_t^T over K = r rounded up to 16
    if (RB > 0 && lora) {
      const int lo = t == 0 ? 0 : (t == 1 ? p.col_k : p.col_v);
      const uint16_t* __restrict__ bt = p.b[t];
      const int r = p.r;
      const int ksteps = (r + 15) >> 4;
      for (int kq = 0; kq < ksteps; ++kq) {
        const int k0 = kq * 16 + h32 * 8;
        bf16x8 af[4], bfr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          af[i] = *reinterpret_cast<const bf16x8*>(s_u + (wm * 128 + i * 32 + l32) * L::kUStride + k0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint16_t* bsrc = bt + (col0 + wn * 128 + j * 32 + l32 - lo) * r + k0;
          if ((r & 7) == 0 && k0 < r) {
            bfr[j] = *reinterpret_cast<const bf16x8*>(bsrc);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              bfr[j][e] = __builtin_bit_cast(__bf16, k0 + e < r ? bsrc[e] : uint16_t{0});
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            ta.acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], ta.acc[i][j], 0, 0, 0);
      }
    }

    // ---- epilogue: row scale, bias, RoPE, store
    const int64_t colw = col0 + wn * 128;
    float bias[4] = {0.f, 0.f, 0.f, 0.f};
    if (p.bias) {
#pragma unroll
      for (int j = 0; j < 4; ++j) bias[j] = bf16_bits_to_f32(p.bias[colw + j * 32 + l32]);
    }
    // Opaque per-tile copies of the lane's row offset and of the row stride: they keep the
    // compiler from hoisting 64 row addresses out of the tile loop (they would spill).
    int lrow = wm * 128 + h32 * 4;
    int64_t n_stride = p.N;
    asm volatile("" : "+v"(lrow), "+s"(n_stride));
    const EpiRows er{{inv_reg[0], inv_reg[1]}, {pos_reg[0], pos_reg[1]},
                     p.out + (row0 + lrow) * n_stride + colw + l32, n_stride, T - (row0 + lrow), h32};
    const bool full = row0 + BM <= T;
    if (t < 2) {
      double om0 = exp2(-(2.0 * l32 / 128.0) * p.log2_theta) * 0.15915494309189533577;
      double om1 = exp2(-(2.0 * (32 + l32) / 128.0) * p.log2_theta) * 0.15915494309189533577;
      if (full)
        store_tile<true, true>(ta.acc, er, bias, om0, om1);
      else
        store_tile<true, false>(ta.acc, er, bias, om0, om1);
    } else {
      if (full)
        store_tile<false, true>(ta.acc, er, bias, 0.0, 0.0);
      else
        store_tile<false, false>(ta.acc, er, bias, 0.0, 0.0);
    }
  }
}

// W' = bf16(W * gamma) and A'_t = bf16(A_t * gamma): rows [0, N) of the destination
// come from W, then r rows per target from A_q, A_k, A_v (targets only).  Each thread
// scales 8 consecutive elements of one row (d % 8 == 0).
struct FoldArgs {
  const uint16_t* w;
  const uint16_t* a[3];
  const uint16_t* gamma;
  uint16_t* dst;
  int64_t rows;     // N + (number of targets) * r
  int N, r, d;
  int slot_t[3];    // target of the slot-th group of r rows after W
};

__global__ __launch_bounds__(256) void fold_gamma_kernel(FoldArgs f) {
  const int64_t chunks_per_row = f.d / 8;
  const int64_t total = f.rows * chunks_per_row;
  for (int64_t c = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; c < total;
       c += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t row = c / chunks_per_row;
    const int k = static_cast<int>(c - row * chunks_per_row) * 8;
    const uint16_t* src;
    if (row < f.N) {
      src = f.w + row * f.d;
    } else {
      const int64_t q = row - f.N;
      const int slot = static_cast<int>(q / f.r);
      src = f.a[f.slot_t[slot]] + (q - static_cast<int64_t>(slot) * f.r) * f.d;
    }
    const uint4 x = *reinterpret_cast<const uint4*>(src + k);
    const uint4 g = *reinterpret_cast<const uint4*>(f.gamma + k);
    const uint32_t xs[4] = {x.x, x.y, x.z, x.w}, gs[4] = {g.x, g.y, g.z, g.w};
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = f32_to_bf16_bits(lo_bf16(xs[e]) * lo_bf16(gs[e]));
      const uint32_t hi = f32_to_bf16_bits(hi_bf16(xs[e]) * hi_bf16(gs[e]));
      o[e] = lo | (hi << 16);
    }
    *reinterpret_cast<uint4*>(f.dst + row * f.d + k) = uint4{o[0], o[1], o[2], o[3]};
  }
}

int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

}  // namespace

bool tiled_supports(const FwdParams& p) {
  return p.T <= (int64_t{1} << 24) && p.D == 128 && p.Hq % 2 == 0 && p.Hkv % 2 == 0 && p.d % BK == 0 &&
         p.d >= BK && p.d <= (1 << 20) && p.r <= kMaxRank;
}

namespace {
int n_targets(const FwdParams& p) { return (p.targets & 1u) + ((p.targets >> 1) & 1u) + ((p.targets >> 2) & 1u); }
size_t align256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }
}  // namespace

// W' then A'_t for every target, bf16, d elements per row.
size_t tiled_workspace_bytes(const FwdParams& p) {
  return align256(static_cast<size_t>(p.N + n_targets(p) * p.r) * static_cast<size_t>(p.d) * 2);
}

hipError_t launch_fwd_tiled(const FwdParams& p, hipStream_t s) {
  uint16_t* ws = static_cast<uint16_t*>(p.ws);
  FoldArgs f;
  f.w = static_cast<const uint16_t*>(p.w);
  f.gamma = static_cast<const uint16_t*>(p.gamma);
  f.dst = ws;
  f.N = p.N;
  f.r = p.r;
  f.d = static_cast<int>(p.d);
  int slots = 0;
  TiledArgs a;
  for (int t = 0; t < 3; ++t) {
    f.a[t] = static_cast<const uint16_t*>(p.a[t]);
    f.slot_t[t] = 0;
    a.ag[t] = nullptr;
    a.b[t] = static_cast<const uint16_t*>(p.b[t]);
    if (p.targets & (1u << t)) {
      a.ag[t] = ws + (static_cast<int64_t>(p.N) + static_cast<int64_t>(slots) * p.r) * p.d;
      f.slot_t[slots++] = t;
    }
  }
  f.rows = static_cast<int64_t>(p.N) + static_cast<int64_t>(slots) * p.r;
  const int64_t chunks = f.rows * (p.d / 8);
  const int fold_blocks = static_cast<int>(std::min<int64_t>((chunks + 255) / 256, 8 * 1024));
  hipLaunchKernelGGL(fold_gamma_kernel, dim3(fold_blocks), dim3(256), 0, s, f);

  a.x = static_cast<const uint16_t*>(p.x);
  a.wg = ws;
  a.bias = p.has_bias ? static_cast<const uint16_t*>(p.bias) : nullptr;
  a.pos = p.pos;
  a.out = static_cast<uint16_t*>(p.out);
  a.T = p.T;
  a.d = static_cast<int>(p.d);
  a.N = p.N;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.col_k = p.col_k;
  a.col_v = p.col_v;
  a.r = p.r;
  a.scale = p.scale;
  a.eps = p.eps;
  a.log2_theta = log2(p.theta);
  a.targets = p.targets;
  const int n_mt = static_cast<int>((p.T + BM - 1) / BM);
  a.n_nt = p.N / BN;
  const int64_t tiles = static_cast<int64_t>(n_mt) * a.n_nt;
  const int cus = cu_count();
  int run = static_cast<int>((tiles + cus - 1) / cus);
  run = run < 1 ? 1 : (run > a.n_nt ? a.n_nt : run);
  a.run = run;
  a.runs_per_m = (a.n_nt + run - 1) / run;
  a.items = n_mt * a.runs_per_m;
  a.remap = a.items % 8 == 0;
  const int rb = p.targets ? (p.r <= 32 ? 1 : 2) : 0;
  dim3 grid(a.items), block(kThreads);
  switch (rb) {
    case 0: hipLaunchKernelGGL(fwd_tiled_kernel<0>, grid, block, 0, s, a); break;
    case 1: hipLaunchKernelGGL(fwd_tiled_kernel<1>, grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL(fwd_tiled_kernel<2>, grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

// ---- the decode and tiled-backward families are not built yet
bool decode_supports(const FwdParams&) { return false; }
size_t decode_workspace_bytes(const FwdParams&) { return 0; }
hipError_t launch_fwd_decode(const FwdParams&, hipStream_t) { return hipErrorNotSupported; }
bool bwd_tiled_supports(const FwdParams&) { return false; }
size_t bwd_tiled_workspace_bytes(const FwdParams&) { return 0; }
hipError_t launch_bwd_tiled(const BwdParams&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace lrq
