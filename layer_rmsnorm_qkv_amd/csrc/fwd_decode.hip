// Decode family of the forward (bf16, at most 256 rows): with so few rows, reading W_qkv
// from HBM is the whole cost, so the work is arranged around streaming W once.
//
//   one kernel, one block per 64 weight rows and 64 token rows.  A "W block" takes the W
//   rows of 32 rotate-half pairs of one head (columns col0 + 0..31 and col0 + D/2 + 0..31);
//   an "A block" (one per LoRA target) takes the 64 (padded) rows of A_t.  x and the weight
//   rows stream through a 4-stage LDS ring (direct-to-LDS loads); each wave forms
//   bf16(x * gamma) from the staged x and gamma, accumulates x^2 for the row statistics and
//   multiplies its share of every stage (32x32x16 bf16 MFMA).  The four waves' partial
//   products are summed through LDS, then
//     A block:  U_t = bf16(s * inv * acc), 64 tokens x 64 ranks, into the workspace, and a
//               count that says so
//     W block:  out = bf16(RoPE(inv * acc + b + B_t U_t)); a block whose columns have an
//               adapter waits for its U_t's count first (B_t is loaded before the stream).
//   The A blocks come first in the grid and wait for nothing: workgroups start in index
//   order on each XCD, so every A block is running or done before a W block that could
//   wait for it starts, and the waits end.  Each wait is bounded all the same.  A count
//   word carries a tag of the launch itself (its packet index in the hardware queue and
//   the queue's address, so it differs between any two launches, replays of a captured
//   launch included): whatever the workspace held before reads as "nothing stored yet",
//   and nothing has to be cleared between launches.
// With a key/value cache, the stores of the k and v columns into out also go to the token's
// cache row.
// With an NF4 W (the QLoRA base) a W block streams the rows' 4-bit codes instead (a quarter of
// the bytes) and dequantises them into the MFMA operand: code book value times the block
// scale, rounded once to bf16; its scales are staged once per block.  Those blocks stream
// x_g = bf16(x * gamma) and read inv, made once by a prep pass, so that their VALU time goes
// to the dequantisation (A blocks and dense W blocks form x * gamma per stage as above).
//
// The operator is RoPE(W h + b + s B (A h)) with h = x * inv * gamma; inv, a per-row scalar,
// is applied after the products and gamma before them.  Every sum runs in a fixed order, so
// results are the same run to run.
#include "lrq_internal.h"
#include "tile_common.h"

namespace lrq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kRows = 64;                         // token rows per row group
constexpr int kBK = 128;                          // columns of d per ring stage
constexpr int kStages = 4;                        // ring depth
constexpr int kPartBytes = kRows * kBK * 2;       // 16 KB: x or weight rows of one stage
constexpr int kStageBytes = 2 * kPartBytes;       // x part, then weight part
constexpr int kRingBytes = kStages * kStageBytes; // 128 KB
constexpr int kMaxD = 8192;                       // gamma is staged whole in LDS
constexpr int kChunks = kBK / 8;                  // 16-byte chunks per staged row
constexpr int kLoads = 2 * kPartBytes / 4096;     // direct-to-LDS loads per thread per stage
constexpr int kMaxTokens = 256;

size_t al256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }


// One 64-bit count word per (row group, A block): the launch tag in bits 8..63, and in bits
// 0..7 the waves of the A block whose U_t stores have landed (0..2).
constexpr int kSyncWords = (kMaxTokens / kRows) * 3;
// Polls of a count word before a wave gives up (never reached when the blocks run: what it
// waits for is done by a running block that waits for nothing).
constexpr int kSpinLimit = 1 << 20;

struct DecodeLayout {
  int Tp;      // rows rounded up to the row group
  int nt;      // number of LoRA targets
  int tgt[3];  // target of A block i
  size_t sync, u, xg, inv, total;
};

DecodeLayout decode_layout(const FwdParams& p) {
  DecodeLayout L{};
  L.Tp = static_cast<int>((p.T + kRows - 1) / kRows * kRows);
  for (int t = 0; t < 3; ++t)
    if (p.targets & (1u << t)) L.tgt[L.nt++] = t;
  size_t o = 0;
  L.sync = o;  // uint64 [kSyncWords]: the U_t count words
  o += al256(L.nt ? kSyncWords * 8 : 0);
  L.u = o;  // bf16 [Tp][nt * 64]: s * inv * U_t, ranks padded to 64
  o += al256(static_cast<size_t>(L.Tp) * L.nt * 64 * 2);
  L.xg = o;  // NF4 weights: bf16 [T][d] x * gamma from the prep pass
  o += al256(p.nf4 ? static_cast<size_t>(p.T) * p.d * 2 : 0);
  L.inv = o;  // NF4 weights: float [T] 1 / rms(x) from the prep pass
  o += al256(p.nf4 ? static_cast<size_t>(p.T) * 4 : 0);
  L.total = o;
  return L;
}

// Cache row of a token (or nullptr): the k or v cache row of the token when the call has a
// cache, `col0` is a k or v column and the slot lies in the cache.  Column c of that block
// lands at row[c - first column of the block].
__device__ __forceinline__ uint16_t* cache_row(uint16_t* kv_k, uint16_t* kv_v, int64_t num_slots, int slot,
                                               int col0, int col_k, int col_v) {
  if (!kv_k || col0 < col_k || slot < 0 || slot >= num_slots) return nullptr;
  return (col0 < col_v ? kv_k : kv_v) + static_cast<int64_t>(slot) * (col_v - col_k);
}

// ---------------------------------------------------------------- main
struct MainArgs {
  const uint16_t* x;
  const uint16_t* xg;      // NF4 W blocks: x * gamma (bf16) from the prep pass
  const float* inv;        // NF4 W blocks: 1 / rms(x) per token row from the prep pass
  const uint16_t* gamma;
  const uint16_t* w;
  Nf4View wq;            // W as NF4 blocks (QLoRA base) when nf4
  int nf4;
  const uint16_t* bias;
  const uint16_t* a[3];  // A of the targets in A-block order
  const uint16_t* b[3];  // B_t by target
  int ublock[3];         // A block of target t, or -1
  const int32_t* pos;
  uint16_t* out;
  uint16_t* u;
  uint64_t* sync;        // U_t count words
  uint16_t* kv_k;           // key/value cache rows (nullptr: none)
  uint16_t* kv_v;
  const int32_t* kv_slots;
  int64_t kv_num_slots;
  int64_t T;
  int d, N, D, r, nt, n_wblocks, groups;
  int col_k, col_v, rot_end;
  uint32_t targets;
  float scale, eps;
  double log2_theta;
};

// XOR pattern of the chunks of staged row `row`: 16 consecutive rows read at one logical
// chunk land in 16 distinct 16-byte bank groups (ds_read_b128 serves 16 lanes per cycle).
__device__ __forceinline__ int sw(int row, int chunk) { return row * (kBK * 2) + ((chunk ^ (row & 15)) << 4); }

// Waits for the last kStages - 1 stages (all issued) and computes them; L loads per stage.
template <int L, int I, typename F>
__device__ __forceinline__ void drain(F& compute, int st) {
  if constexpr (I < kStages - 1) {
    tile::wait_barrier<(kStages - 2 - I) * L>();
    compute(st + I);
    drain<L, I + 1>(compute, st);
  }
}

// NF4 W blocks (QLoRA base): a stage holds the x part and the block's codes, 64 rows x 64
// bytes (16-byte chunk j of row r stored at j ^ ((r / 4) % 4), so the 4-byte reads of 32 rows
// hit at most two rows per bank); the block scales sit transposed, [d / 64][64 rows] float32,
// after the ring, then a 256-entry table: code byte -> its two code-book values (float32
// pair), so one 8-byte LDS read dequantises two weights (value times scale in float32, one
// rounding to bf16, as in the other families).
constexpr int kCodeBytes = kRows * kBK / 2;             // 4 KB
constexpr int kStageNf4 = kPartBytes + kCodeBytes;      // 20 KB
constexpr int kScalesOff = kStages * kStageNf4;         // 80 KB
constexpr int kLevelsOff = kScalesOff + kRows * (kMaxD / 64) * 4;  // 112 KB
static_assert(kLevelsOff + 256 * 8 <= kRingBytes, "NF4 staging fits under gamma");

// bf16(x * g) of 8 values, and ss += sum of x^2 (products exact, fp32 sums)
__device__ __forceinline__ bf16x8 scale8(const bf16x8& x, const bf16x8& g, float& ss) {
  bf16x8 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const bf16x2 v = {x[2 * e], x[2 * e + 1]};
    ss = __builtin_amdgcn_fdot2_f32_bf16(v, v, ss, false);
    o[2 * e] = static_cast<__bf16>(static_cast<float>(x[2 * e]) * static_cast<float>(g[2 * e]));
    o[2 * e + 1] = static_cast<__bf16>(static_cast<float>(x[2 * e + 1]) * static_cast<float>(g[2 * e + 1]));
  }
  return o;
}

// ---------------------------------------------------------------- prep (NF4 weights)
// One wavefront per token row: inv = 1 / rms(x) (fp32 sum of the exact squares) and
// x_g = bf16(x * gamma), once for all NF4 W blocks: their dequantisation takes the VALU time
// that forming x * gamma inside every block would otherwise need.
struct PrepArgs {
  const uint16_t* x;
  const uint16_t* gamma;
  uint16_t* xg;
  float* inv;
  int64_t T;
  int d;
  float eps;
};

__global__ __launch_bounds__(256) void decode_prep_kernel(PrepArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= a.T) return;
  const uint16_t* xr = a.x + row * a.d;
  uint16_t* gr = a.xg + row * a.d;
  float ss = 0.f;
  for (int j = lane * 8; j < a.d; j += 512) {
    const bf16x8 x = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(xr + j));
    const bf16x8 g = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(a.gamma + j));
    *reinterpret_cast<uint4*>(gr + j) = __builtin_bit_cast(uint4, scale8(x, g, ss));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  if (lane == 0) a.inv[row] = 1.0f / sqrtf(ss / static_cast<float>(a.d) + a.eps);
}

// The AQL packet index of this launch in its hardware queue (LLVM's dispatch-id intrinsic).
extern "C" __device__ uint64_t lrq_decode_dispatch_id() __asm("llvm.amdgcn.dispatch.id");

// Tag of this launch in bits 8..63: packet index and queue address mixed, so two launches
// differ, whether on one queue (indices differ) or on two (addresses differ).
__device__ __forceinline__ uint64_t launch_tag() {
  const uint64_t q = reinterpret_cast<uint64_t>(__builtin_amdgcn_queue_ptr());
  const uint64_t h = (lrq_decode_dispatch_id() + 1) * 0x9E3779B97F4A7C15ull ^ (q * 0xC2B2AE3D27D4EB4Full);
  return h & ~uint64_t{255};
}

// Tiles: rt = token-row tile (32 rows), ct = weight-row tile (32 rows).  In a W block the
// weight rows of ct 0 and ct 1 are the two members of rotate-half pairs, so a pair sits in
// the same lane and register of the two tiles.
template <bool NF4>
__device__ __forceinline__ void decode_main_body(const MainArgs& a, unsigned char* smem, int nb, int rg) {
  constexpr int kPer = kLoads / 2;                   // x loads (and dense weight loads) per stage
  constexpr int kLoadsT = NF4 ? kPer + 1 : kLoads;   // loads per thread and stage
  constexpr int kStageT = NF4 ? kStageNf4 : kStageBytes;
  unsigned char* gs = smem + kRingBytes;  // gamma, [d] bf16
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, h32 = lane >> 5;
  const bool wblock = nb < a.n_wblocks;
  const int half = a.D / 2;
  const int per_head = a.D / 64;
  const int head = nb / per_head, sub = nb % per_head;
  const int col0 = head * a.D + sub * 32;  // W blocks
  const int ab = nb - a.n_wblocks;         // A blocks
  const int64_t ld = a.d;

  // gamma into LDS (x * gamma is formed per stage; NF4 W blocks stream x_g instead): 1 KB per
  // load instruction, wave w takes chunks w, w + 4, ...
  if constexpr (!NF4) {
    const uint32_t lds_g = tile::lds_addr(gs);
    const int gchunks = a.d * 2 / 1024;
    for (int c = wave; c < gchunks; c += 4)
      tile::dma16(reinterpret_cast<const unsigned char*>(a.gamma) + c * 1024 + lane * 16, lds_g + c * 1024);
  }

  // NF4: block scales transposed into LDS (plain loads, overlapped with the ring prologue
  // below), and the code book
  float* sc_t = reinterpret_cast<float*>(smem + kScalesOff);
  float2* pairs = reinterpret_cast<float2*>(smem + kLevelsOff);
  const int nblk = a.d / 64;
  float scv[NF4 ? kRows * (kMaxD / 64) / 256 : 1];
  if constexpr (NF4) {
#pragma unroll
    for (int i = 0; i < kRows * (kMaxD / 64) / 256; ++i) {
      const int e = tid + 256 * i;  // (row, block) = (e / nblk, e % nblk)
      const int row = e / nblk, blk = e - (e / nblk) * nblk;
      const int64_t wrow = col0 + (row >> 5) * half + (row & 31);
      scv[i] = row < kRows ? a.wq.scales[wrow * nblk + blk] : 0.f;
    }
  }

  // direct-to-LDS sources: this thread fills slots p = (kLoads/2 * wave + j) * 64 + lane of
  // each part; slot p is (staged row p / kChunks, physical chunk p % kChunks).  Token rows
  // past T re-read row T - 1 and padded A rows re-read row r - 1 (never stored).
  const uint16_t* xsrc[kPer];
  const uint16_t* wsrc[kPer];
  const uint16_t* arows = a.a[0];
#pragma unroll
  for (int i = 1; i < 3; ++i)
    if (i == ab) arows = a.a[i];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int p = (wave * kPer + j) * 64 + lane;
    const int row = p / kChunks, chunk = (p % kChunks) ^ (row & 15);
    const int64_t trow = min(static_cast<int64_t>(rg * kRows + row), a.T - 1);
    xsrc[j] = (NF4 ? a.xg : a.x) + trow * ld + chunk * 8;
    const int64_t wrow = wblock ? col0 + (row >> 5) * half + (row & 31) : min(row, a.r - 1);
    wsrc[j] = (wblock ? a.w : arows) + wrow * ld + chunk * 8;
  }
  // NF4 codes: slot p = wave * 64 + lane is (row p / 4, physical chunk p % 4)
  const uint8_t* csrc = nullptr;
  if constexpr (NF4) {
    const int p = wave * 64 + lane, row = p >> 2, lc = (p & 3) ^ ((row >> 2) & 3);
    const int64_t wrow = col0 + (row >> 5) * half + (row & 31);
    csrc = a.wq.codes + wrow * (ld / 2) + lc * 16;
  }
  // LoRA-up operand of a W block whose columns have an adapter: B_t's fragments for the
  // epilogue waves, loaded before the stream so their latency hides under it.  Ranks past r
  // are zero (16-byte loads clamped into the row, then zeroed; element loads clamped and
  // zeroed), so the four rank steps of the epilogue run unconditionally.
  const int t = col0 < a.col_k ? 0 : (col0 < a.col_v ? 1 : 2);
  const bool adapted = wblock && ((a.targets >> t) & 1u);
  bf16x8 bf[4][2];
  if (adapted && wave < 2) {
    const uint16_t* bt = t == 0 ? a.b[0] : (t == 1 ? a.b[1] : a.b[2]);
    const int lo_t = t == 0 ? 0 : (t == 1 ? a.col_k : a.col_v);
    if ((a.r & 7) == 0) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          const uint16_t* brow = bt + static_cast<int64_t>(col0 + ct * half + l32 - lo_t) * a.r;
          bf[kk][ct] = *reinterpret_cast<const bf16x8*>(brow + min(kk * 16 + 8 * h32, a.r - 8));
        }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        if (kk * 16 + 8 * h32 >= a.r) bf[kk][0] = bf[kk][1] = bf16x8{};
    } else {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          const uint16_t* brow = bt + static_cast<int64_t>(col0 + ct * half + l32 - lo_t) * a.r;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int rank = kk * 16 + 8 * h32 + e;
            const uint16_t v = brow[min(rank, a.r - 1)];
            bf[kk][ct][e] = __builtin_bit_cast(__bf16, rank < a.r ? v : uint16_t{0});
          }
        }
    }
  }
  const uint32_t lds0 = tile::lds_addr(smem) + wave * kPer * 1024;
  const uint32_t ldsc = tile::lds_addr(smem) + kPartBytes + wave * 1024;
  auto issue = [&](int st) {
    const uint32_t base = lds0 + (st % kStages) * kStageT;
    const int k = st * kBK;
#pragma unroll
    for (int j = 0; j < kPer; ++j) tile::dma16(xsrc[j] + k, base + j * 1024);
    if constexpr (NF4) {
      tile::dma16(csrc + k / 2, ldsc + (st % kStages) * kStageT);
    } else {
#pragma unroll
      for (int j = 0; j < kPer; ++j) tile::dma16(wsrc[j] + k, base + kPartBytes + j * 1024);
    }
  };
  const int nst = a.d / kBK;  // >= kStages - 1
#pragma unroll
  for (int st = 0; st < kStages - 1; ++st) issue(st);
  if constexpr (NF4) {
    // the scales' loads are older than the ring's: they have landed by now or soon
#pragma unroll
    for (int i = 0; i < kRows * (kMaxD / 64) / 256; ++i) {
      const int e = tid + 256 * i;
      const int row = e / nblk, blk = e - (e / nblk) * nblk;
      if (row < kRows) sc_t[blk * kRows + row] = scv[i];
    }
    pairs[tid] = make_float2(kNf4Levels[tid & 15], kNf4Levels[tid >> 4]);  // 256 threads, 256 bytes
  }

  floatx16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = floatx16{};
  float ss[2] = {0.f, 0.f};  // token rows l32 and 32 + l32, this lane's columns
  // 8 dequantised weights (row, columns 8 c .. 8 c + 7 of the stage) as a bf16 operand
  auto nf4_frag = [&](const unsigned char* cs, int row, int c, int st) -> bf16x8 {
    const uint32_t code = *reinterpret_cast<const uint32_t*>(
        cs + (row * 4 + ((c >> 2) ^ ((row >> 2) & 3))) * 16 + (c & 3) * 4);
    const float sc = sc_t[(2 * st + (c >> 3)) * kRows + row];
    bf16x8 f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float2 v = pairs[(code >> (8 * e)) & 255u];
      f[2 * e] = static_cast<__bf16>(v.x * sc);
      f[2 * e + 1] = static_cast<__bf16>(v.y * sc);
    }
    return f;
  };
  auto compute = [&](int st) {
    const unsigned char* xs = smem + (st % kStages) * kStageT;
    const unsigned char* ws = xs + kPartBytes;
#pragma unroll
    for (int i = 0; i < kBK / 64; ++i) {
      const int c = (kBK / 64 * wave + i) * 2 + h32;
      bf16x8 a0, a1;
      if constexpr (NF4) {
        a0 = *reinterpret_cast<const bf16x8*>(xs + sw(l32, c));
        a1 = *reinterpret_cast<const bf16x8*>(xs + sw(32 + l32, c));
      } else {
        const bf16x8 g = *reinterpret_cast<const bf16x8*>(gs + (st * kChunks + c) * 16);
        a0 = scale8(*reinterpret_cast<const bf16x8*>(xs + sw(l32, c)), g, ss[0]);
        a1 = scale8(*reinterpret_cast<const bf16x8*>(xs + sw(32 + l32, c)), g, ss[1]);
      }
      bf16x8 b0, b1;
      if constexpr (NF4) {
        b0 = nf4_frag(ws, l32, c, st);
        b1 = nf4_frag(ws, 32 + l32, c, st);
      } else {
        b0 = *reinterpret_cast<const bf16x8*>(ws + sw(l32, c));
        b1 = *reinterpret_cast<const bf16x8*>(ws + sw(32 + l32, c));
      }
      acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, acc[1][1], 0, 0, 0);
    }
  };
  // stage st lives in slot st % kStages; each thread has kLoads loads per stage (gamma's
  // were issued first), so "stage st has landed" is vmcnt <= kLoads * (stages issued after
  // st).  The barrier also tells every wave that the others are done with stage st - 1,
  // whose slot is refilled next.
  int st = 0;
  for (; st + kStages - 1 < nst; ++st) {
    tile::wait_barrier<(kStages - 2) * kLoadsT>();
    issue(st + kStages - 1);
    compute(st);
  }
  drain<kLoadsT, 0>(compute, st);
  tile::barrier_lds();  // the ring is reused below

  // ---- sums of the four waves' column subsets, in wave order: products, then x^2
  float4(*red)[4][4][64] = reinterpret_cast<float4(*)[4][4][64]>(smem);
  float(*rss)[2][64] = reinterpret_cast<float(*)[2][64]>(smem + 4 * 4 * 4 * 64 * 16);
#pragma unroll
  for (int tt = 0; tt < 4; ++tt)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const floatx16& v = acc[tt >> 1][tt & 1];
      red[wave][tt][q][lane] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
    }
  rss[wave][0][lane] = ss[0];
  rss[wave][1][lane] = ss[1];
  __syncthreads();
  if (wave >= 2) return;
  const int rt = wave;
  floatx16 y[2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float4 sum = red[0][rt * 2 + ct][q][lane];
#pragma unroll
      for (int w = 1; w < 4; ++w) {
        const float4 o = red[w][rt * 2 + ct][q][lane];
        sum.x += o.x;
        sum.y += o.y;
        sum.z += o.z;
        sum.w += o.w;
      }
      y[ct][4 * q] = sum.x;
      y[ct][4 * q + 1] = sum.y;
      y[ct][4 * q + 2] = sum.z;
      y[ct][4 * q + 3] = sum.w;
    }
  // row statistics of token row rt * 32 + l32 (lanes l32 and 32 + l32 held its two halves;
  // NF4 W blocks: from the prep pass)
  float inv_l;
  if constexpr (NF4) {
    inv_l = a.inv[min(static_cast<int64_t>(rg * kRows + rt * 32 + l32), a.T - 1)];
  } else {
    float ssum = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) ssum += rss[w][rt][l32] + rss[w][rt][32 + l32];
    inv_l = 1.0f / sqrtf(ssum / static_cast<float>(a.d) + a.eps);
  }

  if (!wblock) {
    // U_t: lane holds rank ct * 32 + l32 of token rows (v / 4) * 8 + h32 * 4 + v % 4
    uint16_t* ub = a.u + ab * 64;
    const int64_t ldu = static_cast<int64_t>(a.nt) * 64;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int rsub = (v >> 2) * 8 + h32 * 4 + (v & 3);
      const int64_t row = rg * kRows + rt * 32 + rsub;
      const float f = a.scale * __shfl(inv_l, rsub);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) ub[row * ldu + ct * 32 + l32] = f32_to_bf16_bits(f * y[ct][v]);
    }
    // this wave's 32 token rows are stored: make them visible device-wide, then count them
    // (a word with another tag is left over from before: this wave is the first)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    if (lane == 0) {
      uint64_t* cw = a.sync + rg * 3 + ab;
      const uint64_t tag = launch_tag();
      uint64_t old = __hip_atomic_load(cw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int n = 0; n < kSpinLimit; ++n) {
        const uint64_t nw = (old & ~uint64_t{255}) == tag ? old + 1 : (tag | 1u);
        if (__hip_atomic_compare_exchange_strong(cw, &old, nw, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT))
          break;
      }
    }
    return;
  }

  const int c0 = col0 + l32, c1 = col0 + half + l32;
  const float b0 = a.bias ? bf16_bits_to_f32(a.bias[c0]) : 0.f;
  const float b1 = a.bias ? bf16_bits_to_f32(a.bias[c1]) : 0.f;
  const bool rot = col0 < a.rot_end;
  const int i_pair = sub * 32 + l32;  // frequency index within the head
  const double om = exp2(-(2.0 * i_pair / a.D) * a.log2_theta) * 0.15915494309189533577;  // turns
  const int64_t myrow = rg * kRows + rt * 32 + l32;
  const int pos_l = myrow < a.T ? a.pos[myrow] : 0;
  const int slot_l = a.kv_slots && myrow < a.T ? a.kv_slots[myrow] : -1;

  // LoRA term B_t U_t of this lane's token rows and columns (the accumulator layout of y)
  floatx16 lo[2] = {floatx16{}, floatx16{}};
  if (adapted) {
    const int ublk = t == 0 ? a.ublock[0] : (t == 1 ? a.ublock[1] : a.ublock[2]);
    // U_t of this row group: both of its A block's waves have counted their stores
    uint64_t* cw = a.sync + rg * 3 + ublk;
    const uint64_t ready = launch_tag() | 2u;
    bool landed = false;
    for (int n = 0; n < kSpinLimit && !landed; ++n) {
      landed = __hip_atomic_load(cw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == ready;
      if (!landed) __builtin_amdgcn_s_sleep(1);
    }
    // U_t is read with device-coherent loads, issued after the count was seen; an acquire
    // fence would instead drop every line of this XCD's L2 (the x rows other blocks stream)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    const uint64_t* urow = reinterpret_cast<const uint64_t*>(a.u + myrow * (static_cast<int64_t>(a.nt) * 64) + ublk * 64);
    bf16x8 uf[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int q = (kk * 16 + 8 * h32) / 4;
      const uint64_t lo64 = __hip_atomic_load(urow + q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint64_t hi64 = __hip_atomic_load(urow + q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      uf[kk] = __builtin_bit_cast(bf16x8, make_ulonglong2(lo64, hi64));
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) lo[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(uf[kk], bf[kk][ct], lo[ct], 0, 0, 0);
    if (!landed) {
      // the wait gave up (never expected): poison these outputs rather than use stale U_t
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) lo[ct] = floatx16{} + __builtin_nanf("");
    }
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int rsub = (v >> 2) * 8 + h32 * 4 + (v & 3);
    const int64_t row = rg * kRows + rt * 32 + rsub;
    const float inv = __shfl(inv_l, rsub);
    const int pos = __shfl(pos_l, rsub);
    const int slot = __shfl(slot_l, rsub);
    float y0 = fmaf(y[0][v], inv, b0);
    float y1 = fmaf(y[1][v], inv, b1);
    if (adapted) {
      y0 += lo[0][v];
      y1 += lo[1][v];
    }
    if (rot) {
      const double tt = static_cast<double>(pos) * om;
      const float f = static_cast<float>(tt - rint(tt));
      const float sn = __builtin_amdgcn_sinf(f), cs = __builtin_amdgcn_cosf(f);
      const float r0 = y0 * cs - y1 * sn, r1 = y1 * cs + y0 * sn;
      y0 = r0;
      y1 = r1;
    }
    if (row < a.T) {
      uint16_t* o = a.out + row * a.N;
      const uint16_t o0 = f32_to_bf16_bits(y0), o1 = f32_to_bf16_bits(y1);
      o[c0] = o0;
      o[c1] = o1;
      uint16_t* kvr = cache_row(a.kv_k, a.kv_v, a.kv_num_slots, slot, col0, a.col_k, a.col_v);
      if (kvr) {
        const int cb = col0 < a.col_v ? a.col_k : a.col_v;
        kvr[c0 - cb] = o0;
        kvr[c1 - cb] = o1;
      }
    }
  }
}

// One-dimensional grid of (n_wblocks + nt) * groups blocks: first the nt * groups A blocks
// (block k: row group k / nt, A block k % nt), then the W blocks (block na + i: row group
// i / n_wblocks, W block i % n_wblocks).
__global__ __launch_bounds__(256, 1) void decode_main_kernel(MainArgs a) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kRingBytes + 2 * kMaxD];
  const int job = static_cast<int>(blockIdx.x);
  const int na = a.nt * a.groups;
  int nb, rg;
  if (job < na) {
    rg = job / a.nt;
    nb = a.n_wblocks + (job - rg * a.nt);
  } else {
    rg = (job - na) / a.n_wblocks;
    nb = (job - na) - rg * a.n_wblocks;
  }
  if (a.nf4 && nb < a.n_wblocks)
    decode_main_body<true>(a, smem, nb, rg);
  else
    decode_main_body<false>(a, smem, nb, rg);
}


}  // namespace

bool decode_supports(const FwdParams& p) {
  return p.D % 64 == 0 && p.d % 512 == 0 && p.d <= kMaxD && p.d / kBK >= kStages - 1 && p.T <= kMaxTokens &&
         p.r <= 64;
}

size_t decode_workspace_bytes(const FwdParams& p) { return decode_layout(p).total; }

hipError_t launch_fwd_decode(const FwdParams& p, hipStream_t s) {
  if (p.T == 0) return hipSuccess;
  const DecodeLayout L = decode_layout(p);
  unsigned char* ws = static_cast<unsigned char*>(p.ws);
  const int groups = L.Tp / kRows;

  MainArgs ma{};
  ma.x = static_cast<const uint16_t*>(p.x);
  ma.gamma = static_cast<const uint16_t*>(p.gamma);
  if (p.nf4) {
    PrepArgs pa{};
    pa.x = ma.x;
    pa.gamma = ma.gamma;
    pa.xg = reinterpret_cast<uint16_t*>(ws + L.xg);
    pa.inv = reinterpret_cast<float*>(ws + L.inv);
    pa.T = p.T;
    pa.d = static_cast<int>(p.d);
    pa.eps = p.eps;
    hipLaunchKernelGGL(decode_prep_kernel, dim3(static_cast<unsigned>((p.T + 3) / 4)), dim3(256), 0, s, pa);
    ma.xg = pa.xg;
    ma.inv = pa.inv;
  }
  ma.w = static_cast<const uint16_t*>(p.w);
  ma.nf4 = p.nf4;
  if (p.nf4) ma.wq = nf4_view(p.w, p.N, p.d);
  ma.bias = p.has_bias ? static_cast<const uint16_t*>(p.bias) : nullptr;
  for (int i = 0; i < 3; ++i) ma.a[i] = static_cast<const uint16_t*>(p.a[L.tgt[i]]);
  ma.pos = p.pos;
  ma.out = static_cast<uint16_t*>(p.out);
  ma.kv_k = static_cast<uint16_t*>(p.kv_k);
  ma.kv_v = static_cast<uint16_t*>(p.kv_v);
  ma.kv_slots = p.kv_slots;
  ma.kv_num_slots = p.kv_num_slots;
  ma.u = reinterpret_cast<uint16_t*>(ws + L.u);
  ma.sync = reinterpret_cast<uint64_t*>(ws + L.sync);
  for (int t = 0; t < 3; ++t) {
    ma.b[t] = static_cast<const uint16_t*>(p.b[t]);
    ma.ublock[t] = -1;
  }
  for (int i = 0; i < L.nt; ++i) ma.ublock[L.tgt[i]] = i;
  ma.T = p.T;
  ma.d = static_cast<int>(p.d);
  ma.N = p.N;
  ma.D = p.D;
  ma.r = p.r;
  ma.nt = L.nt;
  ma.n_wblocks = p.N / 64;
  ma.groups = groups;
  ma.col_k = p.col_k;
  ma.col_v = p.col_v;
  ma.rot_end = p.rot_end;
  ma.targets = p.targets;
  ma.scale = p.scale;
  ma.eps = p.eps;
  ma.log2_theta = log2(p.theta);
  timing_begin(s);
  hipLaunchKernelGGL(decode_main_kernel, dim3(static_cast<unsigned>((ma.n_wblocks + L.nt) * groups)), dim3(256), 0, s, ma);
  timing_end(s);
  return hipGetLastError();
}

}  // namespace lrq
