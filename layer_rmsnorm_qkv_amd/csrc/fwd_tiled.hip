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
//   * K-loop: the shared tile pipeline (tile_common.h) with A = x and B = W': 64-wide steps
//     over d through a two-stage direct-to-LDS ring, one barrier per step.
//   * One workgroup processes one token tile against a run of consecutive column tiles.
//     Before the first tile of the run that needs target t's adapter, a short K pass over
//     the x tile and the rows of A'_t computes U_t = x A'_t^T and keeps bf16(s U_t) in LDS
//     for the rest of the run; the rank-r up projection is an extra K segment of MFMAs
//     (K = r rounded up to 16) before the epilogue of every tile of that target.
//   * Workgroup ids are remapped so that the runs of one token tile share an XCD (and its
//     L2) when the grid is a multiple of the XCD count.
//   * LoRA dropout: the U pass of target t reads x * keep_t (made with the keep bits before
//     this kernel) instead of x; the scale s is then alpha / r / (1 - p).
//   * Epilogue: row sums of squares -> inv, bias, RoPE on q and k heads (angle pos * omega_i
//     reduced in double precision to a fraction of a turn, then the hardware sin / cos),
//     bf16 store.
#include <algorithm>

#include "lrq_internal.h"
#include "tile_common.h"

namespace lrq {
namespace {

using namespace tile;

// LDS map for RB blocks of 32 LoRA ranks: the stage ring, then bf16(s U) [256][32 RB].
// The U pass stages the rows of A'_t in the B half of the ring.  The rows' inv and
// positions live in registers (two per lane, for the wave pair's 128 rows).
template <int RB>
struct Lay {
  static constexpr int U = kRingBytes;
  static constexpr int kUStride = RB * 32;
  static constexpr int TMP = kStageA;  // float [256]: row sums, once per run
  static constexpr int kBytes = U + BM * kUStride * 2;
  static_assert(kBytes <= kLdsMax, "LDS budget");
};

struct TiledArgs {
  const uint16_t* x;
  const uint16_t* wg;     // W' = bf16(W * gamma) [N][d] (workspace)
  const uint16_t* ag[3];  // A'_t = bf16(A_t * gamma) [r][d] (workspace)
  const uint16_t* xm[3];  // LoRA dropout: x * keep_t [T][d], the adapter's input (DROP only)
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

template <int RB, bool DROP>
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

  const Src src = make_src(p.x, d, row0, T, p.wg, d, wave, lane);
  const int nk = p.d / BK;

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
      // U_t = x A'_t^T for the token tile; bf16(s U) kept for the rest of the run (ranks >= r
      // re-read A'_t row r - 1 and are stored as 0)
      floatx16 u[RB == 2 ? 4 : 2];
      if (DROP) {
        // LoRA dropout: the adapter reads its masked copy of the x tile
        const Src sm = make_src(p.xm[t], d, row0, T, p.wg, d, wave, lane);
        rankpass<RB>(smem, sm, make_rank_src(p.ag[t], d, p.r, RB, wave, lane), nk, wave, lane, u);
      } else {
        rankpass<RB>(smem, src, make_rank_src(p.ag[t], d, p.r, RB, wave, lane), nk, wave, lane, u);
      }
#pragma unroll
      for (int i = 0; i < (RB == 2 ? 4 : 2); ++i) {
        const int rank = rank_col<RB>(wn, l32);
#pragma unroll
        for (int v = 0; v < 16; ++v)
          s_u[rank_row<RB>(i, v, wm, wn, h32) * L::kUStride + rank] =
              rank < p.r ? f32_to_bf16_bits(p.scale * u[i][v]) : uint16_t{0};
      }
      barrier_all();
      u_target = t;
    }

    Acc ta;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) ta.acc[i][j] = floatx16{};
#pragma unroll
    for (int i = 0; i < 4; ++i) ta.ss[i] = 0.f;

    if (nt == nt0) {
      kloop<true>(smem, ta, src, col0, nk, wave, lane);
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
      kloop<false>(smem, ta, src, col0, nk, wave, lane);
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

// W' = bf16(W * gamma) and A'_t = bf16(A_t * gamma) (W dequantised first when it is stored as
// NF4 blocks, the QLoRA base): rows [0, N) of the destination
// come from W (N = 0: W is not folded), then r rows per target from A_q, A_k, A_v (targets
// only).  Each thread scales 8 consecutive elements of one row (d % 8 == 0).
struct FoldArgs {
  const uint16_t* w;
  Nf4View wq;       // W as NF4 blocks instead (QLoRA base) when wq.codes != nullptr
  const uint16_t* a[3];
  const uint16_t* gamma;
  uint16_t* dst;
  int64_t rows;     // N + (number of targets) * r
  int N, r, d;
  int slot_t[3];    // target of the slot-th group of r rows after W
};

__global__ __launch_bounds__(256) void fold_gamma_kernel(FoldArgs f) {
  __shared__ float levels[16];
  if (threadIdx.x < 16) levels[threadIdx.x] = kNf4Levels[threadIdx.x];
  __syncthreads();
  const int64_t chunks_per_row = f.d / 8;
  const int64_t total = f.rows * chunks_per_row;
  for (int64_t c = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; c < total;
       c += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t row = c / chunks_per_row;
    const int k = static_cast<int>(c - row * chunks_per_row) * 8;
    if (row < f.N && f.wq.codes) {
      // NF4 base: dequantise 8 weights, times gamma, one rounding to bf16
      float wv[8];
      nf4_at8(f.wq, row, k, levels, wv);
      const uint4 g = *reinterpret_cast<const uint4*>(f.gamma + k);
      const uint32_t gs[4] = {g.x, g.y, g.z, g.w};
      uint32_t o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = f32_to_bf16_bits(wv[2 * e] * lo_bf16(gs[e]));
        const uint32_t hi = f32_to_bf16_bits(wv[2 * e + 1] * hi_bf16(gs[e]));
        o[e] = lo | (hi << 16);
      }
      *reinterpret_cast<uint4*>(f.dst + row * f.d + k) = uint4{o[0], o[1], o[2], o[3]};
      continue;
    }
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
// The NF4 view of W for the fold (QLoRA base), or an empty one for dense weights.
Nf4View weight_view(const FwdParams& p) { return p.nf4 ? nf4_view(p.w, p.N, p.d) : Nf4View{nullptr, nullptr, 0}; }
int n_targets(const FwdParams& p) { return (p.targets & 1u) + ((p.targets >> 1) & 1u) + ((p.targets >> 2) & 1u); }
size_t align256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }
}  // namespace

// Workspace: W' (unless the call brings prepared weights) then A'_t for every target, bf16,
// d elements per row.
size_t tiled_workspace_bytes(const FwdParams& p) {
  const int64_t w_rows = p.use_prepared ? 0 : p.N;
  return align256(static_cast<size_t>(w_rows + n_targets(p) * p.r) * static_cast<size_t>(p.d) * 2);
}

// Prepared forward weights: W' = bf16(W * gamma) [N][d], first in the prepared buffer.
size_t tiled_prepared_bytes(const FwdParams& p) { return align256(static_cast<size_t>(p.N) * p.d * 2); }

namespace {
void launch_fold(const uint16_t* w, const Nf4View& wq, int w_rows, const uint16_t* const a[3], int na,
                 const int slot_t[3], int r, const uint16_t* gamma, uint16_t* dst, int64_t d, hipStream_t s) {
  FoldArgs f;
  f.w = w;
  f.wq = wq;
  f.gamma = gamma;
  f.dst = dst;
  f.N = w_rows;
  f.r = r;
  f.d = static_cast<int>(d);
  for (int t = 0; t < 3; ++t) {
    f.a[t] = a[t];
    f.slot_t[t] = slot_t[t];
  }
  f.rows = static_cast<int64_t>(w_rows) + static_cast<int64_t>(na) * r;
  const int64_t chunks = f.rows * (d / 8);
  if (chunks == 0) return;
  const int fold_blocks = static_cast<int>(std::min<int64_t>((chunks + 255) / 256, 8 * 1024));
  hipLaunchKernelGGL(fold_gamma_kernel, dim3(fold_blocks), dim3(256), 0, s, f);
}
}  // namespace

hipError_t prepare_fwd_tiled(const FwdParams& p, void* prepared, hipStream_t s) {
  const uint16_t* none[3] = {nullptr, nullptr, nullptr};
  const int slot_t[3] = {0, 0, 0};
  launch_fold(static_cast<const uint16_t*>(p.w), weight_view(p), p.N, none, 0, slot_t, 0,
              static_cast<const uint16_t*>(p.gamma), static_cast<uint16_t*>(prepared), p.d, s);
  return hipGetLastError();
}

hipError_t launch_fwd_tiled(const FwdParams& p, hipStream_t s) {
  uint16_t* ws = static_cast<uint16_t*>(p.ws);
  // W' comes prepared, or is folded into the workspace ahead of the A'_t rows
  const int w_rows = p.use_prepared ? 0 : p.N;
  const uint16_t* srcs[3];
  int slot_t[3] = {0, 0, 0};
  int slots = 0;
  TiledArgs a;
  for (int t = 0; t < 3; ++t) {
    srcs[t] = static_cast<const uint16_t*>(p.a[t]);
    a.ag[t] = nullptr;
    a.b[t] = static_cast<const uint16_t*>(p.b[t]);
    a.xm[t] = nullptr;
    if (p.targets & (1u << t)) {
      if (p.dropout) a.xm[t] = p.drop_xm + static_cast<int64_t>(slots) * p.T * p.d;
      a.ag[t] = ws + (static_cast<int64_t>(w_rows) + static_cast<int64_t>(slots) * p.r) * p.d;
      slot_t[slots++] = t;
    }
  }
  launch_fold(static_cast<const uint16_t*>(p.w), weight_view(p), w_rows, srcs, slots, slot_t, p.r,
              static_cast<const uint16_t*>(p.gamma), ws, p.d, s);

  a.x = static_cast<const uint16_t*>(p.x);
  a.wg = p.use_prepared ? static_cast<const uint16_t*>(p.prepared) : ws;
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
  // Without adapters the RB = 1 kernel runs with no target set, so it takes no LoRA pass and
  // no up projection: its register allocation keeps the K-loop free of spills, which an
  // adapter-free instantiation of its own did not.
  const int rb = (!p.targets || p.r <= 32) ? 1 : 2;
  dim3 grid(a.items), block(kThreads);
  timing_begin(s);
  const bool drop = p.dropout;
  switch (rb) {
    case 1:
      if (drop)
        hipLaunchKernelGGL((fwd_tiled_kernel<1, true>), grid, block, 0, s, a);
      else
        hipLaunchKernelGGL((fwd_tiled_kernel<1, false>), grid, block, 0, s, a);
      break;
    default:
      if (drop)
        hipLaunchKernelGGL((fwd_tiled_kernel<2, true>), grid, block, 0, s, a);
      else
        hipLaunchKernelGGL((fwd_tiled_kernel<2, false>), grid, block, 0, s, a);
      break;
  }
  timing_end(s);
  return hipGetLastError();
}

}  // namespace lrq
