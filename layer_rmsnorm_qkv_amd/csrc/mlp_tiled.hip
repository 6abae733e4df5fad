// MFMA tile family of the LoRA-adapted SwiGLU MLP (bf16 operands, fp32 accumulation):
//
//   g = h W_g^T + s (h A_g^T) B_g^T,   u = h W_u^T + s (h A_u^T) B_u^T,   a = SiLU(g) * u
//   y = a W_d^T + s (a A_d^T) B_d^T
//
// in two kernels on the shared tile pipeline (tile_common.h):
//   gate_up  output tile 256 tokens x 128 intermediate columns.  The B tile stages 64 rows of
//            W_g and the same 64 rows of W_u per wave pair: waves 0, 2 of the DMA fill gate
//            rows, waves 1, 3 the matching up rows, so that in the MFMA layout wave (wm, wn)
//            holds gate columns f and up columns f in accumulators j and j + 2 of the same
//            lane -- SwiGLU needs no data exchange, as RoPE's rotate-half partners in the
//            attention projection.  Before the first tile of a run, one K pass computes the
//            LoRA down projections of both adapters (the rows of A_g and A_u stacked as 64
//            rank rows) and keeps bf16(s U) in LDS; the up projections are an extra K segment
//            of MFMAs.  The epilogue forms SiLU(g) * u in fp32 and stores a once, as bf16:
//            g and u never leave the chip.
//   down     y = a W_d^T with the down adapter: the same tile kernel over K = intermediate
//            size (256 x 256 tiles, runs of column tiles, the LoRA K pass per run).
// a is the one intermediate in memory: a full down projection needs all of a row of a, and a
// [256 x d] fp32 accumulator for all of it does not fit on a CU.
#include <algorithm>

#include "lrq_internal.h"
#include "tile_common.h"

namespace lrq {
namespace {

using namespace tile;

size_t al256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

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

// Runs of consecutive column tiles per workgroup so that the grid is about one wave over the
// CUs; ids remapped so the runs of one token tile share an XCD when the grid allows.  (Run
// major order -- one run's weight tiles shared by all token tiles of an XCD -- measured 2-4%
// slower for the gate/up and the down kernel.)
struct Runs {
  int n_ct, run, runs_per_m, items, remap;
};

Runs make_runs(int64_t T, int n_ct) {
  Runs R;
  const int n_mt = static_cast<int>((T + BM - 1) / BM);
  R.n_ct = n_ct;
  const int64_t tiles = static_cast<int64_t>(n_mt) * n_ct;
  const int cus = cu_count();
  int run = static_cast<int>((tiles + cus - 1) / cus);
  R.run = run < 1 ? 1 : (run > n_ct ? n_ct : run);
  R.runs_per_m = (n_ct + R.run - 1) / R.run;
  R.items = n_mt * R.runs_per_m;
  R.remap = R.items % 8 == 0;
  return R;
}

__device__ __forceinline__ void item_of(const Runs& R, int& mt, int& c0, int& c1) {
  int item = blockIdx.x;
  if (R.remap) item = (blockIdx.x & 7) * (R.items >> 3) + (blockIdx.x >> 3);
  mt = item / R.runs_per_m;
  const int run = item - mt * R.runs_per_m;
  c0 = run * R.run;
  c1 = min(c0 + R.run, R.n_ct);
}

// 8 consecutive ranks [k0, k0 + 8) of row `row` of a [rows][r] matrix as an MFMA operand,
// zero past r (a 16-byte load when r is a multiple of 8)
__device__ __forceinline__ bf16x8 rank_frag(const uint16_t* m, int64_t row, int r, int k0) {
  bf16x8 f;
  const uint16_t* src = m + row * r + k0;
  if ((r & 7) == 0 && k0 < r) {
    f = *reinterpret_cast<const bf16x8*>(src);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = __builtin_bit_cast(__bf16, k0 + e < r ? src[e] : uint16_t{0});
  }
  return f;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// ---------------------------------------------------------------- gate + up + SwiGLU
struct GateUpArgs {
  const uint16_t* h;    // [T][d]
  const uint16_t* wg;   // [F][d]
  const uint16_t* wu;   // [F][d]
  const uint16_t* ag;   // [r][d] (nullptr: no gate adapter)
  const uint16_t* au;   // [r][d] (nullptr: no up adapter)
  const uint16_t* bg;   // [F][r]
  const uint16_t* bu;   // [F][r]
  uint16_t* act;        // [T][F]
  int64_t T;
  int d, F, r;
  float scale;
  Runs runs;            // column tiles of 128 intermediate columns
};

template <bool LORA>
__global__ __launch_bounds__(kThreads, 1) void mlp_gate_up_kernel(GateUpArgs p) {
  constexpr int kUStride = 64;  // bf16(s U): ranks 0..31 gate, 32..63 up
  constexpr int kBytes = LORA ? kRingBytes + BM * kUStride * 2 : kRingBytes;
  static_assert(kBytes <= kLdsMax, "LDS budget");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kBytes];
  uint16_t* s_u = reinterpret_cast<uint16_t*>(smem + kRingBytes);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, h32 = lane >> 5;
  int mt, ft0, ft1;
  item_of(p.runs, mt, ft0, ft1);
  const int64_t row0 = static_cast<int64_t>(mt) * BM;
  const int64_t T = p.T, d = p.d;

  // A = h; B: DMA wave w stages rows (w / 2) * 64 .. +64 of W_u (w odd) or W_g (w even) of the
  // tile's 128 intermediate columns (kloop adds the tile's first column times d)
  SrcC src = make_src_c(p.h, d, row0, T, p.wg, d, wave, lane);
  {
    const int rsub = lane >> 3, pc = lane & 7;
    const uint16_t* wb = ((wave & 1) ? p.wu : p.wg) + static_cast<int64_t>((wave >> 1) * 64 + rsub) * d;
    src.b[0] = wb + (pc ^ rsub) * 8;
    src.b[1] = wb + (pc ^ rsub ^ 1) * 8;
  }
  const int nk = p.d / BK;

  if constexpr (LORA) {
    // U of both adapters for the token tile: rank rows 0..31 from A_g, 32..63 from A_u (rows
    // past r, or of an absent adapter, re-read a valid row and are stored as 0)
    RankSrc rs;
    {
      const int pc = lane & 7, rsub = lane >> 3;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int R = 16 * wave + 8 * q + rsub;
        const uint16_t* m = R < 32 ? (p.ag ? p.ag : p.au) : (p.au ? p.au : p.ag);
        rs.r[q] = m + static_cast<int64_t>(min(R & 31, p.r - 1)) * d + (pc ^ chunk_xor(R)) * 8;
      }
    }
    floatx16 u[4];
    rankpass<2>(smem, src, rs, nk, wave, lane, u);
    const int rank = rank_col<2>(wn, l32);  // 32 wn + l32: wn 0 gate, 1 up
    const bool on = (rank < 32 ? p.ag : p.au) != nullptr && (rank & 31) < p.r;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        s_u[rank_row<2>(i, v, wm, wn, h32) * kUStride + rank] = on ? f32_to_bf16_bits(p.scale * u[i][v]) : uint16_t{0};
    barrier_all();
  }

  for (int ft = ft0; ft < ft1; ++ft) {
    const int64_t f0 = static_cast<int64_t>(ft) * 128;
    Acc ta;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) ta.acc[i][j] = floatx16{};
    kloop<false>(smem, ta, src, f0, nk, wave, lane);

    // lane columns: j = 0, 1 gate f0 + 64 wn + 32 (j % 2) + l32; j = 2, 3 the same up columns
    if constexpr (LORA) {
      // opaque per-tile copies (as in the epilogue): nothing of this part is hoisted into
      // registers that would stay live across the K-loop
      int urow = wm * 128 + l32, bcol = wn * 64 + l32;
      asm volatile("" : "+v"(urow), "+v"(bcol));
      const int ksteps = (p.r + 15) >> 4;
      for (int kq = 0; kq < ksteps; ++kq) {
        const int k0 = kq * 16 + h32 * 8;
#pragma unroll
        for (int half = 0; half < 2; ++half) {  // 0: gate (j = 0, 1), 1: up (j = 2, 3)
          const uint16_t* bm = half ? p.bu : p.bg;
          if (!bm) continue;
          bf16x8 af[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            af[i] = *reinterpret_cast<const bf16x8*>(s_u + (urow + i * 32) * kUStride + half * 32 + k0);
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const bf16x8 bf = rank_frag(bm, f0 + bcol + jj * 32, p.r, k0);
#pragma unroll
            for (int i = 0; i < 4; ++i)
              ta.acc[i][2 * half + jj] =
                  __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf, ta.acc[i][2 * half + jj], 0, 0, 0);
          }
        }
      }
    }

    // epilogue: a = SiLU(g) * u, bf16.  Opaque per-tile copies of the lane's first row and of
    // the row stride keep the compiler from hoisting 64 row addresses out of the tile loop.
    int lrow = wm * 128 + h32 * 4;
    int64_t stride = p.F;
    asm volatile("" : "+v"(lrow), "+s"(stride));
    uint16_t* obase = p.act + (row0 + lrow) * stride + f0 + wn * 64 + l32;
    const int64_t left = T - (row0 + lrow);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int ro = i * 32 + (v >> 2) * 8 + (v & 3);
        if (ro >= left) continue;
        uint16_t* o = obase + ro * stride;
        o[0] = f32_to_bf16_bits(silu(ta.acc[i][0][v]) * ta.acc[i][2][v]);
        o[32] = f32_to_bf16_bits(silu(ta.acc[i][1][v]) * ta.acc[i][3][v]);
      }
    }
  }
}

// ---------------------------------------------------------------- down projection
struct DownArgs {
  const uint16_t* act;  // [T][F]
  const uint16_t* wd;   // [d][F]
  const uint16_t* ad;   // [r][F] (nullptr: no adapter)
  const uint16_t* bd;   // [d][r]
  uint16_t* out;        // [T][d]
  int64_t T;
  int d, F, r;
  float scale;
  Runs runs;            // column tiles of 256 output columns
};

template <bool LORA>
__global__ __launch_bounds__(kThreads, 1) void mlp_down_kernel(DownArgs p) {
  constexpr int kUStride = 32;
  constexpr int kBytes = LORA ? kRingBytes + BM * kUStride * 2 : kRingBytes;
  static_assert(kBytes <= kLdsMax, "LDS budget");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kBytes];
  uint16_t* s_u = reinterpret_cast<uint16_t*>(smem + kRingBytes);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, h32 = lane >> 5;
  int mt, nt0, nt1;
  item_of(p.runs, mt, nt0, nt1);
  const int64_t row0 = static_cast<int64_t>(mt) * BM;
  const int64_t T = p.T, F = p.F;
  const SrcC src = make_src_c(p.act, F, row0, T, p.wd, F, wave, lane);
  const int nk = p.F / BK;

  if constexpr (LORA) {
    floatx16 u[2];
    rankpass<1>(smem, src, make_rank_src(p.ad, F, p.r, 1, wave, lane), nk, wave, lane, u);
    const int rank = rank_col<1>(wn, l32);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        s_u[rank_row<1>(i, v, wm, wn, h32) * kUStride + rank] = rank < p.r ? f32_to_bf16_bits(p.scale * u[i][v]) : uint16_t{0};
    barrier_all();
  }

  for (int nt = nt0; nt < nt1; ++nt) {
    const int64_t col0 = static_cast<int64_t>(nt) * BN;
    Acc ta;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) ta.acc[i][j] = floatx16{};
    kloop<false, kXorReads>(smem, ta, src, col0, nk, wave, lane);
    if constexpr (LORA) {
      int urow = wm * 128 + l32, bcol = wn * 128 + l32;
      asm volatile("" : "+v"(urow), "+v"(bcol));
      const int ksteps = (p.r + 15) >> 4;
      for (int kq = 0; kq < ksteps; ++kq) {
        const int k0 = kq * 16 + h32 * 8;
        bf16x8 af[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          af[i] = *reinterpret_cast<const bf16x8*>(s_u + (urow + i * 32) * kUStride + k0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bf16x8 bf = rank_frag(p.bd, col0 + bcol + j * 32, p.r, k0);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            ta.acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf, ta.acc[i][j], 0, 0, 0);
        }
      }
    }
    int lrow = wm * 128 + h32 * 4;
    int64_t stride = p.d;
    asm volatile("" : "+v"(lrow), "+s"(stride));
    uint16_t* obase = p.out + (row0 + lrow) * stride + col0 + wn * 128 + l32;
    const int64_t left = T - (row0 + lrow);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int ro = i * 32 + (v >> 2) * 8 + (v & 3);
        if (ro >= left) continue;
        uint16_t* o = obase + ro * stride;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j * 32] = f32_to_bf16_bits(ta.acc[i][j][v]);
      }
    }
  }
}

}  // namespace

bool mlp_supports(const MlpParams& p) {
  return p.d % BN == 0 && p.F % 128 == 0 && p.d >= BN && p.F >= 128 && p.d <= (1 << 20) && p.F <= (1 << 20) &&
         p.r <= 32 && p.T <= (int64_t{1} << 24);
}

size_t mlp_workspace_bytes(const MlpParams& p) { return al256(static_cast<size_t>(p.T) * p.F * 2); }

hipError_t launch_mlp(const MlpParams& p, hipStream_t s) {
  if (p.T == 0) return hipSuccess;
  uint16_t* act = static_cast<uint16_t*>(p.ws);
  const bool lg = p.targets & 1u, lu = p.targets & 2u, ld = p.targets & 4u;

  GateUpArgs g{};
  g.h = static_cast<const uint16_t*>(p.h);
  g.wg = static_cast<const uint16_t*>(p.wg);
  g.wu = static_cast<const uint16_t*>(p.wu);
  g.ag = lg ? static_cast<const uint16_t*>(p.a[0]) : nullptr;
  g.au = lu ? static_cast<const uint16_t*>(p.a[1]) : nullptr;
  g.bg = lg ? static_cast<const uint16_t*>(p.b[0]) : nullptr;
  g.bu = lu ? static_cast<const uint16_t*>(p.b[1]) : nullptr;
  g.act = act;
  g.T = p.T;
  g.d = static_cast<int>(p.d);
  g.F = static_cast<int>(p.F);
  g.r = p.r;
  g.scale = p.scale;
  g.runs = make_runs(p.T, static_cast<int>(p.F / 128));
  timing_begin(s);
  if (lg || lu)
    hipLaunchKernelGGL(mlp_gate_up_kernel<true>, dim3(g.runs.items), dim3(kThreads), 0, s, g);
  else
    hipLaunchKernelGGL(mlp_gate_up_kernel<false>, dim3(g.runs.items), dim3(kThreads), 0, s, g);
  timing_end(s);

  DownArgs dn{};
  dn.act = act;
  dn.wd = static_cast<const uint16_t*>(p.wd);
  dn.ad = ld ? static_cast<const uint16_t*>(p.a[2]) : nullptr;
  dn.bd = ld ? static_cast<const uint16_t*>(p.b[2]) : nullptr;
  dn.out = static_cast<uint16_t*>(p.out);
  dn.T = p.T;
  dn.d = static_cast<int>(p.d);
  dn.F = static_cast<int>(p.F);
  dn.r = p.r;
  dn.scale = p.scale;
  dn.runs = make_runs(p.T, static_cast<int>(p.d / BN));
  if (ld)
    hipLaunchKernelGGL(mlp_down_kernel<true>, dim3(dn.runs.items), dim3(kThreads), 0, s, dn);
  else
    hipLaunchKernelGGL(mlp_down_kernel<false>, dim3(dn.runs.items), dim3(kThreads), 0, s, dn);
  return hipGetLastError();
}

}  // namespace lrq
