// MFMA tile family of the forward: bf16 operands, fp32 accumulation, head_dim 128.
//
//   out = RoPE( inv_t * ( W (x.gamma) + s B (A (x.gamma)) ) + b )
//
// which equals RoPE(W h + b + s B (A h)) with h = x * inv * gamma, inv = 1/rms(x): the
// row scale commutes with both products, so the kernel streams h' = bf16(x * gamma)
// through LDS, gathers sum(x^2) of its rows in the same K-loop, and applies inv to the
// fp32 accumulators in the epilogue.  Neither h nor U = A h is written to memory.
//
// Work decomposition
//   * Output tile 256 tokens x 256 columns (two heads), 512 threads.  Each of the eight
//     wavefronts owns 64 tokens x one complete head (2 x 4 MFMA 32x32x16 accumulators,
//     128 fp32 per lane), so the rotate-half partners (i, i + 64) sit in the same lane;
//     two wavefronts per SIMD let one stage operands while the other multiplies.
//   * One workgroup processes one 256-token tile against a run of consecutive
//     256-column tiles.  The first tile of the run that needs target t's adapter
//     computes U_t = A_t h' for the 256 rows (MFMA 16x16x32, inside the same K-loop)
//     and keeps bf16(s U_t) in LDS for the rest of the run; the rank-r up projection is
//     an extra K segment of MFMAs (K = r padded to 16) in each tile's epilogue.
//   * K-loop: 32-wide K steps, double-buffered LDS with an XOR swizzle of the 16-byte
//     chunks, global loads for step k+1 in flight while step k is multiplied.
//   * Workgroup ids are remapped so that the runs of one token tile share an XCD (and its
//     L2) when the grid is a multiple of the XCD count.
//   * Epilogue: inv row scale, bias, RoPE on q and k heads (angle pos * omega_i reduced in
//     double precision to a fraction of a turn, then the hardware sin / cos), bf16 store.
#include "lrq_internal.h"

namespace lrq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;
constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 32;
constexpr int kRowBytes = BK * 2;             // one staged row: 32 bf16 = 64 bytes
constexpr int kStageBytes = BM * kRowBytes;   // 16 KB per operand per stage
constexpr int OFF_A = 0;                      // 2 stages of h' tile
constexpr int OFF_B = 2 * kStageBytes;        // 2 stages of W tile
constexpr int OFF_L = 4 * kStageBytes;        // 2 stages of A_t rows (64 x 32 bf16)
constexpr int kLStage = 64 * kRowBytes;
constexpr int OFF_U = OFF_L + 2 * kLStage;    // bf16(s U) [256][16 * RP]
constexpr int kUBytes = BM * 64 * 2;
constexpr int OFF_INV = OFF_U + kUBytes;      // float [256]
constexpr int OFF_POS = OFF_INV + BM * 4;     // int [256]
constexpr int kSmemBytes = OFF_POS + BM * 4;  // 108544

struct TiledArgs {
  FwdParams p;
  int n_mt;        // token tiles
  int n_nt;        // column tiles
  int run;         // column tiles per workgroup
  int runs_per_m;  // workgroups per token tile
  int items;       // grid size
  int remap;       // XCD-aware id remap on/off
};

// byte offset of 16-byte chunk `chunk` (0..3) of row `row` in a [rows][32] bf16 tile
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ ((row >> 1) & 3)) << 4);
}

__device__ __forceinline__ float lo_bf16(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// h' = bf16(x * gamma) for 8 elements; optionally accumulates sum(x^2)
__device__ __forceinline__ bf16x8 scale_pack(uint4 x, uint4 g, bool acc_sq, float& ss) {
  const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
  const uint32_t gs[4] = {g.x, g.y, g.z, g.w};
  bf16x8 h;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float x0 = lo_bf16(xs[e]), x1 = hi_bf16(xs[e]);
    h[2 * e] = static_cast<__bf16>(x0 * lo_bf16(gs[e]));
    h[2 * e + 1] = static_cast<__bf16>(x1 * hi_bf16(gs[e]));
    if (acc_sq) ss = fmaf(x1, x1, fmaf(x0, x0, ss));
  }
  return h;
}

template <int RP>
__global__ __launch_bounds__(kThreads, 1) void fwd_tiled_kernel(TiledArgs ta) {
  constexpr int RPm = RP > 0 ? RP : 1;
  const FwdParams& p = ta.p;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kSmemBytes];
  float* s_inv = reinterpret_cast<float*>(smem + OFF_INV);
  int* s_pos = reinterpret_cast<int*>(smem + OFF_POS);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;  // 64-row quarter of the tile
  const int wn = wave & 1;   // head within the tile
  const int l32 = lane & 31, h32 = lane >> 5;
  const int l16 = lane & 15, h16 = lane >> 4;

  int item = blockIdx.x;
  if (ta.remap) item = (blockIdx.x & 7) * (ta.items >> 3) + (blockIdx.x >> 3);
  const int mt = item / ta.runs_per_m;
  const int run = item - mt * ta.runs_per_m;
  const int nt0 = run * ta.run;
  const int nt1 = min(nt0 + ta.run, ta.n_nt);
  const int64_t row0 = static_cast<int64_t>(mt) * BM;
  const int64_t T = p.T;
  const int d = static_cast<int>(p.d);
  const int nk = d / BK;

  const uint16_t* __restrict__ xg = static_cast<const uint16_t*>(p.x);
  const uint16_t* __restrict__ gg = static_cast<const uint16_t*>(p.gamma);
  const uint16_t* __restrict__ wg = static_cast<const uint16_t*>(p.w);
  uint16_t* __restrict__ out = static_cast<uint16_t*>(p.out);

  for (int i = tid; i < BM; i += kThreads) s_pos[i] = row0 + i < T ? p.pos[row0 + i] : 0;

  // load assignment: thread owns tile rows ld_row and ld_row + 128, 16-byte chunk ld_chunk
  const int ld_row = tid >> 2;
  const int ld_chunk = tid & 3;
  const bool ok0 = row0 + ld_row < T;
  const bool ok1 = row0 + ld_row + 128 < T;
  const uint16_t* xp0 = xg + (row0 + ld_row) * d + ld_chunk * 8;
  const uint16_t* xp1 = xp0 + static_cast<int64_t>(128) * d;
  const uint16_t* gp = gg + ld_chunk * 8;
  const int st_off0 = swz(ld_row, ld_chunk);
  const int st_off1 = swz(ld_row + 128, ld_chunk);
  const bool l_thread = tid < RP * 64;          // loads one chunk of the A_t rows
  const bool l_row_ok = l_thread && ld_row < p.r;

  float ss0 = 0.f, ss1 = 0.f;
  int u_target = -1;

  for (int nt = nt0; nt < nt1; ++nt) {
    const int head0 = 2 * nt;
    const int t = head0 < p.Hq ? 0 : (head0 < p.Hq + p.Hkv ? 1 : 2);
    const bool lora = RP > 0 && ((p.targets >> t) & 1u);
    const bool need_u = lora && u_target != t;
    const bool first = nt == nt0;
    const int64_t col0 = static_cast<int64_t>(nt) * BN;
    const uint16_t* wp0 = wg + (col0 + ld_row) * d + ld_chunk * 8;
    const uint16_t* wp1 = wp0 + static_cast<int64_t>(128) * d;
    const uint16_t* lp = static_cast<const uint16_t*>(p.a[t]) + static_cast<int64_t>(ld_row) * d + ld_chunk * 8;

    floatx16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = floatx16{};
    floatx4 uacc[2][RPm];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < RPm; ++j) uacc[i][j] = floatx4{};

    uint4 xr0, xr1, wr0, wr1, gr, lr = uint4{0, 0, 0, 0};
#define LRQ_LOAD_STEP(ks)                                                            \
    {                                                                                \
      const int koff = (ks) * BK;                                                    \
      xr0 = ok0 ? *reinterpret_cast<const uint4*>(xp0 + koff) : uint4{0, 0, 0, 0};   \
      xr1 = ok1 ? *reinterpret_cast<const uint4*>(xp1 + koff) : uint4{0, 0, 0, 0};   \
      wr0 = *reinterpret_cast<const uint4*>(wp0 + koff);                             \
      wr1 = *reinterpret_cast<const uint4*>(wp1 + koff);                             \
      gr = *reinterpret_cast<const uint4*>(gp + koff);                               \
      if (need_u && l_row_ok) lr = *reinterpret_cast<const uint4*>(lp + koff);       \
    }
#define LRQ_STORE_STEP(stage)                                                        \
    {                                                                                \
      unsigned char* sa_ = smem + OFF_A + (stage) * kStageBytes;                     \
      unsigned char* sb_ = smem + OFF_B + (stage) * kStageBytes;                     \
      *reinterpret_cast<bf16x8*>(sa_ + st_off0) = scale_pack(xr0, gr, first, ss0);   \
      *reinterpret_cast<bf16x8*>(sa_ + st_off1) = scale_pack(xr1, gr, first, ss1);   \
      *reinterpret_cast<uint4*>(sb_ + st_off0) = wr0;                                \
      *reinterpret_cast<uint4*>(sb_ + st_off1) = wr1;                                \
      if (need_u && l_thread)                                                        \
        *reinterpret_cast<uint4*>(smem + OFF_L + (stage) * kLStage + st_off0) = lr;  \
    }

    LRQ_LOAD_STEP(0);
    LRQ_STORE_STEP(0);
    __syncthreads();
    for (int ks = 0; ks < nk; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < nk) LRQ_LOAD_STEP(ks + 1);
      const unsigned char* sa = smem + OFF_A + cur * kStageBytes;
      const unsigned char* sb = smem + OFF_B + cur * kStageBytes;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8 af[2], bfr[4];
#pragma unroll
        for (int i = 0; i < 2; ++i)
          af[i] = *reinterpret_cast<const bf16x8*>(sa + swz(wm * 64 + i * 32 + l32, kk * 2 + h32));
#pragma unroll
        for (int j = 0; j < 4; ++j)
          bfr[j] = *reinterpret_cast<const bf16x8*>(sb + swz(wn * 128 + j * 32 + l32, kk * 2 + h32));
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
      if (RP > 0 && need_u) {
        // U rows 32 * wave + [0, 32) of this tile, all 16 * RP rank columns
        const unsigned char* sl = smem + OFF_L + cur * kLStage;
        bf16x8 au[2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
          au[i] = *reinterpret_cast<const bf16x8*>(sa + swz(wave * 32 + i * 16 + l16, h16));
#pragma unroll
        for (int c = 0; c < RPm; ++c) {
          const bf16x8 bl = *reinterpret_cast<const bf16x8*>(sl + swz(c * 16 + l16, h16));
#pragma unroll
          for (int i = 0; i < 2; ++i)
            uacc[i][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(au[i], bl, uacc[i][c], 0, 0, 0);
        }
      }
      if (ks + 1 < nk) LRQ_STORE_STEP(cur ^ 1);
      __syncthreads();
    }
#undef LRQ_LOAD_STEP
#undef LRQ_STORE_STEP

    // ---- row statistics (first tile of the run): the 4 threads of a row hold its partial sums
    if (first) {
      const float inv_d = 1.0f / static_cast<float>(d);
      float a0 = ss0, a1 = ss1;
      a0 += __shfl_xor(a0, 1);
      a0 += __shfl_xor(a0, 2);
      a1 += __shfl_xor(a1, 1);
      a1 += __shfl_xor(a1, 2);
      if (ld_chunk == 0) {
        s_inv[ld_row] = 1.0f / sqrtf(a0 * inv_d + p.eps);
        s_inv[ld_row + 128] = 1.0f / sqrtf(a1 * inv_d + p.eps);
      }
    }
    // ---- bf16(s * U) for the rest of the run
    if (RP > 0 && need_u) {
      uint16_t* su = reinterpret_cast<uint16_t*>(smem + OFF_U);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int c = 0; c < RPm; ++c)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int row = wave * 32 + i * 16 + h16 * 4 + v;
            su[row * (RPm * 16) + c * 16 + l16] = f32_to_bf16_bits(p.scale * uacc[i][c][v]);
          }
      u_target = t;
    }
    __syncthreads();

    // ---- LoRA up projection: acc += bf16(s U) B_t^T, K = 16 * RP
    if (RP > 0 && lora) {
      int lo, hi;
      target_cols(p, t, lo, hi);
      const uint16_t* __restrict__ bt = static_cast<const uint16_t*>(p.b[t]);
      uint16_t* sbt = reinterpret_cast<uint16_t*>(smem + OFF_A);  // stage buffers are idle here
      constexpr int kp = RPm * 16;
      for (int e = tid; e < BN * kp; e += kThreads) {
        const int c = e / kp, k = e - c * kp;
        sbt[c * kp + k] = k < p.r ? bt[(col0 + c - lo) * p.r + k] : uint16_t{0};
      }
      __syncthreads();
      const unsigned char* su = smem + OFF_U;
      const unsigned char* sbb = smem + OFF_A;
#pragma unroll
      for (int kk = 0; kk < RPm; ++kk) {
        bf16x8 af[2], bfr[4];
#pragma unroll
        for (int i = 0; i < 2; ++i)
          af[i] = *reinterpret_cast<const bf16x8*>(su + (wm * 64 + i * 32 + l32) * (kp * 2) + (kk * 2 + h32) * 16);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          bfr[j] = *reinterpret_cast<const bf16x8*>(sbb + (wn * 128 + j * 32 + l32) * (kp * 2) + (kk * 2 + h32) * 16);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
    }

    // ---- epilogue: row scale, bias, RoPE, store
    const bool rot = t < 2;
    const int64_t colw = col0 + wn * 128;
    float bias0 = 0.f, bias1 = 0.f, bias2 = 0.f, bias3 = 0.f;
    if (p.has_bias) {
      const uint16_t* __restrict__ bg = static_cast<const uint16_t*>(p.bias);
      bias0 = bf16_bits_to_f32(bg[colw + l32]);
      bias1 = bf16_bits_to_f32(bg[colw + 32 + l32]);
      bias2 = bf16_bits_to_f32(bg[colw + 64 + l32]);
      bias3 = bf16_bits_to_f32(bg[colw + 96 + l32]);
    }
    double om0 = 0.0, om1 = 0.0;  // turns per position for frequency l32 and 32 + l32
    if (rot) {
      const double l2t = log2(p.theta);
      om0 = exp2(-(2.0 * l32 / 128.0) * l2t) * 0.15915494309189533577;
      om1 = exp2(-(2.0 * (32 + l32) / 128.0) * l2t) * 0.15915494309189533577;
    }
    // lane rows: wm*64 + h32*4 + i*32 + (v/4)*8 + v%4; all offsets below are compile-time
    const float* inv_b = s_inv + wm * 64 + h32 * 4;
    const int* pos_b = s_pos + wm * 64 + h32 * 4;
    const int64_t rbase = row0 + wm * 64 + h32 * 4;
    uint16_t* obase = out + rbase * p.N + colw + l32;
    const bool full = row0 + BM <= T;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int ro = i * 32 + (v >> 2) * 8 + (v & 3);
        const float inv = inv_b[ro];
        float y0 = fmaf(acc[i][0][v], inv, bias0);
        float y1 = fmaf(acc[i][1][v], inv, bias1);
        float y2 = fmaf(acc[i][2][v], inv, bias2);
        float y3 = fmaf(acc[i][3][v], inv, bias3);
        if (rot) {
          const double pos = static_cast<double>(pos_b[ro]);
          const double t0 = pos * om0, t1 = pos * om1;
          const float f0 = static_cast<float>(t0 - rint(t0));
          const float f1 = static_cast<float>(t1 - rint(t1));
          const float s0 = __builtin_amdgcn_sinf(f0), c0 = __builtin_amdgcn_cosf(f0);
          const float s1 = __builtin_amdgcn_sinf(f1), c1 = __builtin_amdgcn_cosf(f1);
          const float r0 = y0 * c0 - y2 * s0, r2 = y2 * c0 + y0 * s0;
          const float r1 = y1 * c1 - y3 * s1, r3 = y3 * c1 + y1 * s1;
          y0 = r0; y1 = r1; y2 = r2; y3 = r3;
        }
        if (full || rbase + ro < T) {
          uint16_t* o = obase + static_cast<int64_t>(ro) * p.N;
          o[0] = f32_to_bf16_bits(y0);
          o[32] = f32_to_bf16_bits(y1);
          o[64] = f32_to_bf16_bits(y2);
          o[96] = f32_to_bf16_bits(y3);
        }
      }
    }
    __syncthreads();  // the next tile's first stage overwrites the buffers read above
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
  return p.T <= (int64_t{1} << 24) && p.D == 128 && p.Hq % 2 == 0 && p.Hkv % 2 == 0 && p.d % BK == 0 && p.d >= BK &&
         p.d <= (1 << 20) && p.r <= kMaxRank;
}

size_t tiled_workspace_bytes(const FwdParams&) { return 0; }

hipError_t launch_fwd_tiled(const FwdParams& p, hipStream_t s) {
  TiledArgs ta;
  ta.p = p;
  ta.n_mt = static_cast<int>((p.T + BM - 1) / BM);
  ta.n_nt = p.N / BN;
  const int64_t tiles = static_cast<int64_t>(ta.n_mt) * ta.n_nt;
  const int cus = cu_count();
  int run = static_cast<int>((tiles + cus - 1) / cus);
  run = run < 1 ? 1 : (run > ta.n_nt ? ta.n_nt : run);
  ta.run = run;
  ta.runs_per_m = (ta.n_nt + run - 1) / run;
  ta.items = ta.n_mt * ta.runs_per_m;
  ta.remap = ta.items % 8 == 0;
  const int rp = (p.r + 15) / 16;
  dim3 grid(ta.items), block(kThreads);
  switch (p.targets ? rp : 0) {
    case 0: hipLaunchKernelGGL(fwd_tiled_kernel<0>, grid, block, 0, s, ta); break;
    case 1: hipLaunchKernelGGL(fwd_tiled_kernel<1>, grid, block, 0, s, ta); break;
    case 2: hipLaunchKernelGGL(fwd_tiled_kernel<2>, grid, block, 0, s, ta); break;
    case 3: hipLaunchKernelGGL(fwd_tiled_kernel<3>, grid, block, 0, s, ta); break;
    default: hipLaunchKernelGGL(fwd_tiled_kernel<4>, grid, block, 0, s, ta); break;
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
