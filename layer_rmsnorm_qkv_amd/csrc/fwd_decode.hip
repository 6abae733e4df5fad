// Decode family of the forward (bf16, at most 256 rows): with so few rows, reading W_qkv
// from HBM is the whole cost, so the kernels are built around streaming W once at full
// bandwidth while the per-row work (RMSNorm, the rank-r down product) is done up front.
//
//   prep  one block per (slice of d, 32 LoRA ranks, 64 rows):
//           xg = bf16(x * gamma)                       [Tp][d]   (written by rank block 0)
//           ss[ks][row]   = sum over the slice of x^2             (partial row statistics)
//           Up[ks][row][k] = sum over the slice of xg A^T (MFMA)   (partial LoRA-down)
//   main  one block per 64 output columns (32 rotate-half pairs of one head) and 64 rows:
//           acc = xg W^T with d split between the 4 waves (register prefetch ring), summed
//           through LDS; then  y = inv * acc + B_t bf16(s * inv * U_t) + b,  rotate-half
//           on q and k heads, bf16 store.
// inv = 1 / sqrt(sum ss / d + eps) and U_t = sum Up are summed in a fixed order, so results
// are the same run to run.  Operator reading: the fused operator computes
// RoPE(W h + b + s B (A h)) with h = x * inv * gamma; here inv is applied after the
// products (it is a per-row scalar), gamma before them.
#include "lrq_internal.h"

namespace lrq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRows = 64;     // rows per row group
constexpr int kSlices = 8;    // slices of d in the prep kernel
constexpr int kRing = 8;      // main-loop steps (16 columns of d each) in flight per wave
constexpr int kMaxTokens = 256;

size_t al256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

struct DecodeLayout {
  int Tp;  // rows rounded up to the row group
  int R;   // sum of the targets' ranks
  int off[3];
  size_t xg, up, ss, total;
};

DecodeLayout decode_layout(const FwdParams& p) {
  DecodeLayout L{};
  L.Tp = static_cast<int>((p.T + kRows - 1) / kRows * kRows);
  int R = 0;
  for (int t = 0; t < 3; ++t) {
    L.off[t] = (p.targets & (1u << t)) ? R : -1;
    if (p.targets & (1u << t)) R += p.r;
  }
  L.R = R;
  size_t o = 0;
  L.xg = o;
  o += al256(static_cast<size_t>(L.Tp) * p.d * 2);
  L.up = o;
  o += al256(static_cast<size_t>(kSlices) * L.Tp * (R > 0 ? R : 1) * 4);
  L.ss = o;
  o += al256(static_cast<size_t>(kSlices) * L.Tp * 4);
  L.total = o;
  return L;
}

__device__ __forceinline__ float lo_f(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return static_cast<uint32_t>(f32_to_bf16_bits(a)) | (static_cast<uint32_t>(f32_to_bf16_bits(b)) << 16);
}

// ---------------------------------------------------------------- prep
struct PrepArgs {
  const uint16_t* x;
  const uint16_t* gamma;
  const uint16_t* a[3];
  uint16_t* xg;
  float* up;  // [kSlices][Tp][R]
  float* ss;  // [kSlices][Tp]
  int64_t T;
  int d, R, r, Tp;
  int off[3];
};

// Waves: row tile rt = wave & 1 (32 rows), half kh = wave >> 1 of the block's slice.
// MFMA operands come straight from global memory: both x rows and A rows hold the 8
// consecutive columns of d that one lane feeds the 32x32x16 product.
__global__ __launch_bounds__(256) void decode_prep_kernel(PrepArgs a) {
  __shared__ float red[2][17][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, h32 = lane >> 5;
  const int rt = wave & 1, kh = wave >> 1;
  const int ks = blockIdx.x, g = blockIdx.y, rg = blockIdx.z;
  const int tile_row = rg * kRows + rt * 32;
  const int row = tile_row + l32;
  const bool row_ok = row < a.T;
  const int slice = a.d / kSlices;
  const int k_begin = ks * slice + kh * (slice / 2) + 8 * h32;
  const int steps = slice / 32;

  // the lane's LoRA rank (B operand column) and its A row
  const int kr = g * 32 + l32;
  const uint16_t* arow = nullptr;
#pragma unroll
  for (int t = 0; t < 3; ++t)
    if (a.off[t] >= 0 && kr >= a.off[t] && kr < a.off[t] + a.r) arow = a.a[t] + static_cast<int64_t>(kr - a.off[t]) * a.d;

  const uint16_t* xrow = a.x + static_cast<int64_t>(row_ok ? row : 0) * a.d;
  uint16_t* xgrow = a.xg + static_cast<int64_t>(row) * a.d;
  const bool write_xg = g == 0;
  const bool lora = a.R > 0;

  floatx16 acc = {};
  float ss = 0.f;
#pragma unroll 4
  for (int s = 0; s < steps; ++s) {
    const int k = k_begin + 16 * s;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    const u32x4 xv = row_ok ? *reinterpret_cast<const u32x4*>(xrow + k) : zero;
    const u32x4 gv = *reinterpret_cast<const u32x4*>(a.gamma + k);
    const u32x4 av = arow ? *reinterpret_cast<const u32x4*>(arow + k) : zero;
    u32x4 xgv;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t xw = xv[q], gw = gv[q];
      const float x0 = lo_f(xw), x1 = hi_f(xw);
      ss = fmaf(x0, x0, ss);
      ss = fmaf(x1, x1, ss);
      xgv[q] = pack2(x0 * lo_f(gw), x1 * hi_f(gw));
    }
    if (write_xg) *reinterpret_cast<u32x4*>(xgrow + k) = xgv;
    if (lora) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, xgv),
                                                            __builtin_bit_cast(bf16x8, av), acc, 0, 0, 0);
  }

  // the second half of the slice is added to the first through LDS (fixed order)
  if (kh == 1) {
#pragma unroll
    for (int v = 0; v < 16; ++v) red[rt][v][lane] = acc[v];
    red[rt][16][lane] = ss;
  }
  __syncthreads();
  if (kh != 0) return;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] += red[rt][v][lane];
  ss += red[rt][16][lane];
  ss += __shfl_xor(ss, 32);  // lanes l and l + 32 cover the two halves of a step for one row
  if (write_xg && h32 == 0) a.ss[static_cast<int64_t>(ks) * a.Tp + row] = ss;
  if (lora && kr < a.R) {
    float* up = a.up + static_cast<int64_t>(ks) * a.Tp * a.R + kr;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int rr = tile_row + (v >> 2) * 8 + h32 * 4 + (v & 3);
      up[static_cast<int64_t>(rr) * a.R] = acc[v];
    }
  }
}

// ---------------------------------------------------------------- main
struct MainArgs {
  const uint16_t* xg;
  const uint16_t* w;
  const uint16_t* bias;
  const uint16_t* b[3];
  const float* up;
  const float* ss;
  const int32_t* pos;
  uint16_t* out;
  int64_t T;
  int d, N, D, Tp, R, r;
  int col_k, col_v, rot_end;
  int off[3];
  float scale, eps;
  double log2_theta;
};

struct Step {
  bf16x8 a0, a1, b0, b1;  // xg rows l32 and 32 + l32; W columns (pair halves) l32
};

__device__ __forceinline__ void load_step(Step& st, const uint16_t* xa, const uint16_t* wb, int64_t ld, int64_t half_ld,
                                          int k) {
  st.a0 = *reinterpret_cast<const bf16x8*>(xa + k);
  st.a1 = *reinterpret_cast<const bf16x8*>(xa + 32 * ld + k);
  st.b0 = *reinterpret_cast<const bf16x8*>(wb + k);
  st.b1 = *reinterpret_cast<const bf16x8*>(wb + half_ld + k);
}

__device__ __forceinline__ void mfma_step(const Step& st, floatx16 (&acc)[2][2]) {
  acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(st.a0, st.b0, acc[0][0], 0, 0, 0);
  acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(st.a0, st.b1, acc[0][1], 0, 0, 0);
  acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(st.a1, st.b0, acc[1][0], 0, 0, 0);
  acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(st.a1, st.b1, acc[1][1], 0, 0, 0);
}

// Tiles: rt = row tile (32 rows), ct = pair half (ct 0: columns col0 + l32, ct 1: the same
// plus D/2), so both members of a rotate-half pair sit in the same lane and register.
__global__ __launch_bounds__(256, 1) void decode_main_kernel(MainArgs a) {
  __shared__ float4 red[4][4][4][64];  // [wave][tile][quad of registers][lane]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, h32 = lane >> 5;
  const int nb = blockIdx.x, rg = blockIdx.y;
  const int per_head = a.D / 64;
  const int head = nb / per_head, sub = nb % per_head;
  const int half = a.D / 2;
  const int col0 = head * a.D + sub * 32;
  const int64_t ld = a.d;
  const int kq = a.d / 4;  // this wave's quarter of d
  const int steps = kq / 16;

  const uint16_t* xa = a.xg + static_cast<int64_t>(rg * kRows + l32) * ld + wave * kq + 8 * h32;
  const uint16_t* wb = a.w + static_cast<int64_t>(col0 + l32) * ld + wave * kq + 8 * h32;
  const int64_t half_ld = static_cast<int64_t>(half) * ld;

  floatx16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = floatx16{};

  Step ring[kRing];
#pragma unroll
  for (int q = 0; q < kRing; ++q) load_step(ring[q], xa, wb, ld, half_ld, 16 * q);
  int s = 0;
  for (; s + kRing < steps; s += kRing) {
#pragma unroll
    for (int q = 0; q < kRing; ++q) {
      mfma_step(ring[q], acc);
      load_step(ring[q], xa, wb, ld, half_ld, 16 * (s + q + kRing));
    }
  }
#pragma unroll
  for (int q = 0; q < kRing; ++q) mfma_step(ring[q], acc);

  // sum of the four quarters of d, in wave order
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const floatx16& v = acc[t >> 1][t & 1];
      red[wave][t][q][lane] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
    }
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

  // per-row values for row (tile row + l32); other lanes' rows are fetched with __shfl
  const int row_l = rg * kRows + rt * 32 + l32;
  float ssum = 0.f;
#pragma unroll
  for (int ks = 0; ks < kSlices; ++ks) ssum += a.ss[static_cast<int64_t>(ks) * a.Tp + row_l];
  const float inv_l = 1.0f / sqrtf(ssum / static_cast<float>(a.d) + a.eps);
  const int pos_l = row_l < a.T ? a.pos[row_l] : 0;

  // LoRA up: the block's columns lie in one target
  const int t = col0 < a.col_k ? 0 : (col0 < a.col_v ? 1 : 2);
  floatx16 lo[2] = {floatx16{}, floatx16{}};
  if (a.off[t] >= 0) {
    const int lo_t = t == 0 ? 0 : (t == 1 ? a.col_k : a.col_v);
    const float su = a.scale * inv_l;
    for (int kk = 0; kk < a.r; kk += 16) {
      bf16x8 uf;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int rank = kk + 8 * h32 + e;
        float u = 0.f;
        if (rank < a.r) {
          const float* up = a.up + static_cast<int64_t>(row_l) * a.R + a.off[t] + rank;
#pragma unroll
          for (int ks = 0; ks < kSlices; ++ks) u += up[static_cast<int64_t>(ks) * a.Tp * a.R];
        }
        uf[e] = static_cast<__bf16>(u * su);
      }
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const uint16_t* brow = a.b[t] + static_cast<int64_t>(col0 + ct * half + l32 - lo_t) * a.r;
        bf16x8 bf;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int rank = kk + 8 * h32 + e;
          bf[e] = __builtin_bit_cast(__bf16, rank < a.r ? brow[rank] : uint16_t{0});
        }
        lo[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(uf, bf, lo[ct], 0, 0, 0);
      }
    }
  }

  const int c0 = col0 + l32, c1 = col0 + half + l32;
  const float b0 = a.bias ? bf16_bits_to_f32(a.bias[c0]) : 0.f;
  const float b1 = a.bias ? bf16_bits_to_f32(a.bias[c1]) : 0.f;
  const bool rot = col0 < a.rot_end;
  const int i_pair = sub * 32 + l32;  // frequency index within the head
  const double om = exp2(-(2.0 * i_pair / a.D) * a.log2_theta) * 0.15915494309189533577;  // turns
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int rsub = (v >> 2) * 8 + h32 * 4 + (v & 3);
    const int64_t row = rg * kRows + rt * 32 + rsub;
    const float inv = __shfl(inv_l, rsub);
    const int pos = __shfl(pos_l, rsub);
    float y0 = fmaf(y[0][v], inv, lo[0][v] + b0);
    float y1 = fmaf(y[1][v], inv, lo[1][v] + b1);
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
      o[c0] = f32_to_bf16_bits(y0);
      o[c1] = f32_to_bf16_bits(y1);
    }
  }
}

}  // namespace

bool decode_supports(const FwdParams& p) {
  return p.D % 64 == 0 && p.d % 512 == 0 && p.d <= (1 << 20) && p.T <= kMaxTokens && p.r <= kMaxRank;
}

size_t decode_workspace_bytes(const FwdParams& p) { return decode_layout(p).total; }

hipError_t launch_fwd_decode(const FwdParams& p, hipStream_t s) {
  if (p.T == 0) return hipSuccess;
  const DecodeLayout L = decode_layout(p);
  unsigned char* ws = static_cast<unsigned char*>(p.ws);
  const int groups = L.Tp / kRows;

  PrepArgs pa{};
  pa.x = static_cast<const uint16_t*>(p.x);
  pa.gamma = static_cast<const uint16_t*>(p.gamma);
  for (int t = 0; t < 3; ++t) {
    pa.a[t] = static_cast<const uint16_t*>(p.a[t]);
    pa.off[t] = L.off[t];
  }
  pa.xg = reinterpret_cast<uint16_t*>(ws + L.xg);
  pa.up = reinterpret_cast<float*>(ws + L.up);
  pa.ss = reinterpret_cast<float*>(ws + L.ss);
  pa.T = p.T;
  pa.d = static_cast<int>(p.d);
  pa.R = L.R;
  pa.r = p.r;
  pa.Tp = L.Tp;
  const int rank_blocks = L.R > 0 ? (L.R + 31) / 32 : 1;
  hipLaunchKernelGGL(decode_prep_kernel, dim3(kSlices, rank_blocks, groups), dim3(256), 0, s, pa);

  MainArgs ma{};
  ma.xg = pa.xg;
  ma.w = static_cast<const uint16_t*>(p.w);
  ma.bias = p.has_bias ? static_cast<const uint16_t*>(p.bias) : nullptr;
  for (int t = 0; t < 3; ++t) {
    ma.b[t] = static_cast<const uint16_t*>(p.b[t]);
    ma.off[t] = L.off[t];
  }
  ma.up = pa.up;
  ma.ss = pa.ss;
  ma.pos = p.pos;
  ma.out = static_cast<uint16_t*>(p.out);
  ma.T = p.T;
  ma.d = static_cast<int>(p.d);
  ma.N = p.N;
  ma.D = p.D;
  ma.Tp = L.Tp;
  ma.R = L.R;
  ma.r = p.r;
  ma.col_k = p.col_k;
  ma.col_v = p.col_v;
  ma.rot_end = p.rot_end;
  ma.scale = p.scale;
  ma.eps = p.eps;
  ma.log2_theta = log2(p.theta);
  hipLaunchKernelGGL(decode_main_kernel, dim3(p.N / 64, groups), dim3(256), 0, s, ma);
  return hipGetLastError();
}

}  // namespace lrq
