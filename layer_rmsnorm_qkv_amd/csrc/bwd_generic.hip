// Generic fused backward: any shape with an even head size and d <= kMaxCols * 256,
// float32 or bfloat16.  W, gamma and bias are frozen; gradients flow to x and to the
// LoRA factors.
//
// One workgroup owns kRows complete token rows:
//   1. RMSNorm statistics and U_t = A_t h (h recomputed from x, never stored);
//   2. loop over heads: G = inverse rotation of dy (q, k heads; v as is) staged in LDS,
//      V_t += G_t B_t, dB_t += s G_t^T U_t (atomics), dh += G W;
//   3. dh += s V_t A_t and dA_t += s V_t^T h (atomics);
//   4. dx = inv gamma dh - inv^3 x <gamma x, dh> / d, computed from the complete dh row.
// In the bf16 path h, U, G and V are rounded once to bf16 (they are the operands of the
// products) and everything else stays in fp32.  dA / dB are zeroed by a fill kernel first,
// so they are overwritten.  The atomics make the summation order of dA / dB vary between
// runs (within rounding).  With LoRA dropout, U_t, dA_t and target t's dh term see only the
// features that t's keep bits keep, and s = alpha / r / (1 - p).  With an NF4 base (QLoRA), W
// is dequantised as it is read.
#include <algorithm>

#include "lrq_internal.h"

namespace lrq {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 4;
constexpr int kMaxCols = 16;  // columns of dh per thread -> d <= 4096
constexpr int kMaxHead = 256; // head_dim <= 256

__global__ void zero_kernel(float* p, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = 0.f;
}

template <typename TIn, bool kBf16>
__global__ __launch_bounds__(kThreads) void bwd_generic_kernel(BwdParams bp) {
  const FwdParams& p = bp.f;
  __shared__ float s_inv[kRows];
  __shared__ float s_u[kRows][3 * kMaxRank];
  __shared__ float s_v[kRows][3 * kMaxRank];
  __shared__ float s_g[kRows][kMaxHead];
  __shared__ float s_red[kThreads / 64][kRows];
  __shared__ float s_c[kRows];

  const TIn* __restrict__ x = static_cast<const TIn*>(p.x);
  const TIn* __restrict__ gamma = static_cast<const TIn*>(p.gamma);
  const TIn* __restrict__ w = static_cast<const TIn*>(p.w);
  const Nf4View wq = nf4_view(p.w, p.N, p.d);  // used when p.nf4 (the QLoRA base)
  const TIn* __restrict__ dy = static_cast<const TIn*>(bp.dy);
  TIn* __restrict__ dx = static_cast<TIn*>(bp.dx);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * kRows;
  const int64_t d = p.d;
  const int D = p.D, half = p.D / 2;
  const int n_rows = static_cast<int>(min<int64_t>(kRows, p.T - row0));

  // ---- 1. statistics
  for (int rr = wave; rr < kRows; rr += kThreads / 64) {
    float ss = 0.f;
    if (rr < n_rows)
      for (int64_t j = lane; j < d; j += 64) {
        const float v = load_elem(x, (row0 + rr) * d + j);
        ss = fmaf(v, v, ss);
      }
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
    if (lane == 0) s_inv[rr] = 1.0f / sqrtf(ss / static_cast<float>(d) + p.eps);
  }
  __syncthreads();

  auto h_at = [&](int rr, int64_t j) -> float {
    float v = load_elem(x, (row0 + rr) * d + j) * s_inv[rr] * load_elem(gamma, j);
    return kBf16 ? round_bf16(v) : v;
  };
  // LoRA dropout: does target t's adapter keep feature j of row rr?
  const int64_t dw = (d + 31) / 32;
  auto kept = [&](int t, int rr, int64_t j) -> bool {
    if (!p.dropout) return true;
    const uint32_t w = p.drop_bits_r[(static_cast<int64_t>(target_slot(p.targets, t)) * p.T + row0 + rr) * dw + j / 32];
    return (w >> (j % 32)) & 1u;
  };

  // U_t[row][k] = A_t[k] . h[row]: one wave per dot product
  for (int t = 0; t < 3; ++t) {
    if (!(p.targets & (1u << t))) continue;
    const TIn* __restrict__ a = static_cast<const TIn*>(p.a[t]);
    for (int e = wave; e < kRows * p.r; e += kThreads / 64) {
      const int rr = e / p.r, k = e % p.r;
      float s = 0.f;
      if (rr < n_rows)
        for (int64_t j = lane; j < d; j += 64)
          if (kept(t, rr, j)) s = fmaf(h_at(rr, j), load_elem(a, k * d + j), s);
      for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
      if (lane == 0) s_u[rr][t * kMaxRank + k] = kBf16 ? round_bf16(s) : s;
    }
  }
  __syncthreads();

  // ---- 2. heads
  float acc[kRows][kMaxCols];
#pragma unroll
  for (int rr = 0; rr < kRows; ++rr)
#pragma unroll
    for (int m = 0; m < kMaxCols; ++m) acc[rr][m] = 0.f;
  float v_acc[3] = {0.f, 0.f, 0.f};  // V_t[tid / r][tid % r]

  const int n_heads = p.N / D;
  for (int hh = 0; hh < n_heads; ++hh) {
    const int c0 = hh * D;
    for (int e = tid; e < kRows * half; e += kThreads) {
      const int rr = e / half, i = e % half;
      float ga = 0.f, gb = 0.f;
      if (rr < n_rows) {
        const int64_t row = row0 + rr;
        ga = load_elem(dy, row * p.N + c0 + i);
        gb = load_elem(dy, row * p.N + c0 + i + half);
        if (c0 < p.rot_end) {  // transpose of the rotation: angle -phi
          float c, s;
          rope_cos_sin(p.pos[row], rope_omega(p.theta, i, D), c, s);
          const float ra = ga * c + gb * s;
          const float rb = gb * c - ga * s;
          ga = ra;
          gb = rb;
        }
        if (kBf16) {
          ga = round_bf16(ga);
          gb = round_bf16(gb);
        }
      }
      s_g[rr][i] = ga;
      s_g[rr][i + half] = gb;
    }
    __syncthreads();

    const int t = c0 < p.col_k ? 0 : (c0 < p.col_v ? 1 : 2);
    if (p.targets & (1u << t)) {
      int lo, hi;
      target_cols(p, t, lo, hi);
      const TIn* __restrict__ bt = static_cast<const TIn*>(p.b[t]);
      if (tid < kRows * p.r) {
        const int rr = tid / p.r, k = tid % p.r;
        float s = v_acc[t];
        for (int i = 0; i < D; ++i) s = fmaf(s_g[rr][i], load_elem(bt, static_cast<int64_t>(c0 - lo + i) * p.r + k), s);
        v_acc[t] = s;
      }
      float* __restrict__ dbt = bp.db[t];
      for (int e = tid; e < D * p.r; e += kThreads) {
        const int i = e / p.r, k = e % p.r;
        float s = 0.f;
        for (int rr = 0; rr < n_rows; ++rr) s = fmaf(s_g[rr][i], s_u[rr][t * kMaxRank + k], s);
        atomicAdd(&dbt[static_cast<int64_t>(c0 - lo + i) * p.r + k], p.scale * s);
      }
    }
    for (int i = 0; i < D; ++i) {
      const int64_t wrow = static_cast<int64_t>(c0 + i) * d;
#pragma unroll
      for (int m = 0; m < kMaxCols; ++m) {
        const int64_t j = tid + static_cast<int64_t>(m) * kThreads;
        if (j < d) {
          const float wv = p.nf4 ? nf4_at(wq, c0 + i, j) : load_elem(w, wrow + j);
#pragma unroll
          for (int rr = 0; rr < kRows; ++rr) acc[rr][m] = fmaf(s_g[rr][i], wv, acc[rr][m]);
        }
      }
    }
    __syncthreads();
  }

  // ---- 3. LoRA terms of dh, and dA
  for (int t = 0; t < 3; ++t)
    if ((p.targets & (1u << t)) && tid < kRows * p.r) {
      const float v = tid / p.r < n_rows ? v_acc[t] : 0.f;
      s_v[tid / p.r][t * kMaxRank + tid % p.r] = kBf16 ? round_bf16(v) : v;
    }
  __syncthreads();
  for (int t = 0; t < 3; ++t) {
    if (!(p.targets & (1u << t))) continue;
    const TIn* __restrict__ a = static_cast<const TIn*>(p.a[t]);
    float* __restrict__ dat = bp.da[t];
#pragma unroll
    for (int m = 0; m < kMaxCols; ++m) {
      const int64_t j = tid + static_cast<int64_t>(m) * kThreads;
      if (j >= d) continue;
      // the adapter's input feature and the factor of its dh term: h and s, or 0 and 0 where
      // the adapter's dropout drops the feature
      float hj[kRows], fk[kRows];
#pragma unroll
      for (int rr = 0; rr < kRows; ++rr) {
        const bool on = rr < n_rows && kept(t, rr, j);
        hj[rr] = on ? h_at(rr, j) : 0.f;
        fk[rr] = on ? p.scale : 0.f;
      }
      for (int k = 0; k < p.r; ++k) {
        const float av = load_elem(a, k * d + j);
        float da = 0.f;
#pragma unroll
        for (int rr = 0; rr < kRows; ++rr) {
          const float v = s_v[rr][t * kMaxRank + k];
          acc[rr][m] = fmaf(fk[rr] * v, av, acc[rr][m]);
          da = fmaf(v, hj[rr], da);
        }
        atomicAdd(&dat[k * d + j], p.scale * da);
      }
    }
  }

  // ---- 4. RMSNorm backward
  float part[kRows];
#pragma unroll
  for (int rr = 0; rr < kRows; ++rr) part[rr] = 0.f;
#pragma unroll
  for (int m = 0; m < kMaxCols; ++m) {
    const int64_t j = tid + static_cast<int64_t>(m) * kThreads;
    if (j >= d) continue;
    const float g = load_elem(gamma, j);
#pragma unroll
    for (int rr = 0; rr < kRows; ++rr)
      if (rr < n_rows) part[rr] = fmaf(g * load_elem(x, (row0 + rr) * d + j), acc[rr][m], part[rr]);
  }
#pragma unroll
  for (int rr = 0; rr < kRows; ++rr) {
    float s = part[rr];
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
    if (lane == 0) s_red[wave][rr] = s;
  }
  __syncthreads();
  if (tid < kRows) {
    float s = 0.f;
    for (int wv = 0; wv < kThreads / 64; ++wv) s += s_red[wv][tid];
    s_c[tid] = s;
  }
  __syncthreads();
#pragma unroll
  for (int m = 0; m < kMaxCols; ++m) {
    const int64_t j = tid + static_cast<int64_t>(m) * kThreads;
    if (j >= d) continue;
    const float g = load_elem(gamma, j);
#pragma unroll
    for (int rr = 0; rr < kRows; ++rr) {
      if (rr >= n_rows) continue;
      const float inv = s_inv[rr];
      const float xv = load_elem(x, (row0 + rr) * d + j);
      const float v = inv * g * acc[rr][m] - inv * inv * inv * xv * (s_c[rr] / static_cast<float>(d));
      store_elem(dx, (row0 + rr) * d + j, v);
    }
  }
}

template <typename TIn, bool kBf16>
hipError_t launch(const BwdParams& bp, hipStream_t s) {
  const FwdParams& p = bp.f;
  for (int t = 0; t < 3; ++t) {
    if (!(p.targets & (1u << t))) continue;
    int lo, hi;
    target_cols(p, t, lo, hi);
    const int64_t na = static_cast<int64_t>(p.r) * p.d, nb = static_cast<int64_t>(hi - lo) * p.r;
    hipLaunchKernelGGL(zero_kernel, dim3(static_cast<unsigned>(std::min<int64_t>((na + 255) / 256, 1024))),
                       dim3(256), 0, s, bp.da[t], na);
    hipLaunchKernelGGL(zero_kernel, dim3(static_cast<unsigned>(std::min<int64_t>((nb + 255) / 256, 1024))),
                       dim3(256), 0, s, bp.db[t], nb);
  }
  if (p.T > 0) {
    dim3 grid(static_cast<unsigned>((p.T + kRows - 1) / kRows));
    timing_begin(s);
    hipLaunchKernelGGL((bwd_generic_kernel<TIn, kBf16>), grid, dim3(kThreads), 0, s, bp);
    timing_end(s);
  }
  return hipGetLastError();
}

}  // namespace

bool bwd_generic_supports(const FwdParams& p) { return p.d <= static_cast<int64_t>(kMaxCols) * kThreads && p.D <= kMaxHead; }
hipError_t launch_bwd_generic_f32(const BwdParams& p, hipStream_t s) { return launch<float, false>(p, s); }
hipError_t launch_bwd_generic_bf16(const BwdParams& p, hipStream_t s) { return launch<uint16_t, true>(p, s); }

}  // namespace lrq
