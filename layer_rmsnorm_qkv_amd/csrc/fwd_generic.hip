// Generic fused forward: any shape with an even head size, float32 or bfloat16.
//
// One workgroup owns a tile of kRows token rows x kPairs rotation pairs.  A pair is the
// two output columns (h*D + i, h*D + i + D/2) that rotate-half RoPE mixes, so each thread
// holds both partners and applies the rotation in registers.  Per tile:
//   1. RMSNorm row statistics of the tile's rows (wavefront shuffles, fp32);
//   2. K-loop over d: stage h = x * inv * gamma (rounded once to bf16 in the bf16 path),
//      the W rows of the tile's columns and the A rows of the LoRA targets the tile
//      touches in LDS; accumulate W h and U = A h in fp32;
//   3. epilogue: + (alpha/r) B U (U rounded once to bf16 in the bf16 path), + bias,
//      rotation of q and k pairs, one store.
// With LoRA dropout, U_t sums only the features that target t's keep bits keep, and the
// scale is alpha / r / (1 - p).  With an NF4 base (QLoRA), W is dequantised as it is staged.
// h and U live only in LDS and registers.  This family is the float32 path and the
// fallback for shapes the MFMA kernels do not cover; it uses plain FMA arithmetic.
#include "lrq_internal.h"

namespace lrq {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 32;       // token rows per tile
constexpr int kPairs = 32;      // rotation pairs per tile (64 output columns)
constexpr int kChunk = 32;      // K chunk staged per step
constexpr int kMaxU = 3 * kMaxRank;
constexpr int kUPerThread = (kRows * kMaxU + kThreads - 1) / kThreads;  // 24

template <typename TIn, bool kBf16>
__global__ __launch_bounds__(kThreads) void fwd_generic_kernel(FwdParams p) {
  __shared__ float s_inv[kRows];
  __shared__ float s_h[kRows][kChunk + 1];
  __shared__ float s_w[2 * kPairs][kChunk + 1];
  __shared__ float s_a[kMaxU][kChunk + 1];
  __shared__ float s_u[kRows][kMaxU + 1];

  const TIn* __restrict__ x = static_cast<const TIn*>(p.x);
  const TIn* __restrict__ gamma = static_cast<const TIn*>(p.gamma);
  const TIn* __restrict__ w = static_cast<const TIn*>(p.w);
  const Nf4View wq = nf4_view(p.w, p.N, p.d);  // used when p.nf4 (the QLoRA base)
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * kRows;
  const int pair0 = blockIdx.y * kPairs;
  const int half = p.D / 2;
  const int n_pairs = p.N / 2;
  const int64_t d = p.d;

  // ---- which LoRA targets intersect this tile, and where their U columns live
  int u_off[3] = {-1, -1, -1};
  int n_u = 0;
  {
    const int last_pair = min(pair0 + kPairs, n_pairs) - 1;
    const int h_first = pair0 / half, h_last = last_pair / half;
    for (int t = 0; t < 3; ++t) {
      if (!(p.targets & (1u << t))) continue;
      int lo, hi;
      target_cols(p, t, lo, hi);
      const int th_lo = lo / p.D, th_hi = hi / p.D;  // heads [th_lo, th_hi)
      if (h_last >= th_lo && h_first < th_hi) {
        u_off[t] = n_u;
        n_u += p.r;
      }
    }
  }

  // ---- 1. row statistics: each wave reduces rows wave, wave+4, ...
  for (int rr = wave; rr < kRows; rr += kThreads / 64) {
    const int64_t row = row0 + rr;
    float ss = 0.f;
    if (row < p.T) {
      for (int64_t j = lane; j < d; j += 64) {
        const float v = load_elem(x, row * d + j);
        ss = fmaf(v, v, ss);
      }
    }
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
    if (lane == 0) s_inv[rr] = 1.0f / sqrtf(ss / static_cast<float>(d) + p.eps);
  }
  __syncthreads();

  // thread -> (rows tr, tr+16) x (pairs tp, tp+16)
  const int tr = tid >> 4;
  const int tp = tid & 15;
  float acc[2][2][2] = {};  // [row sel][pair sel][a/b]
  float u_acc[kUPerThread];
#pragma unroll
  for (int i = 0; i < kUPerThread; ++i) u_acc[i] = 0.f;

  for (int64_t k0 = 0; k0 < d; k0 += kChunk) {
    // stage h
    for (int e = tid; e < kRows * kChunk; e += kThreads) {
      const int rr = e / kChunk, kk = e % kChunk;
      const int64_t row = row0 + rr, k = k0 + kk;
      float v = 0.f;
      if (row < p.T && k < d) {
        v = load_elem(x, row * d + k) * s_inv[rr] * load_elem(gamma, k);
        if (kBf16) v = round_bf16(v);
      }
      s_h[rr][kk] = v;
    }
    // stage W rows of the tile's columns: tile column c < kPairs is the first partner
    for (int e = tid; e < 2 * kPairs * kChunk; e += kThreads) {
      const int c = e / kChunk, kk = e % kChunk;
      const int pr = pair0 + (c % kPairs);
      const int64_t k = k0 + kk;
      float v = 0.f;
      if (pr < n_pairs && k < d) {
        const int col = (pr / half) * p.D + (pr % half) + (c >= kPairs ? half : 0);
        v = p.nf4 ? nf4_at(wq, col, k) : load_elem(w, static_cast<int64_t>(col) * d + k);
      }
      s_w[c][kk] = v;
    }
    // stage A rows of the touched targets
    for (int t = 0; t < 3; ++t) {
      if (u_off[t] < 0) continue;
      const TIn* __restrict__ a = static_cast<const TIn*>(p.a[t]);
      for (int e = tid; e < p.r * kChunk; e += kThreads) {
        const int j = e / kChunk, kk = e % kChunk;
        const int64_t k = k0 + kk;
        s_a[u_off[t] + j][kk] = k < d ? load_elem(a, static_cast<int64_t>(j) * d + k) : 0.f;
      }
    }
    __syncthreads();

#pragma unroll 4
    for (int kk = 0; kk < kChunk; ++kk) {
      const float h0 = s_h[tr][kk], h1 = s_h[tr + 16][kk];
      const float wa0 = s_w[tp][kk], wb0 = s_w[kPairs + tp][kk];
      const float wa1 = s_w[tp + 16][kk], wb1 = s_w[kPairs + tp + 16][kk];
      acc[0][0][0] = fmaf(h0, wa0, acc[0][0][0]);
      acc[0][0][1] = fmaf(h0, wb0, acc[0][0][1]);
      acc[0][1][0] = fmaf(h0, wa1, acc[0][1][0]);
      acc[0][1][1] = fmaf(h0, wb1, acc[0][1][1]);
      acc[1][0][0] = fmaf(h1, wa0, acc[1][0][0]);
      acc[1][0][1] = fmaf(h1, wb0, acc[1][0][1]);
      acc[1][1][0] = fmaf(h1, wa1, acc[1][1][0]);
      acc[1][1][1] = fmaf(h1, wb1, acc[1][1][1]);
    }
#pragma unroll
    for (int i = 0; i < kUPerThread; ++i) {
      const int e = tid + i * kThreads;
      if (e < kRows * n_u) {
        const int rr = e / n_u, j = e % n_u;
        float s = u_acc[i];
        if (p.dropout) {
          // the adapter's own keep bits of this row and chunk (kChunk = 32: one word)
          int tj = 0;
          for (int t = 0; t < 3; ++t)
            if (u_off[t] >= 0 && j >= u_off[t] && j < u_off[t] + p.r) tj = t;
          const int64_t row = row0 + rr;
          const uint32_t keep =
              row < p.T ? p.drop_bits_r[(static_cast<int64_t>(target_slot(p.targets, tj)) * p.T + row) *
                                            ((d + 31) / 32) + k0 / kChunk]
                        : 0u;
          for (int kk = 0; kk < kChunk; ++kk) s = fmaf((keep >> kk) & 1u ? s_h[rr][kk] : 0.f, s_a[j][kk], s);
        } else {
          for (int kk = 0; kk < kChunk; ++kk) s = fmaf(s_h[rr][kk], s_a[j][kk], s);
        }
        u_acc[i] = s;
      }
    }
    __syncthreads();
  }

  // U to LDS (rounded once to bf16 in the bf16 path)
#pragma unroll
  for (int i = 0; i < kUPerThread; ++i) {
    const int e = tid + i * kThreads;
    if (e < kRows * n_u) s_u[e / n_u][e % n_u] = kBf16 ? round_bf16(u_acc[i]) : u_acc[i];
  }
  __syncthreads();

  // ---- 3. epilogue
  const TIn* __restrict__ bias = static_cast<const TIn*>(p.bias);
  TIn* __restrict__ out = static_cast<TIn*>(p.out);
  for (int rs = 0; rs < 2; ++rs) {
    const int rr = tr + 16 * rs;
    const int64_t row = row0 + rr;
    if (row >= p.T) continue;
    const int pos = p.pos[row];
    for (int ps = 0; ps < 2; ++ps) {
      const int pr = pair0 + tp + 16 * ps;
      if (pr >= n_pairs) continue;
      const int head = pr / half, i = pr % half;
      const int ca = head * p.D + i, cb = ca + half;
      float ya = acc[rs][ps][0], yb = acc[rs][ps][1];
      const int t = ca < p.col_k ? 0 : (ca < p.col_v ? 1 : 2);
      if (u_off[t] >= 0) {
        int lo, hi;
        target_cols(p, t, lo, hi);
        const TIn* __restrict__ bt = static_cast<const TIn*>(p.b[t]);
        float la = 0.f, lb = 0.f;
        for (int j = 0; j < p.r; ++j) {
          const float u = s_u[rr][u_off[t] + j];
          la = fmaf(u, load_elem(bt, static_cast<int64_t>(ca - lo) * p.r + j), la);
          lb = fmaf(u, load_elem(bt, static_cast<int64_t>(cb - lo) * p.r + j), lb);
        }
        ya = fmaf(p.scale, la, ya);
        yb = fmaf(p.scale, lb, yb);
      }
      if (p.has_bias) {
        ya += load_elem(bias, ca);
        yb += load_elem(bias, cb);
      }
      if (ca < p.rot_end) {
        float c, s;
        rope_cos_sin(pos, rope_omega(p.theta, i, p.D), c, s);
        const float ra = ya * c - yb * s;
        const float rb = yb * c + ya * s;
        ya = ra;
        yb = rb;
      }
      store_elem(out, row * p.N + ca, ya);
      store_elem(out, row * p.N + cb, yb);
    }
  }
}

template <typename TIn, bool kBf16>
hipError_t launch(const FwdParams& p, hipStream_t s) {
  const int n_pairs = p.N / 2;
  dim3 grid(static_cast<unsigned>((p.T + kRows - 1) / kRows), (n_pairs + kPairs - 1) / kPairs);
  timing_begin(s);
  hipLaunchKernelGGL((fwd_generic_kernel<TIn, kBf16>), grid, dim3(kThreads), 0, s, p);
  timing_end(s);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_generic_f32(const FwdParams& p, hipStream_t s) { return launch<float, false>(p, s); }
hipError_t launch_fwd_generic_bf16(const FwdParams& p, hipStream_t s) { return launch<uint16_t, true>(p, s); }

}  // namespace lrq
