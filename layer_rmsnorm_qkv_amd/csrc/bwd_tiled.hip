// MFMA family of the backward (bf16, fp32 accumulation): gradients of
//
//   out = RoPE( W h + b + s B (A h) ),   h = x * inv * gamma,   inv = 1/rms(x)
//
// with W, gamma and b frozen, given dy = dL/d(out):
//
//   G   = RoPE^-1(dy) on the q and k heads, dy on v         (transpose of the rotation)
//   V_t = s G_t B_t                                         [T, r] per target
//   dh  = G W + sum_t V_t A_t                               [T, d]
//   dx  = inv * gamma * dh - m * x,  m = inv^2 <dy, y - R b> / d
//   dA_t = sum_tokens V_t^T h,   dB_t = s sum_tokens G_t^T U_t,   U_t = A_t h
//
// The row scalar uses <gamma x, dh> = <dy, y - R b> / inv (R is orthogonal and y - R b is
// the rotated W_eff h), so the RMSNorm backward needs no second pass over dh.
//
// Kernels, in launch order (all on the caller's stream):
//   prep_weights  WT = W^T [d][N] (unless the call brings it prepared; an NF4 W, the QLoRA
//                 base, is dequantised on the way), AT = [A_q^T | A_k^T |
//                 A_v^T | 0] [d][Rp] with Rp = sum r rounded up to 64, B_t^T [r][N_t] and
//                 A'_t = bf16(A_t * gamma) [r][d]
//   rows          per token: inv, m, G (bf16) into Gcat[:, 0:N)
//   rank (V)      V'_t = bf16(s G_t B_t) into Gcat[:, N + off_t ...) (+ zero padding)
//   rank (U)      U_t = bf16(inv * x A'_t^T) into U[T][R]
//   main          dh = Gcat [WT | AT]^T over K = N + Rp (shared tile pipeline), epilogue dx
//   lora_partial  per chunk of tokens: sum V'^T h (all targets) and G_t^T U_t (MFMA)
//   lora_reduce   dA_t, dB_t = sums over chunks (deterministic order), dB scaled by s
// h and U are recomputed from x; G and V' live only in the workspace of this call.
//
// LoRA dropout (s = alpha / r / (1 - p)): the rows pass also makes every target's keep bits and
// masked input x * keep_t for its row (Philox work overlapped with the pass's loads).  U_t and
// dA_t then come from per-target jobs over the masked copies, and target t's dh term
// keep_t * (V'_t A_t) is no longer one K segment shared by all targets: the main kernel starts
// its accumulators at the sum of the targets' masked rank-r products and runs K over N only.
#include <algorithm>

#include "lrq_internal.h"
#include "tile_common.h"

namespace lrq {
namespace {

using namespace tile;

constexpr int kLoraItems = 1152;  // target number of one-wave LoRA-gradient work items

// Workspace of one backward call (byte offsets, 256-aligned) and derived sizes.
struct BwdLayout {
  int R;        // sum of the targets' ranks
  int Rp;       // R rounded up to 64 (0 without targets)
  int64_t K;    // N + Rp: inner size of the main product
  int off[3];   // first LoRA column (within the R block) of each target
  int cpl;      // LoRA gradients: columns per lane (8 when R <= 32, else 4)
  int rpass;    // ranks per pass over M (32 or 64)
  int groups[4];  // work groups per LoRA-gradient job (dA, then each target's dB)
  int groups_da_t;  // with dropout: groups of each target's dA job (groups[0] = their sum)
  int chunk;    // tokens per partial sum (multiple of 16)
  int chunks;   // token chunks of the LoRA-gradient partial sums
  size_t wt, at, bt[3], ap_all, ap[3], gcat, u, inv, m, pda, pdb[3], total;
};

size_t al256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

BwdLayout bwd_layout(const FwdParams& p) {
  BwdLayout L{};
  int R = 0;
  for (int t = 0; t < 3; ++t) {
    L.off[t] = R;
    if (p.targets & (1u << t)) R += p.r;
  }
  L.R = R;
  L.Rp = (R + 63) / 64 * 64;
  L.K = p.N + L.Rp;
  L.cpl = R <= 32 ? 8 : 4;
  L.rpass = L.cpl == 8 ? 32 : 64;
  const int colw = 32 * L.cpl;
  int G = 0;
  // dA: one job over all ranks, or (dropout) one per target over its masked input
  const int dcols = static_cast<int>((p.d + colw - 1) / colw);
  L.groups_da_t = dcols * ((p.r + L.rpass - 1) / L.rpass);
  L.groups[0] = p.dropout ? p.drop_nt * L.groups_da_t : dcols * ((R + L.rpass - 1) / L.rpass);
  G += L.groups[0];
  for (int t = 0; t < 3; ++t) {
    int lo, hi;
    target_cols(p, t, lo, hi);
    L.groups[t + 1] = (p.targets & (1u << t)) ? (hi - lo + colw - 1) / colw * ((p.r + L.rpass - 1) / L.rpass) : 0;
    G += L.groups[t + 1];
  }
  // chunks as long as the work items stay near the target count (fewer partial sums to add)
  L.chunk = 64;
  while (L.chunk < 2048 && (p.T + L.chunk - 1) / L.chunk * G > kLoraItems) L.chunk *= 2;
  L.chunks = static_cast<int>((p.T + L.chunk - 1) / L.chunk);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += al256(bytes);
    return at;
  };
  L.wt = take(p.use_prepared ? 0 : static_cast<size_t>(p.d) * p.N * 2);
  L.at = take(static_cast<size_t>(p.d) * L.Rp * 2);
  for (int t = 0; t < 3; ++t) {
    int lo, hi;
    target_cols(p, t, lo, hi);
    const bool on = p.targets & (1u << t);
    L.bt[t] = take(on ? static_cast<size_t>(p.r) * (hi - lo) * 2 : 0);
  }
  // A'_t of all targets as one [R][d] block (target t at row off_t)
  L.ap_all = take(static_cast<size_t>(R) * p.d * 2);
  for (int t = 0; t < 3; ++t) L.ap[t] = L.ap_all + static_cast<size_t>(L.off[t]) * p.d * 2;
  L.gcat = take(static_cast<size_t>(p.T) * L.K * 2);
  L.u = take(static_cast<size_t>(p.T) * std::max(R, 1) * 2);
  L.inv = take(static_cast<size_t>(p.T) * 4);
  L.m = take(static_cast<size_t>(p.T) * 4);
  L.pda = take(static_cast<size_t>(L.chunks) * R * p.d * 4);
  for (int t = 0; t < 3; ++t) {
    int lo, hi;
    target_cols(p, t, lo, hi);
    L.pdb[t] = take((p.targets & (1u << t)) ? static_cast<size_t>(L.chunks) * p.r * (hi - lo) * 4 : 0);
  }
  L.total = o;
  return L;
}

template <typename T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<unsigned char*>(base) + off);
}

// ---------------------------------------------------------------- prep_weights
// WT[j][n] = W[n][j] (n < N), AT[j][off_t + k] = A_t[k][j] (k < r), AT[j][R ..) = 0;
// BT_t[k][n] = B_t[n][k]; AP_t[k][j] = bf16(A_t[k][j] * gamma[j]).
// 64 x 64 tiles of the source rows [q_begin, N + Rp) -- W rows, then the targets' A rows,
// then zeros -- through LDS; the small B^T / A' products are done by the blocks past the
// transpose grid.
struct PrepArgs {
  const uint16_t* w;
  Nf4View wq;    // W as NF4 blocks instead (QLoRA base) when wq.codes != nullptr
  const uint16_t* a[3];
  const uint16_t* b[3];
  const uint16_t* gamma;
  uint16_t* wt;  // [d][N], written for source rows < N
  uint16_t* at;  // [d][Rp], written for source rows >= N
  uint16_t* bt[3];
  uint16_t* ap[3];
  int N, d, r, Rp, R;
  int q_begin;   // first source row (0, or N when W^T is not transposed)
  int off[3], lo[3], nt[3];  // per target: LoRA column offset, first output column, width
  uint32_t targets;
  int wt_blocks;  // blocks of the transpose part
};

__global__ __launch_bounds__(256) void prep_weights_kernel(PrepArgs a) {
  // [64][64] with the 16-byte chunks of row q stored at chunk (c ^ (q / 8) % 8): the 16-byte
  // writes of a row and the column reads (8 rows q = 8 k + const, one chunk per wave) both
  // hit distinct banks (a padded row pitch cannot do both and stay 16-byte aligned)
  __shared__ uint16_t tile_s[64][64];
  __shared__ float levels[16];
  auto ts = [&](int q, int j) -> uint16_t& { return tile_s[q][(((j >> 3) ^ (q >> 3)) & 7) * 8 + (j & 7)]; };
  const int tid = threadIdx.x;
  if (tid < 16) levels[tid] = kNf4Levels[tid];
  __syncthreads();
  if (static_cast<int>(blockIdx.x) < a.wt_blocks) {
    // transpose a 64 x 64 block: source rows q (LoRA-extended K index) x columns j, moved as
    // 16-byte vectors (8 columns of a source row in, 8 rows of a destination row out)
    const int jb = a.d / 64;
    const int kb = static_cast<int>(blockIdx.x) / jb, cb = static_cast<int>(blockIdx.x) % jb;
    const int q0 = a.q_begin + kb * 64, j0 = cb * 64;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = tid + 256 * h;
      const int qi = c >> 3, jc = (c & 7) * 8;
      const int q = q0 + qi;
      const uint16_t* src = nullptr;
      if (q < a.N) {
        src = a.wq.codes ? nullptr : a.w + static_cast<int64_t>(q) * a.d;
      } else if (q - a.N < a.R) {
        const int cq = q - a.N;
        for (int t = 0; t < 3; ++t)
          if (((a.targets >> t) & 1u) && cq >= a.off[t] && cq < a.off[t] + a.r)
            src = a.a[t] + static_cast<int64_t>(cq - a.off[t]) * a.d;
      }
      uint4 v = src ? *reinterpret_cast<const uint4*>(src + j0 + jc) : uint4{0u, 0u, 0u, 0u};
      if (q < a.N && a.wq.codes) {
        // NF4 base: 8 dequantised weights, rounded once to bf16
        float wv[8];
        nf4_at8(a.wq, q, j0 + jc, levels, wv);
        uint32_t o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = f32_to_bf16_bits(wv[2 * e]) | (f32_to_bf16_bits(wv[2 * e + 1]) << 16);
        v = uint4{o[0], o[1], o[2], o[3]};
      }
      *reinterpret_cast<uint4*>(&ts(qi, jc)) = v;
    }
    __syncthreads();
    // N is a multiple of 64, so a block lies wholly in W^T or wholly in A^T
    uint16_t* dst = q0 < a.N ? a.wt + q0 : a.at + (q0 - a.N);
    const int64_t ldd = q0 < a.N ? a.N : a.Rp;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = tid + 256 * h;
      const int ji = c >> 3, qc = (c & 7) * 8;
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w[e] = static_cast<uint32_t>(ts(qc + 2 * e, ji)) | (static_cast<uint32_t>(ts(qc + 2 * e + 1, ji)) << 16);
      *reinterpret_cast<uint4*>(dst + static_cast<int64_t>(j0 + ji) * ldd + qc) = uint4{w[0], w[1], w[2], w[3]};
    }
    return;
  }
  // B_t^T and A'_t: one thread per output element, grid-stride over all targets
  const int64_t gid = (static_cast<int64_t>(blockIdx.x) - a.wt_blocks) * 256 + tid;
  const int64_t stride = static_cast<int64_t>(gridDim.x - a.wt_blocks) * 256;
  for (int t = 0; t < 3; ++t) {
    if (!((a.targets >> t) & 1u)) continue;
    const int64_t nbt = static_cast<int64_t>(a.r) * a.nt[t];
    for (int64_t e = gid; e < nbt; e += stride) {
      const int64_t k = e / a.nt[t], n = e % a.nt[t];
      a.bt[t][e] = a.b[t][n * a.r + k];
    }
    const int64_t nap = static_cast<int64_t>(a.r) * a.d;
    for (int64_t e = gid; e < nap; e += stride) {
      const int j = static_cast<int>(e % a.d);
      a.ap[t][e] = f32_to_bf16_bits(bf16_bits_to_f32(a.a[t][e]) * bf16_bits_to_f32(a.gamma[j]));
    }
  }
}

// ---------------------------------------------------------------- rows
// One wavefront per token row: inv from sum(x^2); G = inverse rotation of dy (q, k heads) or
// dy (v), rounded once to bf16 into Gcat; m = inv^2 (<dy, y> - <G, b>) / d.  Lane l handles
// the rotation pairs (i, i + D/2) with i = l, l + 64, ...
struct RowsArgs {
  const uint16_t* x;
  const uint16_t* y;
  const uint16_t* dy;
  const uint16_t* bias;  // nullptr without bias
  const int32_t* pos;
  uint16_t* gcat;
  float* inv;
  float* m;
  int64_t T;
  int d, N, D, rot_end;
  int64_t K;
  float eps;
  double log2_theta;
  // LoRA dropout (nt > 0): keep bits [nt][T][d / 8] bytes and x * keep [nt][T][d] per slot
  int nt;
  int target[3];
  uint32_t thr, offset, seed_lo, seed_hi;
  uint8_t* bits;
  uint16_t* xm;
};

__global__ __launch_bounds__(256) void rows_kernel(RowsArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  const uint16_t* xr = a.x + t * a.d;
  float ss = 0.f;
  for (int j = lane * 8; j < a.d; j += 512) {
    const uint4 v = *reinterpret_cast<const uint4*>(xr + j);
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo = __uint_as_float(w4[e] << 16), hi = __uint_as_float(w4[e] & 0xffff0000u);
      ss = fmaf(lo, lo, fmaf(hi, hi, ss));
    }
    for (int sl = 0; sl < a.nt; ++sl) {
      // dropout: this row's keep bits of features j .. j + 7 for slot sl, and its masked input
      const uint32_t keep = dropout_byte(j, static_cast<uint32_t>(t), static_cast<uint32_t>(a.target[sl]),
                                         a.offset, a.thr, a.seed_lo, a.seed_hi);
      const int64_t srow = static_cast<int64_t>(sl) * a.T + t;
      a.bits[srow * (a.d / 8) + j / 8] = static_cast<uint8_t>(keep);
      *reinterpret_cast<uint4*>(a.xm + srow * a.d + j) = mask_bf16x8(v, keep);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  const float inv = 1.0f / sqrtf(ss / static_cast<float>(a.d) + a.eps);

  const int half = a.D / 2;
  const double pos = static_cast<double>(a.pos[t]);
  const uint16_t* dyr = a.dy + t * a.N;
  const uint16_t* yr = a.y + t * a.N;
  uint16_t* gr = a.gcat + t * a.K;
  float dot_y = 0.f, dot_b = 0.f;
  const int gph = half / 8;  // groups of 8 frequencies per head
  if (half % 8 == 0 && 64 % gph == 0) {
    // 16-byte accesses: the lane takes frequencies 8 g .. 8 g + 7 (g = lane % gph, the same
    // in every head it visits) of heads lane / gph, + 64 / gph, ...
    const int g = lane % gph;
    double om[8];  // turns per position
#pragma unroll
    for (int e = 0; e < 8; ++e) om[e] = exp2(-(2.0 * (8 * g + e) / a.D) * a.log2_theta) * 0.15915494309189533577;
    const int heads = a.N / a.D;
    for (int h = lane / gph; h < heads; h += 64 / gph) {
      const int c0 = h * a.D;
      const int ca = c0 + 8 * g, cb = ca + half;
      const uint4 dav = *reinterpret_cast<const uint4*>(dyr + ca), dbv = *reinterpret_cast<const uint4*>(dyr + cb);
      const uint4 yav = *reinterpret_cast<const uint4*>(yr + ca), ybv = *reinterpret_cast<const uint4*>(yr + cb);
      const uint32_t dw[2][4] = {{dav.x, dav.y, dav.z, dav.w}, {dbv.x, dbv.y, dbv.z, dbv.w}};
      const uint32_t yw[2][4] = {{yav.x, yav.y, yav.z, yav.w}, {ybv.x, ybv.y, ybv.z, ybv.w}};
      float da[8], db[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sh = (e & 1) ? 0 : 16;
        da[e] = __uint_as_float((dw[0][e >> 1] << sh) & 0xffff0000u);
        db[e] = __uint_as_float((dw[1][e >> 1] << sh) & 0xffff0000u);
        const float ya = __uint_as_float((yw[0][e >> 1] << sh) & 0xffff0000u);
        const float yb = __uint_as_float((yw[1][e >> 1] << sh) & 0xffff0000u);
        dot_y = fmaf(da[e], ya, fmaf(db[e], yb, dot_y));
      }
      float ga[8], gb[8];
      if (c0 < a.rot_end) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          // angle pos * omega_i as a fraction of a turn, reduced in double precision
          const double turns = pos * om[e];
          const float f = static_cast<float>(turns - rint(turns));
          const float sn = __builtin_amdgcn_sinf(f), cs = __builtin_amdgcn_cosf(f);
          ga[e] = da[e] * cs + db[e] * sn;
          gb[e] = db[e] * cs - da[e] * sn;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          ga[e] = da[e];
          gb[e] = db[e];
        }
      }
      if (a.bias) {
        const uint4 bav = *reinterpret_cast<const uint4*>(a.bias + ca), bbv = *reinterpret_cast<const uint4*>(a.bias + cb);
        const uint32_t bw[2][4] = {{bav.x, bav.y, bav.z, bav.w}, {bbv.x, bbv.y, bbv.z, bbv.w}};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int sh = (e & 1) ? 0 : 16;
          const float ba = __uint_as_float((bw[0][e >> 1] << sh) & 0xffff0000u);
          const float bb = __uint_as_float((bw[1][e >> 1] << sh) & 0xffff0000u);
          dot_b = fmaf(ga[e], ba, fmaf(gb[e], bb, dot_b));
        }
      }
      uint32_t pa[4], pb[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        pa[q] = static_cast<uint32_t>(f32_to_bf16_bits(ga[2 * q])) | (static_cast<uint32_t>(f32_to_bf16_bits(ga[2 * q + 1])) << 16);
        pb[q] = static_cast<uint32_t>(f32_to_bf16_bits(gb[2 * q])) | (static_cast<uint32_t>(f32_to_bf16_bits(gb[2 * q + 1])) << 16);
      }
      *reinterpret_cast<uint4*>(gr + ca) = make_uint4(pa[0], pa[1], pa[2], pa[3]);
      *reinterpret_cast<uint4*>(gr + cb) = make_uint4(pb[0], pb[1], pb[2], pb[3]);
    }
  } else {
    // other head sizes: one frequency pair per lane and head
    double om[4];  // turns per position of the lane's frequencies i = lane + 64 q (D <= 512)
#pragma unroll
    for (int q = 0; q < 4; ++q) om[q] = exp2(-(2.0 * (lane + 64 * q) / a.D) * a.log2_theta) * 0.15915494309189533577;
    for (int c0 = 0; c0 < a.N; c0 += a.D) {
      const bool rot = c0 < a.rot_end;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = lane + 64 * q;
        if (i >= half) break;
        const int ca = c0 + i, cb = c0 + i + half;
        const float da = bf16_bits_to_f32(dyr[ca]), db = bf16_bits_to_f32(dyr[cb]);
        dot_y = fmaf(da, bf16_bits_to_f32(yr[ca]), fmaf(db, bf16_bits_to_f32(yr[cb]), dot_y));
        float ga = da, gb = db;
        if (rot) {
          // angle pos * omega_i as a fraction of a turn, reduced in double precision
          const double turns = pos * om[q];
          const float f = static_cast<float>(turns - rint(turns));
          const float s = __builtin_amdgcn_sinf(f), c = __builtin_amdgcn_cosf(f);
          ga = da * c + db * s;
          gb = db * c - da * s;
        }
        if (a.bias) dot_b = fmaf(ga, bf16_bits_to_f32(a.bias[ca]), fmaf(gb, bf16_bits_to_f32(a.bias[cb]), dot_b));
        gr[ca] = f32_to_bf16_bits(ga);
        gr[cb] = f32_to_bf16_bits(gb);
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    dot_y += __shfl_xor(dot_y, o);
    dot_b += __shfl_xor(dot_b, o);
  }
  if (lane == 0) {
    a.inv[t] = inv;
    a.m[t] = inv * inv * (dot_y - dot_b) / static_cast<float>(a.d);
  }
}

// ---------------------------------------------------------------- rank (V and U)
// One workgroup per (128-token block, job): u = A_rows Bs^T, then out[row][col0 + k] =
// bf16(scale(row) * u) for k < r and 0 for k in [r, pad_to - col0) (the zero padding of Gcat's
// LoRA columns comes with the last V job).
struct RankJob {
  const uint16_t* a;   // A panel source: element (row, kk) at a[row * lda + kk]
  int64_t lda;
  const uint16_t* bs;  // small operand rows [r][nk * 64]
  int64_t ldb;
  int r;               // rows of bs (at most 32 RB)
  int nk;              // K steps of 64
  uint16_t* out;
  int64_t ldo;
  int col0;            // first output column
  int pad_to;          // output columns [col0 + r, pad_to) are written as 0
  float scale;         // constant factor
  const float* inv;    // nullptr, or per-row factor
};

struct RankArgs {
  RankJob job[6];  // up to 3 V jobs and 3 U jobs
  int64_t T;
};

// 128 token rows per workgroup through a three-stage ring (a stage: the A rows [128][64], then
// the small operand's rows [32 RB][64], every row one 128-byte line with its 16-byte chunks
// XOR-swizzled by row), so two workgroups share a CU and two stages are in flight per step.
// Wave w owns rows 32 w .. 32 w + 31 and every rank: RB accumulators.
constexpr int kRankRows = 128;
constexpr int kRankStages = 3;
template <int RB>
struct RankLay {
  static constexpr int kA = kRankRows * kRowBytes;
  static constexpr int kStage = kA + 32 * RB * kRowBytes;
  static constexpr int kBytes = kRankStages * kStage;
};

template <int RB>
__global__ __launch_bounds__(kThreads, 2) void rank_kernel(RankArgs a) {
  using L = RankLay<RB>;
  constexpr int kLoads = 4 + RB;  // DMA instructions per stage and wave
  __shared__ __attribute__((aligned(1024))) unsigned char smem[L::kBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, h32 = lane >> 5;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * kRankRows;
  const RankJob& j = a.job[blockIdx.y];
  // Instruction c of wave w fills A rows R = 32 w + 8 c + lane / 8 (rows past T re-read row
  // T - 1, never stored) and instruction q fills small-operand rows R = 8 (RB w + q) + lane / 8
  // (rows past r re-read row r - 1); the lane's 16 bytes land in chunk lane % 8, which holds
  // logical chunk (lane % 8) ^ chunk_xor(R).
  const int pc = lane & 7, rsub = lane >> 3;
  const uint16_t* asrc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int R = 32 * wave + 8 * c + rsub;
    asrc[c] = j.a + min(row0 + R, a.T - 1) * j.lda + (pc ^ chunk_xor(R)) * 8;
  }
  const uint16_t* bsrc[RB];
#pragma unroll
  for (int q = 0; q < RB; ++q) {
    const int R = 8 * (RB * wave + q) + rsub;
    bsrc[q] = j.bs + static_cast<int64_t>(min(R, j.r - 1)) * j.ldb + (pc ^ chunk_xor(R)) * 8;
  }
  const uint32_t sbase = lds_addr(smem);
  auto issue = [&](int ks) {
    const uint32_t st = sbase + (ks % kRankStages) * L::kStage;
#pragma unroll
    for (int c = 0; c < 4; ++c) dma16(asrc[c] + ks * BK, st + (32 * wave + 8 * c) * kRowBytes);
#pragma unroll
    for (int q = 0; q < RB; ++q) dma16(bsrc[q] + ks * BK, st + L::kA + 8 * (RB * wave + q) * kRowBytes);
  };

  floatx16 u[RB];
#pragma unroll
  for (int b = 0; b < RB; ++b) u[b] = floatx16{};
  const int nk = j.nk;
#pragma unroll
  for (int s0 = 0; s0 < kRankStages - 1; ++s0)
    if (s0 < nk) issue(s0);
  for (int ks = 0; ks < nk; ++ks) {
    // stage ks landed (the one issued after it may still be in flight); every wave is past its
    // reads of stage ks - 1, whose buffer the next issue refills
    if (ks + 1 < nk)
      wait_barrier<kLoads>();
    else
      wait_barrier<0>();
    if (ks + kRankStages - 1 < nk) issue(ks + kRankStages - 1);
    const unsigned char* st = smem + (ks % kRankStages) * L::kStage;
#pragma unroll
    for (int kk = 0; kk < kSlices; ++kk) {
      const bf16x8 af = *reinterpret_cast<const bf16x8*>(st + swz(32 * wave + l32, kk * 2 + h32));
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        const bf16x8 bf = *reinterpret_cast<const bf16x8*>(st + L::kA + swz(32 * b + l32, kk * 2 + h32));
        u[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf, u[b], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    const int k = 32 * b + l32;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t row = row0 + 32 * wave + (v >> 2) * 8 + h32 * 4 + (v & 3);
      if (row >= a.T) continue;
      uint16_t* o = j.out + row * j.ldo + j.col0;
      if (k < j.r) {
        const float f = j.inv ? j.inv[row] * j.scale : j.scale;
        o[k] = f32_to_bf16_bits(f * u[b][v]);
      } else if (j.col0 + k < j.pad_to) {
        o[k] = 0;
      }
    }
  }
  // padding columns beyond the rank blocks (only when pad_to - col0 > 32 RB)
  const int w = j.pad_to - j.col0 - 32 * RB;
  for (int64_t e = tid; e < static_cast<int64_t>(kRankRows) * w; e += kThreads) {
    const int64_t row = row0 + e / w;
    if (row < a.T) j.out[row * j.ldo + j.col0 + 32 * RB + e % w] = 0;
  }
}

// ---------------------------------------------------------------- main: dh and dx
struct MainArgs {
  const uint16_t* gcat;  // [T][K]
  const uint16_t* wt;    // [d][N]
  const uint16_t* at;    // [d][Rp]
  int N, Rp;
  // LoRA dropout (DROP): keep bits [slot][T][d / 32] words and each slot's first LoRA column
  const uint32_t* bits;
  int nslots, r;
  int loff[3];
  const uint16_t* x;
  const uint16_t* gamma;
  const float* inv;
  const float* m;
  uint16_t* dx;
  int64_t T;
  int d;
  int64_t K;
  int n_nt;   // column tiles of d
  int n_mt;   // token tiles
  int group_m;  // token tiles per group of the tile order
  int items;  // grid size
  int remap;
};

// Dropout: acc += keep_s * (V'_s A_s) for every slot s, on the wave's 64 x 128 part of the
// tile before the K loop, one 32 x 32 block at a time and within it one slot at a time (K = r
// rounded up to 16; ranks >= r read 0).  Lane l32's columns are bit l32 of the row's keep
// words (col0 + 128 wn) / 32 + j.
template <int NS>
__device__ __forceinline__ void drop_lora_init(const MainArgs& a, Acc8& ta, int64_t row0, int64_t col0, int wm,
                                               int wn, int l32, int h32) {
  const int ksteps = (a.r + 15) >> 4;
  const bool vec = (a.r & 7) == 0;
  const int64_t dw = a.d / 32;
  const int64_t wcol = (col0 + wn * 128) / 32;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t rblk = row0 + wm * 64 + i * 32;
    const int64_t vrow = min(rblk + l32, a.T - 1);
    const int64_t rbase = rblk + h32 * 4;  // the lane's 16 rows: rbase + 8 (v / 4) + v % 4
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = col0 + wn * 128 + j * 32 + l32;
      asm volatile("" ::: "memory");
#pragma unroll
      for (int sl = 0; sl < NS; ++sl) {
        const uint16_t* vsrc = a.gcat + vrow * a.K + a.N + a.loff[sl];
        const uint16_t* asrc = a.at + col * a.Rp + a.loff[sl];
        const uint32_t* __restrict__ bits = a.bits + static_cast<int64_t>(sl) * a.T * dw + wcol + j;
        floatx16 tmp = floatx16{};
        for (int kq = 0; kq < ksteps; ++kq) {
          const int k0 = kq * 16 + h32 * 8;
          bf16x8 vf, af;
          if (vec && k0 < a.r) {
            vf = *reinterpret_cast<const bf16x8*>(vsrc + k0);
            af = *reinterpret_cast<const bf16x8*>(asrc + k0);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const bool in = k0 + e < a.r;
              vf[e] = __builtin_bit_cast(__bf16, in ? vsrc[k0 + e] : uint16_t{0});
              af[e] = __builtin_bit_cast(__bf16, in ? asrc[k0 + e] : uint16_t{0});
            }
          }
          tmp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, af, tmp, 0, 0, 0);
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const uint32_t keep = bits[min(rbase + (v >> 2) * 8 + (v & 3), a.T - 1) * dw];
          ta.acc[i][j][v] += ((keep >> l32) & 1u) ? tmp[v] : 0.f;
        }
        // the next slot's loads are not hoisted above this block's adds
        asm volatile("" ::: "memory");
      }
    }
  }
}

// NS: number of dropout slots (0: no dropout; the LoRA term is the K segment past N)
template <int NS>
__global__ __launch_bounds__(kThreads8, 1) void bwd_main_kernel(MainArgs a) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kRingBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 3, wn = wave >> 2;
  const int l32 = lane & 31, h32 = lane >> 5;
  int item = blockIdx.x;
  if (a.remap) item = (blockIdx.x & 7) * (a.items >> 3) + (blockIdx.x >> 3);
  // grouped tile order: group_m token tiles by every column tile, token tile fastest, so the
  // workgroups that run together on one XCD share a few Gcat panels and a few W^T panels
  // through its L2 instead of two Gcat panels and every W^T panel
  const int gsz = a.group_m * a.n_nt;
  const int g = item / gsz, gr = item - g * gsz;
  const int gm = min(a.n_mt - g * a.group_m, a.group_m);
  // (wave-uniform: the scalar-base DMA below takes addresses formed from them in SGPRs)
  const int mt = __builtin_amdgcn_readfirstlane(g * a.group_m + gr % gm);
  const int nt = __builtin_amdgcn_readfirstlane(gr / gm);
  const int64_t row0 = static_cast<int64_t>(mt) * BM;
  const int64_t col0 = static_cast<int64_t>(nt) * BN;

  Acc8 ta;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) ta.acc[i][j] = floatx16{};
  if (NS > 0) drop_lora_init<NS>(a, ta, row0, col0, wm, wn, l32, h32);
  const Src8 src = make_src8(a.gcat, a.K, row0, a.T, a.wt, a.N, a.N / BK, a.at, a.Rp, wave, lane);
  kloop8(smem, ta, src, col0, NS > 0 ? a.N / BK : static_cast<int>(a.K / BK), wave, lane);

  // epilogue: dx = inv * gamma * dh - m * x for the lane's rows and columns
  // (lane rows: 64 wm + 32 i + 8 (v / 4) + 4 h32 + v % 4; columns 128 wn + 32 j + l32)
  float gam[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) gam[j] = bf16_bits_to_f32(a.gamma[col0 + wn * 128 + j * 32 + l32]);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t row = row0 + wm * 64 + i * 32 + (v >> 2) * 8 + h32 * 4 + (v & 3);
      if (row >= a.T) continue;
      const float inv = a.inv[row], mm = a.m[row];
      const uint16_t* xr = a.x + row * a.d + col0 + wn * 128 + l32;
      uint16_t* o = a.dx + row * a.d + col0 + wn * 128 + l32;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float xv = bf16_bits_to_f32(xr[j * 32]);
        o[j * 32] = f32_to_bf16_bits(inv * gam[j] * ta.acc[i][j][v] - mm * xv);
      }
    }
  }
}

// ---------------------------------------------------------------- LoRA gradients
// Partial sums over one chunk of tokens, out[k][c] = sum_t P[t][k] M[t][c], as MFMA products
// whose inner dimension is the token index:
//   dA job:  M = x, P = bf16(V' * inv) over all targets' ranks (gamma is applied by the reduce,
//            since h[t][c] = x[t][c] * inv[t] * gamma[c]),
//   dB job:  M = G_t, P = U_t (s is applied by the reduce).
// One wave per work item (job, 32*CPL columns, a pass of 32*RB ranks, one chunk of tokens).
// In each 16-token step lane l reads CPL consecutive columns of 8 tokens (the lane half's
// share of the step) with one vector load per token and transposes them in registers:
// fragment j then holds, for column c0 + CPL*(l%32) + j, the 8 token values that one lane
// feeds the MFMA.  The MFMA's rows are therefore every CPL-th column; the epilogue maps them
// back.  Loads of the next step are issued before the current step's MFMAs.
struct LoraJob {
  const uint16_t* mat;  // M: element (t, c) at mat[t * ldm + c]; rows 16-byte aligned
  int64_t ldm;
  int cols;             // multiple of CPL
  const uint16_t* pv;   // P: element (t, k) at pv[t * ldp + k]
  int64_t ldp;
  int ranks;
  const float* inv;     // per-token factor folded into P, or nullptr
  float* out;           // [chunks][ranks][cols], chunk c at out + c * out_chunk
  int64_t out_chunk;
  int col_groups;       // column groups of 32 * CPL
  int groups;           // col_groups * rank passes
};

struct LoraArgs {
  LoraJob job[6];  // dA (one, or one per target with dropout), then each target's dB
  int njobs;
  int chunk;   // tokens per chunk, a multiple of 16
  int chunks;
  int64_t T;
};

// Buffer loads: every source is addressed as (per-block descriptor, 32-bit byte offset),
// and offsets at or past the descriptor's size read as zero.  That covers tokens past T in
// the last chunk, ranks past the job's count and columns past the job's width without any
// clamping in the loop.
constexpr uint32_t kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format
constexpr int kOutOfRange = 0x7fffffff;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), kRsrcWord3);
}

template <int CPL>
struct LoraVec;
template <>
struct LoraVec<8> {
  typedef uint32_t type __attribute__((ext_vector_type(4)));
  static __device__ __forceinline__ type load(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  }
};
template <>
struct LoraVec<4> {
  typedef uint32_t type __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ type load(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
  }
};

template <int CPL, int RB>
struct LoraStep {
  typename LoraVec<CPL>::type m[8];  // tokens 8 * h32 + u of the step, CPL columns each
  uint16_t p[RB][8];                 // P of the lane's rank in each block, same tokens
  float inv[8];
};

template <int RB>
struct LoraSrc {
  __amdgpu_buffer_rsrc_t m, p, inv;
  int m_off;      // lane's byte offset at the step's first row (its half's row 0)
  int m_row;      // bytes per M row
  int p_off[RB];  // lane's byte offset of (row 0 of its half, its rank), or out of range
  int p_row;
  int inv_off;
};

template <int CPL, int RB, bool SCALED>
__device__ __forceinline__ void lora_load(LoraStep<CPL, RB>& st, const LoraSrc<RB>& src, int row) {
  // row: first token of the step relative to the chunk
#pragma unroll
  for (int u = 0; u < 8; ++u) st.m[u] = LoraVec<CPL>::load(src.m, src.m_off + (row + u) * src.m_row);
#pragma unroll
  for (int b = 0; b < RB; ++b)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      st.p[b][i] = __builtin_amdgcn_raw_buffer_load_b16(src.p, src.p_off[b] + (row + i) * src.p_row, 0, 0);
  if (SCALED) {
    // into the named-component vector type: the builtin's own vector type, subscripted and
    // bit-cast, reads element 0 for every index
    const LoraVec<8>::type v0 = LoraVec<8>::load(src.inv, src.inv_off + row * 4);
    const LoraVec<8>::type v1 = LoraVec<8>::load(src.inv, src.inv_off + row * 4 + 16);
    st.inv[0] = __uint_as_float(v0.x);
    st.inv[1] = __uint_as_float(v0.y);
    st.inv[2] = __uint_as_float(v0.z);
    st.inv[3] = __uint_as_float(v0.w);
    st.inv[4] = __uint_as_float(v1.x);
    st.inv[5] = __uint_as_float(v1.y);
    st.inv[6] = __uint_as_float(v1.z);
    st.inv[7] = __uint_as_float(v1.w);
  }
}

template <int CPL, int RB, bool SCALED>
__device__ __forceinline__ void lora_mfma(const LoraStep<CPL, RB>& st, floatx16 (&acc)[CPL][RB]) {
  bf16x8 pf[RB];
#pragma unroll
  for (int b = 0; b < RB; ++b) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint16_t v = st.p[b][i];
      if (SCALED) v = f32_to_bf16_bits(bf16_bits_to_f32(v) * st.inv[i]);
      pf[b][i] = __builtin_bit_cast(__bf16, v);
    }
  }
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    // column c of the lane's CPL: half (c & 1) of dword c / 2 of each token's vector
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t lo = st.m[2 * q][c >> 1], hi = st.m[2 * q + 1][c >> 1];
      w[q] = (c & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
    }
    const bf16x8 af = __builtin_bit_cast(bf16x8, w);
#pragma unroll
    for (int b = 0; b < RB; ++b) acc[c][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, pf[b], acc[c][b], 0, 0, 0);
  }
}

// Two register sets in turn: the loads of one step are in flight while the other computes.
// Rows are taken 32 at a time; past the chunk's rows every load reads zero.
template <int CPL, int RB, bool SCALED>
__device__ __forceinline__ void lora_steps(const LoraSrc<RB>& src, int rows, floatx16 (&acc)[CPL][RB]) {
  LoraStep<CPL, RB> s0, s1;
  lora_load<CPL, RB, SCALED>(s0, src, 0);
  for (int row = 0; row < rows; row += 32) {
    lora_load<CPL, RB, SCALED>(s1, src, row + 16);
    lora_mfma<CPL, RB, SCALED>(s0, acc);
    lora_load<CPL, RB, SCALED>(s0, src, row + 32);
    lora_mfma<CPL, RB, SCALED>(s1, acc);
  }
}

template <int CPL, int RB>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void lora_partial_kernel(LoraArgs a) {
  const int lane = threadIdx.x, l32 = lane & 31, h32 = lane >> 5;
  const int chunk = blockIdx.x % a.chunks;
  int g = blockIdx.x / a.chunks, jb = 0;
  while (jb < a.njobs - 1 && g >= a.job[jb].groups) g -= a.job[jb++].groups;
  const LoraJob& j = a.job[jb];
  const int c0 = (g % j.col_groups) * 32 * CPL;
  const int k0 = (g / j.col_groups) * 32 * RB;
  const int col = c0 + CPL * l32;
  const int64_t t_begin = static_cast<int64_t>(chunk) * a.chunk;
  const int rows = static_cast<int>(min(static_cast<int64_t>(a.chunk), a.T - t_begin));
  const bool scaled = j.inv != nullptr;

  LoraSrc<RB> src;
  src.m = make_rsrc(j.mat + t_begin * j.ldm, static_cast<int64_t>(rows) * j.ldm * 2);
  src.m_row = static_cast<int>(j.ldm * 2);
  src.m_off = col < j.cols ? (8 * h32 * src.m_row + col * 2) : kOutOfRange;
  src.p = make_rsrc(j.pv + t_begin * j.ldp, static_cast<int64_t>(rows) * j.ldp * 2);
  src.p_row = static_cast<int>(j.ldp * 2);
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    const int k = k0 + 32 * b + l32;
    src.p_off[b] = k < j.ranks ? (8 * h32 * src.p_row + k * 2) : kOutOfRange;
  }
  src.inv = make_rsrc(scaled ? j.inv + t_begin : j.inv, scaled ? rows * 4 : 0);
  src.inv_off = 8 * h32 * 4;

  floatx16 acc[CPL][RB];
#pragma unroll
  for (int c = 0; c < CPL; ++c)
#pragma unroll
    for (int b = 0; b < RB; ++b) acc[c][b] = floatx16{};

  if (scaled)
    lora_steps<CPL, RB, true>(src, rows, acc);
  else
    lora_steps<CPL, RB, false>(src, rows, acc);

  // lane: rank k0 + 32 b + l32; rows i of the 32x32 result are columns c0 + CPL * i + c
  float* o = j.out + static_cast<int64_t>(chunk) * j.out_chunk;
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    const int k = k0 + 32 * b + l32;
    if (k >= j.ranks) continue;
    float* orow = o + static_cast<int64_t>(k) * j.cols;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int c = c0 + CPL * ((v >> 2) * 8 + h32 * 4 + (v & 3));
      if (c >= j.cols) continue;
#pragma unroll
      for (int q = 0; q < CPL; q += 4)
        *reinterpret_cast<float4*>(orow + c + q) =
            make_float4(acc[q][b][v], acc[q + 1][b][v], acc[q + 2][b][v], acc[q + 3][b][v]);
    }
  }
}

// dA_t[k][c] = gamma[c] sum_chunks PdA[ch][off_t + k][c];  dB_t[n][k] = s sum_chunks PdB_t[ch][k][n].
// Chunks are summed in a fixed order (four interleaved running sums), so results are
// reproducible run to run.
struct ReduceArgs {
  const float* pda;
  const float* pdb[3];
  const uint16_t* gamma;
  float* da[3];
  float* db[3];
  int off[3], nt[3];
  int R, r, d, chunks;
  float scale;
  uint32_t targets;
};

__device__ __forceinline__ float sum_chunks(const float* p, int64_t stride, int chunks) {
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
  int c = 0;
  for (; c + 4 <= chunks; c += 4) {
    s0 += p[(c + 0) * stride];
    s1 += p[(c + 1) * stride];
    s2 += p[(c + 2) * stride];
    s3 += p[(c + 3) * stride];
  }
  for (; c < chunks; ++c) s0 += p[c * stride];
  return (s0 + s1) + (s2 + s3);
}

__global__ __launch_bounds__(256) void lora_reduce_kernel(ReduceArgs a) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  const int64_t sa = static_cast<int64_t>(a.R) * a.d;
  for (int t = 0; t < 3; ++t) {
    if (!((a.targets >> t) & 1u)) continue;
    const int64_t na = static_cast<int64_t>(a.r) * a.d;
    for (int64_t e = gid; e < na; e += stride) {
      const int64_t k = e / a.d, c = e % a.d;
      // no token chunks (T == 0): gamma may be NULL and is not read
      a.da[t][e] = a.chunks ? bf16_bits_to_f32(a.gamma[c]) * sum_chunks(a.pda + (a.off[t] + k) * a.d + c, sa, a.chunks)
                            : 0.f;
    }
    const int64_t nb = static_cast<int64_t>(a.nt[t]) * a.r;
    const int64_t sb = nb;
    for (int64_t e = gid; e < nb; e += stride) {
      const int64_t k = e / a.nt[t], n = e % a.nt[t];  // n fastest: coalesced partial reads
      const float s = a.chunks ? sum_chunks(a.pdb[t] + k * a.nt[t] + n, sb, a.chunks) : 0.f;
      a.db[t][n * a.r + k] = a.scale * s;
    }
  }
}

}  // namespace

bool bwd_tiled_supports(const FwdParams& p) {
  return p.D % 2 == 0 && p.D <= 512 && (p.Hq * p.D) % 64 == 0 && (p.Hkv * p.D) % 64 == 0 && p.d % 256 == 0 &&
         p.d < (1 << 19) && p.N + 256 < (1 << 19) && p.r <= kMaxRank && p.T <= (int64_t{1} << 24);
}

size_t bwd_tiled_workspace_bytes(const FwdParams& p) { return bwd_layout(p).total; }

// Prepared backward weights: W^T [d][N] bf16.
size_t bwd_tiled_prepared_bytes(const FwdParams& p) { return al256(static_cast<size_t>(p.d) * p.N * 2); }

hipError_t prepare_bwd_tiled(const FwdParams& p, void* dst, hipStream_t s) {
  PrepArgs pa{};
  pa.w = static_cast<const uint16_t*>(p.w);
  if (p.nf4) pa.wq = nf4_view(p.w, p.N, p.d);
  pa.wt = static_cast<uint16_t*>(dst);
  pa.N = p.N;
  pa.d = static_cast<int>(p.d);
  pa.q_begin = 0;
  pa.targets = 0;
  pa.wt_blocks = (p.N / 64) * static_cast<int>(p.d / 64);
  hipLaunchKernelGGL(prep_weights_kernel, dim3(pa.wt_blocks), dim3(256), 0, s, pa);
  return hipGetLastError();
}

hipError_t launch_bwd_tiled(const BwdParams& bp, hipStream_t s) {
  const FwdParams& p = bp.f;
  const BwdLayout L = bwd_layout(p);
  void* ws = p.ws;
  const bool lora = p.targets != 0;
  int lo[3], nt[3];
  for (int t = 0; t < 3; ++t) {
    int l, h;
    target_cols(p, t, l, h);
    lo[t] = l;
    nt[t] = h - l;
  }

  if (p.T > 0) {
    // ---- weights
    PrepArgs pa{};
    pa.w = static_cast<const uint16_t*>(p.w);
    if (p.nf4) pa.wq = nf4_view(p.w, p.N, p.d);
    pa.gamma = static_cast<const uint16_t*>(p.gamma);
    pa.wt = at<uint16_t>(ws, L.wt);
    pa.at = at<uint16_t>(ws, L.at);
    for (int t = 0; t < 3; ++t) {
      pa.a[t] = static_cast<const uint16_t*>(p.a[t]);
      pa.b[t] = static_cast<const uint16_t*>(p.b[t]);
      pa.bt[t] = at<uint16_t>(ws, L.bt[t]);
      pa.ap[t] = at<uint16_t>(ws, L.ap[t]);
      pa.off[t] = L.off[t];
      pa.lo[t] = lo[t];
      pa.nt[t] = nt[t];
    }
    pa.N = p.N;
    pa.d = static_cast<int>(p.d);
    pa.r = p.r;
    pa.Rp = L.Rp;
    pa.R = L.R;
    pa.q_begin = p.use_prepared ? p.N : 0;
    pa.targets = p.targets;
    pa.wt_blocks = static_cast<int>((L.K - pa.q_begin) / 64) * static_cast<int>(p.d / 64);
    if (pa.wt_blocks + (lora ? 256 : 0) > 0)
      hipLaunchKernelGGL(prep_weights_kernel, dim3(pa.wt_blocks + (lora ? 256 : 0)), dim3(256), 0, s, pa);

    // ---- rows
    RowsArgs ra{};
    ra.x = static_cast<const uint16_t*>(p.x);
    ra.y = static_cast<const uint16_t*>(bp.y);
    ra.dy = static_cast<const uint16_t*>(bp.dy);
    ra.bias = p.has_bias ? static_cast<const uint16_t*>(p.bias) : nullptr;
    ra.pos = p.pos;
    ra.gcat = at<uint16_t>(ws, L.gcat);
    ra.inv = at<float>(ws, L.inv);
    ra.m = at<float>(ws, L.m);
    ra.T = p.T;
    ra.d = static_cast<int>(p.d);
    ra.N = p.N;
    ra.D = p.D;
    ra.rot_end = p.rot_end;
    ra.K = L.K;
    ra.eps = p.eps;
    ra.log2_theta = log2(p.theta);
    if (p.dropout) {
      ra.nt = p.drop_nt;
      for (int t = 0, k = 0; t < 3; ++t)
        if (p.targets & (1u << t)) ra.target[k++] = t;
      ra.thr = p.drop_thr;
      ra.offset = p.drop_offset;
      ra.seed_lo = static_cast<uint32_t>(p.drop_seed);
      ra.seed_hi = static_cast<uint32_t>(p.drop_seed >> 32);
      ra.bits = reinterpret_cast<uint8_t*>(p.drop_bits_r);
      ra.xm = p.drop_xm;
    }
    hipLaunchKernelGGL(rows_kernel, dim3(static_cast<unsigned>((p.T + 3) / 4)), dim3(256), 0, s, ra);

    if (lora) {
      // ---- V' = bf16(s G_t B_t) into Gcat's LoRA columns; U = bf16(inv x A'^T) for the R
      // rows of all targets' A' at once (x is read once per 32 RB of them)
      RankArgs ra2{};
      ra2.T = p.T;
      const int rb = p.r <= 32 ? 1 : 2;
      int nj = 0, last_t = -1;
      for (int t = 0; t < 3; ++t)
        if (p.targets & (1u << t)) last_t = t;
      for (int t = 0; t < 3; ++t) {
        if (!(p.targets & (1u << t))) continue;
        RankJob& vj = ra2.job[nj++];
        vj.a = at<uint16_t>(ws, L.gcat) + lo[t];
        vj.lda = L.K;
        vj.bs = at<uint16_t>(ws, L.bt[t]);
        vj.ldb = nt[t];
        vj.r = p.r;
        vj.nk = nt[t] / BK;
        vj.out = at<uint16_t>(ws, L.gcat);
        vj.ldo = L.K;
        vj.col0 = p.N + L.off[t];
        vj.pad_to = t == last_t ? static_cast<int>(L.K) : vj.col0 + p.r;
        vj.scale = p.scale;
        vj.inv = nullptr;
      }
      for (int t = 0; t < 3 && p.dropout; ++t) {
        // dropout: U_t = bf16(inv (x * keep_t) A'_t^T), one job per target
        if (!(p.targets & (1u << t))) continue;
        RankJob& uj = ra2.job[nj++];
        uj.a = p.drop_xm + static_cast<int64_t>(target_slot(p.targets, t)) * p.T * p.d;
        uj.lda = p.d;
        uj.bs = at<uint16_t>(ws, L.ap[t]);
        uj.ldb = p.d;
        uj.r = p.r;
        uj.nk = static_cast<int>(p.d / BK);
        uj.out = at<uint16_t>(ws, L.u);
        uj.ldo = L.R;
        uj.col0 = L.off[t];
        uj.pad_to = uj.col0 + p.r;
        uj.scale = 1.0f;
        uj.inv = at<float>(ws, L.inv);
      }
      for (int c0 = 0; c0 < L.R && !p.dropout; c0 += 32 * rb) {
        RankJob& uj = ra2.job[nj++];
        uj.a = static_cast<const uint16_t*>(p.x);
        uj.lda = p.d;
        uj.bs = at<uint16_t>(ws, L.ap_all) + static_cast<int64_t>(c0) * p.d;
        uj.ldb = p.d;
        uj.r = std::min(32 * rb, L.R - c0);
        uj.nk = static_cast<int>(p.d / BK);
        uj.out = at<uint16_t>(ws, L.u);
        uj.ldo = L.R;
        uj.col0 = c0;
        uj.pad_to = c0 + uj.r;
        uj.scale = 1.0f;
        uj.inv = at<float>(ws, L.inv);
      }
      const dim3 grid(static_cast<unsigned>((p.T + kRankRows - 1) / kRankRows), nj);
      if (rb == 1)
        hipLaunchKernelGGL(rank_kernel<1>, grid, dim3(kThreads), 0, s, ra2);
      else
        hipLaunchKernelGGL(rank_kernel<2>, grid, dim3(kThreads), 0, s, ra2);
    }

    // ---- dh and dx
    MainArgs ma{};
    ma.gcat = at<uint16_t>(ws, L.gcat);
    ma.wt = p.use_prepared ? static_cast<const uint16_t*>(p.prepared) : at<uint16_t>(ws, L.wt);
    ma.at = at<uint16_t>(ws, L.at);
    ma.N = p.N;
    ma.Rp = L.Rp;
    ma.x = static_cast<const uint16_t*>(p.x);
    ma.gamma = static_cast<const uint16_t*>(p.gamma);
    ma.inv = at<float>(ws, L.inv);
    ma.m = at<float>(ws, L.m);
    ma.dx = static_cast<uint16_t*>(bp.dx);
    ma.T = p.T;
    ma.d = static_cast<int>(p.d);
    ma.K = L.K;
    ma.n_nt = static_cast<int>(p.d / BN);
    const int n_mt = static_cast<int>((p.T + BM - 1) / BM);
    ma.n_mt = n_mt;
    ma.group_m = 4;
    ma.items = n_mt * ma.n_nt;
    ma.remap = ma.items % 8 == 0;
    if (p.dropout) {
      ma.bits = p.drop_bits_r;
      ma.r = p.r;
      for (int t = 0; t < 3; ++t)
        if (p.targets & (1u << t)) ma.loff[ma.nslots++] = L.off[t];
    }
    timing_begin(s);
    switch (p.dropout ? ma.nslots : 0) {
      case 0: hipLaunchKernelGGL(bwd_main_kernel<0>, dim3(ma.items), dim3(kThreads8), 0, s, ma); break;
      case 1: hipLaunchKernelGGL(bwd_main_kernel<1>, dim3(ma.items), dim3(kThreads8), 0, s, ma); break;
      case 2: hipLaunchKernelGGL(bwd_main_kernel<2>, dim3(ma.items), dim3(kThreads8), 0, s, ma); break;
      default: hipLaunchKernelGGL(bwd_main_kernel<3>, dim3(ma.items), dim3(kThreads8), 0, s, ma); break;
    }
    timing_end(s);

    if (lora) {
      // ---- LoRA gradient partial sums
      LoraArgs la{};
      int nj = 0, items = 0;
      if (!p.dropout) {
        LoraJob& ja = la.job[nj++];
        ja.mat = static_cast<const uint16_t*>(p.x);
        ja.ldm = p.d;
        ja.cols = static_cast<int>(p.d);
        ja.pv = at<uint16_t>(ws, L.gcat) + p.N;
        ja.ldp = L.K;
        ja.ranks = L.R;
        ja.inv = at<float>(ws, L.inv);
        ja.out = at<float>(ws, L.pda);
        ja.out_chunk = static_cast<int64_t>(L.R) * p.d;
        ja.groups = L.groups[0];
        ja.col_groups = static_cast<int>(p.d / (32 * L.cpl));
        items += ja.groups;
      }
      for (int t = 0; t < 3 && p.dropout; ++t) {
        // dropout: target t's ranks against its masked input, into the same partial-sum rows
        if (!(p.targets & (1u << t))) continue;
        LoraJob& ja = la.job[nj++];
        ja.mat = p.drop_xm + static_cast<int64_t>(target_slot(p.targets, t)) * p.T * p.d;
        ja.ldm = p.d;
        ja.cols = static_cast<int>(p.d);
        ja.pv = at<uint16_t>(ws, L.gcat) + p.N + L.off[t];
        ja.ldp = L.K;
        ja.ranks = p.r;
        ja.inv = at<float>(ws, L.inv);
        ja.out = at<float>(ws, L.pda) + static_cast<int64_t>(L.off[t]) * p.d;
        ja.out_chunk = static_cast<int64_t>(L.R) * p.d;
        ja.groups = L.groups_da_t;
        ja.col_groups = static_cast<int>(p.d / (32 * L.cpl));
        items += ja.groups;
      }
      for (int t = 0; t < 3; ++t) {
        if (!(p.targets & (1u << t))) continue;
        LoraJob& jb = la.job[nj++];
        jb.mat = at<uint16_t>(ws, L.gcat) + lo[t];
        jb.ldm = L.K;
        jb.cols = nt[t];
        jb.pv = at<uint16_t>(ws, L.u) + L.off[t];
        jb.ldp = L.R;
        jb.ranks = p.r;
        jb.inv = nullptr;
        jb.out = at<float>(ws, L.pdb[t]);
        jb.out_chunk = static_cast<int64_t>(p.r) * nt[t];
        jb.groups = L.groups[t + 1];
        jb.col_groups = (nt[t] + 32 * L.cpl - 1) / (32 * L.cpl);
        items += jb.groups;
      }
      la.njobs = nj;
      la.chunk = L.chunk;
      la.chunks = L.chunks;
      la.T = p.T;
      const dim3 grid(static_cast<unsigned>(items * L.chunks));
      if (L.cpl == 8)
        hipLaunchKernelGGL((lora_partial_kernel<8, 1>), grid, dim3(64), 0, s, la);
      else
        hipLaunchKernelGGL((lora_partial_kernel<4, 2>), grid, dim3(64), 0, s, la);
    }
  }

  if (lora) {
    // ---- dA, dB (zero when T == 0: no chunks)
    ReduceArgs rd{};
    rd.pda = at<float>(ws, L.pda);
    rd.gamma = static_cast<const uint16_t*>(p.gamma);
    for (int t = 0; t < 3; ++t) {
      rd.pdb[t] = at<float>(ws, L.pdb[t]);
      rd.da[t] = bp.da[t];
      rd.db[t] = bp.db[t];
      rd.off[t] = L.off[t];
      rd.nt[t] = nt[t];
    }
    rd.R = L.R;
    rd.r = p.r;
    rd.d = static_cast<int>(p.d);
    rd.chunks = L.chunks;
    rd.scale = p.scale;
    rd.targets = p.targets;
    int64_t n_out = 0;
    for (int t = 0; t < 3; ++t)
      if (p.targets & (1u << t)) n_out = std::max<int64_t>(n_out, static_cast<int64_t>(p.r) * std::max<int64_t>(p.d, nt[t]));
    const unsigned rgrid = static_cast<unsigned>(std::min<int64_t>(std::max<int64_t>((n_out + 255) / 256, 1), 2048));
    hipLaunchKernelGGL(lora_reduce_kernel, dim3(rgrid), dim3(256), 0, s, rd);
  }
  return hipGetLastError();
}

}  // namespace lrq
