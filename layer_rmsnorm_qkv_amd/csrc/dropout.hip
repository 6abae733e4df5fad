// LoRA dropout masks as bits (training-time dropout of the adapters' input; the LoRA
// configurations on the pages carry a lora_dropout rate).  Feature j of token row `row` is kept
// for adapter slot s (target t) iff word j % 4 of Philox4x32-10 applied to the counter
// (j / 4, row, t, offset) with the key (seed low, seed high) is >= floor(p * 2^32).  Philox is
// written from its published definition (Salmon, Moraes, Dror and Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC 2011): ten rounds, each multiplying words 0 and 2 by two
// constants and mixing the 64-bit products' halves with words 1 and 3 and the key, the key
// bumped by two Weyl constants between rounds.  The same bits serve the forward and the
// backward, which regenerates them from (seed, offset).
//   rows  bits_r[s][row][j / 32], bit j % 32           (one thread per 32 features)
//   cols  bits_c[s][j][row / 32], bit row % 32         (a ballot transpose of the rows form)
//   xm    xm[s][row][j] = keep ? x[row][j] : 0, bf16   (the tiled families' adapter input;
//         the 1 / (1 - p) factor is folded into the adapter scale)
#include <algorithm>

#include "lrq_internal.h"

namespace lrq {
namespace {

__device__ __forceinline__ void philox4x32_10(uint32_t (&x)[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = static_cast<uint64_t>(0xD2511F53u) * x[0];
    const uint64_t p1 = static_cast<uint64_t>(0xCD9E8D57u) * x[2];
    const uint32_t hi0 = static_cast<uint32_t>(p0 >> 32), lo0 = static_cast<uint32_t>(p0);
    const uint32_t hi1 = static_cast<uint32_t>(p1 >> 32), lo1 = static_cast<uint32_t>(p1);
    const uint32_t n0 = hi1 ^ x[1] ^ k0, n2 = hi0 ^ x[3] ^ k1;
    x[0] = n0;
    x[1] = lo1;
    x[2] = n2;
    x[3] = lo0;
  }
}

struct MaskArgs {
  uint32_t* bits_r;  // [nt][T][dw]
  uint32_t* bits_c;  // [nt][d][tw] (nullptr: not needed)
  const uint16_t* x; // bf16 [T][d], with xm
  uint16_t* xm;      // [nt][T][d] x * keep (nullptr: not needed)
  int64_t T;
  int d, dw, tw, nt;
  int target[3];     // target index (0 q, 1 k, 2 v) of slot s
  uint32_t thr, offset, seed_lo, seed_hi;
};

// One thread per (slot, row, 32 features): eight Philox blocks give the 32 words.
__global__ __launch_bounds__(256) void dropout_rows_kernel(MaskArgs a) {
  const int64_t total = static_cast<int64_t>(a.nt) * a.T * a.dw;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * 256) {
    const int w = static_cast<int>(e % a.dw);
    const int64_t rs = e / a.dw;
    const int64_t row = rs % a.T;
    const int s = static_cast<int>(rs / a.T);
    const int t = s == 0 ? a.target[0] : (s == 1 ? a.target[1] : a.target[2]);
    uint32_t bits = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      uint32_t x[4] = {static_cast<uint32_t>(8 * w + q), static_cast<uint32_t>(row), static_cast<uint32_t>(t),
                       a.offset};
      philox4x32_10(x, a.seed_lo, a.seed_hi);
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int j = 32 * w + 4 * q + e4;
        if (j < a.d && x[e4] >= a.thr) bits |= 1u << (4 * q + e4);
      }
    }
    a.bits_r[e] = bits;
    if (a.xm) {
      // d % 32 == 0 here (the tiled families): four 16-byte vectors of x, masked per element
      const uint4* src = reinterpret_cast<const uint4*>(a.x + row * a.d + 32 * w);
      uint4* dst = reinterpret_cast<uint4*>(a.xm + (static_cast<int64_t>(s) * a.T + row) * a.d + 32 * w);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint4 v = src[c];
        uint32_t o[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t b2 = bits >> (8 * c + 2 * q);
          o[q] &= ((b2 & 1u) ? 0x0000ffffu : 0u) | ((b2 & 2u) ? 0xffff0000u : 0u);
        }
        dst[c] = uint4{o[0], o[1], o[2], o[3]};
      }
    }
  }
}

// One wave per (slot, 64 rows, 32 features): lane l holds the row word of row 64 rb + l;
// ballot over the lanes turns feature f of the 64 rows into two column words.
__global__ __launch_bounds__(256) void dropout_cols_kernel(MaskArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t rb_count = (a.T + 63) / 64;
  const int64_t items = static_cast<int64_t>(a.nt) * rb_count * a.dw;
  for (int64_t it = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6); it < items;
       it += static_cast<int64_t>(gridDim.x) * 4) {
    const int w = static_cast<int>(it % a.dw);
    const int64_t rbs = it / a.dw;
    const int64_t rb = rbs % rb_count;
    const int s = static_cast<int>(rbs / rb_count);
    const int64_t row = rb * 64 + lane;
    const uint32_t word = row < a.T ? a.bits_r[(static_cast<int64_t>(s) * a.T + row) * a.dw + w] : 0u;
    for (int f = 0; f < 32; ++f) {
      const uint64_t b = __ballot((word >> f) & 1u);
      const int j = 32 * w + f;
      if (j < a.d) {
        const int64_t base = (static_cast<int64_t>(s) * a.d + j) * a.tw + 2 * rb;
        if (lane == 0) a.bits_c[base] = static_cast<uint32_t>(b);
        if (lane == 1 && 2 * rb + 1 < a.tw) a.bits_c[base + 1] = static_cast<uint32_t>(b >> 32);
      }
    }
  }
}

size_t al256(size_t n) { return (n + 255) & ~size_t{255}; }

}  // namespace

size_t dropout_region_bytes(const FwdParams& p, bool cols, bool xm) {
  if (!p.dropout) return 0;
  const size_t nt = static_cast<size_t>(p.drop_nt), T = static_cast<size_t>(p.T), d = static_cast<size_t>(p.d);
  size_t n = al256(nt * T * ((d + 31) / 32) * 4);
  if (cols) n += al256(nt * d * ((T + 31) / 32) * 4);
  if (xm) n += al256(nt * T * d * 2);
  return n;
}

hipError_t launch_dropout_masks(FwdParams& p, void* region, bool cols, bool xm, hipStream_t s) {
  if (!p.dropout) return hipSuccess;
  const size_t nt = static_cast<size_t>(p.drop_nt), T = static_cast<size_t>(p.T), d = static_cast<size_t>(p.d);
  unsigned char* q = static_cast<unsigned char*>(region);
  uint32_t* bits_r = reinterpret_cast<uint32_t*>(q);
  q += al256(nt * T * ((d + 31) / 32) * 4);
  uint32_t* bits_c = nullptr;
  if (cols) {
    bits_c = reinterpret_cast<uint32_t*>(q);
    q += al256(nt * d * ((T + 31) / 32) * 4);
  }
  uint16_t* xmp = xm ? reinterpret_cast<uint16_t*>(q) : nullptr;
  p.drop_bits_r = bits_r;
  p.drop_bits_c = bits_c;
  p.drop_xm = xmp;
  if (p.T == 0) return hipSuccess;
  MaskArgs a{};
  a.bits_r = bits_r;
  a.bits_c = bits_c;
  a.x = static_cast<const uint16_t*>(p.x);
  a.xm = xmp;
  a.T = p.T;
  a.d = static_cast<int>(p.d);
  a.dw = static_cast<int>((p.d + 31) / 32);
  a.tw = static_cast<int>((p.T + 31) / 32);
  a.nt = p.drop_nt;
  for (int t = 0, k = 0; t < 3; ++t)
    if (p.targets & (1u << t)) a.target[k++] = t;
  a.thr = p.drop_thr;
  a.offset = p.drop_offset;
  a.seed_lo = static_cast<uint32_t>(p.drop_seed);
  a.seed_hi = static_cast<uint32_t>(p.drop_seed >> 32);
  const int64_t words = static_cast<int64_t>(a.nt) * a.T * a.dw;
  const unsigned g1 = static_cast<unsigned>(std::min<int64_t>((words + 255) / 256, 8192));
  hipLaunchKernelGGL(dropout_rows_kernel, dim3(g1), dim3(256), 0, s, a);
  if (bits_c) {
    const int64_t items = static_cast<int64_t>(a.nt) * ((a.T + 63) / 64) * a.dw;
    const unsigned g2 = static_cast<unsigned>(std::min<int64_t>((items + 3) / 4, 8192));
    hipLaunchKernelGGL(dropout_cols_kernel, dim3(g2), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace lrq
