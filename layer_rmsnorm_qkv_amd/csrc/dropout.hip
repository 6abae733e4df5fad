// LoRA dropout masks (training-time dropout of the adapters' input; the LoRA configurations on
// the pages carry a lora_dropout rate).  Feature j of token row `row` is kept for adapter slot s
// (target t) iff word j % 4 of Philox4x32-10 applied to the counter (j / 4, row, t, offset)
// with the key (seed low, seed high) is >= floor(p * 2^32) (philox4x32_10 / dropout_byte in
// lrq_internal.h).  The same bits serve the forward and the backward, which regenerates them
// from (seed, offset).  Region layout (each part 256-byte aligned):
//   rows  bits_r[s][row][j / 32], bit j % 32: as bytes, byte j / 8 of the row holds bits
//         j .. j + 7 (little-endian words), so one thread writes one byte per 8 features
//   xm    xm[s][row][j] = keep ? x[row][j] : 0, bf16   (the tiled families' adapter input;
//         the 1 / (1 - p) factor is folded into the adapter scale)
// The generation is bound by Philox's 64-bit products (20 per 4 features); the tiled backward
// therefore makes its masks inside its memory-bound rows pass instead (bwd_tiled.hip).
#include <algorithm>

#include "lrq_internal.h"

namespace lrq {
namespace {

struct MaskArgs {
  uint8_t* bits;      // [nt][T][db] (db = ceil(d / 32) * 4 bytes per row)
  const void* x;      // bf16 [T][d], with xm
  uint16_t* xm;       // [nt][T][d] x * keep (nullptr: not needed)
  int64_t T;
  int d, db, nt;
  int target[3];      // target index (0 q, 1 k, 2 v) of slot s
  uint32_t thr, offset, seed_lo, seed_hi;
};

// One thread per (slot, row, 8 features): two Philox blocks give the 8 words.  Bytes of a row
// past d / 8 (the padding of the last word) are written as 0.
__global__ __launch_bounds__(256) void dropout_rows_kernel(MaskArgs a) {
  const int64_t total = static_cast<int64_t>(a.nt) * a.T * a.db;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * 256) {
    const int c = static_cast<int>(e % a.db);
    const int64_t rs = e / a.db;
    const int64_t row = rs % a.T;
    const int s = static_cast<int>(rs / a.T);
    const int t = s == 0 ? a.target[0] : (s == 1 ? a.target[1] : a.target[2]);
    const int j = 8 * c;
    uint32_t keep = 0;
    if (j < a.d) {
      keep = dropout_byte(j, static_cast<uint32_t>(row), static_cast<uint32_t>(t), a.offset, a.thr, a.seed_lo,
                          a.seed_hi);
      if (a.d - j < 8) keep &= (1u << (a.d - j)) - 1u;
    }
    a.bits[e] = static_cast<uint8_t>(keep);
    if (a.xm && j < a.d) {
      // d % 8 == 0 here (the tiled families): one 16-byte vector of x
      const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.x) + row * a.d + j);
      *reinterpret_cast<uint4*>(a.xm + (static_cast<int64_t>(s) * a.T + row) * a.d + j) = mask_bf16x8(v, keep);
    }
  }
}

size_t al256(size_t n) { return (n + 255) & ~size_t{255}; }
size_t row_bytes(int64_t d) { return static_cast<size_t>((d + 31) / 32) * 4; }

}  // namespace

size_t dropout_region_bytes(const FwdParams& p, bool xm) {
  if (!p.dropout) return 0;
  const size_t nt = static_cast<size_t>(p.drop_nt), T = static_cast<size_t>(p.T), d = static_cast<size_t>(p.d);
  size_t n = al256(nt * T * row_bytes(p.d));
  if (xm) n += al256(nt * T * d * 2);
  return n;
}

hipError_t launch_dropout_masks(FwdParams& p, void* region, bool xm, bool fill, hipStream_t s) {
  if (!p.dropout) return hipSuccess;
  const size_t nt = static_cast<size_t>(p.drop_nt), T = static_cast<size_t>(p.T);
  unsigned char* q = static_cast<unsigned char*>(region);
  p.drop_bits_r = reinterpret_cast<uint32_t*>(q);
  q += al256(nt * T * row_bytes(p.d));
  p.drop_xm = xm ? reinterpret_cast<uint16_t*>(q) : nullptr;
  if (!fill || p.T == 0) return hipSuccess;
  MaskArgs a{};
  a.bits = reinterpret_cast<uint8_t*>(p.drop_bits_r);
  a.x = p.x;
  a.xm = p.drop_xm;
  a.T = p.T;
  a.d = static_cast<int>(p.d);
  a.db = static_cast<int>(row_bytes(p.d));
  a.nt = p.drop_nt;
  for (int t = 0, k = 0; t < 3; ++t)
    if (p.targets & (1u << t)) a.target[k++] = t;
  a.thr = p.drop_thr;
  a.offset = p.drop_offset;
  a.seed_lo = static_cast<uint32_t>(p.drop_seed);
  a.seed_hi = static_cast<uint32_t>(p.drop_seed >> 32);
  const int64_t items = static_cast<int64_t>(a.nt) * a.T * a.db;
  const unsigned g = static_cast<unsigned>(std::min<int64_t>((items + 255) / 256, 16384));
  hipLaunchKernelGGL(dropout_rows_kernel, dim3(g), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace lrq
