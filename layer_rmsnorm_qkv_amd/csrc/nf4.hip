// NF4 quantiser of the frozen W_qkv (the QLoRA base; format in lrq_internal.h / lrq.h).
// One wavefront per block of 64 weights: lane k holds weight k of the block; the block's
// largest magnitude comes from a wavefront max; each lane takes its code from the float32
// midpoints of the code book; even lanes store one byte (their code in the low nibble, the
// odd neighbour's in the high nibble) and lane 0 stores the scale.
#include <algorithm>

#include "lrq_internal.h"

namespace lrq {
namespace {

struct QuantArgs {
  const void* w;     // [n][d] float32 or bf16
  int f32;
  int64_t n, d;
  uint8_t* codes;    // [n][d / 2]
  float* scales;     // [n][d / 64]
};

__global__ __launch_bounds__(256) void quantize_nf4_kernel(QuantArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t nblk = a.n * (a.d / kNf4Block);
  for (int64_t b = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6); b < nblk;
       b += static_cast<int64_t>(gridDim.x) * 4) {
    const int64_t idx = b * kNf4Block + lane;  // row-major element index (blocks tile the rows)
    const float w = a.f32 ? static_cast<const float*>(a.w)[idx]
                          : bf16_bits_to_f32(static_cast<const uint16_t*>(a.w)[idx]);
    float m = fabsf(w);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    uint32_t code = 7;  // the zero level: all-zero blocks
    if (m > 0.f) {
      const float y = w / m;  // correctly rounded float32 division
      code = 0;
#pragma unroll
      for (int i = 0; i < 15; ++i) code += y > (kNf4Levels[i] + kNf4Levels[i + 1]) * 0.5f ? 1u : 0u;
    }
    const uint32_t hi = __shfl_down(code, 1);
    if ((lane & 1) == 0) a.codes[idx >> 1] = static_cast<uint8_t>(code | (hi << 4));
    if (lane == 0) a.scales[b] = m;
  }
}

}  // namespace

hipError_t launch_quantize_nf4(const void* w, bool f32, int64_t n, int64_t d, void* dst, hipStream_t s) {
  QuantArgs a{};
  a.w = w;
  a.f32 = f32 ? 1 : 0;
  a.n = n;
  a.d = d;
  a.codes = static_cast<uint8_t*>(dst);
  a.scales = reinterpret_cast<float*>(static_cast<unsigned char*>(dst) + nf4_codes_bytes(n, d));
  const int64_t nblk = n * (d / kNf4Block);
  if (nblk == 0) return hipSuccess;
  const unsigned g = static_cast<unsigned>(std::min<int64_t>((nblk + 3) / 4, 16384));
  hipLaunchKernelGGL(quantize_nf4_kernel, dim3(g), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace lrq
