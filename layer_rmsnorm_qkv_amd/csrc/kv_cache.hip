// Key/value cache write of a forward call, for the families whose epilogue does not store the
// cache itself (tiled and generic): after the forward, the k and v column blocks of every token
// row of out are copied to row slots[t] of k_cache and v_cache.  The values are the ones in out,
// bit for bit.  Tokens whose slot is negative or past the cache are skipped.
#include "lrq_internal.h"

namespace lrq {
namespace {

struct ScatterArgs {
  const unsigned char* out;
  unsigned char* kc;
  unsigned char* vc;
  const int32_t* slots;
  int64_t T, num_slots;
  int64_t row_bytes;  // N * element size
  int64_t k_off;      // col_k * element size
  int64_t v_off;      // col_v * element size
  int64_t kv_bytes;   // Hkv * D * element size: one cache row
};

// One workgroup per token (grid-stride); V is the copy unit (16 bytes when every offset and
// size is a multiple of 16, else 2 bytes).
template <typename V>
__global__ __launch_bounds__(256) void kv_scatter_kernel(ScatterArgs a) {
  const int64_t n = a.kv_bytes / static_cast<int64_t>(sizeof(V));
  for (int64_t t = blockIdx.x; t < a.T; t += gridDim.x) {
    const int32_t slot = a.slots[t];
    if (slot < 0 || slot >= a.num_slots) continue;
    const unsigned char* row = a.out + t * a.row_bytes;
    for (int64_t i = threadIdx.x; i < 2 * n; i += blockDim.x) {
      const bool is_v = i >= n;
      const int64_t j = is_v ? i - n : i;
      const V val = *reinterpret_cast<const V*>(row + (is_v ? a.v_off : a.k_off) + j * sizeof(V));
      *reinterpret_cast<V*>((is_v ? a.vc : a.kc) + slot * a.kv_bytes + j * sizeof(V)) = val;
    }
  }
}

}  // namespace

hipError_t launch_kv_scatter(const FwdParams& p, hipStream_t s) {
  if (p.T == 0 || !p.kv_slots) return hipSuccess;
  const int64_t es = p.esize;
  ScatterArgs a{};
  a.out = static_cast<const unsigned char*>(p.out);
  a.kc = static_cast<unsigned char*>(p.kv_k);
  a.vc = static_cast<unsigned char*>(p.kv_v);
  a.slots = p.kv_slots;
  a.T = p.T;
  a.num_slots = p.kv_num_slots;
  a.row_bytes = static_cast<int64_t>(p.N) * es;
  a.k_off = static_cast<int64_t>(p.col_k) * es;
  a.v_off = static_cast<int64_t>(p.col_v) * es;
  a.kv_bytes = static_cast<int64_t>(p.Hkv) * p.D * es;
  const int grid = static_cast<int>(p.T < 65536 ? p.T : 65536);
  if (a.row_bytes % 16 == 0 && a.k_off % 16 == 0 && a.v_off % 16 == 0 && a.kv_bytes % 16 == 0)
    hipLaunchKernelGGL(kv_scatter_kernel<uint4>, dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(kv_scatter_kernel<uint16_t>, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace lrq
