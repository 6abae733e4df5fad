// Attention over the key/value cache (bf16 q, k, v; fp32 scores, softmax and accumulation):
// the step after the projection in the decoder layer of the inference-engine page, reading the
// rotated q from the projection's output and k, v from the cache rows the projection wrote.
//
// Work: one workgroup per (sequence, kv head g, block of 128 query rows), a query row being a
// (token, q head of g's group) pair, row = token * G + head (G = Hq / Hkv), so the group's
// heads share every K/V tile.  Four wavefronts, 32 rows each.
// Per tile of 64 keys (gathered through the slot list):
//   load     K rows and V rows into registers (the next tile's, while this one is computed),
//            then into LDS: K row-major [key][d], V transposed [d][key] (pairs of keys packed
//            into one 32-bit LDS word), both padded against bank conflicts; double-buffered.
//   scores   S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (Q stays in registers for the whole
//            kernel): lane (l32, h) then holds the scores of query row l32 for keys
//            8 (v / 4) + 4 h + v % 4, v = 0..15, of each 32-key half.
//   softmax  online, in base 2 (scores pre-multiplied by scale * log2 e): running row max
//            from the two lanes of a row, rescale of the running sum and of the output.
//   P V      the score registers are already the A operand of O = P V for a permuted key order
//            (16-key step s: keys 16 s + 4 h + 0..3 and 16 s + 8 + 4 h + 0..3); the B operand
//            reads the same keys of V^T as two 8-byte LDS reads.
// Causal windows are per query row; keys past a row's window score -inf.  Slots outside the
// cache read as zero vectors (never out of bounds).  Rows with no visible key are written 0.
#include <algorithm>

#include "lrq_internal.h"

namespace lrq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kD = 128;                 // head size
constexpr int kKT = 64;                 // keys per tile
constexpr int kRowsWG = 128;            // query rows per workgroup
constexpr int kKPitch = kD * 2 + 16;    // bytes per K row in LDS (272)
constexpr int kVPitch = kKT * 2 + 8;    // bytes per V^T row in LDS (136)
constexpr int kKBytes = kKT * kKPitch;  // 17408
constexpr int kVBytes = kD * kVPitch;   // 17408
constexpr int kBufBytes = kKBytes + kVBytes;

struct AttnArgs {
  const uint16_t* q;
  int64_t ld_q;
  const uint16_t* kc;
  const uint16_t* vc;
  int64_t ld_kv;
  int64_t num_slots;
  const int32_t* q_indptr;
  const int32_t* kv_indptr;
  const int32_t* kv_slots;
  uint16_t* out;
  int64_t ld_o;
  int Hq, Hkv, G;
  int max_q_len;  // rows of a sequence past this bound are not computed
  float scale_log2e;
  int causal;
};

__device__ __forceinline__ uint4 load_row16(const uint16_t* base, int64_t ld, int64_t slot, int64_t num_slots,
                                            int off) {
  if (slot < 0 || slot >= num_slots) return uint4{0u, 0u, 0u, 0u};
  return *reinterpret_cast<const uint4*>(base + slot * ld + off);
}

__global__ __launch_bounds__(256, 2) void attn_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * kBufBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, h32 = lane >> 5;
  const int b = blockIdx.x, g = blockIdx.z;
  const int64_t q0 = a.q_indptr[b], q_len = a.q_indptr[b + 1] - q0;
  const int64_t kv0 = a.kv_indptr[b], kv_len = a.kv_indptr[b + 1] - kv0;
  const int64_t n_rows = min(q_len, static_cast<int64_t>(a.max_q_len)) * a.G;
  const int64_t rho0 = static_cast<int64_t>(blockIdx.y) * kRowsWG;
  if (rho0 >= n_rows) return;  // uniform over the workgroup

  // keys the workgroup needs: up to the last row's window
  const int64_t last_row = min(n_rows, rho0 + kRowsWG) - 1;
  const int64_t kv_end = a.causal ? min(kv_len, kv_len - q_len + last_row / a.G + 1) : kv_len;
  const int n_tiles = kv_end > 0 ? static_cast<int>((kv_end + kKT - 1) / kKT) : 0;

  // this lane's query row (as the B operand of S^T and the softmax row)
  const int64_t rw0 = rho0 + wave * 32;  // first row of the wave
  const bool wave_active = rw0 < n_rows;
  const int64_t my_row = rw0 + l32;
  const bool row_ok = my_row < n_rows;
  const int64_t my_tok = row_ok ? my_row / a.G : 0;
  const int my_head = g * a.G + static_cast<int>(row_ok ? my_row % a.G : 0);
  const int64_t my_lim = !row_ok ? -1 : (a.causal ? kv_len - q_len + my_tok : kv_len - 1);
  bf16x8 qf[kD / 16];
  {
    const uint16_t* qr = a.q + (q0 + my_tok) * a.ld_q + static_cast<int64_t>(my_head) * kD + 8 * h32;
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) {
      const uint4 v = row_ok ? *reinterpret_cast<const uint4*>(qr + 16 * ks) : uint4{0u, 0u, 0u, 0u};
      qf[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // ---- tile loads: K rows (tid / 16) + 16 c, chunk tid % 16; V key pairs (tid / 16) + 16 c
  const int chunk = tid & 15, rsub = tid >> 4;
  const int64_t koff = static_cast<int64_t>(g) * kD + chunk * 8;
  // slot numbers are loaded two tiles ahead of their rows, so a tile's row loads never wait for
  // a slot-list load
  uint4 kreg[4], vreg[2][2];
  int32_t kslot[4], vslot[4];
  auto load_slots = [&](int t) {
    const int64_t base = static_cast<int64_t>(t) * kKT;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int64_t key = base + rsub + 16 * c;
      kslot[c] = key < kv_end ? a.kv_slots[kv0 + key] : -1;
    }
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int64_t key = base + 2 * (rsub + 16 * c) + e;
        vslot[2 * c + e] = key < kv_end ? a.kv_slots[kv0 + key] : -1;
      }
  };
  auto load_tile = [&]() {
#pragma unroll
    for (int c = 0; c < 4; ++c) kreg[c] = load_row16(a.kc, a.ld_kv, kslot[c], a.num_slots, static_cast<int>(koff));
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int e = 0; e < 2; ++e)
        vreg[c][e] = load_row16(a.vc, a.ld_kv, vslot[2 * c + e], a.num_slots, static_cast<int>(koff));
  };
  auto store_tile = [&](int buf) {
    unsigned char* kb = smem + buf * kBufBytes;
    unsigned char* vb = kb + kKBytes;
#pragma unroll
    for (int c = 0; c < 4; ++c) *reinterpret_cast<uint4*>(kb + (rsub + 16 * c) * kKPitch + chunk * 16) = kreg[c];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint32_t w0[4] = {vreg[c][0].x, vreg[c][0].y, vreg[c][0].z, vreg[c][0].w};
      const uint32_t w1[4] = {vreg[c][1].x, vreg[c][1].y, vreg[c][1].z, vreg[c][1].w};
      const int pair = rsub + 16 * c;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t lo = (e & 1) ? (w0[e >> 1] >> 16) : (w0[e >> 1] & 0xffffu);
        const uint32_t hi = (e & 1) ? (w1[e >> 1] >> 16) : (w1[e >> 1] & 0xffffu);
        *reinterpret_cast<uint32_t*>(vb + (chunk * 8 + e) * kVPitch + pair * 4) = lo | (hi << 16);
      }
    }
  };

  floatx16 o[kD / 32];
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt) o[dt] = floatx16{};
  float m_run = -INFINITY, l_run = 0.f;

  if (n_tiles > 0) {
    load_slots(0);
    load_tile();
    if (n_tiles > 1) load_slots(1);
    store_tile(0);
  }
  __syncthreads();
  for (int t = 0; t < n_tiles; ++t) {
    if (t + 1 < n_tiles) {
      load_tile();  // rows of tile t + 1 (their slots were loaded an iteration ago)
      if (t + 2 < n_tiles) load_slots(t + 2);
    }
    if (wave_active) {
      const unsigned char* kb = smem + (t & 1) * kBufBytes;
      const unsigned char* vb = kb + kKBytes;
      // ---- S^T = K Q^T for the two 32-key halves
      floatx16 s[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        s[st] = floatx16{};
        const unsigned char* krow = kb + (st * 32 + l32) * kKPitch + h32 * 16;
#pragma unroll
        for (int ks = 0; ks < kD / 16; ++ks) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(krow + ks * 32);
          s[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s[st], 0, 0, 0);
        }
      }
      // ---- scale, mask, running max
      const int64_t kbase = static_cast<int64_t>(t) * kKT + 4 * h32;
      float mloc = -INFINITY;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t key = kbase + st * 32 + (v >> 2) * 8 + (v & 3);
          const float x = key <= my_lim ? s[st][v] * a.scale_log2e : -INFINITY;
          s[st][v] = x;
          mloc = fmaxf(mloc, x);
        }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
      const float m_new = fmaxf(m_run, mloc);
      // rows that have seen no key yet keep m = -inf: scale 1, probabilities 0
      const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      float lsum = 0.f;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = __builtin_amdgcn_exp2f(s[st][v] - m_use);
          s[st][v] = p;
          lsum += p;
        }
      l_run = l_run * alpha + lsum;
      m_run = m_new;
      // ---- rescale O: its rows are 8 (v / 4) + 4 h + v % 4, whose alpha lane l32 = that row holds
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float al = __shfl(alpha, (v >> 2) * 8 + h32 * 4 + (v & 3));
#pragma unroll
        for (int dt = 0; dt < kD / 32; ++dt) o[dt][v] *= al;
      }
      // ---- O += P V over 4 steps of 16 keys
#pragma unroll
      for (int sstep = 0; sstep < kKT / 16; ++sstep) {
        bf16x8 pf;
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[e] = static_cast<__bf16>(s[sstep >> 1][8 * (sstep & 1) + e]);
        const int k0 = 16 * sstep + 4 * h32;
#pragma unroll
        for (int dt = 0; dt < kD / 32; ++dt) {
          const unsigned char* vrow = vb + (dt * 32 + l32) * kVPitch;
          const uint2 lo = *reinterpret_cast<const uint2*>(vrow + k0 * 2);
          const uint2 hi = *reinterpret_cast<const uint2*>(vrow + (k0 + 8) * 2);
          const uint4 vv = uint4{lo.x, lo.y, hi.x, hi.y};
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pf, __builtin_bit_cast(bf16x8, vv), o[dt], 0, 0, 0);
        }
      }
    }
    if (t + 1 < n_tiles) store_tile((t + 1) & 1);
    __syncthreads();
  }

  if (!wave_active) return;
  // ---- normalise and store: O row q' = 8 (v / 4) + 4 h + v % 4 of the wave
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv_l = l_tot > 0.f ? 1.0f / l_tot : 0.f;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int qr = (v >> 2) * 8 + h32 * 4 + (v & 3);
    const float il = __shfl(inv_l, qr);
    const int64_t row = rw0 + qr;
    if (row >= n_rows) continue;
    const int64_t tok = row / a.G;
    const int head = g * a.G + static_cast<int>(row % a.G);
    uint16_t* orow = a.out + (q0 + tok) * a.ld_o + static_cast<int64_t>(head) * kD + l32;
#pragma unroll
    for (int dt = 0; dt < kD / 32; ++dt) orow[dt * 32] = f32_to_bf16_bits(o[dt][v] * il);
  }
}

}  // namespace

bool attn_supports(int head_dim) { return head_dim == kD; }

hipError_t launch_attention(const AttnParams& p, hipStream_t s) {
  if (p.n_seqs == 0 || p.max_q_len == 0) return hipSuccess;
  AttnArgs a{};
  a.q = static_cast<const uint16_t*>(p.q);
  a.ld_q = p.ld_q;
  a.kc = static_cast<const uint16_t*>(p.k_cache);
  a.vc = static_cast<const uint16_t*>(p.v_cache);
  a.ld_kv = static_cast<int64_t>(p.Hkv) * kD;
  a.num_slots = p.num_slots;
  a.q_indptr = p.q_indptr;
  a.kv_indptr = p.kv_indptr;
  a.kv_slots = p.kv_slots;
  a.out = static_cast<uint16_t*>(p.out);
  a.ld_o = static_cast<int64_t>(p.Hq) * kD;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.G = p.Hq / p.Hkv;
  a.max_q_len = p.max_q_len;
  a.scale_log2e = p.scale * 1.4426950408889634f;
  a.causal = p.causal;
  const int64_t mblocks = (static_cast<int64_t>(p.max_q_len) * a.G + kRowsWG - 1) / kRowsWG;
  dim3 grid(static_cast<unsigned>(p.n_seqs), static_cast<unsigned>(mblocks), static_cast<unsigned>(p.Hkv));
  timing_begin(s);
  hipLaunchKernelGGL(attn_kernel, grid, dim3(256), 0, s, a);
  timing_end(s);
  return hipGetLastError();
}

}  // namespace lrq
