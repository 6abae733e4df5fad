// Internal declarations shared by the liblrq translation units (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lrq {

constexpr int kMaxRank = 64;  // LRQ_MAX_LORA_RANK

// Everything a forward launch needs, resolved on the host from lrq_desc.
struct FwdParams {
  int64_t T;        // tokens
  int64_t d;        // model dim
  int Hq, Hkv, D;   // heads and head size
  int N;            // (Hq + 2 Hkv) * D
  int col_k;        // first k column = Hq * D
  int col_v;        // first v column = (Hq + Hkv) * D
  int rot_end;      // columns [0, rot_end) are rotated = col_v
  float eps;
  float scale;      // alpha / r (0 without targets)
  double theta;
  int r;            // LoRA rank (0 without targets)
  uint32_t targets; // bit t set: target t (0 q, 1 k, 2 v) has an adapter
  int has_bias;
  const void* x;
  const void* gamma;
  const void* w;
  const void* bias;
  const void* a[3];
  const void* b[3];
  const int32_t* pos;
  void* out;
  const void* prepared;     // frozen-weight layout of this call's family, or nullptr
  bool use_prepared;        // sizes and launches assume `prepared` (set with it)
  void* ws;
  size_t ws_bytes;
  int esize;                // bytes per element of the call's dtype
  // optional key/value cache destination (kv_slots == nullptr: none)
  void* kv_k;               // [kv_num_slots][Hkv * D]
  void* kv_v;
  const int32_t* kv_slots;  // [T]; slots outside [0, kv_num_slots) are skipped
  int64_t kv_num_slots;
  // LoRA dropout of the adapters' input (dropout.hip); scale above is then alpha / r / (1 - p)
  bool dropout;             // p > 0 with targets
  int drop_nt;              // mask slots = number of targets, in target order
  uint32_t drop_thr;        // floor(p * 2^32): a generator word below it drops its feature
  uint32_t drop_offset;
  uint64_t drop_seed;
  uint32_t* drop_bits_r;        // [drop_nt][T][ceil(d / 32)] keep bits, row-major
  uint16_t* drop_xm;            // [drop_nt][T][d] bf16 x * keep (tiled families), or nullptr
  // QLoRA base: w is an NF4 buffer (codes [N][d / 2], then float32 scales [N][d / 64])
  int nf4;
};

struct BwdParams {
  FwdParams f;      // out unused
  const void* y;
  const void* dy;
  void* dx;
  float* da[3];
  float* db[3];
};

// The LoRA-adapted SwiGLU MLP: y = down(SiLU(gate(h)) * up(h)) (mlp_tiled.hip).
struct MlpParams {
  int64_t T, d, F;        // tokens, model size, intermediate size
  int r;                  // LoRA rank (0 without targets)
  float scale;            // alpha / r
  uint32_t targets;       // bit 0 gate, 1 up, 2 down
  const void* h;          // [T][d]
  const void* wg;         // [F][d]
  const void* wu;         // [F][d]
  const void* wd;         // [d][F]
  const void* a[3];       // gate, up: [r][d]; down: [r][F]
  const void* b[3];       // gate, up: [F][r]; down: [d][r]
  void* out;              // [T][d]
  void* ws;               // a = SiLU(g) * u, [T][F] bf16
  size_t ws_bytes;
};
bool mlp_supports(const MlpParams& p);
size_t mlp_workspace_bytes(const MlpParams& p);
hipError_t launch_mlp(const MlpParams& p, hipStream_t s);

// LoRA dropout (dropout.hip): bytes of the mask region that follows a family's workspace
// (row bits, then the masked inputs if `xm`), and the launch that points p.drop_* into it and
// fills it (unless `fill` is false: the tiled backward fills it from its own rows pass).
// Slot s of the region belongs to the s-th target in q, k, v order.
size_t dropout_region_bytes(const FwdParams& p, bool xm);
hipError_t launch_dropout_masks(FwdParams& p, void* region, bool xm, bool fill, hipStream_t s);
__host__ __device__ inline int target_slot(uint32_t targets, int t) {
  return static_cast<int>((targets & 1u) * (t > 0) + ((targets >> 1) & 1u) * (t > 1));
}

// ---- NF4 weights (QLoRA base): the QLoRA paper's published 4-bit NormalFloat code book,
// blocks of 64 weights along d with a float32 scale each (nf4.hip quantises).
constexpr int kNf4Block = 64;
__host__ __device__ inline size_t nf4_codes_bytes(int64_t n, int64_t d) {
  return (static_cast<size_t>(n) * static_cast<size_t>(d) / 2 + 255) & ~static_cast<size_t>(255);
}
__host__ __device__ inline size_t nf4_buffer_bytes(int64_t n, int64_t d) {
  return nf4_codes_bytes(n, d) + static_cast<size_t>(n) * static_cast<size_t>(d / kNf4Block) * 4;
}
static __device__ __constant__ const float kNf4Levels[16] = {
    -1.0f, -0.6961928009986877f, -0.5250730514526367f, -0.39491748809814453f,
    -0.28444138169288635f, -0.18477343022823334f, -0.09105003625154495f, 0.0f,
    0.07958029955625534f, 0.16093020141124725f, 0.24611230194568634f, 0.33791524171829224f,
    0.44070982933044434f, 0.5626170039176941f, 0.7229568362236023f, 1.0f};

// Read-only view of an NF4 buffer of an [n, d] weight.
struct Nf4View {
  const uint8_t* codes;
  const float* scales;
  int64_t d;
};
__host__ __device__ inline Nf4View nf4_view(const void* buf, int64_t n, int64_t d) {
  const uint8_t* c = static_cast<const uint8_t*>(buf);
  return Nf4View{c, reinterpret_cast<const float*>(c + nf4_codes_bytes(n, d)), d};
}
// Weight (row, k) of the buffer.
__device__ __forceinline__ float nf4_at(const Nf4View& v, int64_t row, int64_t k) {
  const uint32_t byte = v.codes[(row * v.d + k) >> 1];
  const uint32_t code = (k & 1) ? (byte >> 4) : (byte & 15u);
  return kNf4Levels[code] * v.scales[row * (v.d / kNf4Block) + k / kNf4Block];
}
// Weights (row, k .. k + 7) (k % 8 == 0) as float, from 4 code bytes and the block scale;
// `levels` is the code book (in LDS or constant memory).
__device__ __forceinline__ void nf4_at8(const Nf4View& v, int64_t row, int64_t k, const float* levels,
                                        float (&out)[8]) {
  const uint32_t c4 = *reinterpret_cast<const uint32_t*>(v.codes + ((row * v.d + k) >> 1));
  const float sc = v.scales[row * (v.d / kNf4Block) + k / kNf4Block];
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = levels[(c4 >> (4 * e)) & 15u] * sc;
}

hipError_t launch_quantize_nf4(const void* w, bool f32, int64_t n, int64_t d, void* dst, hipStream_t s);

// Attention over the key/value cache (attn.hip).
struct AttnParams {
  const void* q;          // [T_q][ld_q] bf16, q heads in the first Hq * D columns
  int64_t ld_q;
  const void* k_cache;    // [num_slots][Hkv * D] bf16
  const void* v_cache;
  int64_t num_slots;
  const int32_t* q_indptr;   // [n_seqs + 1]
  const int32_t* kv_indptr;  // [n_seqs + 1]
  const int32_t* kv_slots;   // cache rows of each sequence's keys, in token order
  void* out;              // [T_q][Hq * D] bf16
  int n_seqs, max_q_len, Hq, Hkv;
  float scale;
  int causal;
};
bool attn_supports(int head_dim);
hipError_t launch_attention(const AttnParams& p, hipStream_t s);

// Column range [lo, hi) of target t.
__host__ __device__ inline void target_cols(const FwdParams& p, int t, int& lo, int& hi) {
  lo = t == 0 ? 0 : (t == 1 ? p.col_k : p.col_v);
  hi = t == 0 ? p.col_k : (t == 1 ? p.col_v : p.N);
}

// ---- measurement hook: events around the dominant kernel of a call (lrq_api.hip) ----
void timing_begin(hipStream_t s);
void timing_end(hipStream_t s);

// ---- launchers (defined in the kernel translation units) ----
hipError_t launch_kv_scatter(const FwdParams& p, hipStream_t s);
hipError_t launch_fwd_generic_f32(const FwdParams& p, hipStream_t s);
hipError_t launch_fwd_generic_bf16(const FwdParams& p, hipStream_t s);
hipError_t launch_bwd_generic_f32(const BwdParams& p, hipStream_t s);
hipError_t launch_bwd_generic_bf16(const BwdParams& p, hipStream_t s);
bool bwd_generic_supports(const FwdParams& p);

// ---- device helpers ----
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t u) {
  return __uint_as_float(static_cast<uint32_t>(u) << 16);
}
// Round-to-nearest-even float -> bfloat16 (hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
__device__ __forceinline__ float round_bf16(float f) { return bf16_bits_to_f32(f32_to_bf16_bits(f)); }

__device__ __forceinline__ float load_elem(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_elem(const uint16_t* p, int64_t i) { return bf16_bits_to_f32(p[i]); }
__device__ __forceinline__ void store_elem(float* p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void store_elem(uint16_t* p, int64_t i, float v) { p[i] = f32_to_bf16_bits(v); }

// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2,
// 3", SC 2011) on counter x with key (k0, k1): ten rounds, each multiplying words 0 and 2 by
// the two multipliers and mixing the 64-bit products' halves with words 1 and 3 and the key;
// the key is bumped by the two Weyl constants between rounds.  x is replaced by the output.
__device__ __forceinline__ void philox4x32_10(uint32_t (&x)[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = static_cast<uint64_t>(0xD2511F53u) * x[0];
    const uint64_t p1 = static_cast<uint64_t>(0xCD9E8D57u) * x[2];
    const uint32_t n0 = static_cast<uint32_t>(p1 >> 32) ^ x[1] ^ k0;
    const uint32_t n2 = static_cast<uint32_t>(p0 >> 32) ^ x[3] ^ k1;
    x[0] = n0;
    x[1] = static_cast<uint32_t>(p1);
    x[2] = n2;
    x[3] = static_cast<uint32_t>(p0);
  }
}

// LoRA dropout keep bits of features j .. j + 7 (j % 4 == 0) of one token row for target t:
// bit e set iff word (j + e) % 4 of Philox4x32-10 on ((j + e) / 4, row, t, offset) >= thr.
__device__ __forceinline__ uint32_t dropout_byte(int j, uint32_t row, uint32_t t, uint32_t offset, uint32_t thr,
                                                 uint32_t k0, uint32_t k1) {
  uint32_t bits = 0;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    uint32_t x[4] = {static_cast<uint32_t>(j / 4 + q), row, t, offset};
    philox4x32_10(x, k0, k1);
#pragma unroll
    for (int e = 0; e < 4; ++e) bits |= (x[e] >= thr ? 1u : 0u) << (4 * q + e);
  }
  return bits;
}

// x * keep for 8 bf16 values packed in a 16-byte vector (bit e of keep: element e).
__device__ __forceinline__ uint4 mask_bf16x8(uint4 v, uint32_t keep) {
  uint32_t o[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t b2 = keep >> (2 * q);
    o[q] &= ((b2 & 1u) ? 0x0000ffffu : 0u) | ((b2 & 2u) ? 0xffff0000u : 0u);
  }
  return uint4{o[0], o[1], o[2], o[3]};
}

// RoPE frequency omega_i = theta^(-2i/D) in double precision.
__device__ __forceinline__ double rope_omega(double theta, int i, int D) {
  return exp2(-(2.0 * i / D) * log2(theta));
}

// cos/sin of pos * omega.  The angle is formed and reduced to [-pi, pi] in double
// precision, so large positions lose no accuracy before the float32 sincos.
__device__ __forceinline__ void rope_cos_sin(int pos, double omega, float& c, float& s) {
  const double two_pi = 6.283185307179586476925286766559;
  double phi = static_cast<double>(pos) * omega;
  double k = rint(phi * (1.0 / two_pi));
  double red = fma(-k, two_pi, phi);
  sincosf(static_cast<float>(red), &s, &c);
}

}  // namespace lrq
