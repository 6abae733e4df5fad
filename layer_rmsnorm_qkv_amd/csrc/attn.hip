// Attention over the key/value cache (bf16 q, k, v; fp32 scores, softmax and accumulation):
// the step after the projection in the decoder layer of the inference-engine page, reading the
// rotated q from the projection's output and k, v from the cache rows the projection wrote.
//
// Work: one workgroup per (sequence, kv head g, block of 128 query rows), a query row being a
// (token, q head of g's group) pair, row = token * G + head (G = Hq / Hkv), so the group's
// heads share every K/V tile.  Four wavefronts, 32 rows each.  The blocks of one (sequence,
// kv head) pair all land on one XCD (they read the same keys and values through its L2), and
// with a causal mask the blocks with the longest key windows are dispatched first.
// Per tile of 64 keys (gathered through the slot list):
//   load     K and V rows go from global memory straight into LDS (16 bytes per lane,
//            global_load_lds_dwordx4; no registers, no LDS store instructions), through a
//            ring of two stages; each row is 256 bytes with its 16-byte chunks XOR-swizzled
//            by key.  A key past the sequence or a slot outside the cache loads a zero row.
//            Slot numbers are read two tiles ahead of their rows.
//   scores   S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (Q stays in registers for the whole
//            kernel): lane (l32, h) then holds the scores of query row l32 for keys
//            8 (v / 4) + 4 h + v % 4, v = 0..15, of each 32-key half.
//   softmax  online, in base 2: running row max of the raw scores over the row's two lanes
//            (v_permlane32_swap), probabilities exp2(s * scale * log2 e - max * scale * log2 e)
//            (one fma each), rescale of the running sum and (when a row's max moved) of O.
//   P V      computed transposed, O^T += V^T P^T: the score registers are already the B
//            operand for a permuted key order (16-key step s: keys 16 s + 4 h + 0..3 and
//            16 s + 8 + 4 h + 0..3), and the A operand V^T is read from the row-major V tile
//            with the LDS transpose read (ds_read_b64_tr_b16).  Each lane's accumulators then
//            belong to its own query row (head-dim columns 32 dt + 8 j + 4 h + 0..3), so the
//            rescale and the final normalisation need no cross-lane traffic, and each lane
//            stores 8-byte runs of its row.
// Causal windows are per query row; keys past a row's window score -inf.  Rows with no
// visible key are written 0.
#include <algorithm>

#include "lrq_internal.h"
#include "tile_common.h"

namespace lrq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

constexpr int kD = 128;                      // head size
constexpr int kKT = 64;                      // keys per tile
constexpr int kRowsWG = 128;                 // query rows per workgroup
constexpr int kRowBytes = kD * 2;            // one K or V row in LDS: 256 bytes, unpadded
constexpr int kTileBytes = kKT * kRowBytes;  // 16 KB
constexpr int kStageBytes = 2 * kTileBytes;  // K tile, then V tile
constexpr int kPairsPerXcd = 8;
constexpr float kLazyLog2 = 8.f;             // rescale threshold of the running max (exp2 units)              // XCDs: consecutive workgroups go to consecutive XCDs

// The DMA source of keys past the sequence and of slots outside the cache.
__device__ __attribute__((aligned(256))) uint16_t g_zero_row[kD] = {};

// XOR of the 16-byte chunk index of V row `key` (by key % 4: 0, 10, 4, 14).  A transpose read
// takes four consecutive keys at two adjacent chunks in each 16-lane group and four keys at four
// adjacent chunks in each 32 lanes: these masks send both sets to distinct bank groups of a
// 128-byte and of a 256-byte window.  K rows use key % 16 (16 consecutive keys at one chunk).
__device__ __forceinline__ int v_xor(int key) { return ((key & 1) ? 10 : 0) ^ ((key & 2) ? 4 : 0); }

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
  int Hkv, G;
  int pairs, pairs8;  // (sequence, kv head) pairs, rounded up to a multiple of 8
  int mblocks;        // 128-row blocks per sequence
  int max_q_len;      // rows of a sequence past this bound are not computed
  float scale_log2e;
  int causal;
};

__device__ __forceinline__ float pair_max(float x) {
  // max of x over lanes l and l ^ 32
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__global__ __launch_bounds__(256, 2) void attn_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * kStageBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, h32 = lane >> 5;
  // block -> (pair, row block): ids m * pairs8 + pair, so a pair's blocks share id % 8 (one XCD)
  const int m_ord = static_cast<int>(blockIdx.x) / a.pairs8;
  const int pair = static_cast<int>(blockIdx.x) - m_ord * a.pairs8;
  if (pair >= a.pairs) return;
  const int b = pair / a.Hkv, g = pair - b * a.Hkv;
  const int mblk = a.causal ? a.mblocks - 1 - m_ord : m_ord;  // longest windows first
  const int64_t q0 = a.q_indptr[b];
  const int q_len = a.q_indptr[b + 1] - static_cast<int>(q0);
  const int64_t kv0 = a.kv_indptr[b];
  const int kv_len = a.kv_indptr[b + 1] - static_cast<int>(kv0);
  const int n_rows = min(q_len, a.max_q_len) * a.G;
  const int rho0 = mblk * kRowsWG;
  if (rho0 >= n_rows) return;  // uniform over the workgroup

  // keys the workgroup needs: up to the last row's window
  const int last_row = min(n_rows, rho0 + kRowsWG) - 1;
  const int kv_end = a.causal ? min(kv_len, kv_len - q_len + last_row / a.G + 1) : kv_len;
  const int n_tiles = kv_end > 0 ? (kv_end + kKT - 1) / kKT : 0;

  // this lane's query row (the B operand of S^T, the softmax row and the output row)
  const int rw0 = rho0 + wave * 32;  // first row of the wave
  const bool wave_active = rw0 < n_rows;
  const int my_row = rw0 + l32;
  const bool row_ok = my_row < n_rows;
  const int my_tok = row_ok ? my_row / a.G : 0;
  const int my_head = g * a.G + (row_ok ? my_row - my_tok * a.G : 0);
  const int my_lim = !row_ok ? -1 : (a.causal ? kv_len - q_len + my_tok : kv_len - 1);
  // smallest window end of the wave's rows (-1 when some row is past the sequence)
  const int wave_min_lim = rw0 + 31 < n_rows ? (a.causal ? kv_len - q_len + rw0 / a.G : kv_len - 1) : -1;
  // ---- DMA: instruction c of wave w fills keys 16 w + 4 c .. + 3 of the tile (1 KB); lane
  // `lane` takes LDS chunk position lane % 16 of key 16 w + 4 c + lane / 16, whose source is
  // the logical chunk position ^ (key % 16) of K and position ^ v_xor(key) of V.
  const int kq = lane >> 4, pos = lane & 15;
  int kchunk[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) kchunk[c] = pos ^ (4 * c + kq);
  const int vchunk = pos ^ v_xor(kq);
  const char* kc_g = reinterpret_cast<const char*>(a.kc + static_cast<int64_t>(g) * kD);
  const char* vc_g = reinterpret_cast<const char*>(a.vc + static_cast<int64_t>(g) * kD);
  const uint32_t row_bytes = static_cast<uint32_t>(a.ld_kv) * 2u;
  // the zero row's address, kept in scalar registers (not reloaded in the loop)
  const char* zrow = reinterpret_cast<const char*>(g_zero_row);
  asm volatile("" : "+s"(zrow));
  const uint32_t lds0 = tile::lds_addr(smem) + static_cast<uint32_t>(wave) * 4096u;
  // Slot numbers of the next tile to load, as read from the list: they are checked only where
  // the DMA uses them (an iteration later), so no wave waits for the slot-list loads.
  int32_t sl[4];
  int sl_tile = 0;  // the tile sl belongs to
  auto load_slots = [&](int t) {
#pragma unroll
    for (int c = 0; c < 4; ++c) sl[c] = a.kv_slots[kv0 + min(t * kKT + 16 * wave + 4 * c + kq, kv_end - 1)];
    sl_tile = t;
  };
  auto issue_dma = [&](int buf) {
    const uint32_t dst = lds0 + static_cast<uint32_t>(buf * kStageBytes);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int key = sl_tile * kKT + 16 * wave + 4 * c + kq;
      const bool ok = key < kv_end && sl[c] >= 0 && sl[c] < a.num_slots;  // else a zero row
      // one 32 x 32 -> 64-bit multiply (sl[c] >= 0 wherever the row is used), in bytes
      const uint64_t row = static_cast<uint64_t>(static_cast<uint32_t>(sl[c])) * row_bytes;
      const char* ks = ok ? kc_g + row + 16 * kchunk[c] : zrow + 16 * kchunk[c];
      const char* vs = ok ? vc_g + row + 16 * vchunk : zrow + 16 * vchunk;
      tile::dma16(ks, dst + c * 1024);
      tile::dma16(vs, dst + kTileBytes + c * 1024);
    }
  };

  // ---- LDS read offsets of this lane
  // K (A operand of S^T): key 32 st + l32, logical chunk 2 ks + h32 at position ^ (l32 % 16)
  const int k_row_off = l32 * kRowBytes;
  const int k_xor = (l32 & 15) ^ h32;  // (2 ks + h32) ^ (l32 % 16) = 2 ks ^ k_xor
  // V (A operand of O^T, transpose read): in 16-lane group q = lane / 16, lane j reads the
  // 8 bytes of key 4 (q / 2) + j / 4 (+ 16 s + 8 half) at head-dim columns 32 dt + 16 (q % 2)
  // + 4 (j % 4) .. + 3; the read hands lane j of the group that key's column 32 dt + 16 (q % 2)
  // + j for each of the four keys.
  int v_off[kD / 32];
  {
    const int q = lane >> 4, j = lane & 15;
    const int key = 4 * (q >> 1) + (j >> 2);
#pragma unroll
    for (int dt = 0; dt < kD / 32; ++dt) {
      const int chunk = 4 * dt + 2 * (q & 1) + ((j & 3) >> 1);
      v_off[dt] = key * kRowBytes + ((chunk ^ v_xor(key)) << 4) + 8 * (j & 1);
    }
  }

  floatx16 o[kD / 32];
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt) o[dt] = floatx16{};
  float m_run = -INFINITY;
  // row sums: every entry of lane (l32, h) accumulates row l32's sum; entry 0 is kept scaled
  floatx16 lsum = floatx16{};
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = static_cast<__bf16>(1.0f);

  // ---- Q rows and output rows: lane `lane` moves 16-byte chunk lane % 16 of the wave's rows
  // 4 c + lane / 16, c = 0..7 (four whole 256-byte rows per instruction)
  auto row_off = [&](int c, int64_t ld) -> int64_t {  // -1: row past the sequence's rows
    const int rho = rw0 + 4 * c + kq;
    if (rho >= n_rows) return -1;
    const int tok = rho / a.G;
    return (q0 + tok) * ld + static_cast<int64_t>(g * a.G + rho - tok * a.G) * kD;
  };
  bf16x8 qf[kD / 16];
  if (n_tiles > 0) {
    load_slots(0);
    {
      // Q rows of the wave into stage 1 (row r of the workgroup at r * 256, chunks XOR r % 16)
      const uint32_t dst = tile::lds_addr(smem) + kStageBytes + static_cast<uint32_t>(wave) * 8192u;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int chunk = pos ^ ((4 * c + kq) & 15);
        const int64_t off = row_off(c, a.ld_q);
        tile::dma16(off >= 0 ? reinterpret_cast<const char*>(a.q + off) + 16 * chunk : zrow + 16 * chunk, dst + c * 1024);
      }
    }
    issue_dma(0);
    if (n_tiles > 1) load_slots(1);
    tile::wait_barrier<0>();
    const unsigned char* qrow = smem + kStageBytes + (32 * wave + l32) * kRowBytes;
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + ((2 * ks ^ k_xor) << 4));
  }
  for (int t = 0; t < n_tiles; ++t) {
    // tile t is in LDS (every wave's loads), and every wave is done with tile t - 1
    tile::wait_barrier<0>();
    auto next_tile = [&]() {
      if (t + 1 < n_tiles) {
        issue_dma((t + 1) & 1);  // slots of tile t + 1 were read an iteration ago
        if (t + 2 < n_tiles) load_slots(t + 2);
      }
    };
    if (!wave_active) {
      next_tile();
      continue;
    }
    const unsigned char* kb = smem + (t & 1) * kStageBytes;
    const unsigned char* vb = kb + kTileBytes;
    // ---- S^T = K Q^T for the two 32-key halves (their accumulation chains interleaved), the K
    // fragments read two steps ahead of their MFMAs; the next tile's loads are issued after the
    // first steps, while the matrix cores work
    floatx16 s[2] = {floatx16{}, floatx16{}};
    auto kread = [&](int ks, int st) {
      return *reinterpret_cast<const bf16x8*>(kb + st * 32 * kRowBytes + k_row_off + ((2 * ks ^ k_xor) << 4));
    };
    bf16x8 kfr[3][2];
    kfr[0][0] = kread(0, 0);
    kfr[0][1] = kread(0, 1);
    kfr[1][0] = kread(1, 0);
    kfr[1][1] = kread(1, 1);
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) {
      if (ks + 2 < kD / 16) {
        kfr[(ks + 2) % 3][0] = kread(ks + 2, 0);
        kfr[(ks + 2) % 3][1] = kread(ks + 2, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
      s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfr[ks % 3][0], qf[ks], s[0], 0, 0, 0);
      s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfr[ks % 3][1], qf[ks], s[1], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (ks == 1) {
        next_tile();
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // ---- mask: only a tile that reaches past some row's window (wave-uniform test); the lane's
    // keys sit at 4 h + (compile-time offsets) within the tile
    const int t0 = t * kKT;
    if (t0 + kKT - 1 > wave_min_lim) {
      const int lim = max(min(my_lim - t0, kKT), -1) - 4 * h32;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int v = 0; v < 16; ++v) s[st][v] = st * 32 + (v >> 2) * 8 + (v & 3) > lim ? -INFINITY : s[st][v];
    }
    // ---- reference max on the raw scores (the scale is positive), probabilities in base 2.
    // The reference moves only when the row's max exceeds it by more than kLazyLog2 (in exp2
    // units), so most tiles rescale nothing; probabilities stay below 2^kLazyLog2.
    float mloc = -INFINITY;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int v = 0; v < 16; ++v) mloc = fmaxf(mloc, s[st][v]);
    const float m_tile = pair_max(mloc);
    // a row that has seen no key keeps m = -inf (scale 1, probabilities 0); -inf - -inf is NaN
    const bool grow = (m_tile - m_run) * a.scale_log2e > kLazyLog2;
    const float m_new = grow ? m_tile : m_run;
    const float alpha = grow ? __builtin_amdgcn_exp2f((m_run - m_new) * a.scale_log2e) : 1.f;
    const float mc = m_new == -INFINITY ? 0.f : m_new * a.scale_log2e;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int v = 0; v < 16; ++v) s[st][v] = __builtin_amdgcn_exp2f(fmaf(s[st][v], a.scale_log2e, -mc));
    m_run = m_new;
    if (!__all(alpha == 1.f)) {
#pragma unroll
      for (int dt = 0; dt < kD / 32; ++dt) o[dt] *= alpha;
      lsum[0] *= alpha;
    }
    // ---- O^T += V^T P^T over 4 steps of 16 keys; the row sums of the (bf16) probabilities come
    // from the same product with an all-ones A operand
#pragma unroll
    for (int sstep = 0; sstep < kKT / 16; ++sstep) {
      bf16x8 pf;
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[e] = static_cast<__bf16>(s[sstep >> 1][8 * (sstep & 1) + e]);
#pragma unroll
      for (int dt = 0; dt < kD / 32; ++dt) {
        const unsigned char* vp = vb + v_off[dt] + 16 * sstep * kRowBytes;
        const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(vp));
        const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(vp + 8 * kRowBytes));
        const shortx4 vv[2] = {lo, hi};
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv), pf, o[dt], 0, 0, 0);
      }
      lsum = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones, pf, lsum, 0, 0, 0);
    }
  }

  if (!wave_active) return;
  // ---- normalise, stage the wave's 32 x 128 output block in LDS (a stage no wave reads any
  // more: the one tile n_tiles - 1 did not use), then store whole rows
  const float l_tot = lsum[0];
  const float inv_l = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  unsigned char* ob = smem + (n_tiles & 1) * kStageBytes + wave * 8192;
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x4 r;
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = static_cast<__bf16>(o[dt][4 * j + e] * inv_l);
      *reinterpret_cast<bf16x4*>(ob + l32 * kRowBytes + (((4 * dt + j) ^ (l32 & 15)) << 4) + 8 * h32) = r;
    }
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wave's LDS writes are done
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int rr = 4 * c + kq;
    const uint4 v = *reinterpret_cast<const uint4*>(ob + rr * kRowBytes + ((pos ^ (rr & 15)) << 4));
    const int64_t off = row_off(c, a.ld_o);
    if (off >= 0) *reinterpret_cast<uint4*>(a.out + off + 8 * pos) = v;
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
  a.Hkv = p.Hkv;
  a.G = p.Hq / p.Hkv;
  a.pairs = p.n_seqs * p.Hkv;
  a.pairs8 = (a.pairs + kPairsPerXcd - 1) / kPairsPerXcd * kPairsPerXcd;
  a.mblocks = static_cast<int>((static_cast<int64_t>(p.max_q_len) * a.G + kRowsWG - 1) / kRowsWG);
  a.max_q_len = p.max_q_len;
  a.scale_log2e = p.scale * 1.4426950408889634f;
  a.causal = p.causal;
  const int64_t blocks = static_cast<int64_t>(a.mblocks) * a.pairs8;
  timing_begin(s);
  hipLaunchKernelGGL(attn_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, a);
  timing_end(s);
  return hipGetLastError();
}

}  // namespace lrq
