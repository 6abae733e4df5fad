// liblrq C ABI: host-side validation, kernel-family selection and launch.
// Every check happens before anything is enqueued; see include/lrq.h for the contract.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "lrq.h"
#include "lrq_internal.h"

namespace lrq {
bool bwd_generic_supports(const FwdParams& p);
bool tiled_supports(const FwdParams& p);
bool decode_supports(const FwdParams& p);
bool bwd_tiled_supports(const FwdParams& p);
size_t tiled_workspace_bytes(const FwdParams& p);
size_t decode_workspace_bytes(const FwdParams& p);
size_t bwd_tiled_workspace_bytes(const FwdParams& p);
size_t tiled_prepared_bytes(const FwdParams& p);
size_t bwd_tiled_prepared_bytes(const FwdParams& p);
hipError_t prepare_fwd_tiled(const FwdParams& p, void* dst, hipStream_t s);
hipError_t prepare_bwd_tiled(const FwdParams& p, void* dst, hipStream_t s);
hipError_t launch_fwd_tiled(const FwdParams& p, hipStream_t s);
hipError_t launch_fwd_decode(const FwdParams& p, hipStream_t s);
hipError_t launch_bwd_tiled(const BwdParams& p, hipStream_t s);
}  // namespace lrq

namespace {

// Measurement hook state (process-wide; the hook is meant for a single benchmarking thread).
struct Timing {
  bool on = false;
  int kind = 0;                   // 0: the current call is a forward, 1: a backward
  std::vector<hipEvent_t> ev[2];  // start, stop pairs; created on demand, kept until exit
  size_t used[2] = {0, 0};        // pairs recorded since the hook was (re)enabled
  bool open = false;              // a start was recorded and its stop is due
};
Timing g_timing;
constexpr size_t kMaxTimedCalls = 4096;

}  // namespace

namespace lrq {

void timing_begin(hipStream_t s) {
  Timing& t = g_timing;
  if (!t.on || t.used[t.kind] >= kMaxTimedCalls) return;
  std::vector<hipEvent_t>& v = t.ev[t.kind];
  const size_t u = t.used[t.kind];
  while (v.size() < 2 * (u + 1)) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return;
    v.push_back(e);
  }
  t.open = hipEventRecord(v[2 * u], s) == hipSuccess;
}

void timing_end(hipStream_t s) {
  Timing& t = g_timing;
  if (!t.on || !t.open) return;
  t.open = false;
  const size_t u = t.used[t.kind];
  if (hipEventRecord(t.ev[t.kind][2 * u + 1], s) == hipSuccess) ++t.used[t.kind];
}

}  // namespace lrq

// ---- the no-allocation entry point's scratch (lrq_forward_noalloc)
// One array per GPU, part of the library's device code object: it exists on every device the
// library is loaded on and lives until the process ends.  Host code never uses its name as an
// address; it uses the device address that hipGetSymbolAddress returns for the current device.
constexpr size_t kScratchBytes = size_t{16} << 20;  // LRQ_NOALLOC_SCRATCH_BYTES
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per device.
hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

namespace {

thread_local char g_err[512] = "";

lrq_status fail(lrq_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

lrq_status ok() {
  g_err[0] = '\0';
  return LRQ_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

// Largest token count sent to the decode family when the choice is automatic.
constexpr int64_t kDecodeMaxTokens = 256;

// Checks the descriptor and fills the shape part of FwdParams.
lrq_status check_desc(const lrq_desc* d, lrq::FwdParams& p) {
  if (!d) return fail(LRQ_ERR_INVALID_ARG, "desc is NULL");
  if (d->n_tokens < 0) return fail(LRQ_ERR_INVALID_ARG, "n_tokens < 0");
  if (d->d_model < 1) return fail(LRQ_ERR_INVALID_ARG, "d_model < 1");
  if (d->n_q_heads < 1 || d->n_kv_heads < 1) return fail(LRQ_ERR_INVALID_ARG, "head counts must be >= 1");
  if (d->n_q_heads % d->n_kv_heads != 0) return fail(LRQ_ERR_INVALID_ARG, "n_q_heads %% n_kv_heads != 0");
  if (d->head_dim < 2 || (d->head_dim & 1)) return fail(LRQ_ERR_INVALID_ARG, "head_dim must be even and >= 2");
  if (d->dtype != LRQ_F32 && d->dtype != LRQ_BF16) return fail(LRQ_ERR_INVALID_ARG, "unknown dtype %d", d->dtype);
  if (!std::isfinite(d->eps) || d->eps < 0.f) return fail(LRQ_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (!std::isfinite(d->rope_theta) || d->rope_theta <= 0.f)
    return fail(LRQ_ERR_INVALID_ARG, "rope_theta must be finite and > 0");
  if (d->lora_targets & ~7u) return fail(LRQ_ERR_INVALID_ARG, "lora_targets has unknown bits");
  if (d->lora_targets) {
    if (d->lora_rank < 1) return fail(LRQ_ERR_INVALID_ARG, "lora_rank < 1 with targets set");
    if (!std::isfinite(d->lora_alpha)) return fail(LRQ_ERR_INVALID_ARG, "lora_alpha not finite");
  }
  if (d->has_bias != 0 && d->has_bias != 1) return fail(LRQ_ERR_INVALID_ARG, "has_bias must be 0 or 1");
  if (d->variant < LRQ_VARIANT_AUTO || d->variant > LRQ_VARIANT_DECODE)
    return fail(LRQ_ERR_INVALID_ARG, "unknown variant %d", d->variant);
  const int64_t N = static_cast<int64_t>(d->n_q_heads + 2 * d->n_kv_heads) * d->head_dim;
  if (N > (1 << 24) || d->d_model > (1 << 24) || d->n_tokens > (int64_t{1} << 31) - 1)
    return fail(LRQ_ERR_UNSUPPORTED, "sizes beyond the supported range");
  if (!std::isfinite(d->lora_dropout) || d->lora_dropout < 0.f || d->lora_dropout >= 1.f)
    return fail(LRQ_ERR_INVALID_ARG, "lora_dropout must be finite and in [0, 1)");
  if (d->weight_format != LRQ_WEIGHT_DENSE && d->weight_format != LRQ_WEIGHT_NF4)
    return fail(LRQ_ERR_INVALID_ARG, "unknown weight_format %d", d->weight_format);
  if (d->weight_format == LRQ_WEIGHT_NF4 && d->d_model % lrq::kNf4Block != 0)
    return fail(LRQ_ERR_UNSUPPORTED, "NF4 weights need d_model %% 64 == 0");
  if (d->lora_targets && d->lora_rank > LRQ_MAX_LORA_RANK)
    return fail(LRQ_ERR_UNSUPPORTED, "lora_rank %d > %d", d->lora_rank, LRQ_MAX_LORA_RANK);

  std::memset(&p, 0, sizeof p);
  p.T = d->n_tokens;
  p.d = d->d_model;
  p.Hq = d->n_q_heads;
  p.Hkv = d->n_kv_heads;
  p.D = d->head_dim;
  p.N = static_cast<int>(N);
  p.col_k = d->n_q_heads * d->head_dim;
  p.col_v = (d->n_q_heads + d->n_kv_heads) * d->head_dim;
  p.rot_end = p.col_v;
  p.eps = d->eps;
  p.theta = static_cast<double>(d->rope_theta);
  p.targets = d->lora_targets;
  p.r = d->lora_targets ? d->lora_rank : 0;
  p.scale = d->lora_targets ? d->lora_alpha / static_cast<float>(d->lora_rank) : 0.f;
  p.has_bias = d->has_bias;
  p.esize = d->dtype == LRQ_F32 ? 4 : 2;
  p.nf4 = d->weight_format == LRQ_WEIGHT_NF4;
  p.dropout = d->lora_targets != 0 && d->lora_dropout > 0.f;
  if (p.dropout) {
    // inverted dropout: the kept features' 1 / (1 - p) joins the adapter scale
    p.scale = d->lora_alpha / static_cast<float>(d->lora_rank) / (1.f - d->lora_dropout);
    p.drop_nt = __builtin_popcount(d->lora_targets);
    p.drop_thr = static_cast<uint32_t>(std::floor(static_cast<double>(d->lora_dropout) * 4294967296.0));
    p.drop_offset = d->dropout_offset;
    p.drop_seed = d->dropout_seed;
  }
  return LRQ_OK;
}

// Kernel family for a valid descriptor, or -1 (message set) if the forced one cannot run.
int select(const lrq_desc* d, const lrq::FwdParams& p, bool backward) {
  if (backward) {
    const bool tiled = d->dtype == LRQ_BF16 && lrq::bwd_tiled_supports(p);
    if (d->variant == LRQ_VARIANT_AUTO) {
      if (tiled) return LRQ_VARIANT_TILED;
      if (lrq::bwd_generic_supports(p)) return LRQ_VARIANT_GENERIC;
      fail(LRQ_ERR_UNSUPPORTED, "no backward kernel covers this shape");
      return -1;
    }
    if (d->variant == LRQ_VARIANT_GENERIC && lrq::bwd_generic_supports(p)) return LRQ_VARIANT_GENERIC;
    if (d->variant == LRQ_VARIANT_TILED && tiled) return LRQ_VARIANT_TILED;
    fail(LRQ_ERR_UNSUPPORTED, "backward variant %d cannot run this shape", d->variant);
    return -1;
  }
  const bool bf16 = d->dtype == LRQ_BF16;
  const bool tiled = bf16 && lrq::tiled_supports(p);
  const bool decode = bf16 && !p.dropout && lrq::decode_supports(p);
  switch (d->variant) {
    case LRQ_VARIANT_AUTO:
      if (decode && p.T <= kDecodeMaxTokens) return LRQ_VARIANT_DECODE;
      if (tiled) return LRQ_VARIANT_TILED;
      return LRQ_VARIANT_GENERIC;
    case LRQ_VARIANT_GENERIC:
      return LRQ_VARIANT_GENERIC;
    case LRQ_VARIANT_TILED:
      if (tiled) return LRQ_VARIANT_TILED;
      break;
    case LRQ_VARIANT_DECODE:
      if (decode) return LRQ_VARIANT_DECODE;
      break;
  }
  fail(LRQ_ERR_UNSUPPORTED, "forward variant %d cannot run this shape", d->variant);
  return -1;
}

// Prepared-weight buffer: the tiled forward's W' first (when that family covers the shape),
// then, for a backward preparation, the tiled backward's W^T.  Independent of T.
struct PrepLayout {
  size_t fwd_off, fwd_bytes, bwd_off, bwd_bytes, total;
};

PrepLayout prep_layout(const lrq_desc* d, const lrq::FwdParams& p, bool for_backward) {
  PrepLayout L{};
  if (d->dtype != LRQ_BF16) return L;
  lrq::FwdParams q = p;
  q.T = 0;
  if (lrq::tiled_supports(q)) L.fwd_bytes = lrq::tiled_prepared_bytes(q);
  L.bwd_off = L.fwd_bytes;
  if (for_backward && lrq::bwd_tiled_supports(q)) L.bwd_bytes = lrq::bwd_tiled_prepared_bytes(q);
  L.total = L.bwd_off + L.bwd_bytes;
  return L;
}

size_t family_workspace(int variant, const lrq::FwdParams& p, bool backward) {
  if (backward) return variant == LRQ_VARIANT_TILED ? lrq::bwd_tiled_workspace_bytes(p) : 0;
  if (variant == LRQ_VARIANT_TILED) return lrq::tiled_workspace_bytes(p);
  if (variant == LRQ_VARIANT_DECODE) return lrq::decode_workspace_bytes(p);
  return 0;
}

size_t al256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

// The family's own workspace, then (with LoRA dropout) the mask region: keep bits, and for the
// tiled families the masked adapter inputs too.
size_t workspace_for(int variant, const lrq::FwdParams& p, bool backward) {
  const size_t base = family_workspace(variant, p, backward);
  if (!p.dropout) return base;
  return al256(base) + lrq::dropout_region_bytes(p, variant == LRQ_VARIANT_TILED);
}

// Points p's dropout fields into the region and fills it, except for the tiled backward, whose
// rows pass makes the masks itself.
hipError_t launch_dropout(int variant, lrq::FwdParams& p, bool backward, hipStream_t s) {
  if (!p.dropout) return hipSuccess;
  const bool tiled = variant == LRQ_VARIANT_TILED;
  void* region = static_cast<unsigned char*>(p.ws) + al256(family_workspace(variant, p, backward));
  return lrq::launch_dropout_masks(p, region, tiled, !(tiled && backward), s);
}

lrq_status check_common_ptrs(const lrq_desc* d, lrq::FwdParams& p, const void* x, const void* gamma,
                             const void* w, const void* bias, const void* const* a, const void* const* b,
                             const int32_t* pos) {
  if (p.T > 0 && (!x || !gamma || !w || !pos)) return fail(LRQ_ERR_INVALID_ARG, "x, gamma, w_qkv and positions are required");
  if (d->has_bias && !bias) return fail(LRQ_ERR_INVALID_ARG, "bias is NULL with has_bias");
  if (d->lora_targets && (!a || !b)) return fail(LRQ_ERR_INVALID_ARG, "lora_a / lora_b arrays are NULL");
  for (int t = 0; t < 3; ++t)
    if ((d->lora_targets & (1u << t)) && (!a[t] || !b[t]))
      return fail(LRQ_ERR_INVALID_ARG, "lora_a[%d] / lora_b[%d] is NULL for a target", t, t);
  const void* all[] = {x, gamma, w, d->has_bias ? bias : nullptr, pos};
  for (const void* q : all)
    if (q && !aligned16(q)) return fail(LRQ_ERR_UNSUPPORTED, "array pointers must be 16-byte aligned");
  p.x = x;
  p.gamma = gamma;
  p.w = w;
  p.bias = d->has_bias ? bias : nullptr;
  p.pos = pos;
  for (int t = 0; t < 3; ++t) {
    if (!(d->lora_targets & (1u << t))) continue;
    if (!aligned16(a[t]) || !aligned16(b[t])) return fail(LRQ_ERR_UNSUPPORTED, "LoRA pointers must be 16-byte aligned");
    p.a[t] = a[t];
    p.b[t] = b[t];
  }
  return LRQ_OK;
}

lrq_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(LRQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int lrq_abi_version(void) { return LRQ_ABI_VERSION; }

lrq_status lrq_attention(const lrq_attn_desc* d, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* q_indptr, const int32_t* kv_indptr, const int32_t* kv_slots, void* out,
                         void* stream) {
  if (!d) return fail(LRQ_ERR_INVALID_ARG, "desc is NULL");
  if (d->n_seqs < 0 || d->max_q_len < 0 || d->num_slots < 0)
    return fail(LRQ_ERR_INVALID_ARG, "n_seqs, max_q_len and num_slots must be >= 0");
  if (d->n_q_heads < 1 || d->n_kv_heads < 1 || d->n_q_heads % d->n_kv_heads != 0)
    return fail(LRQ_ERR_INVALID_ARG, "head counts must be >= 1 with n_q_heads %% n_kv_heads == 0");
  if (d->head_dim < 1) return fail(LRQ_ERR_INVALID_ARG, "head_dim < 1");
  if (d->ld_q < static_cast<int64_t>(d->n_q_heads) * d->head_dim)
    return fail(LRQ_ERR_INVALID_ARG, "ld_q < n_q_heads * head_dim");
  if (!std::isfinite(d->scale) || d->scale < 0.f) return fail(LRQ_ERR_INVALID_ARG, "scale must be finite and >= 0");
  if (d->causal != 0 && d->causal != 1) return fail(LRQ_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (d->dtype != LRQ_BF16) return fail(LRQ_ERR_UNSUPPORTED, "attention runs in bf16 only");
  if (!lrq::attn_supports(d->head_dim)) return fail(LRQ_ERR_UNSUPPORTED, "head_dim %d not supported", d->head_dim);
  if (d->ld_q % 8 != 0) return fail(LRQ_ERR_UNSUPPORTED, "ld_q must be a multiple of 8");
  const int64_t group = d->n_q_heads / d->n_kv_heads;
  if ((static_cast<int64_t>(d->max_q_len) * group + 127) / 128 > 65535)
    return fail(LRQ_ERR_UNSUPPORTED, "too many query rows per sequence");
  if (d->n_seqs == 0 || d->max_q_len == 0) return ok();
  if (!q || !k_cache || !v_cache || !q_indptr || !kv_indptr || !kv_slots || !out)
    return fail(LRQ_ERR_INVALID_ARG, "q, caches, index arrays and out are required");
  for (const void* p : {q, k_cache, v_cache, static_cast<const void*>(out)})
    if (!aligned16(p)) return fail(LRQ_ERR_UNSUPPORTED, "q, caches and out must be 16-byte aligned");
  for (const void* p : {static_cast<const void*>(q_indptr), static_cast<const void*>(kv_indptr),
                        static_cast<const void*>(kv_slots)})
    if (reinterpret_cast<uintptr_t>(p) & 3u) return fail(LRQ_ERR_UNSUPPORTED, "index arrays must be 4-byte aligned");
  lrq::AttnParams p{};
  p.q = q;
  p.ld_q = d->ld_q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.num_slots = d->num_slots;
  p.q_indptr = q_indptr;
  p.kv_indptr = kv_indptr;
  p.kv_slots = kv_slots;
  p.out = out;
  p.n_seqs = d->n_seqs;
  p.max_q_len = d->max_q_len;
  p.Hq = d->n_q_heads;
  p.Hkv = d->n_kv_heads;
  p.scale = d->scale > 0.f ? d->scale : 1.0f / std::sqrt(static_cast<float>(d->head_dim));
  p.causal = d->causal;
  g_timing.kind = 0;  // timed with the forward-direction calls
  return hip_status(lrq::launch_attention(p, static_cast<hipStream_t>(stream)), "attention launch");
}

size_t lrq_nf4_weight_size(const lrq_desc* desc) {
  lrq::FwdParams p;
  if (check_desc(desc, p) != LRQ_OK || p.d % lrq::kNf4Block != 0) return 0;
  return lrq::nf4_buffer_bytes(p.N, p.d);
}

lrq_status lrq_quantize_nf4(const lrq_desc* desc, const void* w_qkv, void* w_nf4, size_t nf4_bytes, void* stream) {
  lrq::FwdParams p;
  lrq_status st = check_desc(desc, p);
  if (st != LRQ_OK) return st;
  if (p.d % lrq::kNf4Block != 0) return fail(LRQ_ERR_UNSUPPORTED, "NF4 weights need d_model %% 64 == 0");
  if (!w_qkv || !w_nf4) return fail(LRQ_ERR_INVALID_ARG, "w_qkv and w_nf4 are required");
  const size_t need = lrq::nf4_buffer_bytes(p.N, p.d);
  if (nf4_bytes < need) return fail(LRQ_ERR_INVALID_ARG, "NF4 buffer too small: %zu < %zu", nf4_bytes, need);
  if (!aligned16(w_qkv) || !aligned16(w_nf4)) return fail(LRQ_ERR_UNSUPPORTED, "pointers must be 16-byte aligned");
  return hip_status(lrq::launch_quantize_nf4(w_qkv, desc->dtype == LRQ_F32, p.N, p.d, w_nf4,
                                             static_cast<hipStream_t>(stream)),
                    "NF4 quantisation");
}

const char* lrq_status_string(lrq_status s) {
  switch (s) {
    case LRQ_OK: return "LRQ_OK";
    case LRQ_ERR_INVALID_ARG: return "LRQ_ERR_INVALID_ARG";
    case LRQ_ERR_UNSUPPORTED: return "LRQ_ERR_UNSUPPORTED";
    case LRQ_ERR_HIP: return "LRQ_ERR_HIP";
  }
  return "LRQ_UNKNOWN_STATUS";
}

const char* lrq_last_error(void) { return g_err; }

int lrq_select_variant(const lrq_desc* desc, int for_backward) {
  lrq::FwdParams p;
  if (check_desc(desc, p) != LRQ_OK) return -1;
  return select(desc, p, for_backward != 0);
}

size_t lrq_workspace_size(const lrq_desc* desc, int for_backward) {
  lrq::FwdParams p;
  if (check_desc(desc, p) != LRQ_OK) return 0;
  const int v = select(desc, p, for_backward != 0);
  if (v < 0) return 0;
  return workspace_for(v, p, for_backward != 0);
}

size_t lrq_prepared_size(const lrq_desc* desc, int for_backward) {
  lrq::FwdParams p;
  if (check_desc(desc, p) != LRQ_OK) return 0;
  return prep_layout(desc, p, for_backward != 0).total;
}

size_t lrq_workspace_size_prepared(const lrq_desc* desc, int for_backward) {
  lrq::FwdParams p;
  if (check_desc(desc, p) != LRQ_OK) return 0;
  const int v = select(desc, p, for_backward != 0);
  if (v < 0) return 0;
  const PrepLayout L = prep_layout(desc, p, for_backward != 0);
  p.use_prepared = v == LRQ_VARIANT_TILED && (for_backward ? L.bwd_bytes : L.fwd_bytes) > 0;
  return workspace_for(v, p, for_backward != 0);
}

lrq_status lrq_prepare_weights(const lrq_desc* desc, int for_backward, const void* gamma, const void* w_qkv,
                               void* prepared, size_t prepared_bytes, void* stream) {
  lrq::FwdParams p;
  lrq_status st = check_desc(desc, p);
  if (st != LRQ_OK) return st;
  const PrepLayout L = prep_layout(desc, p, for_backward != 0);
  if (L.total == 0) return ok();
  if (!gamma || !w_qkv) return fail(LRQ_ERR_INVALID_ARG, "gamma and w_qkv are required");
  if (!prepared) return fail(LRQ_ERR_INVALID_ARG, "prepared is NULL");
  if (prepared_bytes < L.total)
    return fail(LRQ_ERR_INVALID_ARG, "prepared buffer too small: %zu < %zu", prepared_bytes, L.total);
  if (!aligned16(gamma) || !aligned16(w_qkv)) return fail(LRQ_ERR_UNSUPPORTED, "array pointers must be 16-byte aligned");
  if (!aligned256(prepared)) return fail(LRQ_ERR_UNSUPPORTED, "prepared must be 256-byte aligned");
  p.gamma = gamma;
  p.w = w_qkv;
  hipStream_t s = static_cast<hipStream_t>(stream);
  unsigned char* base = static_cast<unsigned char*>(prepared);
  hipError_t e = hipSuccess;
  if (L.fwd_bytes) e = lrq::prepare_fwd_tiled(p, base + L.fwd_off, s);
  if (e == hipSuccess && L.bwd_bytes) e = lrq::prepare_bwd_tiled(p, base + L.bwd_off, s);
  return hip_status(e, "weight preparation");
}

lrq_status lrq_forward_prepared(const lrq_desc* desc, const void* x, const void* gamma, const void* w_qkv,
                                const void* prepared, size_t prepared_bytes, const void* bias,
                                const void* const* lora_a, const void* const* lora_b, const int32_t* positions,
                                void* out, const lrq_kv_cache* kv, void* workspace, size_t workspace_bytes,
                                void* stream) {
  lrq::FwdParams p;
  lrq_status st = check_desc(desc, p);
  if (st != LRQ_OK) return st;
  st = check_common_ptrs(desc, p, x, gamma, w_qkv, bias, lora_a, lora_b, positions);
  if (st != LRQ_OK) return st;
  if (prepared && !aligned256(prepared)) return fail(LRQ_ERR_UNSUPPORTED, "prepared must be 256-byte aligned");
  if (p.T > 0 && !out) return fail(LRQ_ERR_INVALID_ARG, "out is NULL");
  if (out && !aligned16(out)) return fail(LRQ_ERR_UNSUPPORTED, "out must be 16-byte aligned");
  if (kv) {
    if (kv->num_slots < 0) return fail(LRQ_ERR_INVALID_ARG, "kv->num_slots < 0");
    if (p.T > 0 && (!kv->k_cache || !kv->v_cache || !kv->slots))
      return fail(LRQ_ERR_INVALID_ARG, "kv->k_cache, kv->v_cache and kv->slots are required");
    for (const void* q : {static_cast<const void*>(kv->k_cache), static_cast<const void*>(kv->v_cache),
                          static_cast<const void*>(kv->slots)})
      if (q && !aligned16(q)) return fail(LRQ_ERR_UNSUPPORTED, "kv cache pointers must be 16-byte aligned");
  }
  const int v = select(desc, p, false);
  if (v < 0) return LRQ_ERR_UNSUPPORTED;
  if (prepared && v == LRQ_VARIANT_TILED) {
    const PrepLayout L = prep_layout(desc, p, false);
    if (L.fwd_bytes) {
      if (prepared_bytes < L.fwd_off + L.fwd_bytes)
        return fail(LRQ_ERR_INVALID_ARG, "prepared buffer too small: %zu < %zu", prepared_bytes,
                    L.fwd_off + L.fwd_bytes);
      p.prepared = static_cast<const unsigned char*>(prepared) + L.fwd_off;
      p.use_prepared = true;
    }
  }
  const size_t need = workspace_for(v, p, false);
  if (workspace_bytes < need) return fail(LRQ_ERR_INVALID_ARG, "workspace too small: %zu < %zu", workspace_bytes, need);
  if (need > 0 && !workspace) return fail(LRQ_ERR_INVALID_ARG, "workspace is NULL");
  if (need > 0 && !aligned256(workspace)) return fail(LRQ_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
  if (p.T == 0) return ok();
  p.out = out;
  p.ws = workspace;
  p.ws_bytes = workspace_bytes;
  if (kv && kv->num_slots > 0) {
    p.kv_k = kv->k_cache;
    p.kv_v = kv->v_cache;
    p.kv_slots = kv->slots;
    p.kv_num_slots = kv->num_slots;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_dropout(v, p, false, s);
  if (e != hipSuccess) return hip_status(e, "dropout masks");
  g_timing.kind = 0;
  switch (v) {
    case LRQ_VARIANT_TILED: e = lrq::launch_fwd_tiled(p, s); break;
    case LRQ_VARIANT_DECODE: e = lrq::launch_fwd_decode(p, s); break;
    default:
      e = desc->dtype == LRQ_F32 ? lrq::launch_fwd_generic_f32(p, s) : lrq::launch_fwd_generic_bf16(p, s);
  }
  // the decode family stores the cache rows from its own epilogues
  if (e == hipSuccess && v != LRQ_VARIANT_DECODE) e = lrq::launch_kv_scatter(p, s);
  return hip_status(e, "forward launch");
}

lrq_status lrq_forward_kv(const lrq_desc* desc, const void* x, const void* gamma, const void* w_qkv,
                          const void* bias, const void* const* lora_a, const void* const* lora_b,
                          const int32_t* positions, void* out, const lrq_kv_cache* kv, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return lrq_forward_prepared(desc, x, gamma, w_qkv, nullptr, 0, bias, lora_a, lora_b, positions, out, kv,
                              workspace, workspace_bytes, stream);
}

lrq_status lrq_forward(const lrq_desc* desc, const void* x, const void* gamma, const void* w_qkv,
                       const void* bias, const void* const* lora_a, const void* const* lora_b,
                       const int32_t* positions, void* out, void* workspace, size_t workspace_bytes,
                       void* stream) {
  return lrq_forward_prepared(desc, x, gamma, w_qkv, nullptr, 0, bias, lora_a, lora_b, positions, out, nullptr,
                              workspace, workspace_bytes, stream);
}

lrq_status lrq_forward_noalloc(const lrq_desc* desc, const void* x, const void* gamma, const void* w_qkv,
                               const void* prepared, size_t prepared_bytes, const void* bias,
                               const void* const* lora_a, const void* const* lora_b, const int32_t* positions,
                               void* out, const lrq_kv_cache* kv, void* stream) {
  // every argument check of lrq_forward_prepared, plus the scratch bound, before any HIP call
  lrq::FwdParams p;
  lrq_status st = check_desc(desc, p);
  if (st != LRQ_OK) return st;
  st = check_common_ptrs(desc, p, x, gamma, w_qkv, bias, lora_a, lora_b, positions);
  if (st != LRQ_OK) return st;
  const int v = select(desc, p, false);
  if (v < 0) return LRQ_ERR_UNSUPPORTED;
  if (prepared && v == LRQ_VARIANT_TILED && prep_layout(desc, p, false).fwd_bytes) p.use_prepared = true;
  const size_t need = workspace_for(v, p, false);
  if (need > kScratchBytes)
    return fail(LRQ_ERR_UNSUPPORTED,
                "lrq_forward_noalloc: this call needs %zu bytes of scratch, above the library's %zu "
                "(pass prepared weights, or use lrq_forward_prepared with a workspace)",
                need, kScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = scratch_address(&ws);
    if (e != hipSuccess) return hip_status(e, "scratch address");
  }
  return lrq_forward_prepared(desc, x, gamma, w_qkv, prepared, prepared_bytes, bias, lora_a, lora_b, positions,
                              out, kv, ws, need > 0 ? kScratchBytes : 0, stream);
}

lrq_status lrq_backward_prepared(const lrq_desc* desc, const void* x, const void* gamma, const void* w_qkv,
                                 const void* prepared, size_t prepared_bytes, const void* bias,
                                 const void* const* lora_a, const void* const* lora_b, const int32_t* positions,
                                 const void* y, const void* dy, void* dx, float* const* d_lora_a,
                                 float* const* d_lora_b, void* workspace, size_t workspace_bytes, void* stream) {
  lrq::BwdParams bp;
  std::memset(&bp, 0, sizeof bp);
  lrq_status st = check_desc(desc, bp.f);
  if (st != LRQ_OK) return st;
  st = check_common_ptrs(desc, bp.f, x, gamma, w_qkv, bias, lora_a, lora_b, positions);
  if (st != LRQ_OK) return st;
  if (prepared && !aligned256(prepared)) return fail(LRQ_ERR_UNSUPPORTED, "prepared must be 256-byte aligned");
  if (bp.f.T > 0 && (!y || !dy || !dx)) return fail(LRQ_ERR_INVALID_ARG, "y, dy and dx are required");
  for (const void* q : {y, dy, static_cast<const void*>(dx)})
    if (q && !aligned16(q)) return fail(LRQ_ERR_UNSUPPORTED, "y, dy, dx must be 16-byte aligned");
  if (desc->lora_targets && (!d_lora_a || !d_lora_b)) return fail(LRQ_ERR_INVALID_ARG, "d_lora_a / d_lora_b arrays are NULL");
  for (int t = 0; t < 3; ++t) {
    if (!(desc->lora_targets & (1u << t))) continue;
    if (!d_lora_a[t] || !d_lora_b[t]) return fail(LRQ_ERR_INVALID_ARG, "d_lora_a[%d] / d_lora_b[%d] is NULL", t, t);
    if (!aligned16(d_lora_a[t]) || !aligned16(d_lora_b[t]))
      return fail(LRQ_ERR_UNSUPPORTED, "LoRA gradient pointers must be 16-byte aligned");
    bp.da[t] = d_lora_a[t];
    bp.db[t] = d_lora_b[t];
  }
  const int v = select(desc, bp.f, true);
  if (v < 0) return LRQ_ERR_UNSUPPORTED;
  if (prepared && v == LRQ_VARIANT_TILED) {
    const PrepLayout L = prep_layout(desc, bp.f, true);
    if (L.bwd_bytes) {
      if (prepared_bytes < L.bwd_off + L.bwd_bytes)
        return fail(LRQ_ERR_INVALID_ARG, "prepared buffer too small for the backward: %zu < %zu", prepared_bytes,
                    L.bwd_off + L.bwd_bytes);
      bp.f.prepared = static_cast<const unsigned char*>(prepared) + L.bwd_off;
      bp.f.use_prepared = true;
    }
  }
  const size_t need = workspace_for(v, bp.f, true);
  if (workspace_bytes < need) return fail(LRQ_ERR_INVALID_ARG, "workspace too small: %zu < %zu", workspace_bytes, need);
  if (need > 0 && !workspace) return fail(LRQ_ERR_INVALID_ARG, "workspace is NULL");
  if (need > 0 && !aligned256(workspace)) return fail(LRQ_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
  if (bp.f.T == 0 && !desc->lora_targets) return ok();
  bp.y = y;
  bp.dy = dy;
  bp.dx = dx;
  bp.f.ws = workspace;
  bp.f.ws_bytes = workspace_bytes;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_dropout(v, bp.f, true, s);
  if (e != hipSuccess) return hip_status(e, "dropout masks");
  g_timing.kind = 1;
  if (v == LRQ_VARIANT_TILED)
    e = lrq::launch_bwd_tiled(bp, s);
  else
    e = desc->dtype == LRQ_F32 ? lrq::launch_bwd_generic_f32(bp, s) : lrq::launch_bwd_generic_bf16(bp, s);
  return hip_status(e, "backward launch");
}

lrq_status lrq_backward(const lrq_desc* desc, const void* x, const void* gamma, const void* w_qkv,
                        const void* bias, const void* const* lora_a, const void* const* lora_b,
                        const int32_t* positions, const void* y, const void* dy, void* dx,
                        float* const* d_lora_a, float* const* d_lora_b, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return lrq_backward_prepared(desc, x, gamma, w_qkv, nullptr, 0, bias, lora_a, lora_b, positions, y, dy, dx,
                               d_lora_a, d_lora_b, workspace, workspace_bytes, stream);
}

// ---- SwiGLU MLP
namespace {
lrq_status check_mlp_desc(const lrq_mlp_desc* d, lrq::MlpParams& p) {
  if (!d) return fail(LRQ_ERR_INVALID_ARG, "desc is NULL");
  if (d->n_tokens < 0) return fail(LRQ_ERR_INVALID_ARG, "n_tokens < 0");
  if (d->d_model < 1 || d->d_ff < 1) return fail(LRQ_ERR_INVALID_ARG, "d_model and d_ff must be >= 1");
  if (d->dtype != LRQ_F32 && d->dtype != LRQ_BF16) return fail(LRQ_ERR_INVALID_ARG, "unknown dtype %d", d->dtype);
  if (d->lora_targets & ~7u) return fail(LRQ_ERR_INVALID_ARG, "lora_targets has unknown bits");
  if (d->lora_targets) {
    if (d->lora_rank < 1) return fail(LRQ_ERR_INVALID_ARG, "lora_rank < 1 with targets set");
    if (!std::isfinite(d->lora_alpha)) return fail(LRQ_ERR_INVALID_ARG, "lora_alpha not finite");
  }
  std::memset(&p, 0, sizeof p);
  p.T = d->n_tokens;
  p.d = d->d_model;
  p.F = d->d_ff;
  p.targets = d->lora_targets;
  p.r = d->lora_targets ? d->lora_rank : 0;
  p.scale = d->lora_targets ? d->lora_alpha / static_cast<float>(d->lora_rank) : 0.f;
  if (d->dtype != LRQ_BF16) return fail(LRQ_ERR_UNSUPPORTED, "the MLP kernels take bf16 only");
  if (!lrq::mlp_supports(p))
    return fail(LRQ_ERR_UNSUPPORTED, "MLP shape not covered (d %% 256, d_ff %% 128, rank <= 32, T <= 2^24)");
  return LRQ_OK;
}
}  // namespace

size_t lrq_mlp_workspace_size(const lrq_mlp_desc* desc) {
  lrq::MlpParams p;
  if (check_mlp_desc(desc, p) != LRQ_OK) return 0;
  return lrq::mlp_workspace_bytes(p);
}

lrq_status lrq_mlp_forward(const lrq_mlp_desc* desc, const void* h, const void* w_gate, const void* w_up,
                           const void* w_down, const void* const* lora_a, const void* const* lora_b, void* out,
                           void* workspace, size_t workspace_bytes, void* stream) {
  lrq::MlpParams p;
  lrq_status st = check_mlp_desc(desc, p);
  if (st != LRQ_OK) return st;
  if (p.T > 0 && (!h || !w_gate || !w_up || !w_down || !out))
    return fail(LRQ_ERR_INVALID_ARG, "h, w_gate, w_up, w_down and out are required");
  if (desc->lora_targets && (!lora_a || !lora_b)) return fail(LRQ_ERR_INVALID_ARG, "lora_a / lora_b arrays are NULL");
  for (int t = 0; t < 3; ++t) {
    if (!(desc->lora_targets & (1u << t))) continue;
    if (!lora_a[t] || !lora_b[t]) return fail(LRQ_ERR_INVALID_ARG, "lora_a[%d] / lora_b[%d] is NULL for a target", t, t);
    if (!aligned16(lora_a[t]) || !aligned16(lora_b[t]))
      return fail(LRQ_ERR_UNSUPPORTED, "LoRA pointers must be 16-byte aligned");
    p.a[t] = lora_a[t];
    p.b[t] = lora_b[t];
  }
  for (const void* q : {h, w_gate, w_up, w_down, static_cast<const void*>(out)})
    if (q && !aligned16(q)) return fail(LRQ_ERR_UNSUPPORTED, "array pointers must be 16-byte aligned");
  const size_t need = lrq::mlp_workspace_bytes(p);
  if (workspace_bytes < need) return fail(LRQ_ERR_INVALID_ARG, "workspace too small: %zu < %zu", workspace_bytes, need);
  if (need > 0 && !workspace) return fail(LRQ_ERR_INVALID_ARG, "workspace is NULL");
  if (need > 0 && !aligned256(workspace)) return fail(LRQ_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
  if (p.T == 0) return ok();
  p.h = h;
  p.wg = w_gate;
  p.wu = w_up;
  p.wd = w_down;
  p.out = out;
  p.ws = workspace;
  p.ws_bytes = workspace_bytes;
  g_timing.kind = 0;
  return hip_status(lrq::launch_mlp(p, static_cast<hipStream_t>(stream)), "MLP launch");
}

lrq_status lrq_kernel_timing(int enable) {
  g_timing.on = enable != 0;
  g_timing.used[0] = g_timing.used[1] = 0;
  g_timing.open = false;
  return ok();
}

lrq_status lrq_kernel_time_ms(int for_backward, double* mean_ms, int* count) {
  if (!mean_ms || !count) return fail(LRQ_ERR_INVALID_ARG, "mean_ms and count are required");
  const int k = for_backward ? 1 : 0;
  const size_t n = g_timing.used[k];
  double sum = 0.0;
  for (size_t i = 0; i < n; ++i) {
    hipEvent_t a = g_timing.ev[k][2 * i], b = g_timing.ev[k][2 * i + 1];
    hipError_t e = hipEventSynchronize(b);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, a, b);
    if (e != hipSuccess) return hip_status(e, "kernel timing");
    sum += ms;
  }
  *mean_ms = n ? sum / static_cast<double>(n) : 0.0;
  *count = static_cast<int>(n);
  return ok();
}

}  // extern "C"
