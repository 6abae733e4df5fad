// MFMA tile family (bf16, head_dim 128) -- placeholder until the kernel lands.
#include "lrq_internal.h"
namespace lrq {
bool tiled_supports(const FwdParams&) { return false; }
size_t tiled_workspace_bytes(const FwdParams&) { return 0; }
hipError_t launch_fwd_tiled(const FwdParams&, hipStream_t) { return hipErrorNotSupported; }
bool decode_supports(const FwdParams&) { return false; }
size_t decode_workspace_bytes(const FwdParams&) { return 0; }
hipError_t launch_fwd_decode(const FwdParams&, hipStream_t) { return hipErrorNotSupported; }
bool bwd_tiled_supports(const FwdParams&) { return false; }
size_t bwd_tiled_workspace_bytes(const FwdParams&) { return 0; }
hipError_t launch_bwd_tiled(const BwdParams&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace lrq
