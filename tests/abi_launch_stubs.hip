// Launch-function stubs for the host AddressSanitizer build of the C ABI (tests/test_abi_host_asan.py):
// that build compiles qattn_abi.hip alone, with its host code instrumented, and links these in place
// of the kernel translation units. Argument validation returns before any launch, so the stubs are
// never reached by the validation tests; if one were, the call would fail with a HIP error status.
#include "qattn_internal.h"

namespace qattn {

hipError_t launch_attn_bwd(const BwdParams&, int, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_attn_fwd_bf16(const FwdParams&, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_attn_fwd_f16(const FwdParams&, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_attn_qbsa(const FwdParams&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_quant_qk(const uint16_t*, int, int, int, int, int8_t*, float*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_quant_v(const uint16_t*, int, int, int, int, uint8_t*, float*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_block_list(const uint8_t*, int, int, int, int, int32_t*, int32_t*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_qblock_order(const int32_t*, int, int, int, int32_t*, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_mask_pack(const uint8_t*, int64_t, int, int64_t, int32_t*, hipStream_t) { return hipErrorNotSupported; }

}  // namespace qattn
