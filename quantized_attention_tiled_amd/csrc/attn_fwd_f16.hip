// The fused attention forward kernel of attn_fwd_kernel.h instantiated for float16 Q, K, V and O.
#include "attn_fwd_kernel.h"

namespace qattn {

hipError_t launch_attn_fwd_f16(const FwdParams& p, int mode, hipStream_t stream) {
  return launch_attn_fwd<_Float16>(p, mode, stream);
}

}  // namespace qattn
