// Block-scaled fp8 (e4m3) exact attention forward for gfx950.
#include "attn_common.h"
#include "attn_kernels.h"

namespace iaea {

hipError_t launch_attn_fwd_fp8(const FwdArgs&, bool, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace iaea
