// BF16 instantiations of the causal forward kernel: d_qk 128 and 192 (MLA), 64-key
// tiles, 8 waves.  Built with the default floating-point semantics: the schedule the
// compiler produces for these kernels measured 6% slower without NaN semantics.
#include "attn_fwd.h"

namespace attn {

hipError_t launch_attn_fwd_bf16(const FwdParams& p, int d_qk, hipStream_t stream) {
  if (d_qk == 128) return launch_cfg<false, 128, 64, 8>(p, stream);
  return launch_cfg<false, 192, 64, 8>(p, stream);
}

}  // namespace attn
