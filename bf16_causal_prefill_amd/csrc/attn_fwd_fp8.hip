// FP8 e4m3 instantiations of the causal forward kernel: d_qk 128 and 192 (MLA), 128-key
// tiles, 8 waves.  Built without NaN semantics (no NaN arises from valid inputs), which
// drops the canonicalising instructions the compiler would put before the float maxima.
#include "attn_fwd.h"

namespace attn {

hipError_t launch_attn_fwd_fp8(const FwdParams& p, int d_qk, hipStream_t stream) {
  if (d_qk == 128) return launch_cfg<true, 128, 128, 8>(p, stream);
  return launch_cfg<true, 192, 128, 8>(p, stream);
}

}  // namespace attn
