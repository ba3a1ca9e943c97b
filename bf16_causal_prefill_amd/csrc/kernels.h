// Internal launch interface between the C-ABI entry points and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;          // may be null
  const float* qds;    // FP8 descales (device), null for BF16
  const float* kds;
  const float* vds;
  int per_head;
  int B, Hq, Hkv, N;
  float scale;
  int n_qtiles;        // filled in by the launcher
};

// Enqueues the causal forward kernel; d_v is 128 for both supported shapes.
hipError_t launch_attn_fwd(const FwdParams& p, bool fp8, int d_qk, hipStream_t stream);

// Enqueues the four kernels of absmax e4m3 quantisation.
hipError_t launch_quantize_e4m3(const float* x, uint8_t* out, float* descale, int B, int N,
                                int H, int d, int per_head, hipStream_t stream);

}  // namespace attn
