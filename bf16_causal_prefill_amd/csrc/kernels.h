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
  int B, Hq, Hkv;
  int Nq, Nk;          // query rows and key rows per (batch, head)
  int q_off;           // key j is visible to query i iff j <= i + q_off (0 <= q_off <= Nk)
  float scale;
  int n_qtiles;        // filled in by the launcher
  int lse_rounded;     // FP8: lse from the rounded-probability row sums (consistent with O)
  int split;           // FP8, d_qk 128: the last 32 channels of Q and K on the BF16 pipe,
  const void* q_exact; // from these bf16 side arrays (B, Nq, Hq, 32) and (B, Nk, Hkv, 32)
  const void* k_exact;
  int q_f32;           // FP8: q is float32, encoded on load with q's descales
  int xcd_swap;        // items each odd XCD trades with its even partner, and the place
  int xcd_swap_at;     // in the even one's list of the items it takes (the launcher)
  int se_rotate;       // rotate items over each XCD's shader engines (the launcher)
  int late_rows_ahead; // the wave group ahead in the key loop owns the later rows (the launcher)
#ifdef ATTN_PHASE_TIMERS
  // Phase-timer build only (libattn_phase_timers.so): ATTN_PHASE_TIMER_WORDS words per
  // (workgroup, wave) of the first timer_blocks workgroups, see include/attn_phase_timers.h.
  unsigned long long* timers;
  int timer_blocks;
#endif
};

// Enqueue the causal forward kernel (d_qk 128 or 192; d_v is 128 for both shapes).
hipError_t launch_attn_fwd_fp8(const FwdParams& p, int d_qk, hipStream_t stream);
hipError_t launch_attn_fwd_bf16(const FwdParams& p, int d_qk, hipStream_t stream);

// Enqueues the merge of two partial attentions over disjoint key sets:
// o = (e^(lse_a - m) o_a + e^(lse_b - m) o_b) / (e^(lse_a - m) + e^(lse_b - m)), lse = m + ln(..).
hipError_t launch_attn_merge(const void* o_a, const float* lse_a, const void* o_b,
                             const float* lse_b, void* o, float* lse, int B, int N, int Hq,
                             int d_v, hipStream_t stream);

// Enqueues the four kernels of absmax e4m3 quantisation, optionally of the
// Hadamard-rotated values (hadamard != 0).
hipError_t launch_quantize_e4m3(const float* x, uint8_t* out, float* descale, int B, int N,
                                int H, int d, int per_head, int hadamard, hipStream_t stream);
hipError_t launch_quantize_e4m3_q_pow2(const float* x, uint8_t* out, float* descale, int B,
                                       int N, int H, int d, int per_head,
                                       const float* k_descale, int Hkv, float softmax_scale,
                                       hipStream_t stream);

// Enqueues the quantisation of Q, K and V in four kernels (clear, absmax, finalize,
// encode, each over the three tensors); Q as launch_quantize_e4m3_q_pow2 (q_pow2) or
// launch_quantize_e4m3, K and V as launch_quantize_e4m3.  q_out null: Q's descales
// only.
hipError_t launch_quantize_e4m3_qkv(const float* q, const float* k, const float* v,
                                    uint8_t* q_out, uint8_t* k_out, uint8_t* v_out,
                                    float* q_descale, float* k_descale, float* v_descale,
                                    int B, int Nq, int Nk, int Hq, int Hkv, int d_qk, int d_v,
                                    int per_head, int q_pow2, float softmax_scale,
                                    hipStream_t stream);

// Enqueues the joint Q/K quantisation that stores each KV head's largest-product
// channels last (workspace: (Hq + Hkv) * d uint32 accumulators).
hipError_t launch_quantize_e4m3_qk_outliers(const float* q, const float* k, uint8_t* q_out,
                                            uint8_t* k_out, void* q_exact, void* k_exact,
                                            float* q_descale, float* k_descale, uint8_t* perm,
                                            uint32_t* workspace, int B, int N, int Hq,
                                            int Hkv, int d, int per_head, int q_pow2,
                                            float softmax_scale, hipStream_t stream);

// Device address of the file-scope scratch array of quantize_e4m3_qk_outliers_noalloc on
// `device` (which must be current), or nullptr.
constexpr int kMaxDevices = 64;
uint32_t* scratch_ptr(int device);

}  // namespace attn
