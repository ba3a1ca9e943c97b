// C-ABI entry points of libattn: argument validation, then launches on the caller's
// stream.  Every check that can fail runs before the first HIP call, so invalid
// arguments are reported without touching a device.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "../../include/attn.h"
#ifdef ATTN_PHASE_TIMERS
#include "../../include/attn_phase_timers.h"
#endif
#include "kernels.h"

namespace {

constexpr long long kMaxElems = 1LL << 31;

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int check_shape(int B, int Hq, int Hkv, int Nq, int Nk, int d_qk, int d_v, float scale) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nk < 1) return ATTN_E_INVAL;
  if (Hq % Hkv != 0) return ATTN_E_INVAL;
  if (!(isfinite(scale) && scale > 0.f)) return ATTN_E_INVAL;
  if (!((d_qk == 128 && d_v == 128) || (d_qk == 192 && d_v == 128))) return ATTN_E_UNSUPPORTED;
  const long long bq = (long long)B * Nq, bk = (long long)B * Nk;
  if (bq * Hq * d_qk >= kMaxElems || bq * Hq * d_v >= kMaxElems) return ATTN_E_INVAL;
  if (bk * Hkv * d_qk >= kMaxElems || bk * Hkv * d_v >= kMaxElems) return ATTN_E_INVAL;
  return ATTN_OK;
}

int check_tensors(const void* q, const void* k, const void* v, const void* o, const float* lse) {
  if (!q || !k || !v || !o) return ATTN_E_INVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
    return ATTN_E_ALIGN;
  if (lse && !aligned(lse, 4)) return ATTN_E_ALIGN;
  return ATTN_OK;
}

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return ATTN_E_NODEVICE;
  }
  return ATTN_OK;
}

int launch_status(hipError_t e) {
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return ATTN_E_LAUNCH;
  }
  return ATTN_OK;
}

#ifdef ATTN_PHASE_TIMERS
// The phase-timer buffer every attention launch of this build records into (set by
// attn_phase_timers_set; null records nothing).
unsigned long long* g_timers = nullptr;
int g_timer_blocks = 0;
void set_timers(attn::FwdParams& p) {
  p.timers = g_timers;
  p.timer_blocks = g_timer_blocks;
}
#else
void set_timers(attn::FwdParams&) {}
#endif

int fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
             int Hkv, int Nq, int Nk, int q_offset, int d_qk, int d_v, float softmax_scale,
             void* stream) {
  int st = check_shape(B, Hq, Hkv, Nq, Nk, d_qk, d_v, softmax_scale);
  if (st == ATTN_OK && q_offset < 0) st = ATTN_E_INVAL;
  if (st == ATTN_OK) st = check_tensors(q, k, v, o, lse);
  if (st == ATTN_OK) st = check_device();
  if (st != ATTN_OK) return st;
  attn::FwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Nq = Nq; p.Nk = Nk; p.q_off = q_offset < Nk ? q_offset : Nk;
  p.scale = softmax_scale;
  set_timers(p);
  return launch_status(attn::launch_attn_fwd_bf16(p, d_qk, (hipStream_t)stream));
}

int fwd_fp8(const uint8_t* q, const uint8_t* k, const uint8_t* v, const float* q_descale,
            const float* k_descale, const float* v_descale, int descale_per_head, void* o,
            float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int q_offset, int d_qk, int d_v,
            float softmax_scale, void* stream, int lse_rounded = 0, int split = 0,
            const void* q_exact = nullptr, const void* k_exact = nullptr, int q_f32 = 0) {
  int st = check_shape(B, Hq, Hkv, Nq, Nk, d_qk, d_v, softmax_scale);
  if (st == ATTN_OK && split && d_qk != 128) st = ATTN_E_UNSUPPORTED;
  if (st == ATTN_OK && split && (!q_exact || !k_exact)) st = ATTN_E_INVAL;
  if (st == ATTN_OK && split && (!aligned(q_exact, 16) || !aligned(k_exact, 16)))
    st = ATTN_E_ALIGN;
  if (st == ATTN_OK && q_offset < 0) st = ATTN_E_INVAL;
  if (st == ATTN_OK) st = check_tensors(q, k, v, o, lse);
  if (st == ATTN_OK && (!q_descale || !k_descale || !v_descale)) st = ATTN_E_INVAL;
  if (st == ATTN_OK && (descale_per_head != 0 && descale_per_head != 1)) st = ATTN_E_INVAL;
  if (st == ATTN_OK && (!aligned(q_descale, 4) || !aligned(k_descale, 4) ||
                        !aligned(v_descale, 4)))
    st = ATTN_E_ALIGN;
  if (st == ATTN_OK) st = check_device();
  if (st != ATTN_OK) return st;
  attn::FwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.qds = q_descale; p.kds = k_descale; p.vds = v_descale; p.per_head = descale_per_head;
  p.lse_rounded = lse_rounded;
  p.split = split;
  p.q_exact = q_exact;
  p.k_exact = k_exact;
  p.q_f32 = q_f32;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Nq = Nq; p.Nk = Nk; p.q_off = q_offset < Nk ? q_offset : Nk;
  p.scale = softmax_scale;
  set_timers(p);
  return launch_status(attn::launch_attn_fwd_fp8(p, d_qk, (hipStream_t)stream));
}

}  // namespace

extern "C" {

#ifdef ATTN_PHASE_TIMERS
int attn_phase_timers_set(void* buf, size_t bytes) {
  if (buf && !aligned(buf, 8)) return ATTN_E_ALIGN;
  const size_t rec = (size_t)ATTN_PHASE_TIMER_WAVES * ATTN_PHASE_TIMER_WORDS * 8;
  if (buf && bytes < rec) return ATTN_E_INVAL;
  const size_t blocks = buf ? bytes / rec : 0;
  g_timers = (unsigned long long*)buf;
  g_timer_blocks = blocks > 0x7fffffff ? 0x7fffffff : (int)blocks;
  return ATTN_OK;
}
#endif

int attn_fwd_causal_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                         int B, int Hq, int Hkv, int N, int d_qk, int d_v,
                         float softmax_scale, void* stream) {
  return fwd_bf16(q, k, v, o, lse, B, Hq, Hkv, N, N, 0, d_qk, d_v, softmax_scale, stream);
}

int attn_fwd_causal_fp8(const uint8_t* q, const uint8_t* k, const uint8_t* v,
                        const float* q_descale, const float* k_descale,
                        const float* v_descale, int descale_per_head, void* o, float* lse,
                        int B, int Hq, int Hkv, int N, int d_qk, int d_v,
                        float softmax_scale, void* stream) {
  return fwd_fp8(q, k, v, q_descale, k_descale, v_descale, descale_per_head, o, lse, B, Hq, Hkv,
                 N, N, 0, d_qk, d_v, softmax_scale, stream);
}

int attn_fwd_causal_fp8_qf32(const float* q, const uint8_t* k, const uint8_t* v,
                             const float* q_descale, const float* k_descale,
                             const float* v_descale, int descale_per_head, void* o, float* lse,
                             int B, int Hq, int Hkv, int N, int d_qk, int d_v,
                             float softmax_scale, void* stream) {
  return fwd_fp8((const uint8_t*)q, k, v, q_descale, k_descale, v_descale, descale_per_head, o,
                 lse, B, Hq, Hkv, N, N, 0, d_qk, d_v, softmax_scale, stream, 0, 0, nullptr,
                 nullptr, 1);
}

int attn_fwd_causal_offset_bf16(const void* q, const void* k, const void* v, void* o,
                                float* lse, int B, int Hq, int Hkv, int Nq, int Nk,
                                int q_offset, int d_qk, int d_v, float softmax_scale,
                                void* stream) {
  return fwd_bf16(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, q_offset, d_qk, d_v, softmax_scale,
                  stream);
}

int attn_fwd_causal_offset_fp8(const uint8_t* q, const uint8_t* k, const uint8_t* v,
                               const float* q_descale, const float* k_descale,
                               const float* v_descale, int descale_per_head, void* o,
                               float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int q_offset,
                               int d_qk, int d_v, float softmax_scale, void* stream) {
  return fwd_fp8(q, k, v, q_descale, k_descale, v_descale, descale_per_head, o, lse, B, Hq, Hkv,
                 Nq, Nk, q_offset, d_qk, d_v, softmax_scale, stream);
}

int attn_fwd_causal_offset_fp8_rounded_lse(const uint8_t* q, const uint8_t* k, const uint8_t* v,
                                           const float* q_descale, const float* k_descale,
                                           const float* v_descale, int descale_per_head, void* o,
                                           float* lse, int B, int Hq, int Hkv, int Nq, int Nk,
                                           int q_offset, int d_qk, int d_v, float softmax_scale,
                                           void* stream) {
  if (!lse) return ATTN_E_INVAL;
  return fwd_fp8(q, k, v, q_descale, k_descale, v_descale, descale_per_head, o, lse, B, Hq, Hkv,
                 Nq, Nk, q_offset, d_qk, d_v, softmax_scale, stream, 1);
}

int attn_fwd_causal_fp8_outliers(const uint8_t* q, const uint8_t* k, const uint8_t* v,
                                 const void* q_exact, const void* k_exact,
                                 const float* q_descale, const float* k_descale,
                                 const float* v_descale, int descale_per_head, void* o,
                                 float* lse, int B, int Hq, int Hkv, int N, int d_qk, int d_v,
                                 float softmax_scale, void* stream) {
  return fwd_fp8(q, k, v, q_descale, k_descale, v_descale, descale_per_head, o, lse, B, Hq, Hkv,
                 N, N, 0, d_qk, d_v, softmax_scale, stream, 0, 1, q_exact, k_exact);
}

int attn_fwd_causal_offset_fp8_outliers(const uint8_t* q, const uint8_t* k, const uint8_t* v,
                                        const void* q_exact, const void* k_exact,
                                        const float* q_descale, const float* k_descale,
                                        const float* v_descale, int descale_per_head, void* o,
                                        float* lse, int B, int Hq, int Hkv, int Nq, int Nk,
                                        int q_offset, int d_qk, int d_v, float softmax_scale,
                                        void* stream) {
  return fwd_fp8(q, k, v, q_descale, k_descale, v_descale, descale_per_head, o, lse, B, Hq, Hkv,
                 Nq, Nk, q_offset, d_qk, d_v, softmax_scale, stream, 0, 1, q_exact, k_exact);
}

int attn_merge_partials(const void* o_a, const float* lse_a, const void* o_b,
                        const float* lse_b, void* o, float* lse, int B, int N, int Hq, int d_v,
                        void* stream) {
  if (!o_a || !lse_a || !o_b || !lse_b || !o) return ATTN_E_INVAL;
  if (B < 1 || N < 1 || Hq < 1) return ATTN_E_INVAL;
  if (d_v < 8 || d_v > 512 || (d_v & (d_v - 1)) != 0) return ATTN_E_INVAL;
  if ((long long)B * N * Hq * d_v >= kMaxElems) return ATTN_E_INVAL;
  if (!aligned(o_a, 16) || !aligned(o_b, 16) || !aligned(o, 16) || !aligned(lse_a, 4) ||
      !aligned(lse_b, 4) || (lse && !aligned(lse, 4)))
    return ATTN_E_ALIGN;
  const int st = check_device();
  if (st != ATTN_OK) return st;
  return launch_status(attn::launch_attn_merge(o_a, lse_a, o_b, lse_b, o, lse, B, N, Hq, d_v,
                                               (hipStream_t)stream));
}

static int quantize_impl(const float* x, uint8_t* out, float* descale, int B, int N, int H,
                         int d, int per_head, int hadamard, void* stream) {
  if (!x || !out || !descale) return ATTN_E_INVAL;
  if (B < 1 || N < 1 || H < 1 || d < 4 || (d & 3) != 0) return ATTN_E_INVAL;
  if (per_head != 0 && per_head != 1) return ATTN_E_INVAL;
  if (H > 65535) return ATTN_E_INVAL;
  if ((long long)B * N * H * d >= kMaxElems) return ATTN_E_INVAL;
  if (!aligned(x, 16) || !aligned(out, 4) || !aligned(descale, 4)) return ATTN_E_ALIGN;
  const int st = check_device();
  if (st != ATTN_OK) return st;
  return launch_status(attn::launch_quantize_e4m3(x, out, descale, B, N, H, d, per_head,
                                                  hadamard, (hipStream_t)stream));
}

int quantize_e4m3(const float* x, uint8_t* out, float* descale, int B, int N, int H, int d,
                  int per_head, void* stream) {
  return quantize_impl(x, out, descale, B, N, H, d, per_head, 0, stream);
}

int quantize_e4m3_q_pow2(const float* x, uint8_t* out, float* descale, int B, int N, int H,
                         int d, int per_head, const float* k_descale, int Hkv,
                         float softmax_scale, void* stream) {
  if (!x || !out || !descale || !k_descale) return ATTN_E_INVAL;
  if (B < 1 || N < 1 || H < 1 || d < 4 || (d & 3) != 0) return ATTN_E_INVAL;
  if (per_head != 0 && per_head != 1) return ATTN_E_INVAL;
  if (H > 65535 || Hkv < 1 || (per_head && H % Hkv != 0)) return ATTN_E_INVAL;
  if (!(isfinite(softmax_scale) && softmax_scale > 0.f)) return ATTN_E_INVAL;
  if ((long long)B * N * H * d >= kMaxElems) return ATTN_E_INVAL;
  if (!aligned(x, 16) || !aligned(out, 4) || !aligned(descale, 4) || !aligned(k_descale, 4))
    return ATTN_E_ALIGN;
  const int st = check_device();
  if (st != ATTN_OK) return st;
  return launch_status(attn::launch_quantize_e4m3_q_pow2(x, out, descale, B, N, H, d, per_head,
                                                         k_descale, Hkv, softmax_scale,
                                                         (hipStream_t)stream));
}

int quantize_e4m3_qkv(const float* q, const float* k, const float* v, uint8_t* q_out,
                      uint8_t* k_out, uint8_t* v_out, float* q_descale, float* k_descale,
                      float* v_descale, int B, int Nq, int Nk, int Hq, int Hkv, int d_qk,
                      int d_v, int per_head, int q_pow2, float softmax_scale, void* stream) {
  if (!q || !k || !v || !k_out || !v_out || !q_descale || !k_descale || !v_descale)
    return ATTN_E_INVAL;
  if (B < 1 || Nq < 1 || Nk < 1 || Hq < 1 || Hkv < 1) return ATTN_E_INVAL;
  if (d_qk < 4 || (d_qk & 3) != 0 || d_v < 4 || (d_v & 3) != 0) return ATTN_E_INVAL;
  if (per_head != 0 && per_head != 1) return ATTN_E_INVAL;
  if (q_pow2 != 0 && q_pow2 != 1) return ATTN_E_INVAL;
  if (Hq > 65535 || Hkv > 65535) return ATTN_E_INVAL;
  if (q_pow2 && per_head && Hq % Hkv != 0) return ATTN_E_INVAL;
  if (q_pow2 && !(isfinite(softmax_scale) && softmax_scale > 0.f)) return ATTN_E_INVAL;
  if ((long long)B * Nq * Hq * d_qk >= kMaxElems || (long long)B * Nk * Hkv * d_qk >= kMaxElems ||
      (long long)B * Nk * Hkv * d_v >= kMaxElems)
    return ATTN_E_INVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || (q_out && !aligned(q_out, 4)) ||
      !aligned(k_out, 4) || !aligned(v_out, 4) || !aligned(q_descale, 4) ||
      !aligned(k_descale, 4) || !aligned(v_descale, 4))
    return ATTN_E_ALIGN;
  const int st = check_device();
  if (st != ATTN_OK) return st;
  return launch_status(attn::launch_quantize_e4m3_qkv(
      q, k, v, q_out, k_out, v_out, q_descale, k_descale, v_descale, B, Nq, Nk, Hq, Hkv, d_qk,
      d_v, per_head, q_pow2, softmax_scale, (hipStream_t)stream));
}

int quantize_e4m3_hadamard(const float* x, uint8_t* out, float* descale, int B, int N, int H,
                           int d, int per_head, void* stream) {
  return quantize_impl(x, out, descale, B, N, H, d, per_head, 1, stream);
}

static int quantize_e4m3_qk_outliers_check(const float* q, const float* k, uint8_t* q_out,
                                           uint8_t* k_out, void* q_exact, void* k_exact,
                                           float* q_descale, float* k_descale, uint8_t* perm,
                                           int B, int N, int Hq, int Hkv, int d, int per_head,
                                           int q_pow2, float softmax_scale) {
  if (!q || !k || !q_out || !k_out || !q_exact || !k_exact || !q_descale || !k_descale || !perm)
    return ATTN_E_INVAL;
  if (B < 1 || N < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return ATTN_E_INVAL;
  if (d < ATTN_OUTLIER_CHANNELS || d > 256 || (d & 3) != 0) return ATTN_E_INVAL;
  if (per_head != 0 && per_head != 1) return ATTN_E_INVAL;
  if (q_pow2 != 0 && q_pow2 != 1) return ATTN_E_INVAL;
  if (q_pow2 && !(isfinite(softmax_scale) && softmax_scale > 0.f)) return ATTN_E_INVAL;
  if (Hq > 65535) return ATTN_E_INVAL;
  if ((long long)B * N * Hq * d >= kMaxElems) return ATTN_E_INVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(q_out, 4) || !aligned(k_out, 4) ||
      !aligned(q_exact, 16) || !aligned(k_exact, 16) || !aligned(q_descale, 4) ||
      !aligned(k_descale, 4) || !aligned(perm, 4))
    return ATTN_E_ALIGN;
  return ATTN_OK;
}

int quantize_e4m3_qk_outliers(const float* q, const float* k, uint8_t* q_out, uint8_t* k_out,
                              void* q_exact, void* k_exact, float* q_descale, float* k_descale,
                              uint8_t* perm, void* workspace, size_t workspace_bytes, int B,
                              int N, int Hq, int Hkv, int d, int per_head, int q_pow2,
                              float softmax_scale, void* stream) {
  if (!workspace) return ATTN_E_INVAL;
  int st0 = quantize_e4m3_qk_outliers_check(q, k, q_out, k_out, q_exact, k_exact, q_descale,
                                            k_descale, perm, B, N, Hq, Hkv, d, per_head, q_pow2,
                                            softmax_scale);
  if (st0 != ATTN_OK) return st0;
  if (workspace_bytes < quantize_e4m3_qk_outliers_workspace_bytes(Hq, Hkv, d))
    return ATTN_E_INVAL;
  if (!aligned(workspace, 4)) return ATTN_E_ALIGN;
  const int st = check_device();
  if (st != ATTN_OK) return st;
  return launch_status(attn::launch_quantize_e4m3_qk_outliers(
      q, k, q_out, k_out, q_exact, k_exact, q_descale, k_descale, perm, (uint32_t*)workspace, B,
      N, Hq, Hkv, d, per_head, q_pow2, softmax_scale, (hipStream_t)stream));
}

int quantize_e4m3_qk_outliers_noalloc(const float* q, const float* k, uint8_t* q_out,
                                      uint8_t* k_out, void* q_exact, void* k_exact,
                                      float* q_descale, float* k_descale, uint8_t* perm, int B,
                                      int N, int Hq, int Hkv, int d, int per_head, int q_pow2,
                                      float softmax_scale, void* stream) {
  // Every argument check before the first HIP call; the scratch address is only looked
  // up for a call that will run (the first one on each device).
  const int st = quantize_e4m3_qk_outliers_check(q, k, q_out, k_out, q_exact, k_exact,
                                                 q_descale, k_descale, perm, B, N, Hq, Hkv, d,
                                                 per_head, q_pow2, softmax_scale);
  if (st != ATTN_OK) return st;
  if ((long long)(Hq + Hkv) * d > (long long)ATTN_NOALLOC_SCRATCH_WORDS) return ATTN_E_TOO_LARGE;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return ATTN_E_NODEVICE;
  }
  uint32_t* ws = attn::scratch_ptr(dev);
  if (!ws) return ATTN_E_LAUNCH;
  return launch_status(attn::launch_quantize_e4m3_qk_outliers(
      q, k, q_out, k_out, q_exact, k_exact, q_descale, k_descale, perm, ws, B, N, Hq, Hkv, d,
      per_head, q_pow2, softmax_scale, (hipStream_t)stream));
}

size_t quantize_e4m3_qk_outliers_workspace_bytes(int Hq, int Hkv, int d) {
  if (Hq < 1 || Hkv < 1 || d < 1) return 0;
  return (size_t)(Hq + Hkv) * (size_t)d * sizeof(uint32_t);
}

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_E_INVAL: return "invalid argument";
    case ATTN_E_UNSUPPORTED: return "unsupported head dims (need d_qk/d_v 128/128 or 192/128)";
    case ATTN_E_ALIGN: return "misaligned tensor pointer";
    case ATTN_E_NODEVICE: return "no usable HIP device";
    case ATTN_E_LAUNCH: return "kernel launch failed";
    case ATTN_E_TOO_LARGE:
      return "(Hq + Hkv) * d exceeds the scratch of the allocation-free entry point";
    default: return "unknown status";
  }
}

}  // extern "C"
