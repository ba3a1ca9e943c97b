// Device helpers of the e4m3 quantisers (quantize.hip, outliers.hip): streaming loads,
// the descale of an absmax, the round-to-nearest-even e4m3 encoder (per element on the
// bit pattern, and branch-free through a correctly rounded quotient and the hardware
// conversion) and the power-of-two Q descale.
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace attn {

// Non-temporal 16-byte load: the float32 input is streamed through once per pass.
typedef float f32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load_stream(const float4* p) {
  const f32x4_nt v = __builtin_nontemporal_load((const f32x4_nt*)p);
  return make_float4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ float descale_of(uint32_t amax_bits) {
  const float a = __uint_as_float(amax_bits);
  return a > 0.f ? a / 448.f : 1.f;
}

// Round-to-nearest-even e4m3fn code of a float32, saturating at +-448, NaN -> 0x7F.
// Works on the bit pattern: normal results round the 23-bit mantissa to 3 bits by
// adding half-an-ulp-minus-one plus the kept lsb; below 2^-6 the spacing is 2^-9.
__device__ __forceinline__ uint32_t e4m3_code(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;               // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;       // |f| >= 448: saturate
  if (a < 0x3c800000u) {                           // |f| < 2^-6: multiples of 2^-9
    const float s = __uint_as_float(a) * 512.f;    // exact power-of-two scaling
    return sign | (uint32_t)__builtin_rintf(s);    // 0..8 (8 is the code of 2^-6)
  }
  const uint32_t r = (a + 0x7ffffu + ((a >> 20) & 1u)) >> 20;   // (E << 3) | m3, rounded
  return sign | (r - (120u << 3));                 // exponent bias 127 -> 7
}

__device__ __forceinline__ uint32_t e4m3_word(float4 a, float ds) {
  return e4m3_code(a.x / ds) | (e4m3_code(a.y / ds) << 8) | (e4m3_code(a.z / ds) << 16) |
         (e4m3_code(a.w / ds) << 24);
}

// The same codes without branches, for divisors in [2^-100, 2^100] (every descale of a
// tensor whose absmax is a normal float32 above 2^-90).
//  * Quotient: the reciprocal of ds refined by one Newton step, then two residual
//    corrections whose residuals the FMA forms exactly; for these divisors this is the
//    correctly rounded quotient, and copying the sign of x keeps the sign of a zero
//    quotient.  Checked against the IEEE division on the device over 4M pairs and every
//    e4m3 value, tie and neighbour times random descales.
//  * Code: clamped to +-448 (beyond it the hardware conversion gives NaN codes), then
//    gfx950's f32 -> e4m3 conversion, which rounds to nearest even with subnormals and
//    signed zeros exactly as e4m3_code for |q| < 448 (checked on the same values).
//  * A NaN quotient (seen through the sum of the four, which is also NaN when they
//    hold infinities of both signs) takes e4m3_code for the whole word.
struct Divisor {
  float b, r;
};

__device__ __forceinline__ Divisor make_divisor(float b) {
  float r = __builtin_amdgcn_rcpf(b);
  r = fmaf(fmaf(-b, r, 1.f), r, r);
  return {b, r};
}

__device__ __forceinline__ bool fast_divisor(float b) {
  return b >= 0x1p-100f && b <= 0x1p100f;
}

__device__ __forceinline__ float quotient(float a, Divisor d) {
  float q = a * d.r;
  q = fmaf(fmaf(-d.b, q, a), d.r, q);
  q = fmaf(fmaf(-d.b, q, a), d.r, q);
  return copysignf(q, a);
}

// NaN test on the bit pattern, which holds also where the compiler is told that no
// NaNs occur (the FP8 attention kernels, which encode float32 Q with these helpers).
__device__ __forceinline__ bool nan_bits(float x) {
  return (__float_as_uint(x) & 0x7fffffffu) > 0x7f800000u;
}

// The code word of four quotients already formed (as e4m3_word_fast below).
__device__ __forceinline__ uint32_t e4m3_word_of_quotients(float4 q) {
  if (__builtin_expect(nan_bits((q.x + q.y) + (q.z + q.w)), 0))
    return e4m3_code(q.x) | (e4m3_code(q.y) << 8) | (e4m3_code(q.z) << 16) |
           (e4m3_code(q.w) << 24);
  const float m = 448.f;
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(q.x, -m, m),
                                          __builtin_amdgcn_fmed3f(q.y, -m, m), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(q.z, -m, m),
                                      __builtin_amdgcn_fmed3f(q.w, -m, m), w, true);
  return (uint32_t)w;
}

__device__ __forceinline__ uint32_t e4m3_word_fast(float4 a, Divisor d) {
  const float4 q = make_float4(quotient(a.x, d), quotient(a.y, d), quotient(a.z, d),
                               quotient(a.w, d));
  if (__builtin_expect(nan_bits((q.x + q.y) + (q.z + q.w)), 0))
    return e4m3_code(q.x) | (e4m3_code(q.y) << 8) | (e4m3_code(q.z) << 16) |
           (e4m3_code(q.w) << 24);
  const float m = 448.f;
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(q.x, -m, m),
                                          __builtin_amdgcn_fmed3f(q.y, -m, m), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(q.z, -m, m),
                                      __builtin_amdgcn_fmed3f(q.w, -m, m), w, true);
  return (uint32_t)w;
}

// Q descale for which the FP8 attention's float32 softmax constant
// c = fl(fl(scale * log2 e) * fl(dq * dk)) lies within 4 ulps of a power of two: the
// smallest power of two at or above fl(fl(absmax / 448) * fl(sl * dk)), sl =
// fl(scale * log2 e), divided by fl(sl * dk), then moved one ulp at a time (at most 16)
// towards it until c is there.  A zero or non-finite absmax, or no such descale, gives
// the plain absmax / 448 (1 for zero).  Every step is one float32 operation, correctly
// rounded, so the result is reproducible off the device.
__device__ __forceinline__ float pow2_q_descale(float amax, float dk, float sl) {
  const float plain = amax > 0.f ? amax / 448.f : 1.f;
  if (!(isfinite(amax) && amax > 0.f && isfinite(dk) && dk > 0.f)) return plain;
  const float a = sl * dk;
  const float tmin = (amax / 448.f) * a;
  if (!(isfinite(tmin) && tmin > 0.f)) return plain;
  const uint32_t b = __float_as_uint(tmin);
  const uint32_t ex = (b >> 23) & 0xffu;
  if (ex == 0u || ex >= 0xfeu) return plain;
  const float target = (b & 0x7fffffu) == 0u ? tmin : __uint_as_float((ex + 1u) << 23);
  float d = target / a;
  for (int i = 0; i < 16; ++i) {
    const float c = sl * (d * dk);
    const uint32_t cb = __float_as_uint(c), cm = cb & 0x7fffffu, ce = (cb >> 23) & 0xffu;
    if (ce != 0u && ce != 0xffu && (cm <= 4u || cm >= 0x7ffffcu) &&
        fabsf(c / target - 1.f) < 0x1p-20f)
      return d;
    d = __uint_as_float(__float_as_uint(d) + (c < target ? 1u : 0xffffffffu));   // +-1 ulp
  }
  return plain;
}

}  // namespace attn
