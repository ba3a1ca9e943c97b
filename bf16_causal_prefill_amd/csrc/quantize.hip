// Absmax quantisation of float32 (B, N, H, d) tensors into OCP e4m3fn codes.
//
// Each tensor (or each head) gets one scale factor that maps it into the e4m3 range
// (kongchang.com, "ZYFA 的性能与精度数据": per-tensor or per-head scaling).
// descale = absmax / 448 in float32, code = e4m3 round-to-nearest-even of the float32
// quotient x / descale, saturating at +-448.  The pass is bound by HBM bandwidth:
// one read for the absmax, one read plus a quarter-size write for the codes.
//
// Kernels, in stream order:
//   1. clear     descale[] <- 0 (used as the absmax accumulator, as float bits)
//   2. absmax    per workgroup max |x| over its rows of one head, then an integer
//                atomicMax on the float bits (non-negative floats order like their
//                bit patterns), which is order-independent and so deterministic
//   3. encode    reads the absmax, forms the descale and writes the codes
//   4. finalize  descale[] <- absmax / 448 (1 for an all-zero tensor or head)
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace attn {

constexpr int QZ_THREADS = 256;
constexpr int QZ_ROWS = 64;     // (b, n) rows of one head per workgroup

__global__ void qz_clear(uint32_t* amax_bits, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) amax_bits[i] = 0u;
}

// Grid: (ceil(B*N / QZ_ROWS), H).  A row of one head has d floats, read as float4.
__global__ __launch_bounds__(QZ_THREADS) void qz_absmax(const float* __restrict__ x,
                                                       uint32_t* amax_bits, int rows, int H,
                                                       int d, int per_head) {
  const int h = blockIdx.y;
  const int r0 = blockIdx.x * QZ_ROWS;
  const int v4 = d >> 2;                       // float4 per row
  const int total = min(QZ_ROWS, rows - r0) * v4;
  float m = 0.f;
  for (int e = threadIdx.x; e < total; e += QZ_THREADS) {
    const int r = r0 + e / v4, c4 = e - (e / v4) * v4;
    const float4 val = *(const float4*)(x + ((size_t)r * H + h) * d + 4 * c4);
    m = fmaxf(m, fmaxf(fmaxf(fabsf(val.x), fabsf(val.y)), fmaxf(fabsf(val.z), fabsf(val.w))));
  }
  // bit patterns of non-negative floats order like the values, so reduce as integers
  uint32_t u = __float_as_uint(m);
  for (int off = 32; off > 0; off >>= 1) u = max(u, (uint32_t)__shfl_xor((int)u, off));
  __shared__ uint32_t red[QZ_THREADS / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = u;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t v = red[0];
    for (int w = 1; w < QZ_THREADS / 64; ++w) v = max(v, red[w]);
    atomicMax(amax_bits + (per_head ? h : 0), v);
  }
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

__global__ __launch_bounds__(QZ_THREADS) void qz_encode(const float* __restrict__ x,
                                                       uint8_t* __restrict__ out,
                                                       const uint32_t* amax_bits, int rows,
                                                       int H, int d, int per_head) {
  const int h = blockIdx.y;
  const int r0 = blockIdx.x * QZ_ROWS;
  const int v4 = d >> 2;
  const int total = min(QZ_ROWS, rows - r0) * v4;
  const float ds = descale_of(amax_bits[per_head ? h : 0]);
  for (int e = threadIdx.x; e < total; e += QZ_THREADS) {
    const int r = r0 + e / v4, c4 = e - (e / v4) * v4;
    const size_t off = ((size_t)r * H + h) * d + 4 * c4;
    const float4 val = *(const float4*)(x + off);
    const uint32_t w = e4m3_code(val.x / ds) | (e4m3_code(val.y / ds) << 8) |
                       (e4m3_code(val.z / ds) << 16) | (e4m3_code(val.w / ds) << 24);
    *(uint32_t*)(out + off) = w;
  }
}

__global__ void qz_finalize(float* descale, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) descale[i] = descale_of(__float_as_uint(descale[i]));
}

hipError_t launch_quantize_e4m3(const float* x, uint8_t* out, float* descale, int B, int N,
                                int H, int d, int per_head, hipStream_t stream) {
  const int rows = B * N;
  const int ns = per_head ? H : 1;
  uint32_t* bits = (uint32_t*)descale;
  const dim3 grid((rows + QZ_ROWS - 1) / QZ_ROWS, H);
  hipLaunchKernelGGL(qz_clear, dim3((ns + 255) / 256), dim3(256), 0, stream, bits, ns);
  hipLaunchKernelGGL(qz_absmax, grid, dim3(QZ_THREADS), 0, stream, x, bits, rows, H, d,
                     per_head);
  hipLaunchKernelGGL(qz_encode, grid, dim3(QZ_THREADS), 0, stream, x, out,
                     (const uint32_t*)bits, rows, H, d, per_head);
  hipLaunchKernelGGL(qz_finalize, dim3((ns + 255) / 256), dim3(256), 0, stream, descale, ns);
  return hipGetLastError();
}

}  // namespace attn
