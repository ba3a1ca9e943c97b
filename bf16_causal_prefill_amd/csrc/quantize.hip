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
//   2. absmax    per workgroup max |x| over a band of whole rows (per head, gathered
//                in LDS), then one integer atomicMax per head on the float bits
//                (non-negative floats order like their bit patterns), which is
//                order-independent and so deterministic
//   3. encode    reads the absmax, forms the descale and writes the codes
//   4. finalize  descale[] <- absmax / 448 (1 for an all-zero tensor or head)
//
// Optional Hadamard rotation (spke.com "ZYFAのFP8アテンションの精度はどのくらいか?":
// rotating Q and K roughly halves the FP8 input error): the values quantised are
// x H / sqrt(hb) with H the Sylvester Hadamard matrix of order hb applied to each block
// of hb channels (hb = the largest power of two dividing d, at most 128).  Q H (K H)^T
// = Q K^T, so scores are unchanged while outlier channels are spread over the block.
// Passes 2 and 3 transform the unnormalised blocks in float32 (wht_block) and the
// normalisation 1/sqrt(hb) goes into the descale, so the codes are those of x H.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kernels.h"

namespace attn {

constexpr int QZ_THREADS = 256;
constexpr int QZ_LDS_HEADS = 1024;   // per-head maxima kept in LDS up to this many heads
constexpr int QZ_TARGET_WGS = 1024;  // workgroups per pass (about four per CU)

// Work split shared by both passes.  The tensor is B*N rows of L4 = H*d/4 float4
// values (head h owns columns h*d4 .. h*d4 + d4-1, d4 = d/4).  A workgroup takes a band
// of `band` consecutive rows; thread t handles the columns t, t + 256, ... of every row
// in the band, so each column's head is fixed per thread and the workgroup reads whole
// rows (contiguous memory) at a time.

__global__ void qz_clear(uint32_t* amax_bits, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) amax_bits[i] = 0u;
}

// Walsh-Hadamard transform (Sylvester order, unnormalised) of a block of hb = 4*hb4
// consecutive channels held by hb4 consecutive lanes, 4 channels each (hb4 divides 64
// and blocks start at multiples of hb4 lanes).  Radix-2 butterflies in float32, stage
// half-sizes 1, 2, 4, ..., hb/2 in that order: the element with the stage bit clear
// becomes a + b, its partner a - b.  Every lane of a block must be active.
__device__ __forceinline__ float4 wht_block(float4 v, int hb4, int lane) {
  const float a0 = v.x + v.y, a1 = v.x - v.y, a2 = v.z + v.w, a3 = v.z - v.w;
  v = make_float4(a0 + a2, a1 + a3, a0 - a2, a1 - a3);
  for (int m = 1; m < hb4; m <<= 1) {
    const float4 q = make_float4(__shfl_xor(v.x, m), __shfl_xor(v.y, m), __shfl_xor(v.z, m),
                                 __shfl_xor(v.w, m));
    if (lane & m) v = make_float4(q.x - v.x, q.y - v.y, q.z - v.z, q.w - v.w);
    else v = make_float4(v.x + q.x, v.y + q.y, v.z + q.z, v.w + q.w);
  }
  return v;
}

// Bit patterns of non-negative floats order like the values, so maxima are taken as
// unsigned integers (atomicMax is then exact and order-independent).  With hb4 > 0
// the values are the Walsh-Hadamard transforms of blocks of 4*hb4 channels.
__global__ __launch_bounds__(QZ_THREADS) void qz_absmax(const float* __restrict__ x,
                                                       uint32_t* amax_bits, int rows, int L4,
                                                       int d4, int H, int per_head, int band,
                                                       int hb4) {
  const int lane = threadIdx.x & 63;
  __shared__ uint32_t hmax[QZ_LDS_HEADS];
  const int nslots = per_head ? min(H, QZ_LDS_HEADS) : 1;
  for (int i = threadIdx.x; i < nslots; i += QZ_THREADS) hmax[i] = 0u;
  __syncthreads();
  const int r0 = blockIdx.x * band;
  const int r1 = min(rows, r0 + band);
  uint32_t all = 0u;                       // per-tensor mode: this thread's maximum
  for (int c = threadIdx.x; c < L4; c += QZ_THREADS) {
    const float4* col = (const float4*)x + (size_t)r0 * L4 + c;
    float m0 = 0.f, m1 = 0.f;
    int r = r0;
    for (; r + 1 < r1; r += 2) {           // two loads in flight per thread
      float4 a = col[0], b = col[L4];
      col += 2 * (size_t)L4;
      if (hb4) {
        a = wht_block(a, hb4, lane);
        b = wht_block(b, hb4, lane);
      }
      m0 = fmaxf(m0, fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))));
      m1 = fmaxf(m1, fmaxf(fmaxf(fabsf(b.x), fabsf(b.y)), fmaxf(fabsf(b.z), fabsf(b.w))));
    }
    if (r < r1) {
      float4 a = col[0];
      if (hb4) a = wht_block(a, hb4, lane);
      m0 = fmaxf(m0, fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))));
    }
    const uint32_t u = __float_as_uint(fmaxf(m0, m1));
    if (!per_head) {
      all = max(all, u);
    } else {
      const int h = c / d4;
      if (h < QZ_LDS_HEADS) atomicMax(&hmax[h], u);
      else atomicMax(amax_bits + h, u);
    }
  }
  if (!per_head) {
    for (int off = 32; off > 0; off >>= 1) all = max(all, (uint32_t)__shfl_xor((int)all, off));
    if ((threadIdx.x & 63) == 0) atomicMax(&hmax[0], all);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nslots; i += QZ_THREADS)
    if (hmax[i] != 0u) atomicMax(amax_bits + i, hmax[i]);
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
                                                       uint32_t* __restrict__ out,
                                                       const uint32_t* amax_bits, int rows,
                                                       int L4, int d4, int per_head, int band,
                                                       int hb4) {
  const int lane = threadIdx.x & 63;
  const int r0 = blockIdx.x * band;
  const int r1 = min(rows, r0 + band);
  const float ds_t = per_head ? 0.f : descale_of(amax_bits[0]);
  for (int c = threadIdx.x; c < L4; c += QZ_THREADS) {
    const float ds = per_head ? descale_of(amax_bits[c / d4]) : ds_t;
    const float4* src = (const float4*)x + (size_t)r0 * L4 + c;
    uint32_t* dst = out + (size_t)r0 * L4 + c;
    int r = r0;
    for (; r + 1 < r1; r += 2) {
      float4 a = src[0], b = src[L4];
      src += 2 * (size_t)L4;
      if (hb4) {
        a = wht_block(a, hb4, lane);
        b = wht_block(b, hb4, lane);
      }
      dst[0] = e4m3_code(a.x / ds) | (e4m3_code(a.y / ds) << 8) | (e4m3_code(a.z / ds) << 16) |
               (e4m3_code(a.w / ds) << 24);
      dst[L4] = e4m3_code(b.x / ds) | (e4m3_code(b.y / ds) << 8) | (e4m3_code(b.z / ds) << 16) |
                (e4m3_code(b.w / ds) << 24);
      dst += 2 * (size_t)L4;
    }
    if (r < r1) {
      float4 a = src[0];
      if (hb4) a = wht_block(a, hb4, lane);
      dst[0] = e4m3_code(a.x / ds) | (e4m3_code(a.y / ds) << 8) | (e4m3_code(a.z / ds) << 16) |
               (e4m3_code(a.w / ds) << 24);
    }
  }
}

// descale = (absmax / 448) * post, post = 1 or the Hadamard normalisation 1/sqrt(hb).
__global__ void qz_finalize(float* descale, int n, float post) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) descale[i] = descale_of(__float_as_uint(descale[i])) * post;
}

hipError_t launch_quantize_e4m3(const float* x, uint8_t* out, float* descale, int B, int N,
                                int H, int d, int per_head, int hadamard, hipStream_t stream) {
  const int rows = B * N;
  // Hadamard block: the largest power of two dividing d, at most 128 (d is a multiple of
  // 4); in float4 columns, 0 when no rotation is asked for.
  int hb = 4;
  while (hb < 128 && d % (2 * hb) == 0) hb *= 2;
  const int hb4 = hadamard ? hb / 4 : 0;
  const float post = hadamard ? (float)(1.0 / sqrt((double)hb)) : 1.f;
  const int ns = per_head ? H : 1;
  const int L4 = H * (d / 4), d4 = d / 4;
  const int band = (rows + QZ_TARGET_WGS - 1) / QZ_TARGET_WGS;
  const int nwg = (rows + band - 1) / band;
  uint32_t* bits = (uint32_t*)descale;
  hipLaunchKernelGGL(qz_clear, dim3((ns + 255) / 256), dim3(256), 0, stream, bits, ns);
  hipLaunchKernelGGL(qz_absmax, dim3(nwg), dim3(QZ_THREADS), 0, stream, x, bits, rows, L4, d4,
                     H, per_head, band, hb4);
  hipLaunchKernelGGL(qz_encode, dim3(nwg), dim3(QZ_THREADS), 0, stream, x, (uint32_t*)out,
                     (const uint32_t*)bits, rows, L4, d4, per_head, band, hb4);
  hipLaunchKernelGGL(qz_finalize, dim3((ns + 255) / 256), dim3(256), 0, stream, descale, ns,
                     post);
  return hipGetLastError();
}

}  // namespace attn
