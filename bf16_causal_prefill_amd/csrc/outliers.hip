// Joint e4m3 quantisation of Q and K that stores, per KV head, the channels with the
// largest products last in every row (for the FP8 attention that multiplies those
// channels exactly, attn_fwd_causal_fp8_outliers).
//
// Why: gfx950's FP8 matrix instructions add each run of 8 channel products after
// truncating every product toward zero to 13 bits below the run's largest exponent sum
// (e_q + e_k of the factors), so one
// channel whose Q or K magnitude is far above the others swamps the small products of
// its run, and on activations with outlier channels that moves scores and log-sum-exps
// by far more than the rounding of the inputs (the pages name the FP8 error of Q and K
// as the one that matters, spke.com "ZYFAのFP8アテンションの精度はどのくらいか?").
// Permuting the channels of Q and of K the same way leaves every score Q.K unchanged,
// so the quantiser is free to choose the stored channel order.
//
// Rule (the same steps as the oracle's quantize_e4m3_qk_outliers):
//   amax_q[h][c], amax_k[g][c]  max |x| over all (b, n), NaN elements ignored;
//   importance_g[c] = fl32(max_{h in g} amax_q[h][c]) * amax_k[g][c] (0 if either is 0);
//   the ATTN_OUTLIER_CHANNELS channels of largest importance (ties: the lower channel)
//   are stored last, in ascending channel order, after the others in ascending order;
//   codes and descales are exactly quantize_e4m3's (Q's descale optionally
//   quantize_e4m3_q_pow2's), only the channel order changes;
//   the last ATTN_OUTLIER_CHANNELS stored channels are also written as bf16 side arrays
//   (round to nearest even of the float32 quotient x / descale), which the exact-channel
//   attention multiplies on the BF16 matrix pipe instead of the codes.
//
// Kernels, in stream order:
//   1. clear    the per-channel absmax accumulators in the workspace
//   2. absmax   per-channel max |x| of Q and of K (64-column blocks times row bands per
//               workgroup, one integer atomicMax per channel and workgroup on the bits)
//   3. select   one workgroup per KV head: importance, rank, permutation, descales
//   4. encode   Q and K rows gathered through the permutation and encoded
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "../../include/attn.h"
#include "kernels.h"
#include "quantize_common.h"

namespace attn {

namespace {

constexpr int QO_THREADS = 256;
constexpr int QO_ABSMAX_WGS = 512;   // workgroups of the absmax pass (per tensor)
constexpr int QO_ROWS_IN_FLIGHT = 4;

__global__ void qo_clear(uint32_t* bits, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) bits[i] = 0u;
}

// Per-channel max |x| of a (rows, L4) float4 matrix (column c holds channels 4c .. 4c+3
// of the flat head-major channel index h*d + ch).  Workgroup (bx, by) takes the 64 float4
// columns 64 bx .. (one per lane, so each wave reads 1 KiB of a row) over the rows of band
// by; its four waves take every fourth row of the band, QO_ROWS_IN_FLIGHT rows at a time,
// and meet in LDS.  One integer atomicMax per channel and workgroup on the float bits
// (order-independent): splitting the columns over workgroups keeps the bands, and with
// them the atomics on each channel, few.  fmaxf ignores NaN elements.
__global__ __launch_bounds__(QO_THREADS) void qo_channel_absmax(const float* __restrict__ x,
                                                               uint32_t* amax_bits, int rows,
                                                               int L4, int band) {
  constexpr int NWAVE = QO_THREADS / 64;
  __shared__ float4 part[NWAVE][64];
  const int lane = threadIdx.x & 63, rp = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + lane;
  const int r0 = blockIdx.y * band;
  const int r1 = min(rows, r0 + band);
  float4 m = make_float4(0.f, 0.f, 0.f, 0.f);
  if (c < L4) {
    const float4* col = (const float4*)x + c;
    int r = r0 + rp;
    for (; r + NWAVE * (QO_ROWS_IN_FLIGHT - 1) < r1; r += NWAVE * QO_ROWS_IN_FLIGHT) {
      float4 a[QO_ROWS_IN_FLIGHT];
#pragma unroll
      for (int u = 0; u < QO_ROWS_IN_FLIGHT; ++u)
        a[u] = load_stream(col + (size_t)(r + NWAVE * u) * L4);
#pragma unroll
      for (int u = 0; u < QO_ROWS_IN_FLIGHT; ++u)
        m = make_float4(fmaxf(m.x, fabsf(a[u].x)), fmaxf(m.y, fabsf(a[u].y)),
                        fmaxf(m.z, fabsf(a[u].z)), fmaxf(m.w, fabsf(a[u].w)));
    }
    for (; r < r1; r += NWAVE) {
      const float4 a = load_stream(col + (size_t)r * L4);
      m = make_float4(fmaxf(m.x, fabsf(a.x)), fmaxf(m.y, fabsf(a.y)), fmaxf(m.z, fabsf(a.z)),
                      fmaxf(m.w, fabsf(a.w)));
    }
  }
  part[rp][lane] = m;
  __syncthreads();
  if (rp == 0 && c < L4) {
#pragma unroll
    for (int w = 1; w < NWAVE; ++w) {
      const float4 o = part[w][lane];
      m = make_float4(fmaxf(m.x, o.x), fmaxf(m.y, o.y), fmaxf(m.z, o.z), fmaxf(m.w, o.w));
    }
    uint32_t* dst = amax_bits + 4 * c;
    if (m.x > 0.f) atomicMax(dst + 0, __float_as_uint(m.x));
    if (m.y > 0.f) atomicMax(dst + 1, __float_as_uint(m.y));
    if (m.z > 0.f) atomicMax(dst + 2, __float_as_uint(m.z));
    if (m.w > 0.f) atomicMax(dst + 3, __float_as_uint(m.w));
  }
}

// Max over the workgroup of v (non-negative float bits compared as integers).
__device__ __forceinline__ uint32_t wg_max(uint32_t v, uint32_t* red) {
  for (int off = 32; off > 0; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t r = 0u;
  for (int w = 0; w < QO_THREADS / 64; ++w) r = max(r, red[w]);
  return r;
}

// Max over all n entries of bits (every thread of the workgroup takes part).
__device__ __forceinline__ uint32_t wg_max_of(const uint32_t* bits, int n, uint32_t* red) {
  uint32_t v = 0u;
  for (int i = threadIdx.x; i < n; i += QO_THREADS) v = max(v, bits[i]);
  return wg_max(v, red);
}

// Workgroup g (one per KV head; d <= QO_THREADS): the permutation of KV head g and the
// descales.  Per head: K's descale of head g and Q's of the heads in g's group.  Per
// tensor: workgroup 0 writes both (from the maxima over every channel).
__global__ __launch_bounds__(QO_THREADS) void qo_select(const uint32_t* amax_q,
                                                       const uint32_t* amax_k, uint8_t* perm,
                                                       float* q_descale, float* k_descale,
                                                       int Hq, int Hkv, int d, int per_head,
                                                       int q_pow2, float sl) {
  __shared__ float imp[256];
  __shared__ int chosen[256];
  __shared__ uint32_t red[QO_THREADS / 64];
  const int g = blockIdx.x;
  const int G = Hq / Hkv;
  const int c = threadIdx.x;
  if (c < d) {
    uint32_t aq = 0u;
    for (int h = g * G; h < (g + 1) * G; ++h) aq = max(aq, amax_q[(size_t)h * d + c]);
    const float fq = __uint_as_float(aq);
    const float fk = __uint_as_float(amax_k[(size_t)g * d + c]);
    imp[c] = (fq == 0.f || fk == 0.f) ? 0.f : fq * fk;
  }
  __syncthreads();
  if (c < d) {
    const float mine = imp[c];
    int rank = 0;
    for (int o = 0; o < d; ++o) {
      const float v = imp[o];
      rank += (v > mine || (v == mine && o < c)) ? 1 : 0;
    }
    chosen[c] = rank < ATTN_OUTLIER_CHANNELS ? 1 : 0;
  }
  __syncthreads();
  if (c < d) {
    int before = 0;                                    // channels below c in c's part
    for (int o = 0; o < c; ++o) before += chosen[o] == chosen[c] ? 1 : 0;
    const int pos = chosen[c] ? d - ATTN_OUTLIER_CHANNELS + before : before;
    perm[(size_t)g * d + pos] = (uint8_t)c;
  }
  if (per_head) {
    const float dk = descale_of(wg_max_of(amax_k + (size_t)g * d, d, red));
    if (threadIdx.x == 0) k_descale[g] = dk;
    for (int h = g * G; h < (g + 1) * G; ++h) {
      const uint32_t a = wg_max_of(amax_q + (size_t)h * d, d, red);
      if (threadIdx.x == 0)
        q_descale[h] = q_pow2 ? pow2_q_descale(__uint_as_float(a), dk, sl) : descale_of(a);
    }
  } else if (g == 0) {
    const float dk = descale_of(wg_max_of(amax_k, Hkv * d, red));
    const uint32_t a = wg_max_of(amax_q, Hq * d, red);
    if (threadIdx.x == 0) {
      k_descale[0] = dk;
      q_descale[0] = q_pow2 ? pow2_q_descale(__uint_as_float(a), dk, sl) : descale_of(a);
    }
  }
}

// bf16 bits of a float32, round to nearest even (overflow to infinity), NaN -> 0x7FC0.
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Stored word w of every row (4 channels): word w of row r belongs to head
// h = w / d4 at stored channels 4(w % d4) .. +3, which hold source channels
// perm[(h / G) * d + ...].  The gathered values are divided by the head's descale and
// encoded as in quantize_e4m3; words of the last ATTN_OUTLIER_CHANNELS stored channels
// also write the bf16 quotients into the side array exact (rows of H * 32 values).
__global__ __launch_bounds__(QO_THREADS) void qo_encode(const float* __restrict__ x,
                                                       uint32_t* __restrict__ out,
                                                       uint2* __restrict__ exact,
                                                       const float* descale,
                                                       const uint8_t* perm, long long words,
                                                       int L4, int d4, int G, int per_head) {
  const int d = 4 * d4;
  const float ds_t = per_head ? 0.f : descale[0];
  for (long long w = (long long)blockIdx.x * QO_THREADS + threadIdx.x; w < words;
       w += (long long)gridDim.x * QO_THREADS) {
    const long long r = w / L4;
    const int cw = (int)(w - r * L4);
    const int h = cw / d4;
    const int j = 4 * (cw - h * d4);
    const uint32_t src = *(const uint32_t*)(perm + (size_t)(h / G) * d + j);
    const float* row = x + (size_t)r * (size_t)(4 * L4) + (size_t)h * d;
    // (the clamp only keeps a malformed permutation inside the row; select writes
    // every entry below d)
    const uint32_t last = (uint32_t)d - 1u;
    const float4 a = make_float4(row[min(src & 0xffu, last)], row[min((src >> 8) & 0xffu, last)],
                                 row[min((src >> 16) & 0xffu, last)], row[min(src >> 24, last)]);
    const float ds = per_head ? descale[h] : ds_t;
    float4 qt;                     // the correctly rounded quotients x / ds
    if (fast_divisor(ds)) {
      const Divisor dv = make_divisor(ds);
      qt = make_float4(quotient(a.x, dv), quotient(a.y, dv), quotient(a.z, dv), quotient(a.w, dv));
      out[w] = e4m3_word_of_quotients(qt);
    } else {
      qt = make_float4(a.x / ds, a.y / ds, a.z / ds, a.w / ds);
      out[w] = e4m3_word(a, ds);
    }
    const int js = j - (d - ATTN_OUTLIER_CHANNELS);   // position among the exact channels
    if (js >= 0) {
      const int H = L4 / d4;
      exact[((size_t)r * H + h) * (ATTN_OUTLIER_CHANNELS / 4) + js / 4] =
          make_uint2(bf16_bits(qt.x) | (bf16_bits(qt.y) << 16),
                     bf16_bits(qt.z) | (bf16_bits(qt.w) << 16));
    }
  }
}

// Scratch of quantize_e4m3_qk_outliers_noalloc: the per-channel absmax accumulators,
// (Hq + Hkv) * d words at most ATTN_NOALLOC_SCRATCH_WORDS.  One copy per device, held
// until the process ends; host code uses the device address from hipGetSymbolAddress
// (scratch_ptr below), never this name.
__device__ __align__(256) uint32_t scratch[ATTN_NOALLOC_SCRATCH_WORDS];

}  // namespace

// Device address of this device's scratch array, looked up once per device with that
// device current (the first call on it); nullptr if the lookup fails.
uint32_t* scratch_ptr(int device) {
  static std::mutex mu;
  static uint32_t* ptrs[kMaxDevices] = {};
  static bool done[kMaxDevices] = {};
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!done[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;          // not cached: a later call may retry
    }
    ptrs[device] = (uint32_t*)p;
    done[device] = true;
  }
  return ptrs[device];
}

hipError_t launch_quantize_e4m3_qk_outliers(const float* q, const float* k, uint8_t* q_out,
                                            uint8_t* k_out, void* q_exact, void* k_exact,
                                            float* q_descale, float* k_descale, uint8_t* perm,
                                            uint32_t* workspace, int B, int N, int Hq,
                                            int Hkv, int d, int per_head, int q_pow2,
                                            float softmax_scale, hipStream_t stream) {
  const int rows = B * N;
  const int d4 = d / 4;
  uint32_t* amax_q = workspace;
  uint32_t* amax_k = workspace + (size_t)Hq * d;
  const int nws = (Hq + Hkv) * d;
  hipLaunchKernelGGL(qo_clear, dim3((nws + 255) / 256), dim3(256), 0, stream, workspace, nws);
  // about QO_ABSMAX_WGS workgroups per tensor: 64-column blocks times row bands
  auto absmax = [&](const float* x, uint32_t* amax, int L4) {
    const int cb = (L4 + 63) / 64;
    const int nb0 = std::max(1, std::min(rows, QO_ABSMAX_WGS / cb));
    const int band = (rows + nb0 - 1) / nb0;
    const int nb = (rows + band - 1) / band;
    hipLaunchKernelGGL(qo_channel_absmax, dim3(cb, nb), dim3(QO_THREADS), 0, stream, x, amax,
                       rows, L4, band);
  };
  absmax(q, amax_q, Hq * d4);
  absmax(k, amax_k, Hkv * d4);
  const float sl = softmax_scale * 1.4426950408889634f;
  hipLaunchKernelGGL(qo_select, dim3(Hkv), dim3(QO_THREADS), 0, stream, (const uint32_t*)amax_q,
                     (const uint32_t*)amax_k, perm, q_descale, k_descale, Hq, Hkv, d, per_head,
                     q_pow2, sl);
  const long long wq = (long long)rows * Hq * d4, wk = (long long)rows * Hkv * d4;
  auto grid = [](long long words) {
    return (unsigned)std::min<long long>((words + QO_THREADS - 1) / QO_THREADS, 8192);
  };
  hipLaunchKernelGGL(qo_encode, dim3(grid(wq)), dim3(QO_THREADS), 0, stream, q,
                     (uint32_t*)q_out, (uint2*)q_exact, (const float*)q_descale,
                     (const uint8_t*)perm, wq, Hq * d4, d4, Hq / Hkv, per_head);
  hipLaunchKernelGGL(qo_encode, dim3(grid(wk)), dim3(QO_THREADS), 0, stream, k,
                     (uint32_t*)k_out, (uint2*)k_exact, (const float*)k_descale,
                     (const uint8_t*)perm, wk, Hkv * d4, d4, 1, per_head);
  return hipGetLastError();
}

}  // namespace attn
