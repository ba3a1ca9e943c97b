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
// Passes 2 and 3 transform the unnormalised blocks in float32 (wht_block, one kernel
// instantiation per block size, cross-lane stages on the DPP lane network) and the
// normalisation 1/sqrt(hb) goes into the descale, so the codes are those of x H.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kernels.h"
#include "quantize_common.h"

namespace attn {

constexpr int QZ_THREADS = 256;
constexpr int QZ_LDS_HEADS = 1024;   // per-head maxima kept in LDS up to this many heads
// Workgroups per pass (about four per CU) and rows in flight per thread: measured best
// of 512/768/1024/2048/4096 workgroups and 2/4/8 rows on the 16K-32K-row tensors (with
// the non-temporal loads as well).
constexpr int QZ_TARGET_WGS = 1024;
constexpr int QZ_U = 4;

// Work split shared by both passes.  The tensor is B*N rows of L4 = H*d/4 float4
// values (head h owns columns h*d4 .. h*d4 + d4-1, d4 = d/4).  A workgroup takes a band
// of `band` consecutive rows; thread t handles the columns t, t + 256, ... of every row
// in the band, so each column's head is fixed per thread and the workgroup reads whole
// rows (contiguous memory) at a time, QZ_U rows in flight per thread.

__global__ void qz_clear(uint32_t* amax_bits, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) amax_bits[i] = 0u;
}

// x[lane ^ M] within the wave (M < 32): quad permutations and row shifts of the DPP
// lane network for M <= 8 (a row shift serves the 4-lane banks whose partner lies in
// its direction; two of them, with complementary bank masks, cover the row), a
// swizzle for M = 16.
template <int M>
__device__ __forceinline__ float lane_xor(float x) {
  const int v = __float_as_int(x);
  int r;
  if constexpr (M == 1) {
    r = __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);         // quad_perm 1,0,3,2
  } else if constexpr (M == 2) {
    r = __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);         // quad_perm 2,3,0,1
  } else if constexpr (M == 4) {
    r = __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xA, false);  // row_shr:4, banks 1,3
    r = __builtin_amdgcn_update_dpp(r, v, 0x104, 0xF, 0x5, false);  // row_shl:4, banks 0,2
  } else if constexpr (M == 8) {
    r = __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xC, false);  // row_shr:8, banks 2,3
    r = __builtin_amdgcn_update_dpp(r, v, 0x108, 0xF, 0x3, false);  // row_shl:8, banks 0,1
  } else {
    static_assert(M == 16, "lane_xor: M must be 1, 2, 4, 8 or 16");
    r = __builtin_amdgcn_ds_swizzle(v, 0x1F | (16 << 10));          // and 31, xor 16
  }
  return __int_as_float(r);
}

// Walsh-Hadamard transform (Sylvester order, unnormalised) of a block of hb = 4*HB4
// consecutive channels held by HB4 consecutive lanes, 4 channels each (blocks start at
// multiples of HB4 lanes).  Radix-2 butterflies in float32, stage half-sizes 1, 2, 4,
// ..., hb/2 in that order: the element with the stage bit clear becomes a + b, its
// partner a - b (written q - v = fma(-1, v, q) in the upper lane, one rounding as for
// the subtraction).  Every lane of a block must be active.
template <int M, int HB4>
__device__ __forceinline__ float4 wht_stages(float4 v, int lane) {
  if constexpr (M < HB4) {
    const float sg = (lane & M) ? -1.f : 1.f;
    v = make_float4(fmaf(sg, v.x, lane_xor<M>(v.x)), fmaf(sg, v.y, lane_xor<M>(v.y)),
                    fmaf(sg, v.z, lane_xor<M>(v.z)), fmaf(sg, v.w, lane_xor<M>(v.w)));
    return wht_stages<2 * M, HB4>(v, lane);
  } else {
    return v;
  }
}

template <int HB4>
__device__ __forceinline__ float4 wht_block(float4 v, int lane) {
  if constexpr (HB4 == 0) {
    return v;
  } else {
    const float a0 = v.x + v.y, a1 = v.x - v.y, a2 = v.z + v.w, a3 = v.z - v.w;
    v = make_float4(a0 + a2, a1 + a3, a0 - a2, a1 - a3);
    return wht_stages<1, HB4>(v, lane);
  }
}

__device__ __forceinline__ float absmax4(float4 a) {
  return fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w)));
}

// Bit patterns of non-negative floats order like the values, so maxima are taken as
// unsigned integers (atomicMax is then exact and order-independent).  With HB4 > 0
// the values are the Walsh-Hadamard transforms of blocks of 4*HB4 channels.
// Workgroup `wg` of a pass over one tensor (hmax: the workgroup's LDS maxima).
template <int HB4>
__device__ __forceinline__ void qz_absmax_body(const float* __restrict__ x, uint32_t* amax_bits,
                                               int rows, int L4, int d4, int H, int per_head,
                                               int band, int wg, uint32_t* hmax) {
  const int lane = threadIdx.x & 63;
  const int nslots = per_head ? min(H, QZ_LDS_HEADS) : 1;
  for (int i = threadIdx.x; i < nslots; i += QZ_THREADS) hmax[i] = 0u;
  __syncthreads();
  const int r0 = wg * band;
  const int r1 = min(rows, r0 + band);
  uint32_t all = 0u;                       // per-tensor mode: this thread's maximum
  for (int c = threadIdx.x; c < L4; c += QZ_THREADS) {
    const float4* col = (const float4*)x + (size_t)r0 * L4 + c;
    float m[QZ_U];
#pragma unroll
    for (int u = 0; u < QZ_U; ++u) m[u] = 0.f;
    int r = r0;
    for (; r + QZ_U <= r1; r += QZ_U) {    // QZ_U loads in flight per thread
      float4 a[QZ_U];
#pragma unroll
      for (int u = 0; u < QZ_U; ++u) a[u] = load_stream(col + (size_t)u * L4);
      col += (size_t)QZ_U * L4;
#pragma unroll
      for (int u = 0; u < QZ_U; ++u) m[u] = fmaxf(m[u], absmax4(wht_block<HB4>(a[u], lane)));
    }
    for (; r < r1; ++r) {
      m[0] = fmaxf(m[0], absmax4(wht_block<HB4>(load_stream(col), lane)));
      col += L4;
    }
    float mm = m[0];
#pragma unroll
    for (int u = 1; u < QZ_U; ++u) mm = fmaxf(mm, m[u]);
    const uint32_t u = __float_as_uint(mm);
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

template <int HB4>
__global__ __launch_bounds__(QZ_THREADS) void qz_absmax(const float* __restrict__ x,
                                                       uint32_t* amax_bits, int rows, int L4,
                                                       int d4, int H, int per_head, int band) {
  __shared__ uint32_t hmax[QZ_LDS_HEADS];
  qz_absmax_body<HB4>(x, amax_bits, rows, L4, d4, H, per_head, band, blockIdx.x, hmax);
}

// Rows r0 .. r1-1 of float4 column c (FAST: the branch-free word for a divisor in range).
template <int HB4, bool FAST>
__device__ __forceinline__ void encode_column(const float4* src, uint32_t* dst, int r0, int r1,
                                              int L4, float ds, int lane) {
  const Divisor dv = make_divisor(ds);
  auto word = [&](float4 a) {
    return FAST ? e4m3_word_fast(wht_block<HB4>(a, lane), dv)
                : e4m3_word(wht_block<HB4>(a, lane), ds);
  };
  int r = r0;
  for (; r + QZ_U <= r1; r += QZ_U) {    // QZ_U loads in flight per thread
    float4 a[QZ_U];
#pragma unroll
    for (int u = 0; u < QZ_U; ++u) a[u] = load_stream(src + (size_t)u * L4);
    src += (size_t)QZ_U * L4;
#pragma unroll
    for (int u = 0; u < QZ_U; ++u) dst[(size_t)u * L4] = word(a[u]);
    dst += (size_t)QZ_U * L4;
  }
  for (; r < r1; ++r) {
    dst[0] = word(load_stream(src));
    src += L4;
    dst += L4;
  }
}

// amax_bits holds the absmax bits (ds_final == 0) or the finished descale (ds_final == 1).
template <int HB4>
__device__ __forceinline__ void qz_encode_body(const float* __restrict__ x,
                                               uint32_t* __restrict__ out,
                                               const uint32_t* amax_bits, int rows, int L4,
                                               int d4, int per_head, int band, int ds_final,
                                               int wg) {
  const int lane = threadIdx.x & 63;
  const int r0 = wg * band;
  const int r1 = min(rows, r0 + band);
  auto ds_of = [&](uint32_t bits) { return ds_final ? __uint_as_float(bits) : descale_of(bits); };
  const float ds_t = per_head ? 0.f : ds_of(amax_bits[0]);
  for (int c = threadIdx.x; c < L4; c += QZ_THREADS) {
    const float ds = per_head ? ds_of(amax_bits[c / d4]) : ds_t;
    const float4* src = (const float4*)x + (size_t)r0 * L4 + c;
    uint32_t* dst = out + (size_t)r0 * L4 + c;
    if (fast_divisor(ds))
      encode_column<HB4, true>(src, dst, r0, r1, L4, ds, lane);
    else
      encode_column<HB4, false>(src, dst, r0, r1, L4, ds, lane);
  }
}

template <int HB4>
__global__ __launch_bounds__(QZ_THREADS) void qz_encode(const float* __restrict__ x,
                                                       uint32_t* __restrict__ out,
                                                       const uint32_t* amax_bits, int rows,
                                                       int L4, int d4, int per_head, int band,
                                                       int ds_final) {
  qz_encode_body<HB4>(x, out, amax_bits, rows, L4, d4, per_head, band, ds_final, blockIdx.x);
}

// descale[i] <- the Q descale above from the absmax it holds (as float bits, which for a
// non-negative float are the float itself); query head (or tensor) i pairs with
// k_descale[i / group].
__global__ void qz_finalize_q_pow2(float* descale, int n, const float* k_descale, int group,
                                   float sl) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) descale[i] = pow2_q_descale(descale[i], k_descale[i / group], sl);
}

// descale = (absmax / 448) * post, post = 1 or the Hadamard normalisation 1/sqrt(hb).
__global__ void qz_finalize(float* descale, int n, float post) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) descale[i] = descale_of(__float_as_uint(descale[i])) * post;
}

template <int HB4>
static void qz_passes(const float* x, uint8_t* out, uint32_t* bits, int rows, int L4, int d4,
                      int H, int per_head, int band, int nwg, hipStream_t stream) {
  hipLaunchKernelGGL(qz_absmax<HB4>, dim3(nwg), dim3(QZ_THREADS), 0, stream, x, bits, rows, L4,
                     d4, H, per_head, band);
  hipLaunchKernelGGL(qz_encode<HB4>, dim3(nwg), dim3(QZ_THREADS), 0, stream, x, (uint32_t*)out,
                     (const uint32_t*)bits, rows, L4, d4, per_head, band, 0);
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
  switch (hb4) {
    case 0: qz_passes<0>(x, out, bits, rows, L4, d4, H, per_head, band, nwg, stream); break;
    case 1: qz_passes<1>(x, out, bits, rows, L4, d4, H, per_head, band, nwg, stream); break;
    case 2: qz_passes<2>(x, out, bits, rows, L4, d4, H, per_head, band, nwg, stream); break;
    case 4: qz_passes<4>(x, out, bits, rows, L4, d4, H, per_head, band, nwg, stream); break;
    case 8: qz_passes<8>(x, out, bits, rows, L4, d4, H, per_head, band, nwg, stream); break;
    case 16: qz_passes<16>(x, out, bits, rows, L4, d4, H, per_head, band, nwg, stream); break;
    default: qz_passes<32>(x, out, bits, rows, L4, d4, H, per_head, band, nwg, stream); break;
  }
  hipLaunchKernelGGL(qz_finalize, dim3((ns + 255) / 256), dim3(256), 0, stream, descale, ns,
                     post);
  return hipGetLastError();
}

hipError_t launch_quantize_e4m3_q_pow2(const float* x, uint8_t* out, float* descale, int B,
                                       int N, int H, int d, int per_head,
                                       const float* k_descale, int Hkv, float softmax_scale,
                                       hipStream_t stream) {
  const int rows = B * N;
  const int ns = per_head ? H : 1;
  const int group = per_head ? H / Hkv : 1;
  const int L4 = H * (d / 4), d4 = d / 4;
  const int band = (rows + QZ_TARGET_WGS - 1) / QZ_TARGET_WGS;
  const int nwg = (rows + band - 1) / band;
  uint32_t* bits = (uint32_t*)descale;
  const float sl = softmax_scale * 1.4426950408889634f;
  hipLaunchKernelGGL(qz_clear, dim3((ns + 255) / 256), dim3(256), 0, stream, bits, ns);
  hipLaunchKernelGGL(qz_absmax<0>, dim3(nwg), dim3(QZ_THREADS), 0, stream, x, bits, rows, L4,
                     d4, H, per_head, band);
  hipLaunchKernelGGL(qz_finalize_q_pow2, dim3((ns + 255) / 256), dim3(256), 0, stream, descale,
                     ns, k_descale, group, sl);
  hipLaunchKernelGGL(qz_encode<0>, dim3(nwg), dim3(QZ_THREADS), 0, stream, x, (uint32_t*)out,
                     (const uint32_t*)bits, rows, L4, d4, per_head, band, 1);
  return hipGetLastError();
}

// ---- Q, K and V in one call (quantize_e4m3_qkv) ------------------------------------
// The same passes over the three tensors, one launch each: the grid is the three
// tensors' workgroups back to back (Q's first, the largest), each workgroup running the
// pass of the tensor its index falls in.  Codes and descales are those of the separate
// calls: the same per-element arithmetic, and the finalize below forms the same values.
struct QzTensor {
  const float* x;
  uint32_t* out;
  uint32_t* bits;      // the tensor's descale array (absmax bits until finalized)
  int rows, L4, d4, H, band;
};
struct QzSet {
  QzTensor t0, t1, t2;
  int wg1, wg2;        // first workgroups of tensors 1 and 2
  int per_head;
};

// Tensor of workgroup w (field by field, so the set stays in scalar registers).
__device__ __forceinline__ QzTensor qz_pick(const QzSet& s, int w, int& wg) {
  const bool in2 = w >= s.wg2, in1 = !in2 && w >= s.wg1;
  wg = in2 ? w - s.wg2 : in1 ? w - s.wg1 : w;
  QzTensor t;
  t.x = in2 ? s.t2.x : in1 ? s.t1.x : s.t0.x;
  t.out = in2 ? s.t2.out : in1 ? s.t1.out : s.t0.out;
  t.bits = in2 ? s.t2.bits : in1 ? s.t1.bits : s.t0.bits;
  t.rows = in2 ? s.t2.rows : in1 ? s.t1.rows : s.t0.rows;
  t.L4 = in2 ? s.t2.L4 : in1 ? s.t1.L4 : s.t0.L4;
  t.d4 = in2 ? s.t2.d4 : in1 ? s.t1.d4 : s.t0.d4;
  t.H = in2 ? s.t2.H : in1 ? s.t1.H : s.t0.H;
  t.band = in2 ? s.t2.band : in1 ? s.t1.band : s.t0.band;
  return t;
}

__global__ void qz_clear3(uint32_t* a, int na, uint32_t* b, int nb, uint32_t* c, int nc) {
  for (int i = threadIdx.x; i < na + nb + nc; i += blockDim.x) {
    if (i < na) a[i] = 0u;
    else if (i < na + nb) b[i - na] = 0u;
    else c[i - na - nb] = 0u;
  }
}

__global__ __launch_bounds__(QZ_THREADS) void qz_absmax3(QzSet s) {
  __shared__ uint32_t hmax[QZ_LDS_HEADS];
  int wg;
  const QzTensor t = qz_pick(s, blockIdx.x, wg);
  qz_absmax_body<0>(t.x, t.bits, t.rows, t.L4, t.d4, t.H, s.per_head, t.band, wg, hmax);
}

// One workgroup: Q's descales first, while K's array still holds its absmax bits (the Q
// power-of-two descale pairs query head i with K's descale descale_of(bits[i / group]),
// the value K's finalize writes), then K's and V's.
__global__ void qz_finalize3(float* qd, int nq, float* kd, int nk, float* vd, int nv, int group,
                             int q_pow2, float sl) {
  for (int i = threadIdx.x; i < nq; i += blockDim.x)
    qd[i] = q_pow2 ? pow2_q_descale(qd[i], descale_of(__float_as_uint(kd[i / group])), sl)
                   : descale_of(__float_as_uint(qd[i]));
  __syncthreads();
  for (int i = threadIdx.x; i < nk; i += blockDim.x) kd[i] = descale_of(__float_as_uint(kd[i]));
  for (int i = threadIdx.x; i < nv; i += blockDim.x) vd[i] = descale_of(__float_as_uint(vd[i]));
}

__global__ __launch_bounds__(QZ_THREADS) void qz_encode3(QzSet s) {
  int wg;
  const QzTensor t = qz_pick(s, blockIdx.x, wg);
  qz_encode_body<0>(t.x, t.out, t.bits, t.rows, t.L4, t.d4, s.per_head, t.band, 1, wg);
}

hipError_t launch_quantize_e4m3_qkv(const float* q, const float* k, const float* v,
                                    uint8_t* q_out, uint8_t* k_out, uint8_t* v_out,
                                    float* q_descale, float* k_descale, float* v_descale,
                                    int B, int Nq, int Nk, int Hq, int Hkv, int d_qk, int d_v,
                                    int per_head, int q_pow2, float softmax_scale,
                                    hipStream_t stream) {
  auto tensor = [&](const float* x, uint8_t* out, float* ds, int rows, int H, int d, int& nwg) {
    QzTensor t;
    t.x = x;
    t.out = (uint32_t*)out;
    t.bits = (uint32_t*)ds;
    t.rows = rows;
    t.L4 = H * (d / 4);
    t.d4 = d / 4;
    t.H = H;
    t.band = (rows + QZ_TARGET_WGS - 1) / QZ_TARGET_WGS;
    nwg = (rows + t.band - 1) / t.band;
    return t;
  };
  int nq, nk, nv;
  QzSet s;
  s.t0 = tensor(q, q_out, q_descale, B * Nq, Hq, d_qk, nq);
  s.t1 = tensor(k, k_out, k_descale, B * Nk, Hkv, d_qk, nk);
  s.t2 = tensor(v, v_out, v_descale, B * Nk, Hkv, d_v, nv);
  s.wg1 = nq;
  s.wg2 = nq + nk;
  s.per_head = per_head;
  const int sq = per_head ? Hq : 1, skv = per_head ? Hkv : 1;
  hipLaunchKernelGGL(qz_clear3, dim3(1), dim3(256), 0, stream, s.t0.bits, sq, s.t1.bits, skv,
                     s.t2.bits, skv);
  hipLaunchKernelGGL(qz_absmax3, dim3(nq + nk + nv), dim3(QZ_THREADS), 0, stream, s);
  hipLaunchKernelGGL(qz_finalize3, dim3(1), dim3(256), 0, stream, q_descale, sq, k_descale, skv,
                     v_descale, skv, per_head ? Hq / Hkv : 1, q_pow2,
                     softmax_scale * 1.4426950408889634f);
  if (q_out) {
    hipLaunchKernelGGL(qz_encode3, dim3(nq + nk + nv), dim3(QZ_THREADS), 0, stream, s);
  } else {
    // Q's descales only (for the attention entry points that take float32 Q): the
    // encode pass covers K and V
    QzSet e = s;
    e.t0 = s.t1;
    e.t1 = s.t2;
    e.wg1 = nk;
    e.wg2 = nk + nv;
    hipLaunchKernelGGL(qz_encode3, dim3(nk + nv), dim3(QZ_THREADS), 0, stream, e);
  }
  return hipGetLastError();
}

}  // namespace attn
