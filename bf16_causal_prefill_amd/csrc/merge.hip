// Merge of two partial attentions of the same queries over disjoint key sets.
//
// Each partial is normalised over its own keys, so with m = max(lse_a, lse_b) the
// exact combination is O = (e^(lse_a - m) O_a + e^(lse_b - m) O_b) / (e^(lse_a - m) +
// e^(lse_b - m)) and LSE = m + ln(e^(lse_a - m) + e^(lse_b - m)).  A partial with
// LSE = -inf (no keys) gets weight 0.  This is the combination step that splitting the
// key axis (KV-prefix chunks, context-parallel rings) needs.  O is bf16 (B, N, Hq, d_v),
// LSE fp32 (B, Hq, N); computed in fp32, O rounded to nearest even.
//
// Work split: d_v/8 lanes per (b, n, h) row, 16 bytes each, whole rows inside one wave,
// so the lanes of a row read both LSE values in the same instruction before the row's
// first lane writes the merged LSE: the outputs may alias the inputs.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kernels.h"

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int MG_THREADS = 256;

__global__ __launch_bounds__(MG_THREADS) void attn_merge_kernel(
    const bf16x8* o_a, const float* lse_a, const bf16x8* o_b, const float* lse_b, bf16x8* o,
    float* lse, long long rows, int c8, int Hq, int N) {
  const int lane = threadIdx.x & 63;
  const int rpw = 64 / c8;                        // rows per wave
  const int sub = lane / c8, chunk = lane - sub * c8;
  const long long waves = (long long)gridDim.x * (MG_THREADS / 64);
  for (long long w = (long long)blockIdx.x * (MG_THREADS / 64) + (threadIdx.x >> 6);
       w * rpw < rows; w += waves) {
    const long long r = w * rpw + sub;            // row (b, n, h), h fastest
    if (r >= rows) continue;
    const int h = (int)(r % Hq);
    const long long bn = r / Hq;
    const long long b = bn / N, n = bn - b * N;
    const size_t li = ((size_t)b * Hq + h) * N + n;
    const float la = lse_a[li], lb = lse_b[li];
    const float m = fmaxf(la, lb);
    float wa = 0.f, wb = 0.f, lo = -INFINITY;
    if (m != -INFINITY) {
      wa = expf(la - m);
      wb = expf(lb - m);
      const float sum = wa + wb;
      lo = m + logf(sum);
      wa /= sum;
      wb /= sum;
    }
    const size_t oi = (size_t)r * c8 + chunk;
    const bf16x8 xa = o_a[oi], xb = o_b[oi];
    bf16x8 y;
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = (__bf16)(wa * (float)xa[e] + wb * (float)xb[e]);
    o[oi] = y;
    if (lse && chunk == 0) lse[li] = lo;
  }
}

hipError_t launch_attn_merge(const void* o_a, const float* lse_a, const void* o_b,
                             const float* lse_b, void* o, float* lse, int B, int N, int Hq,
                             int d_v, hipStream_t stream) {
  const long long rows = (long long)B * N * Hq;
  const int c8 = d_v / 8;
  const long long waves = (rows + (64 / c8) - 1) / (64 / c8);
  const long long blocks = (waves + (MG_THREADS / 64) - 1) / (MG_THREADS / 64);
  const unsigned grid = (unsigned)(blocks < 65536 ? blocks : 65536);
  hipLaunchKernelGGL(attn_merge_kernel, dim3(grid), dim3(MG_THREADS), 0, stream,
                     (const bf16x8*)o_a, lse_a, (const bf16x8*)o_b, lse_b, (bf16x8*)o, lse, rows,
                     c8, Hq, N);
  return hipGetLastError();
}

}  // namespace attn
