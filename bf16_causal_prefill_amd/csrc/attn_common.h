// Device helpers shared by the causal attention kernels (gfx950): vector types,
// constants of the softmax, LDS swizzles, direct-to-LDS copies, the workgroup-to-tile
// map and small cross-lane and scheduling helpers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v2s __attribute__((ext_vector_type(2)));

constexpr int DV = 128;    // value head dim (both supported shapes)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
// Offset of the FP8 probability code: code = 8 * log2(p) + C0 before the integer
// conversion, which rounds to nearest; 56 - 0.5 makes it act as truncation of
// 8*log2(p) + 56, which keeps the piecewise-linear code close to unbiased.
constexpr float LEANP_C0 = 55.5f;
// Lazy-rescale threshold in log2 units (probabilities relative to a stale max stay
// below 2^TAU).
constexpr float TAU = 8.0f;

// The 16-byte chunks of key row k of the LDS V tile are XOR-permuted by vswz<FP8>(k).
// A transposing operand read makes each 16-lane group fetch 16 bytes from each of 8
// (fp8) or 4 (bf16) key rows that share their chunk index, and two groups (the two
// 16-channel halves of a 32-channel block) are served per LDS cycle; this permutation
// puts those 16 row segments in 16 different 4-bank groups.
template <bool FP8>
__device__ __forceinline__ int vswz(int key) {
  return FP8 ? 2 * ((key >> 1) & 1) + 4 * ((key >> 3) & 1) : 4 * (key & 3);
}

// The 16-byte chunks of key row r of the LDS K tile are XOR-permuted by kswz<R16>(r)
// (R16 = chunks per row).  An MFMA operand read makes 16 lanes fetch the same chunk of
// 16 consecutive rows; with unpadded rows those would share a handful of banks, the
// permutation spreads them over all 16 4-bank groups.  It never leaves the row (for
// 12 and 24 chunks it permutes within aligned groups of 4 or 8).
template <int R16>
__device__ __forceinline__ int kswz(int row) {
  static_assert(R16 == 8 || R16 == 12 || R16 == 16 || R16 == 24, "K row size");
  if (R16 == 16) return row & 15;
  if (R16 == 12) return (row >> 2) & 3;
  return (row >> 1) & 7;
}

typedef int i32x4_t __attribute__((ext_vector_type(4)));

// 16 bytes per lane from global memory straight into LDS: lane i's bytes land at
// lds_addr + 16 i.  `rsrc` is a raw buffer descriptor (reads past its range return
// zeros), `voff` the lane's byte offset in it.  Written as an instruction the compiler
// does not model, so it neither waits for these copies at every barrier nor before LDS
// reads of other stages: the caller waits with s_waitcnt vmcnt before publishing.
__device__ __forceinline__ void copy16_to_lds(i32x4_t rsrc, uint32_t voff, uint32_t lds_addr) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(lds_addr) : "memory", "m0");
#endif
}

// A raw buffer descriptor for `bytes` bytes at `base` (wave-uniform).
__device__ __forceinline__ i32x4_t buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  i32x4_t r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;
  return r;
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Maps the flat workgroup id to (batch, query head, query tile).  Heaviest causal
// tiles (last query rows) go first.  When B*Hkv is a multiple of 8, each of the 8
// XCDs (workgroups are dealt to XCDs round-robin) gets whole KV-head groups, so the
// query heads that share K/V run on one XCD and share its L2.  On that path the odd
// XCD of each pair (2i, 2i+1) hands its sw = p.xcd_swap heaviest items to the even
// one, which runs them first, and takes the even one's items at places j .. j+sw-1 of
// its list (j = p.xcd_swap_at >= sw, lighter ones), run where their weight puts them:
// both keep the same number of workgroups, which round-robin dealing fixes.  The odd
// XCDs measured a few percent slower on every MI355X tried, and a launch ends with its
// slowest XCD.  Within an XCD, workgroups are dealt in order to its 4 shader engines,
// place k to engine (k mod 4) (a fixed order per XCD, measured), and a workgroup waits
// for a free CU on its own engine.  With p.se_rotate each group of 4 consecutive places
// takes the group's 4 items rotated by the group index, so every engine gets, over 4
// groups, every position of a group (the heavier and the lighter row when a row has
// fewer than 4 items, every head of a KV group when it has 4) instead of always the
// same one; the launcher sets it for the FP8 kernels, except for the exact-LSE one when
// a row has 4 or more items: the cases it measured faster.
__host__ __device__ __forceinline__ void map_block(int bid, const FwdParams& p, int& b, int& h,
                                                   int& qt) {
  const int G = p.Hq / p.Hkv;
  const int BHkv = p.B * p.Hkv;
  if ((BHkv & 7) == 0) {
    int xcd = bid & 7, local = bid >> 3;      // local: the item's place in its XCD's list
    const int per = (BHkv >> 3) * G;
    if (p.se_rotate) {
      const int grp = local >> 2;
      if (4 * grp + 4 <= p.n_qtiles * per) local = 4 * grp + (((local & 3) + grp) & 3);
    }
    const int sw = p.xcd_swap, j = p.xcd_swap_at;
    if (sw > 0) {
      if ((xcd & 1) == 0) {
        if (local < sw) xcd |= 1;             // the odd partner's heaviest items,
        else if (local < j + sw) local -= sw; // then its own before place j,
                                              // then its own after place j + sw - 1
      } else {
        if (local < j - sw) local += sw;      // its own after its sw heaviest,
        else if (local < j) {                 // then the even partner's j .. j+sw-1,
          xcd &= ~1;
          local += sw;
        }                                     // then its own from place j
      }
    }
    const int t = local / per, r = local - t * per;
    qt = p.n_qtiles - 1 - t;
    const int og = r / G, hg = r - og * G;
    const int bk = xcd + 8 * og;
    b = bk / p.Hkv;
    h = (bk - b * p.Hkv) * G + hg;
  } else {
    const int per = p.B * p.Hq;
    const int t = bid / per, r = bid - t * per;
    qt = p.n_qtiles - 1 - t;
    b = r / p.Hq;
    h = r - b * p.Hq;
  }
}

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32); }

// max(x[lane], x[lane ^ 32]) in every lane: one lane-half swap and one max.
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// An empty instruction that reads x: the value must be computed by this point.
template <typename T>
__device__ __forceinline__ void keep_in_vgprs(const T& x) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" ::"v"(x));
#endif
}

// Eight e4m3 codes (bytes of lo, then hi, in order) as bf16, exactly: every e4m3 value
// is a bf16 value (3 of bf16's 7 mantissa bits, exponents 2^-9 .. 2^8).
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.f, true);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

__device__ __forceinline__ i32x8 load_i32x8(const char* p) {
  const uint4 a = *(const uint4*)p;
  const uint4 b = *(const uint4*)(p + 16);
  i32x8 f;
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  return f;
}

}  // namespace attn
