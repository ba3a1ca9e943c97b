// Causal forward (prefill) attention kernels for gfx950 (CDNA4), BF16 and FP8 e4m3:
// the kernel template and its launcher, instantiated by attn_fwd_fp8.hip and
// attn_fwd_bf16.hip (separate files so that each precision gets its own compile flags).
//
// What is computed: O = softmax(mask(Q K^T * scale)) V per (batch, query head), with
// the query head h reading KV head h / (Hq / Hkv), and the log-sum-exp of each row.
// The whole-row softmax is evaluated tile by tile with an online (running-max)
// softmax so the score matrix never leaves registers (kongchang.com,
// "为什么 prefill attention 值得单独优化").
//
// Work split.  A workgroup owns NW*32 consecutive queries of one (batch, head); each of
// its NW waves owns 32 of them.  The workgroup walks the key axis in tiles of BN keys
// up to its causal diagonal; each K/V tile is copied HBM -> LDS once per workgroup by
// the buffer loads' direct-to-LDS mode (no registers involved; the copy of tile j+2 is
// in flight while tiles j and j+1 are used) and every wave reads its matrix operands
// from LDS.  The launch asks for two
// waves per SIMD, so while one wave waits on its matrix instructions the other issues
// its softmax arithmetic.
//
// Formulation.  Each wave forms the TRANSPOSED scores S^T = K Q^T with 32x32 MFMAs
// (A = K rows from LDS, B = Q^T held in registers for the whole loop), so that in the
// 32x32 accumulator a lane holds one query column and 16 keys of it: the row max, the
// exponentials and the row sums are per-lane work.  The second product is also
// transposed, O^T = V^T P^T: the B operand P^T needs, per lane, probabilities of its own
// query, which are exactly the values the lane already holds, so P goes from the score
// accumulator to the MFMA operand without any cross-lane movement.  The keys a lane
// holds are not contiguous (rows 8*(i/4) + 4*(lane/32) + i%4 of the accumulator); the
// contraction over keys does not care about key order as long as both operands use the
// same one, so the V^T operand is gathered in exactly that key order.  V stays in LDS
// as it is stored in memory (one row of channels per key) and gfx950's transposing LDS
// reads (ds_read_b64_tr_b8 / _b16) turn 8 key rows x 8 bytes into one channel's 8 keys
// per lane, with each lane of a 16-lane group addressing the key row it contributes.
//
// Lazy rescaling.  The running max m of a query only moves when a tile's max exceeds it
// by more than TAU (log2 units); otherwise the tile's probabilities are taken relative to
// the stale m (so they are at most 2^TAU, harmless in fp32 accumulators, in bf16, and
// for FP8 absorbed by the block exponent below).  The rescale of O by 2^(m_old - m_new)
// then runs on only a handful of tiles per row instead of on every tile.
//
// FP8 probabilities (the-ai.news "Drie technieken om de bottleneck te omzeilen";
// spke.com "Lean P" and "ブロックごとのスケーリングと丸められた行和"): the e4m3 code of
// 2^y is 8y + 56 exactly at integer y and in between linear in y, so a probability
// 2^(x + k) is written as the integer conversion of one FMA, s * 8c + (8k + C0 - 8c m).
// k is a power-of-two block exponent chosen per query and 64-key block, so that the
// block maximum lands in (2^7, 2^8] (codes <= 0x78) and small probabilities stay in
// the normal range; the scaled MFMA's E8M0 operand scale 2^-k (the same value for
// both of its 32-key scale blocks) undoes it at no cost.  O is
// divided by the sum of the same rounded probabilities, taken with one extra MFMA per
// 64-key block against a matrix of ones, so the approximation's bias cancels in the
// normalisation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>


#include <cmath>
#include <type_traits>

#include "attn_common.h"
#include "kernels.h"
#include "quantize_common.h"
#ifdef ATTN_PHASE_TIMERS
#include "../../include/attn_phase_timers.h"
// s_getreg operands (id | offset << 6 | (bits - 1) << 11): the wave's hardware ids
// (wave, SIMD, CU in bits 8-11, shader array, shader engine in bits 13-15, ...) and the
// index of its compute die
#define HWREG_HW_ID (4 | (31 << 11))
#define HWREG_XCC_ID (20 | (15 << 11))
#endif

namespace attn {

template <bool FP8, int DQK, int BN, int NW>
struct Cfg {
  static constexpr int EB = FP8 ? 1 : 2;            // bytes per element
  static constexpr int NT = NW * 64;                 // threads per workgroup
  static constexpr int BM = NW * 32;                 // queries per workgroup
  static constexpr int KRB = DQK * EB;               // K row bytes = LDS row (unpadded)
  static constexpr int R16 = KRB / 16;               // 16-byte chunks per K row
  static constexpr int VROW = DV * EB;               // LDS row of the V tile (one key)
  static constexpr int VCPR = VROW / 16;             // 16-byte chunks per V row
  static constexpr int K_BYTES = BN * KRB;
  static constexpr int V_BYTES = BN * VROW;
  static constexpr int KDMA = K_BYTES / (1024 * NW);  // 1 KiB direct copies per wave, K
  static constexpr int VDMA = V_BYTES / (1024 * NW);  // and V
  static constexpr int NKS = 3;                      // K tiles resident in LDS
  static constexpr int NVS = 4;                      // V tiles resident in LDS
  static constexpr int LDS = NKS * K_BYTES + NVS * V_BYTES;
  // exact channels (FP8, d_qk 128): their bf16 K values, 64 bytes per key, one stage per
  // K stage, copied with the tile (one 1 KiB block per wave)
  static constexpr int KX_ROW = 64;
  static constexpr int KX_BYTES = BN * KX_ROW;
  static constexpr int KXDMA = KX_BYTES / (1024 * NW);
  static constexpr int LDS_SPLIT = LDS + NKS * KX_BYTES;
  // float32 Q (FP8): each wave turns the codes of one 64-channel k-step of its 32 rows
  // from row order into the MFMA operand order through a private LDS block past the
  // stages, rows padded from 64 to 80 bytes (16-byte reads of 8 consecutive rows hit
  // 8 different 4-bank groups)
  static constexpr int QX_ROW = 80;
  static constexpr int LDS_QF32 = LDS + NW * 32 * QX_ROW;
  static constexpr int KS = FP8 ? DQK / 64 : DQK / 16;  // MFMA k-steps of Q K^T
  static constexpr int MT = BN / 32;                 // 32-key M-tiles of S^T
  static constexpr int NB = BN / 64;                 // 64-key blocks
  static_assert(BN % 64 == 0, "key tile must be a multiple of 64");
  static_assert(K_BYTES % (1024 * NW) == 0 && V_BYTES % (1024 * NW) == 0,
                "each wave copies whole 1 KiB blocks of every tile");
  static_assert(LDS <= 160 * 1024, "LDS budget of a workgroup");
  static_assert(!FP8 || DQK != 128 || (LDS_SPLIT <= 160 * 1024 && KXDMA == 1),
                "LDS budget and copy split of the exact-channel kernel");
  static_assert(!FP8 || LDS_QF32 <= 160 * 1024, "LDS budget of the float32-Q kernel");
  static_assert(NW == 8, "two groups of four waves, one wave of each per SIMD");
};

template <bool FP8, int DQK, int BN, int NW, int LSE, bool SPLIT, bool QF32>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64),
                          amdgpu_waves_per_eu(2, 2)))
void attn_fwd_kernel(FwdParams p) {
  using C = Cfg<FP8, DQK, BN, NW>;
  // LSE: 0 none; 1 the exact log-sum-exp (FP8: exact probabilities, O normalised by
  // their fp32 sum); 2 (FP8) the log of the rounded-probability row sum that
  // normalises the Lean P output, i.e. the LSE consistent with O.
  // SPLIT (FP8, d_qk 128): the last NSPC channels of every Q and K row are multiplied on
  // the BF16 matrix pipe, from the bf16 side arrays p.q_exact / p.k_exact (values in
  // descale units, as the codes), and left out of the FP8 products.  The FP8 instructions add each run of 8 channel products after
  // truncating them toward zero 13 bits below the run's largest exponent sum, so a channel whose
  // magnitude is far above the rest swamps its run; quantize_e4m3_qk_outliers stores each
  // KV head's largest-product channels there.  The BF16 products are exact and their
  // float32 sums as accurate as float32.
  static_assert(!SPLIT || (FP8 && DQK == 128 && LSE != 2), "exact channels: FP8, d_qk 128");
  // QF32 (FP8): Q is float32 and encoded on load (see the prologue)
  static_assert(!QF32 || (FP8 && !SPLIT), "float32 Q: the FP8 kernels without exact channels");
  constexpr int NSPC = 32;                               // exact channels (stored last)
  constexpr bool WANT_LSE = LSE != 0;
  constexpr bool EXACT = FP8 && LSE == 1;
  extern __shared__ __attribute__((aligned(16))) char lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int l32 = lane & 31;
  const int g = lane >> 5;
#ifdef ATTN_PHASE_TIMERS
  const unsigned long long rt_entry = __builtin_amdgcn_s_memrealtime();
#endif

  int b, h, qt;
  map_block(blockIdx.x, p, b, h, qt);
  const int hkv = h / (p.Hq / p.Hkv);
  const int Nq = p.Nq, Nk = p.Nk, q_off = p.q_off;
  const int q0 = qt * C::BM;
  // With late_rows_ahead, waves 0..NW/2-1 (group A, half a phase ahead in the key loop)
  // own the later half of the rows. The group that ends the loop last then has no key in
  // the last tile, so the loop ends with the leading group's masked softmax and last P V,
  // not with a softmax and a P V after it.
  const int q0w = q0 + (p.late_rows_ahead ? wave ^ (NW / 2) : wave) * 32;

  const size_t kstride = (size_t)p.Hkv * DQK * C::EB;   // bytes between keys
  const size_t vstride = (size_t)p.Hkv * DV * C::EB;
  const char* kbase = (const char*)p.k + ((size_t)b * Nk * p.Hkv + hkv) * DQK * C::EB;
  const char* vbase = (const char*)p.v + ((size_t)b * Nk * p.Hkv + hkv) * DV * C::EB;

  // Softmax constant in log2 units per raw score unit (descales folded in for FP8), V's
  // descale, Q's descale, and the power-of-two form of c (below).  They are set after the
  // Q loads and the first tile's copy are issued: the descales are memory loads, and the
  // decision on c branches, so taking them first put a second memory round trip in front
  // of the Q and K/V loads of every workgroup.
  float c = p.scale * LOG2E;
  float vds = 1.f;
  float dq = 1.f;   // FP8: Q's descale (float32 Q is encoded with it in the prologue)
  bool P2 = false;
  int qsc = 0x7f7f7f7f;   // E8M0 scale of the Q operand, one byte per 32-element block

  // ---- Q^T fragments (B operand), held for the whole key loop -------------------
  // Rows past Nq read row Nq-1 (finite data); their outputs are never stored.
  typedef typename std::conditional<FP8, i32x8, bf16x8>::type QFrag;
  QFrag qf[C::KS];
  bf16x8 qsp[SPLIT ? NSPC / 16 : 1];   // exact channels of Q^T, one per BF16 k-step
  // QF32: float32 Q read in row order, whole rows per load: q32[8ks + i] holds channels
  // 64ks + 4(lane & 15) .. +3 of the wave's row 4i + lane / 16 (16 lanes cover the 256
  // contiguous bytes of one k-step of a row), encoded into qf in the prologue
  float4 q32[QF32 ? 8 * C::KS : 1];
  if constexpr (QF32) {
    const size_t qstride = (size_t)p.Hq * DQK * 4;
    const char* qbase = (const char*)p.q + ((size_t)b * Nq * p.Hq + h) * DQK * 4;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = min(q0w + 4 * i + (lane >> 4), Nq - 1);
      const float4* rp = (const float4*)(qbase + (size_t)row * qstride) + (lane & 15);
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) q32[8 * ks + i] = rp[16 * ks];
    }
  } else {
    const size_t qstride = (size_t)p.Hq * DQK * C::EB;
    const char* qbase = (const char*)p.q + ((size_t)b * Nq * p.Hq + h) * DQK * C::EB;
    const int qrow = min(q0w + l32, Nq - 1);
    const char* rp = qbase + (size_t)qrow * qstride;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      if constexpr (FP8) {
        qf[ks] = load_i32x8(rp + 64 * ks + 32 * g);
      } else {
        const uint4 a = *(const uint4*)(rp + 2 * (16 * ks + 8 * g));
        qf[ks] = *(const QFrag*)&a;
      }
    }
    if constexpr (SPLIT) {
      // The FP8 operand of the last k-step holds channels DQK-64+32g ..: in the upper
      // lane half those are exactly the exact channels, which leave the FP8 products.
      static_assert(NSPC == 32, "the exact channels are the upper lane half's last k-step");
      if (g == 1) {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[C::KS - 1][e] = 0;
      }
      // BF16 k-step sk: lane (query l32, half g) holds exact channels 16sk+8g .. +7 of its
      // row of q_exact.  On the power-of-two path they are scaled by 2^ce further down,
      // once c is known (exact unless it leaves bf16's normal range, which the bound on
      // ce keeps away from the values quantisation produces).
      const __bf16* xrow = (const __bf16*)p.q_exact +
                           ((size_t)((size_t)b * Nq + qrow) * p.Hq + h) * NSPC;
#pragma unroll
      for (int sk = 0; sk < NSPC / 16; ++sk) qsp[sk] = *(const bf16x8*)(xrow + 16 * sk + 8 * g);
    }
  }

  // ---- K/V tile copies: global -> LDS -------------------------------------------
  // Each wave copies KDMA (K) and VDMA (V) 1 KiB blocks of every tile; lane i of block q
  // fills LDS chunk 64q + i of the tile, i.e. row (64q + i) / R16 at position
  // (64q + i) % R16, with the global chunk that the row's swizzle puts there.  The
  // descriptors cover this (b, kv head)'s keys 0..Nk-1, so keys past Nk read as zeros
  // (and are masked).
  uint32_t kdoff[C::KDMA], vdoff[C::VDMA];
#pragma unroll
  for (int i = 0; i < C::KDMA; ++i) {
    const int cc = (wave * C::KDMA + i) * 64 + lane;
    const int row = cc / C::R16, pos = cc - row * C::R16;
    kdoff[i] = (uint32_t)row * (uint32_t)kstride + 16u * (uint32_t)(pos ^ kswz<C::R16>(row));
  }
#pragma unroll
  for (int i = 0; i < C::VDMA; ++i) {
    const int cc = (wave * C::VDMA + i) * 64 + lane;
    const int row = cc / C::VCPR, pos = cc - row * C::VCPR;
    vdoff[i] = (uint32_t)row * (uint32_t)vstride + 16u * (uint32_t)(pos ^ vswz<FP8>(row));
  }
  const i32x4_t krsrc = buffer_rsrc(kbase, (uint32_t)((Nk - 1) * kstride + C::KRB));
  const i32x4_t vrsrc = buffer_rsrc(vbase, (uint32_t)((Nk - 1) * vstride + C::VROW));
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds;
  char* const kst = lds;                                // NKS K stages
  char* const vst = lds + C::NKS * C::K_BYTES;          // NVS V stages
  char* const kxst = vst + C::NVS * C::V_BYTES;         // NKS exact-channel K stages
  constexpr int KXD = SPLIT ? C::KXDMA : 0;
  constexpr int NDMA = C::KDMA + C::VDMA + KXD;         // copies per wave per tile
  // Exact-channel K rows (64 bytes, 4 chunks) are stored with chunk c of key r at
  // c ^ xswz(r), xswz(r) = (r >> 2) & 3, so the 16 lanes reading one chunk of 16
  // consecutive keys hit 16 different 4-bank groups.  This wave copies LDS chunks
  // 64 * wave + lane of the stage.
  const size_t kxstride = (size_t)p.Hkv * NSPC * 2;
  uint32_t kxoff = 0;
  i32x4_t kxrsrc = {0, 0, 0, 0};
  if constexpr (SPLIT) {
    const int cc = wave * 64 + lane;
    const int row = cc >> 2, pos = cc & 3;
    kxoff = (uint32_t)row * (uint32_t)kxstride + 16u * (uint32_t)(pos ^ ((row >> 2) & 3));
    const char* kxbase = (const char*)p.k_exact + ((size_t)b * Nk * p.Hkv + hkv) * NSPC * 2;
    kxrsrc = buffer_rsrc(kxbase, (uint32_t)((Nk - 1) * kxstride + NSPC * 2));
  }

  auto copy_tile = [&](int kt) {
    const uint32_t kt_off = (uint32_t)kt * BN * (uint32_t)kstride;
    const uint32_t vt_off = (uint32_t)kt * BN * (uint32_t)vstride;
    const uint32_t kl = lds_base + (uint32_t)((kt % C::NKS) * C::K_BYTES + wave * C::KDMA * 1024);
    const uint32_t vl = lds_base + (uint32_t)(C::NKS * C::K_BYTES + (kt % C::NVS) * C::V_BYTES +
                                              wave * C::VDMA * 1024);
#pragma unroll
    for (int i = 0; i < C::KDMA; ++i) copy16_to_lds(krsrc, kdoff[i] + kt_off, kl + 1024u * i);
#pragma unroll
    for (int i = 0; i < C::VDMA; ++i) copy16_to_lds(vrsrc, vdoff[i] + vt_off, vl + 1024u * i);
    if constexpr (SPLIT) {
      const uint32_t xl = lds_base + (uint32_t)(C::NKS * C::K_BYTES + C::NVS * C::V_BYTES +
                                                (kt % C::NKS) * C::KX_BYTES + wave * 1024);
      copy16_to_lds(kxrsrc, kxoff + (uint32_t)kt * BN * (uint32_t)kxstride, xl);
    }
  };

  // ---- per-query running state ---------------------------------------------------
  f32x16 oacc[DV / 32];
#pragma unroll
  for (int md = 0; md < DV / 32; ++md)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[md][i] = 0.f;
  float m_run = -INFINITY;   // running max (raw score units), same in both lane halves
  float l_run = 0.f;         // row sum relative to m_run (FP8: of the rounded P, full row;
                             // BF16: this lane's keys only)
  float lx_run = 0.f;        // FP8 + LSE: exact row sum over this lane's keys
  float r_run = 0.f;         // FP8 + LSE with P2: running max in log2 units (c m)

  // Query row i sees keys 0 .. min(i + q_off, Nk - 1).
  const int wg_end = min(q0 + C::BM, Nq);
  const int n_kt = (min(wg_end + q_off, Nk) + BN - 1) / BN;                  // workgroup's tiles
  const int w_end = min(q0w + 32, Nq);
  const int w_kt = q0w < Nq ? (min(w_end + q_off, Nk) + BN - 1) / BN : 0;    // this wave's
  const int w_lim = min(q0w + q_off, Nk - 1);   // last key every row of the wave sees

  // ---- ping-pong main loop ----------------------------------------------------------
  // The tile loop alternates a matrix phase, MFMA(t) = S(t) = K_t Q^T plus O += P(t-1)
  // V_(t-1), with a softmax phase, VALU(t), which turns S(t) into P(t) (P V is thus
  // software-pipelined by one tile).  Waves 0..3 (group A) and 4..7 (group B), one of
  // each per SIMD, run the same sequence half a phase apart, separated by workgroup
  // barriers: while one group issues matrix instructions the other does its softmax
  // arithmetic on the same SIMD, and the matrix group runs at raised issue priority.
  // Copies run two tiles ahead: MFMA(t) starts the copy of tile t+2, into the K stage
  // of tile t-1 and the V stage of tile t-2, which the other group's MFMA(t-1) (the
  // last reader) finished before the barrier that opened this phase; hence 3 K and 4 V
  // stages.  Before each barrier a wave waits for its own copy of tile t+1, so tile
  // t+1 is complete in LDS when either group's MFMA(t+1) begins.
  const bool grp_b = wave >= NW / 2;
  f32x16 s[C::MT];
  i32x8 pf8[C::NB];             // FP8 P(t-1) operand, one per 64-key block
  int psc[C::NB];               // its E8M0 block scales
  bf16x8 pfb[2 * C::MT];        // BF16 P(t-1) operand, one per 16-key k-step

  // Matrix-phase slots: the P V MFMAs of tile t-1 (NPV of them) followed by the Q K^T
  // MFMAs of tile t (NQK).  The LDS operand of slot j+LA is requested while slot j's
  // MFMA runs, so the matrix pipe does not wait on LDS latency between MFMAs.
  constexpr int NMD = DV / 32;
  constexpr int NPV = FP8 ? C::NB * NMD : 2 * C::MT * NMD;
  constexpr int NQK = C::KS * C::MT;
  constexpr int NSP = SPLIT ? (NSPC / 16) * C::MT : 0;   // BF16 slots of the exact channels
  // (3 for the d128 exact-probability kernel: +0.5% measured; neutral for the MLA shape)
  // (the exact-channel kernel keeps 2: its BF16 Q operands take the registers)
  constexpr int LA = FP8 ? (EXACT && DQK == 128 && !SPLIT ? 3 : 2) : 3;
  typedef typename std::conditional<FP8, i32x8, bf16x8>::type Frag;
  f32x16 zero16;
#pragma unroll
  for (int i = 0; i < 16; ++i) zero16[i] = 0.f;
  f32x16 init16 = zero16;       // first-k-step accumulator of Q K^T: -r_run with P2

  // Transposing V reads.  A P V MFMA needs, in lane l, channel 32md + l%32 of the keys
  // whose probabilities lane l holds, in the order it holds them:
  //   FP8, 64-key block n, operand byte j (k-index 32g + j):
  //     key 64n + 32(j/16) + 8((j%16)/4) + 4g + j%4
  //   BF16, 16-key step kk, operand element i (k-index 8g + i):
  //     key 32(kk/2) + 16(kk%2) + 8(i/4) + 4g + i%4
  // ds_read_b64_tr_b8 gives lane L of a 16-lane group byte (L%8) of the 8-byte chunks
  // addressed by group lanes 2j + L/8 (j = 0..7); ds_read_b64_tr_b16 gives it halfword
  // (L%4) of the chunks addressed by group lanes 4j + L/4 (j = 0..3).  So group lane s
  // addresses, for FP8 read r (operand bytes 8r..8r+7), key row 16r + 8(s/8) + 4g +
  // (s/2)%4 at channels 16(s/16 of the 32-lane half) + 8(s%2); for BF16 read r (elements
  // 4r..4r+3), key row 8r + 4g + s/4 at channels 4(s%4).  The lane-dependent part of
  // that address (and the channel block md) is precomputed; block, step and read
  // indices add compile-time row offsets, which leave vswz unchanged (it only looks at
  // key bits the lane fixes).
  int vrd[NMD];
  {
    const int s16 = lane & 15, grp = (lane >> 4) & 1;
    if constexpr (FP8) {
      const int kl = 8 * (s16 >> 3) + 4 * g + ((s16 >> 1) & 3);
      const int f = vswz<true>(kl);
#pragma unroll
      for (int md = 0; md < NMD; ++md)
        vrd[md] = kl * C::VROW + 16 * (((2 * md) ^ f) + grp) + 8 * (s16 & 1);
    } else {
      const int kl = 4 * g + (s16 >> 2);
      const int f = vswz<false>(kl);
#pragma unroll
      for (int md = 0; md < NMD; ++md)
        vrd[md] = kl * C::VROW + 16 * (((4 * md) ^ f) + 2 * grp + ((s16 >> 1) & 1)) +
                  8 * (s16 & 1);
    }
  }

  const int kx = kswz<C::R16>(l32);   // swizzle of every K row this lane reads

  const int kxr = 16 * ((l32 >> 2) & 3);   // xswz of every exact-channel K row this lane reads
  auto load_frag = [&](int j, const char* ks_, const char* vs_, const char* xs_) -> Frag {
    if (j < NPV) {                       // V^T rows 32md.., keys of block nb / step kk
      const int md = j % NMD;
      if constexpr (FP8) {
        const char* rp = vs_ + vrd[md] + 64 * (j / NMD) * C::VROW;
        i32x8 f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const v2i x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (__attribute__((address_space(3))) v2i*)(rp + 16 * r * C::VROW));
          f[2 * r] = x[0];
          f[2 * r + 1] = x[1];
        }
        return f;
      } else {
        const char* rp = vs_ + vrd[md] + 16 * (j / NMD) * C::VROW;
        const v4s x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4s*)rp);
        const v4s x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4s*)(rp + 8 * C::VROW));
        const uint2 a = __builtin_bit_cast(uint2, x0), b2 = __builtin_bit_cast(uint2, x1);
        return __builtin_bit_cast(Frag, make_uint4(a.x, a.y, b2.x, b2.y));
      }
    } else if (j >= NPV + NQK) {         // exact channels: 8 bf16 of key row 32m + l32
      Frag f{};
      if constexpr (SPLIT) {
        const int jj = j - NPV - NQK, sk = jj / C::MT, m = jj % C::MT;
        const uint4 a = *(const uint4*)(xs_ + (32 * m + l32) * C::KX_ROW +
                                        ((16 * (2 * sk + g)) ^ kxr));
        f[0] = (int)a.x; f[1] = (int)a.y; f[2] = (int)a.z; f[3] = (int)a.w;
      }
      return f;
    } else {                             // K rows 32m.., channels of k-step ks
      const int jj = j - NPV, ks = jj / C::MT, m = jj % C::MT;
      const char* rp = ks_ + (32 * m + l32) * C::KRB;
      if constexpr (FP8) {
        const int c0 = 4 * ks + 2 * g;                  // chunks c0, c0 + 1 of the row
        const uint4 a = *(const uint4*)(rp + 16 * (c0 ^ kx));
        const uint4 b2 = *(const uint4*)(rp + 16 * ((c0 + 1) ^ kx));
        i32x8 f;
        f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
        f[4] = b2.x; f[5] = b2.y; f[6] = b2.z; f[7] = b2.w;
        return f;
      } else {
        const uint4 a = *(const uint4*)(rp + 16 * ((2 * ks + g) ^ kx));
        return *(const Frag*)&a;
      }
    }
  };

  // Row sums by matrix instruction.  A 16x16 MFMA whose B operand is the probability
  // operand (lane l: query l%32, 32 keys) and whose A operand selects, for output rows
  // 4i..4i+3 (read by lanes 16i..16i+15), the k-groups of the lanes holding the same
  // query (lanes l and l+32 of each 32-lane half), leaves in every lane the sum over
  // both lane halves of its own query.  rsel marks the A entries that are 1.
  const bool rsel = ((lane >> 2) & 1) == ((lane >> 4) & 1);
  f32x4 zrow[C::NB];   // FP8 Lean P: rounded-code row sums of tile t-1, per block,
                       // still scaled by the block's 2^kb (element 0)
  f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  auto do_mfma = [&](int j, const Frag& f) {
    if (j < NPV) {
      const int md = j % NMD, blk = j / NMD;
      if constexpr (FP8) {
        oacc[md] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            f, pf8[blk], oacc[md], 0, 0, 0, 0x7f7f7f7f, 0, psc[blk]);
        if (!EXACT && md == NMD - 1) {
          // row sums of the rounded probabilities: one 16x16x128 MFMA per block with
          // unit scales (the block scale is removed on the VALU below)
          i32x8 sel;
#pragma unroll
          for (int e = 0; e < 8; ++e) sel[e] = rsel ? 0x38383838 : 0;   // e4m3 1.0 or 0
          zrow[blk] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              sel, pf8[blk], zero4, 0, 0, 0, 0x7f7f7f7f, 0, 0x7f7f7f7f);
        }
      } else {
        oacc[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, pfb[blk], oacc[md], 0, 0, 0);
      }
    } else if (j >= NPV + NQK) {
      if constexpr (SPLIT) {
        const int jj = j - NPV - NQK, sk = jj / C::MT, m = jj % C::MT;
        const uint4 a = make_uint4((uint32_t)f[0], (uint32_t)f[1], (uint32_t)f[2], (uint32_t)f[3]);
        s[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), qsp[sk],
                                                       s[m], 0, 0, 0);
      }
    } else {
      const int jj = j - NPV, ks = jj / C::MT, m = jj % C::MT;
      if (ks == 0) {
        if constexpr (FP8) {
          if constexpr (EXACT)
            s[m] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                f, *(const i32x8*)&qf[ks], init16, 0, 0, 0, 0x7f7f7f7f, 0, qsc);
          else
            s[m] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                f, *(const i32x8*)&qf[ks], zero16, 0, 0, 0, 0x7f7f7f7f, 0, 0x7f7f7f7f);
        } else {
          s[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, *(const bf16x8*)&qf[ks], zero16,
                                                         0, 0, 0);
        }
      } else {
        if constexpr (FP8) {
          s[m] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              f, *(const i32x8*)&qf[ks], s[m], 0, 0, 0, 0x7f7f7f7f, 0,
              EXACT ? qsc : 0x7f7f7f7f);
        } else {
          s[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, *(const bf16x8*)&qf[ks], s[m],
                                                         0, 0, 0);
        }
      }
    }
  };

  // FP8 with exact probabilities (LSE requested) has the longer softmax phase, so its
  // matrix phase takes over the per-block maxima of S(t): it issues the Q K^T MFMAs
  // first and forms the maxima while its P V MFMAs run (the scores are complete by
  // then); a tile that needs the causal mask recomputes them after masking.  In the
  // other variants the two phases are balanced and moving VALU work into the matrix
  // phase only lengthens it (measured), so they keep P V first and the max in the
  // softmax phase.
  constexpr bool MAX_IN_MFMA = EXACT;
  constexpr int NE = 16 * C::MT;          // scores per lane per tile
  float bmx_pre[C::NB];
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb) bmx_pre[nb] = -INFINITY;
  float pmx[C::NB][4];                    // independent max chains per block
  auto max_chunk = [&](int p) {           // p-th of NPV chunks of this lane's scores
#pragma unroll
    for (int e = (NE * p) / NPV; e < (NE * (p + 1)) / NPV; ++e) {
      float& acc = pmx[e >> 5][e & 3];
      acc = fmaxf(acc, s[e >> 4][e & 15]);
    }
    if (p == NPV - 1) {
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) {
        bmx_pre[nb] = fmaxf(fmaxf(pmx[nb][0], pmx[nb][1]), fmaxf(pmx[nb][2], pmx[nb][3]));
        if constexpr (FP8) bmx_pre[nb] = max_halves(bmx_pre[nb]);
      }
    }
  };

  // Block exponent of a 64-key block with maximum bmx, relative to the running max
  // (nmc = -m c): the block maximum maps into (2^7, 2^8].
  auto block_exp = [&](float bmx, float nmc) -> float {
    return fminf(floorf(8.f - fmaf(bmx, c, nmc)), 127.f);
  };
  // The 8 words of block nb (4 probabilities each, already exponentiated in place of
  // the scores and scaled by the block exponent) rounded to e4m3 into pf8[nb]; bs[j]
  // receives the sum of the j-th probabilities of the words (four independent chains,
  // started from the first word rather than from zero, which would cost an add of 0 per
  // chain).
  auto exact_words = [&](int nb, float* bs) {
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      float pv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = 4 * w + j;
        pv[j] = s[2 * nb + (e >> 4)][e & 15];
        bs[j] = w == 0 ? pv[j] : bs[j] + pv[j];
      }
      // high half first into the word being replaced, so no zeroed register
      int word = __builtin_amdgcn_cvt_pk_fp8_f32(pv[2], pv[3], pf8[nb][w], true);
      word = __builtin_amdgcn_cvt_pk_fp8_f32(pv[0], pv[1], word, false);
      pf8[nb][w] = word;
    }
  };

  // The matrix phase's slots in issue order: with MAX_IN_MFMA the Q K^T MFMAs of tile t
  // first (slot indices NPV.. of load_frag / do_mfma, the FP8 k-steps and then those of
  // the exact channels), then the P V MFMAs of tile t-1 (0..NPV-1), each P V slot also
  // taking a share of the max over S(t); otherwise P V then Q K^T.  An LA-deep operand pipeline requests slot j+LA's LDS operand while
  // slot j's MFMA runs.
  // The pipeline's first matrix phase (t = 0) has no P V to do (P(-1) is zero) and its
  // last (t = n_kt) no Q K^T (there is no tile n_kt): mode_tag selects all slots (0), the
  // Q K^T slots only (1, with the maxima after them) or the P V slots only (2).
  auto run_slots = [&](const char* ks_, const char* vs_, const char* xs_, auto mode_tag) {
    constexpr int MODE = decltype(mode_tag)::value;
    constexpr int NK = NQK + NSP;   // Q K^T slots (FP8, then the exact channels)
    constexpr int NS = MODE == 0 ? NPV + NK : MODE == 1 ? NK : NPV;
    auto vs = [](int j) {
      if (MODE == 1) return NPV + j;
      if (MODE == 2) return j;
      return !MAX_IN_MFMA ? j : j < NK ? NPV + j : j - NK;
    };
    if (MODE != 2) {
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
        for (int e = 0; e < 4; ++e) pmx[nb][e] = -INFINITY;
    }
    Frag fr[LA + 1];
#pragma unroll
    for (int j = 0; j < LA; ++j) fr[j % (LA + 1)] = load_frag(vs(j), ks_, vs_, xs_);
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      // keep the slots in program order: the scheduler would otherwise hoist every
      // operand read to the top of the phase and run out of registers
      __builtin_amdgcn_sched_barrier(0);
      if (j + LA < NS) fr[(j + LA) % (LA + 1)] = load_frag(vs(j + LA), ks_, vs_, xs_);
      do_mfma(vs(j), fr[j % (LA + 1)]);
      if (MODE == 0 && MAX_IN_MFMA && j >= NK) max_chunk(j - NK);
    }
    if (MODE == 1 && MAX_IN_MFMA) {
#pragma unroll
      for (int c = 0; c < NPV; ++c) max_chunk(c);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  auto mfma_phase = [&](int t, auto mode_tag) {
    constexpr int MODE = decltype(mode_tag)::value;
    __builtin_amdgcn_s_setprio(1);
    copy_tile(t + 2);   // past the last tile this reads zeros into a free stage
    // Inside the loop every matrix phase runs all slots, so the phase is one
    // straight-line schedule.  Where a wave has no work the slots are made harmless
    // instead of skipped: the P operand is zero (set by the softmax phase) and a Q K^T
    // past the wave's last tile is never used.
    // FP8: stage offsets as opaque scalars, so that every K fragment address is one
    // per-lane base plus an immediate (derived from t, the compiler folds them into
    // negative constants that the LDS offset field cannot hold and adds them per read;
    // +2-3% measured).  BF16 measured 3-4% slower that way and keeps the plain form.
    int kso = (t % C::NKS) * C::K_BYTES;
    int vso = (t == 0 ? 0 : (t - 1) % C::NVS) * C::V_BYTES;
    if constexpr (FP8) {
      kso = __builtin_amdgcn_readfirstlane(kso);
      vso = __builtin_amdgcn_readfirstlane(vso);
    }
    const char* ks_ = kst + kso;
    const char* vs_ = vst + vso;
    const char* xs_ = kxst + (SPLIT ? (t % C::NKS) * C::KX_BYTES : 0);
    run_slots(ks_, vs_, xs_, mode_tag);
    if (FP8 && !EXACT && MODE != 1) {
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) l_run += __builtin_ldexpf(zrow[nb][0], psc[nb] - 127);
    }
    // Pin the scores and their maxima to this phase (the compiler would otherwise sink
    // the Q K^T MFMAs, which touch no memory, and the max past the barrier).
    if constexpr (MODE != 2) {
#pragma unroll
      for (int m = 0; m < C::MT; ++m) keep_in_vgprs(s[m]);
      if constexpr (MAX_IN_MFMA) {
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) keep_in_vgprs(bmx_pre[nb]);
      }
    }
  };

  auto zero_p = [&]() {
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) {
      psc[nb] = 127;
#pragma unroll
      for (int w = 0; w < 8; ++w) pf8[nb][w] = 0;
    }
#pragma unroll
    for (int kk = 0; kk < 2 * C::MT; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) pfb[kk][e] = (__bf16)0.f;
  };

  // Softmax phase of the P2 path: the scores are x = c S - r_run already.  The first
  // tile sets r_run to its row max; later a row moves it only when its tile max exceeds
  // it by more than TAU.  The block exponent goes into the scaled conversion
  // (v_cvt_scalef32_pk_fp8_f32 converts x / 2^-kb), so the exponentials and their fp32
  // sums are taken on the unscaled arguments.
  auto valu_p2 = [&](int t, float* bmx, float mx) {
    if constexpr (!EXACT) return;
    const bool first = t == 0;
    if (first || __any(mx > TAU)) {
      const float sh = first ? mx : fmaxf(mx, 0.f);
      const float alpha = first ? 1.f : __builtin_amdgcn_exp2f(-sh);
      r_run += sh;
      lx_run *= alpha;
#pragma unroll
      for (int md = 0; md < DV / 32; ++md)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[md][i] *= alpha;
#pragma unroll
      for (int m = 0; m < C::MT; ++m)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[m][i] -= sh;
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) bmx[nb] -= sh;
#pragma unroll
      for (int i = 0; i < 16; ++i) init16[i] = -r_run;
    }
    float scl[C::NB];
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) {
      // block maximum into (2^7, 2^8]; at most 126 so that the scale 2^-kb is a normal
      // float (its exponent is the conversion's scale)
      const int kb = (int)fminf(floorf(8.f - bmx[nb]), 126.f);
      psc[nb] = 127 - kb;
      scl[nb] = __uint_as_float((uint32_t)(127 - kb) << 23);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
      for (int e = 0; e < 32; ++e)
        s[2 * nb + (e >> 4)][e & 15] = __builtin_amdgcn_exp2f(s[2 * nb + (e >> 4)][e & 15]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) {
      float bs[4];
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        float pv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = 4 * w + j;
          pv[j] = s[2 * nb + (e >> 4)][e & 15];
          bs[j] = w == 0 ? pv[j] : bs[j] + pv[j];
        }
        // both halves are overwritten, so the first conversion writes into the register
        // of a probability the sums have already read (no zeroed register is needed)
        const v2s hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(
            __builtin_bit_cast(v2s, pv[3]), pv[2], pv[3], scl[nb], true);
        const v2s wd = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(hi, pv[0], pv[1], scl[nb], false);
        pf8[nb][w] = __builtin_bit_cast(int, wd);
      }
      lx_run += (bs[0] + bs[1]) + (bs[2] + bs[3]);
    }
  };

  auto valu_phase = [&](int t, auto p2_tag) {
    constexpr bool PP = decltype(p2_tag)::value;
    __builtin_amdgcn_s_setprio(0);
    if (t >= w_kt) {        // past this wave's last tile: the next P V adds nothing
      zero_p();
      return;
    }
    float bmx[C::NB];
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) bmx[nb] = bmx_pre[nb];
    // causal mask on the tile(s) that cross this wave's diagonal or the end of the keys
    // (then the block maxima are taken again over the masked scores)
    const bool masked = t * BN + BN - 1 > w_lim;
    if (masked) {
      // element i of M-tile m holds key t*BN + 32m + 4g + off_i, off_i = 8(i/4) + i%4;
      // it is masked when 32m + off_i > d0 = lim - (t*BN + 4g), lim = the row's last
      // visible key: one compare of d0 with a constant per element.
      const int d0 = min(q0w + l32 + q_off, Nk - 1) - (t * BN + 4 * g);
#pragma unroll
      for (int m = 0; m < C::MT; ++m)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          s[m][i] = d0 < 32 * m + 8 * (i >> 2) + (i & 3) ? -INFINITY : s[m][i];
    }
    if (masked || !MAX_IN_MFMA) {
      // max over each 64-key block (this lane's 32 keys, then the other lane half's)
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) {
        float pm[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};   // independent chains
#pragma unroll
        for (int e = 0; e < 32; ++e) pm[e & 3] = fmaxf(pm[e & 3], s[2 * nb + (e >> 4)][e & 15]);
        bmx[nb] = fmaxf(fmaxf(pm[0], pm[1]), fmaxf(pm[2], pm[3]));
        if constexpr (FP8) bmx[nb] = max_halves(bmx[nb]);
      }
    }
    float mx = bmx[0];
#pragma unroll
    for (int nb = 1; nb < C::NB; ++nb) mx = fmaxf(mx, bmx[nb]);
    if constexpr (EXACT && PP) {
      valu_p2(t, bmx, mx);
      return;
    }
    // lazy running max: rescale only when some row's tile max exceeds m by > TAU
    if (__any((mx - m_run) * c > TAU)) {
      // (FP8 block maxima already cover both lane halves of the query)
      const float m_new = FP8 ? fmaxf(m_run, mx) : fmaxf(m_run, fmaxf(mx, xor32(mx)));
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
      m_run = m_new;
      l_run *= alpha;
      if (EXACT) lx_run *= alpha;
#pragma unroll
      for (int md = 0; md < DV / 32; ++md)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[md][i] *= alpha;
    }
    const float nmc = -m_run * c;

    if constexpr (EXACT) {
      // Exact probabilities scaled by 2^kb (<= 2^8), rounded to e4m3; their exact fp32
      // sum (scale removed) normalises O and gives the log-sum-exp.  Staged like the
      // Lean P words below: all exponent arguments, then all exponentials (in place of
      // the scores), then the words and the sums.
      float kbf[C::NB];
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) {
        // one block exponent per query and 64-key block (both operand scale blocks)
        kbf[nb] = block_exp(bmx[nb], nmc);
        psc[nb] = 127 - (int)kbf[nb];
        const float off = nmc + kbf[nb];
#pragma unroll
        for (int e = 0; e < 32; ++e)
          s[2 * nb + (e >> 4)][e & 15] = fmaf(s[2 * nb + (e >> 4)][e & 15], c, off);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
        for (int e = 0; e < 32; ++e)
          s[2 * nb + (e >> 4)][e & 15] = __builtin_amdgcn_exp2f(s[2 * nb + (e >> 4)][e & 15]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) {
        float bs[4];
        exact_words(nb, bs);
        lx_run += __builtin_ldexpf((bs[0] + bs[1]) + (bs[2] + bs[3]), -(int)kbf[nb]);
      }
    } else if constexpr (FP8) {
      // Lean P: e4m3 code = integer conversion of 8 (x + kb) + C0, one FMA each.  All
      // code arguments are formed first (in place of the scores), then the words are
      // packed a byte position at a time across all of them, so that no instruction
      // waits on the one just before it (+1% against packing one word at a time).
      const float A = 8.f * c;
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) {
        // one block exponent per query and 64-key block (both operand scale blocks)
        const float kbf = block_exp(bmx[nb], nmc);
        psc[nb] = 127 - (int)kbf;
        const float Bc = fmaf(8.f, kbf, fmaf(8.f, nmc, LEANP_C0));
#pragma unroll
        for (int e = 0; e < 32; ++e)
          s[2 * nb + (e >> 4)][e & 15] = fmaf(s[2 * nb + (e >> 4)][e & 15], A, Bc);
      }
      uint32_t words[C::NB][8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
          for (int w = 0; w < 8; ++w) {
            const int e = 4 * w + j;
            words[nb][w] = __builtin_amdgcn_cvt_pk_u8_f32(s[2 * nb + (e >> 4)][e & 15], j,
                                                          j == 0 ? 0u : words[nb][w]);
          }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
        for (int w = 0; w < 8; ++w) pf8[nb][w] = (int)words[nb][w];
    } else {
      // staged: all exponent arguments, then all exponentials (in place of the
      // scores), then the bf16 operands and the sums (four independent chains, each
      // started from its first probability)
#pragma unroll
      for (int e = 0; e < 16 * C::MT; ++e) s[e >> 4][e & 15] = fmaf(s[e >> 4][e & 15], c, nmc);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int e = 0; e < 16 * C::MT; ++e)
        s[e >> 4][e & 15] = __builtin_amdgcn_exp2f(s[e >> 4][e & 15]);
      __builtin_amdgcn_sched_barrier(0);
      float rs[4];
#pragma unroll
      for (int e = 0; e < 16 * C::MT; ++e) {
        const float pv = s[e >> 4][e & 15];
        rs[e & 3] = e < 4 ? pv : rs[e & 3] + pv;
        pfb[e >> 3][e & 7] = (__bf16)pv;
      }
      l_run += (rs[0] + rs[1]) + (rs[2] + rs[3]);
    }
  };

  // Workgroup barrier that the compiler may not schedule anything across (matrix
  // instructions touch no memory, so it would otherwise move them over barriers).
  auto phase_barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };

  // Every matrix phase issues exactly one tile copy (tiles past the end read zeros
  // into a free stage), so "this wave's copy of tile t+1 has landed" is always the
  // same wait, vmcnt <= NDMA, and the phases stay free of branches (the compiler
  // would sink the P V MFMAs into a branch that followed them).
  zero_p();                             // the first matrix phase has no P yet
  copy_tile(0);
  if (FP8) {
    dq = p.qds[p.per_head ? h : 0];
    const float dk = p.kds[p.per_head ? hkv : 0];
    vds = p.vds[p.per_head ? hkv : 0];
    c *= dq * dk;
  }
  // FP8 with the exact LSE, c within 4 ulps of a power of two 2^ce (a relative change
  // below 2^-21, the size of the rounding already in c's float32 product; a Q descale
  // chosen for it makes this the case): the Q operand's E8M0 scale applies c inside the
  // matrix instruction and its first k-step starts from -r_run, the running max in log2
  // units, so the scores leave the MFMA as the exponent arguments themselves and the
  // softmax phase needs no FMA per score.  Otherwise qsc is 1.0 and init16 stays zero.
  if constexpr (EXACT) {
    const uint32_t cb = __float_as_uint(c);
    const uint32_t man = cb & 0x7fffffu;
    const int ce = (int)((cb >> 23) & 0xffu) - 127 + (man >= 0x400000u ? 1 : 0);
    P2 = ((cb >> 23) & 0xffu) != 0u && ((cb >> 23) & 0xffu) != 0xffu &&
         (man <= 4u || man >= 0x7ffffcu) && ce >= -120 && ce <= 120;
    // with exact channels, 2^ce also scales their bf16 Q values: keep those normal
    if (SPLIT) P2 = P2 && ce >= -100 && ce <= 100;
    if (P2) qsc = (127 + ce) * 0x01010101;
  }
  if constexpr (SPLIT) {
    // On the power-of-two path the Q operand's scale 2^ce applies to the FP8 products, so
    // the exact channels' bf16 Q values carry it too.
    if (P2) {
      const float qmul = __uint_as_float((uint32_t)(qsc & 0xff) << 23);   // 2^ce
#pragma unroll
      for (int sk = 0; sk < NSPC / 16; ++sk)
#pragma unroll
        for (int e = 0; e < 8; ++e) qsp[sk][e] = (__bf16)((float)qsp[sk][e] * qmul);
    }
  }
  if constexpr (QF32) {
    // The codes quantize_e4m3 / quantize_e4m3_q_pow2 write with this descale (round to
    // nearest even of x / descale, saturating at +-448, NaN to 0x7F; the same encoder),
    // formed while the first tile is being copied, then moved to the operand order one
    // k-step at a time through the wave's LDS block: code word 4i + lane / 16, lane & 15
    // of the row-order block, read back as 32 bytes of row l32 at byte 32g.  The block
    // is this wave's alone and a wave's LDS accesses execute in issue order, so fences
    // at wavefront scope (ordering for the compiler, no wait) are all it needs.
    const float dsq = dq;
    uint32_t qw[8 * C::KS];
    if (fast_divisor(dsq)) {
      const Divisor dv = make_divisor(dsq);
#pragma unroll
      for (int e = 0; e < 8 * C::KS; ++e) qw[e] = e4m3_word_fast(q32[e], dv);
    } else {
#pragma unroll
      for (int e = 0; e < 8 * C::KS; ++e) qw[e] = e4m3_word(q32[e], dsq);
    }
    char* const qx = lds + C::LDS + wave * 32 * C::QX_ROW;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        *(uint32_t*)(qx + (4 * i + (lane >> 4)) * C::QX_ROW + 4 * (lane & 15)) = qw[8 * ks + i];
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      const uint4* src = (const uint4*)(qx + l32 * C::QX_ROW + 32 * g);
      const uint4 lo = src[0], hi = src[1];
      qf[ks] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                     (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    }
  }
  // The Q fragments and tile 0 have landed (loads complete in issue order); the
  // compiler also learns here that nothing it issued is outstanding.
  wait_vmcnt<0>();
  copy_tile(1);
  phase_barrier();
  if (grp_b) phase_barrier();           // group B runs half a phase behind group A
#ifdef ATTN_PHASE_TIMERS
  const unsigned long long rt_loop0 = __builtin_amdgcn_s_memrealtime();
#endif

  // The P2 choice is taken once per workgroup, outside the key loop: each loop copy
  // holds the registers of its own softmax path only (a loop wrapped in a lambda spills,
  // hence the macro).
  // The pipeline's fill (t = 0: Q K^T only, while group B waits at its extra barrier) and
  // drain (t = n_kt: P V only; group B's comes after group A has finished) run outside the
  // loop with only the slots they need (measured +2.4-3.3% at 4K, +1.1-1.3% at mla32k, outputs
  // unchanged).  Peeling the fill puts a second copy of the softmax phase outside the
  // loop; in the two exact-LSE kernels nearest the 256-VGPR limit (the exact channels,
  // and d192 with float32 Q) that made the register allocator spill, so they keep the
  // fill inside the loop (with all its slots) and peel only the drain.  A wave whose
  // rows see no key of the last tile (w_kt < n_kt: the first half of the workgroup's
  // rows when the tile crosses their diagonal) has a zero P(n_kt - 1) and skips the
  // drain's P V; it still issues its share of the (unused) copy, as every phase does.
  constexpr bool PEEL_FILL = !(EXACT && (SPLIT || (QF32 && DQK == 192)));
#ifdef ATTN_PHASE_TIMERS
  // Measurement build: shader-clock reads around each phase of the tiles past the
  // pipeline's fill (t >= 2) and before its drain (t + 2 < n_kt); record layout in
  // include/attn_phase_timers.h.
  unsigned tm_mb = 0, tm_vb = 0, tm_t0 = 0, tm_t1 = 0;
#define ATTN_TM(...) __VA_ARGS__
#else
#define ATTN_TM(...)
#endif
#define ATTN_KEY_LOOP(P2_TAG)                \
  int t_first = 0;                           \
  if constexpr (PEEL_FILL) {                 \
    mfma_phase(0, std::integral_constant<int, 1>{}); \
    wait_vmcnt<NDMA>();                      \
    phase_barrier();                         \
    valu_phase(0, P2_TAG);                   \
    wait_vmcnt<NDMA>();                      \
    phase_barrier();                         \
    t_first = 1;                             \
  }                                          \
  for (int t = t_first; t < n_kt; ++t) {     \
    ATTN_TM(const unsigned c0 = (unsigned)__builtin_amdgcn_s_memtime(); \
            if (t == 2) tm_t0 = c0;          \
            if (t + 2 == n_kt) tm_t1 = c0;)  \
    mfma_phase(t, std::integral_constant<int, 0>{}); \
    ATTN_TM(__builtin_amdgcn_sched_barrier(0); \
            const unsigned c1 = (unsigned)__builtin_amdgcn_s_memtime(); \
            if (t >= 2 && t + 2 < n_kt) tm_mb += c1 - c0;) \
    wait_vmcnt<NDMA>();                      \
    phase_barrier();                         \
    ATTN_TM(const unsigned c2 = (unsigned)__builtin_amdgcn_s_memtime();) \
    valu_phase(t, P2_TAG);                   \
    ATTN_TM(__builtin_amdgcn_sched_barrier(0); \
            const unsigned c3 = (unsigned)__builtin_amdgcn_s_memtime(); \
            if (t >= 2 && t + 2 < n_kt) tm_vb += c3 - c2;) \
    wait_vmcnt<NDMA>();                      \
    phase_barrier();                         \
  }                                          \
  if (w_kt == n_kt) {                        \
    mfma_phase(n_kt, std::integral_constant<int, 2>{}); \
  } else {                                   \
    __builtin_amdgcn_s_setprio(1);           \
    copy_tile(n_kt + 2);                     \
  }                                          \
  wait_vmcnt<NDMA>();                        \
  phase_barrier();
  if constexpr (EXACT) {
    if (P2) {
      ATTN_KEY_LOOP(std::true_type{})
    } else {
      ATTN_KEY_LOOP(std::false_type{})
    }
  } else {
    ATTN_KEY_LOOP(std::false_type{})
  }
#undef ATTN_KEY_LOOP
#undef ATTN_TM
  wait_vmcnt<0>();                      // no copy into LDS outlives the loop
  if (!grp_b) phase_barrier();          // equal barrier counts in both groups
  __builtin_amdgcn_s_setprio(0);
#ifdef ATTN_PHASE_TIMERS
  const unsigned long long rt_loop1 = __builtin_amdgcn_s_memrealtime();
#endif

  // ---- epilogue: normalise, write O (bf16) and LSE ---------------------------------
  const int qrow = q0w + l32;
  float l = l_run;
  if (!FP8) l += xor32(l);
  if (EXACT) l = lx_run + xor32(lx_run);
  const float lsum = l;
  const float inv = (FP8 ? vds : 1.f) / l;
  // O leaves through LDS so that each store instruction writes whole rows: the wave's
  // 32 rows go to a private block (rows padded from 256 to 272 bytes, so the 8-byte
  // writes of one column of the accumulators spread over the banks), then each lane
  // stores 16 contiguous bytes, 16 lanes per row, 4 rows per instruction (full cache
  // lines, a quarter of the write requests of storing from the accumulator layout,
  // where every instruction touches 32 rows).  The stages are free once every wave's
  // copies have landed (the barrier below; each wave waited for its own above), and a
  // wave's LDS accesses execute in issue order, so its own block needs only a
  // wavefront fence between the writes and the reads.
  phase_barrier();
  {
    constexpr int OROW = DV * 2 + 16;
    static_assert(8 * 32 * OROW <= C::LDS, "O staging fits in the stages");
    char* const ost = lds + wave * 32 * OROW;
#pragma unroll
    for (int md = 0; md < DV / 32; ++md)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        bf16x4 ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = (__bf16)(oacc[md][4 * r + e] * inv);
        *(bf16x4*)(ost + l32 * OROW + 2 * (32 * md + 8 * r + 4 * g)) = ov;
      }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    constexpr int CPR = DV * 2 / 16;          // 16-byte chunks per O row
    constexpr int RPI = 64 / CPR;             // rows per store instruction
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int rr = RPI * i + lane / CPR;
      const uint4 v = *(const uint4*)(ost + rr * OROW + 16 * (lane % CPR));
      if (q0w + rr < Nq)
        *(uint4*)((char*)p.o + ((size_t)((size_t)b * Nq + q0w + rr) * p.Hq + h) * DV * 2 +
                  16 * (lane % CPR)) = v;
    }
  }
  if (WANT_LSE && g == 0 && qrow < Nq)
    p.lse[((size_t)b * p.Hq + h) * Nq + qrow] =
        ((EXACT && P2 ? r_run : m_run * c) + __builtin_amdgcn_logf(lsum)) * LN2;
#ifdef ATTN_PHASE_TIMERS
  // Record layout in include/attn_phase_timers.h; the exit stamp follows the issue of
  // this wave's O and LSE stores, which complete later (as in the product build, which
  // does not wait for them).
  const unsigned long long rt_exit = __builtin_amdgcn_s_memrealtime();
  if (lane == 0 && p.timers && (int)blockIdx.x < p.timer_blocks) {
    unsigned long long* rec =
        p.timers + ((size_t)blockIdx.x * NW + wave) * ATTN_PHASE_TIMER_WORDS;
    rec[0] = (unsigned long long)(n_kt > 4 ? n_kt - 4 : 0);
    rec[1] = tm_mb;
    rec[2] = tm_vb;
    rec[3] = n_kt > 4 ? tm_t1 - tm_t0 : 0u;
    rec[4] = rt_entry;
    rec[5] = rt_loop0;
    rec[6] = rt_loop1;
    rec[7] = rt_exit;
    rec[8] = (unsigned long long)n_kt;
    rec[9] = (unsigned long long)(unsigned)__builtin_amdgcn_s_getreg(HWREG_HW_ID) |
             ((unsigned long long)(unsigned)__builtin_amdgcn_s_getreg(HWREG_XCC_ID) << 32);
  }
#endif
}

// The exchange between the XCDs of a pair (map_block): the odd XCD hands its sw
// heaviest items to the even one for the even one's items at places j .. j+sw-1, so
// that the moved work, in key tiles, comes closest to XCD_SHIFT of one XCD's work: the
// fewest items that can move that much, and the block of the even XCD's list whose
// weight leaves the closest difference; none unless it lands within half of the target.
// XCD_SHIFT = (r - 1) / (r + 1) for an odd/even time ratio r = 1.03 at equal work, the
// low end of what the phase-timer build measured (1.027-1.048 over five boxes, every
// kernel and size; rotating the KV heads over the XCDs left the odd XCDs the slow ones).
constexpr double XCD_SHIFT = 0.03 / 2.03;
// Only with at least this many items per CU of an XCD (32 CUs each on MI355X): with two
// (4K, B=1) one traded item upset the balance between the XCD's own CUs, and the
// exchange cost 3-4% there instead of gaining.
constexpr long long XCD_SWAP_MIN_ITEMS = 6 * 32;

template <int BM, int BN>
static void xcd_swap_plan(FwdParams& p) {
  p.xcd_swap = 0;
  p.xcd_swap_at = 0;
  const int BHkv = p.B * p.Hkv;
  if ((BHkv & 7) != 0) return;
  const long long per = (long long)(BHkv >> 3) * (p.Hq / p.Hkv);
  const long long total = (long long)p.n_qtiles * per;
  if (total < XCD_SWAP_MIN_ITEMS) return;
  // key tiles of the item at place i of an XCD's list (query tile n_qtiles - 1 - i/per)
  auto w = [&](long long i) -> long long {
    const long long qt = p.n_qtiles - 1 - i / per;
    const long long wg_end = qt * BM + BM < p.Nq ? qt * BM + BM : p.Nq;
    const long long keys = wg_end + p.q_off < p.Nk ? wg_end + p.q_off : p.Nk;
    return (keys + BN - 1) / BN;
  };
  long long work = 0;
  for (long long t = 0; t < p.n_qtiles; ++t) work += per * w(t * per);
  const double target = XCD_SHIFT * (double)work;
  long long heavy = 0, light = 0;
  for (long long s = 1; 2 * s <= total; ++s) {
    // the most s items can move: the s heaviest for the s lightest; once one more pair
    // moves nothing (falling weights), no larger s moves more
    if (w(s - 1) <= w(total - s)) return;
    heavy += w(s - 1);
    light += w(total - s);
    if ((double)(heavy - light) < target) continue;
    // blocks get lighter as j grows: take the first j whose block moves at least the
    // target, or the one before it if that comes closer
    long long lo = s, hi = total - s;         // block(lo) heaviest, block(hi) lightest
    auto block = [&](long long jj) {
      long long b = 0;
      for (long long i = jj; i < jj + s; ++i) b += w(i);
      return b;
    };
    const double need = (double)heavy - target;
    while (lo < hi) {                         // first j with block(j) <= need
      const long long mid = (lo + hi) / 2;
      if ((double)block(mid) <= need) hi = mid; else lo = mid + 1;
    }
    long long jb = lo;
    double err = std::fabs((double)(heavy - block(jb)) - target);
    if (jb > s) {
      const double e2 = std::fabs((double)(heavy - block(jb - 1)) - target);
      if (e2 < err) { err = e2; jb -= 1; }
    }
    if (err <= 0.5 * target) {
      p.xcd_swap = (int)s;
      p.xcd_swap_at = (int)jb;
    }
    return;
  }
}

// The tile map's parameters for one launch (p.n_qtiles set): the XCD pair exchange and
// the shader-engine rotation (map_block).
template <bool FP8, int BM, int BN>
static void schedule_tiles(FwdParams& p) {
  xcd_swap_plan<BM, BN>(p);
  // Same-box A/B of the shader-engine rotation, four alternations on each of two boxes:
  // FP8 without the LSE +0.4% to +1.9% on every shape; BF16 -0.2% to -0.65%; FP8 with the
  // exact LSE +0.3% and +0.4% where a row of the XCD's list has fewer than 4 items
  // (mla32k: the lighter row of each pair always fell to the same two engines) and
  // -0.75% to -0.1% where it has 4 (only the heads rotate then).
  const int row_items = (p.B * p.Hkv) % 8 == 0 ? (p.B * p.Hkv / 8) * (p.Hq / p.Hkv) : 0;
  p.se_rotate = FP8 && (!p.lse || p.lse_rounded || (row_items > 0 && row_items < 4)) ? 1 : 0;
  // Later rows in the leading wave group: same-box A/B, outputs unchanged, at 4K (2 query
  // tiles per CU) +0.5% to +1.1% for every kernel; at 8 and 16 per CU (mla32k, gauss32k)
  // -0.4% to +0.9% with FP8 and the exact LSE at gauss32k consistently -0.4%.  So only
  // launches with at most 4 query tiles per CU (256 CUs) use it.
  p.late_rows_ahead = (long long)p.n_qtiles * p.B * p.Hq <= 4LL * 256 ? 1 : 0;
}

template <bool FP8, int DQK, int BN, int NW>
static hipError_t launch_cfg(const FwdParams& p0, hipStream_t stream) {
  using C = Cfg<FP8, DQK, BN, NW>;
  FwdParams p = p0;
  p.n_qtiles = (p.Nq + C::BM - 1) / C::BM;
  schedule_tiles<FP8, C::BM, BN>(p);
  const long long grid = (long long)p.n_qtiles * p.B * p.Hq;
  if (grid <= 0 || grid > 0x7fffffffLL) return hipErrorInvalidValue;
  auto kern = !p.lse ? attn_fwd_kernel<FP8, DQK, BN, NW, 0, false, false>
                     : attn_fwd_kernel<FP8, DQK, BN, NW, 1, false, false>;
  if constexpr (FP8) {
    if (p.lse && p.lse_rounded) kern = attn_fwd_kernel<FP8, DQK, BN, NW, 2, false, false>;
    if (p.q_f32) {
      if (p.lse_rounded || p.split) return hipErrorInvalidValue;
      kern = !p.lse ? attn_fwd_kernel<FP8, DQK, BN, NW, 0, false, true>
                    : attn_fwd_kernel<FP8, DQK, BN, NW, 1, false, true>;
    }
  } else {
    if (p.q_f32) return hipErrorInvalidValue;
  }
  if constexpr (FP8 && DQK == 128) {
    if (p.split) {
      if (p.lse_rounded) return hipErrorInvalidValue;
      kern = !p.lse ? attn_fwd_kernel<FP8, DQK, BN, NW, 0, true, false>
                    : attn_fwd_kernel<FP8, DQK, BN, NW, 1, true, false>;
    }
  } else {
    if (p.split) return hipErrorInvalidValue;
  }
  const int lds = p.split ? C::LDS_SPLIT : p.q_f32 ? C::LDS_QF32 : C::LDS;
  hipError_t e = hipFuncSetAttribute((const void*)kern,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(C::NT), lds, stream, p);
  return hipGetLastError();
}

}  // namespace attn
