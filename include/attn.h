/*
 * attn.h -- C ABI of libattn: causal forward (prefill) attention for AMD
 * Instinct MI355X (CDNA4, gfx950), in BF16 and FP8 e4m3, for head dim 128
 * with grouped KV heads and for the MLA shape (d_qk = 192, d_v = 128).
 *
 * What is computed (the-ai.news "Waarom presteert FP8 minder goed op de
 * MI355X?"; spke.com "TL;DR"; ai-daily-news.org "Qué cubren los kernels"):
 * for every batch b, query head h and query i,
 *     O[b,i,h,:]  = sum_{j<=i} softmax_j(scale * Q[b,i,h,:].K[b,j,g,:]) V[b,j,g,:]
 *     LSE[b,h,i]  = log sum_{j<=i} exp(scale * Q[b,i,h,:].K[b,j,g,:])
 * with g = h / (Hq / Hkv) (consecutive query heads share a KV head), computed
 * tile by tile with an online softmax so the N x N score matrix is never
 * stored (kongchang.com "为什么 prefill attention 值得单独优化").
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *     allocates no memory, keeps no state between calls and never
 *     synchronises: work is enqueued on `stream` (a hipStream_t passed as
 *     void*; NULL means the null stream) and the call returns at once.
 *   - Layouts are contiguous "BSHD", head dim innermost:
 *       q (B, N, Hq,  d_qk)   k (B, N, Hkv, d_qk)   v (B, N, Hkv, d_v)
 *       o (B, N, Hq,  d_v)  bf16        lse (B, Hq, N) float32
 *     q, k, v, o must be 16-byte aligned; lse and descale pointers 4-byte
 *     aligned.
 *   - Accepted shapes: B >= 1, N >= 1, Hq >= 1, Hkv >= 1, Hq % Hkv == 0,
 *     (d_qk, d_v) in {(128, 128), (192, 128)}, softmax_scale finite and > 0,
 *     and every tensor smaller than 2^31 elements.  Anything else is rejected
 *     before any launch.
 *   - Return value: ATTN_OK (0) or a negative ATTN_E_* code; no call aborts
 *     and no exception crosses the ABI.  attn_status_string() names a code.
 *   - NaN or Inf inputs give undefined output values but no fault.
 *   - Calls are thread-safe.  Results are bit-identical across repeated runs
 *     on the same device (no atomics or split reductions in the attention
 *     kernels; spke.com "ZYFAのFP8アテンションの精度はどのくらいか?" reports
 *     bit-identical outputs across repeated runs).
 */
#ifndef LIBATTN_ATTN_H
#define LIBATTN_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum attn_status {
  ATTN_OK = 0,
  ATTN_E_INVAL = -1,        /* bad size, scale, NULL pointer or flag           */
  ATTN_E_UNSUPPORTED = -2,  /* (d_qk, d_v) not one of the supported pairs      */
  ATTN_E_ALIGN = -3,        /* a tensor pointer is not 16-byte aligned         */
  ATTN_E_NODEVICE = -4,     /* no usable HIP device                            */
  ATTN_E_LAUNCH = -5,       /* the HIP runtime reported a launch error (this
                               includes a device without gfx950 code)          */
  ATTN_E_TOO_LARGE = -6     /* sizes beyond the fixed scratch of an
                               allocation-free entry point                     */
};

/*
 * BF16 causal attention.
 *   q, k, v   bf16 inputs in the layouts above.
 *   o         bf16 output (B, N, Hq, d_v), written in full.
 *   lse       float32 (B, Hq, N) natural-log log-sum-exp of the scaled scores,
 *             or NULL to skip it.
 *   softmax_scale  multiplies Q.K before the softmax (usually 1/sqrt(d_qk)).
 * Scores and the O accumulator are float32; probabilities enter the P.V
 * product as bf16.
 */
int attn_fwd_causal_bf16(const void* q, const void* k, const void* v,
                         void* o, float* lse,
                         int B, int Hq, int Hkv, int N, int d_qk, int d_v,
                         float softmax_scale, void* stream);

/*
 * FP8 causal attention (spke.com "ZYFAはどのように動作するのか?"; the-ai.news
 * "Drie technieken om de bottleneck te omzeilen").
 *   q, k, v   OCP e4m3fn codes (uint8) in the layouts above; the value of a
 *             code c of head h is e4m3(c) * descale.
 *   q_descale, k_descale, v_descale  DEVICE float32 pointers: one value each
 *             when descale_per_head == 0, else Hq (q) / Hkv (k, v) values.
 *   o, lse    as for the BF16 entry point (o is bf16).
 * Q.K^T and P.V run on the e4m3 matrix instructions with float32
 * accumulation; each 64-key block of probabilities is scaled by a power of two
 * that the scaled matrix instruction removes.
 *   lse == NULL: each probability is written straight as an e4m3 code from one
 *             multiply-add and one integer conversion, using that the code of 2^x
 *             is about 8x plus a constant, and O is divided by the sum of the
 *             rounded probabilities (one extra matrix instruction per block).
 *   lse != NULL: the probabilities are exact exponentials rounded to e4m3, and
 *             their exact float32 sum both normalises O and gives the LSE (the
 *             rounded-code sum is too coarse for an LSE).  When the float32
 *             softmax constant fl(fl(softmax_scale * log2 e) * fl(dq * dk)) lies
 *             within 4 ulps of a power of two (quantize_e4m3_q_pow2 chooses such
 *             a Q descale), that power of two is applied by the Q operand's
 *             scale of the matrix instruction, which then yields the exponent
 *             arguments directly (no multiply-add per score, about 8% faster).
 * The FP8 matrix instructions sum each run of 8 consecutive channel products
 * after truncating every product toward zero to a multiple of 2^(E - 13), E the
 * largest exponent sum e_q + e_k of the run's factors (measured), so a score
 * carries an error below 7 * 2^(E-13) per run of 8 channels; O and LSE inherit
 * it.  On inputs with outlier channels that reaches 0.1-0.3 in the LSE: use
 * quantize_e4m3_qk_outliers with attn_fwd_causal_fp8_outliers there.
 */
int attn_fwd_causal_fp8(const uint8_t* q, const uint8_t* k, const uint8_t* v,
                        const float* q_descale, const float* k_descale,
                        const float* v_descale, int descale_per_head,
                        void* o, float* lse,
                        int B, int Hq, int Hkv, int N, int d_qk, int d_v,
                        float softmax_scale, void* stream);

/*
 * attn_fwd_causal_fp8 on float32 Q: q is DEVICE float32 (B, N, Hq, d_qk),
 * 16-byte aligned, and q_descale its descales (from quantize_e4m3,
 * quantize_e4m3_q_pow2, or quantize_e4m3_qkv with q_out == NULL).  The kernel
 * encodes each Q row as it loads it, with the quantisers' encoder (round to
 * nearest even of x / descale, saturating at +-448, NaN to 0x7F), so O and the
 * LSE are byte-identical to quantising Q and calling attn_fwd_causal_fp8; the
 * separate pass that writes Q's codes (a read of the float32 tensor and a write
 * of a quarter of its size) is not needed.  Other arguments and the results as
 * for attn_fwd_causal_fp8 (d_qk 128 or 192).
 */
int attn_fwd_causal_fp8_qf32(const float* q, const uint8_t* k, const uint8_t* v,
                             const float* q_descale, const float* k_descale,
                             const float* v_descale, int descale_per_head,
                             void* o, float* lse,
                             int B, int Hq, int Hkv, int N, int d_qk, int d_v,
                             float softmax_scale, void* stream);

/*
 * Causal attention of Nq queries over Nk keys with a query offset: key j is
 * visible to query i iff j <= i + q_offset.  This is the same computation with
 * the causal diagonal shifted, for query chunks that follow a KV prefix
 * (chunked prefill: q_offset = Nk - Nq for the last Nq of Nk positions) and for
 * a chunk of keys that lies entirely before the queries (q_offset >= Nk - 1:
 * every key visible).  The pages' kernels stop at Nq = Nk and name
 * variable-length work as future work (ai-daily-news.org "Qué cubren los
 * kernels"); this is that extension, with the partials combined by
 * attn_merge_partials below.
 *   q (B, Nq, Hq, d_qk), k (B, Nk, Hkv, d_qk), v (B, Nk, Hkv, d_v),
 *   o (B, Nq, Hq, d_v) bf16, lse (B, Hq, Nq) float32 or NULL.
 *   q_offset  >= 0; values above Nk act as Nk.  Every query sees key 0.
 * Everything else (arguments, numerics, errors) as for the entry points above;
 * attn_fwd_causal_bf16/_fp8 are these with Nq = Nk = N and q_offset = 0.
 */
int attn_fwd_causal_offset_bf16(const void* q, const void* k, const void* v,
                                void* o, float* lse,
                                int B, int Hq, int Hkv, int Nq, int Nk, int q_offset,
                                int d_qk, int d_v, float softmax_scale, void* stream);

int attn_fwd_causal_offset_fp8(const uint8_t* q, const uint8_t* k, const uint8_t* v,
                               const float* q_descale, const float* k_descale,
                               const float* v_descale, int descale_per_head,
                               void* o, float* lse,
                               int B, int Hq, int Hkv, int Nq, int Nk, int q_offset,
                               int d_qk, int d_v, float softmax_scale, void* stream);

/*
 * attn_fwd_causal_offset_fp8 on the fast path (probabilities written straight as
 * e4m3 codes, O divided by the sum of the rounded probabilities: spke.com
 * "ブロックごとのスケーリングと丸められた行和"), which also writes the LSE of
 * that same row sum: lse = m + ln(sum of the rounded probabilities).  That LSE is
 * the one consistent with O's normaliser, which is what the merge of partial
 * attentions needs; it differs from the exact log-sum-exp by the rounding of the
 * probabilities: each rounded probability is within a factor 0.917 .. 1.061 of
 * the exact one, so the LSE is within 0.087 of the exact LSE (less with many keys
 * per row), not a substitute where the exact LSE is required.  o is byte-identical to the
 * lse == NULL call.
 *   lse       required (NULL returns ATTN_E_INVAL); everything else as for
 *             attn_fwd_causal_offset_fp8.
 */
int attn_fwd_causal_offset_fp8_rounded_lse(const uint8_t* q, const uint8_t* k,
                                           const uint8_t* v, const float* q_descale,
                                           const float* k_descale, const float* v_descale,
                                           int descale_per_head, void* o, float* lse,
                                           int B, int Hq, int Hkv, int Nq, int Nk,
                                           int q_offset, int d_qk, int d_v,
                                           float softmax_scale, void* stream);

/*
 * Merge of two partial attentions of the same queries over disjoint key sets
 * (e.g. a KV-prefix chunk and the causal chunk, from the offset entry points):
 *   m   = max(lse_a, lse_b)
 *   o   = (e^(lse_a-m) o_a + e^(lse_b-m) o_b) / (e^(lse_a-m) + e^(lse_b-m))
 *   lse = m + ln(e^(lse_a-m) + e^(lse_b-m))
 * which is the attention over the union of the two key sets.  A partial whose
 * LSE is -inf carries weight 0 (both -inf: o = 0, lse = -inf).
 *   o_a, o_b, o   DEVICE bf16 (B, N, Hq, d_v), 16-byte aligned.
 *   lse_a, lse_b  DEVICE float32 (B, Hq, N); lse (output) may be NULL.
 *   d_v           a power of two in [8, 512].
 * Computed in float32, o rounded to nearest even.  Outputs may alias the
 * inputs (in-place merge).  One kernel is enqueued.
 */
int attn_merge_partials(const void* o_a, const float* lse_a,
                        const void* o_b, const float* lse_b,
                        void* o, float* lse, int B, int N, int Hq, int d_v,
                        void* stream);

/*
 * Absmax quantisation of a float32 (B, N, H, d) tensor into e4m3fn codes
 * (kongchang.com "ZYFA 的性能与精度数据": per-tensor or per-head scale
 * factors map values into the e4m3 range).
 *   x         DEVICE float32 input, contiguous (B, N, H, d), 16-byte aligned.
 *   out       DEVICE uint8 output of the same shape, 4-byte aligned.
 *   descale   DEVICE float32 output: 1 value (per_head == 0) or H values.
 *             descale = absmax / 448 in float32 (1 for an all-zero tensor or
 *             head); it is also used as scratch during the call.
 *   code      = round-to-nearest-even e4m3 of the float32 quotient x / descale,
 *             saturating at +-448; NaN maps to 0x7F.  NaN elements take no
 *             part in the absmax; an infinity makes the descale infinite (then
 *             finite elements encode to signed zeros).
 * d must be a multiple of 4, H <= 65535 and the tensor below 2^31 elements.
 * Invalid arguments return ATTN_E_INVAL / ATTN_E_ALIGN before any launch.  The absmax reduction is order-independent, so
 * results are bit-identical across runs.  Four kernels are enqueued.
 */
int quantize_e4m3(const float* x, uint8_t* out, float* descale,
                  int B, int N, int H, int d, int per_head, void* stream);

/*
 * quantize_e4m3 for Q with a descale chosen for the FP8 attention that follows:
 * any descale at or above absmax / 448 keeps every value in range (the pages fix
 * per-tensor or per-head scale factors, kongchang.com "ZYFA 的性能与精度数据",
 * not their value), and this one makes the kernel's float32 softmax constant
 * c = fl(fl(softmax_scale * log2 e) * fl(descale * k_descale)) lie within 4 ulps
 * of a power of two.  attn_fwd_causal_fp8 (and the offset form) with an LSE
 * then applies c through the matrix instruction's power-of-two operand scale
 * instead of one multiply-add per score (about 8% faster at 32K tokens).
 *   k_descale DEVICE float32: K's descales from quantize_e4m3, 1 value
 *             (per_head == 0) or Hkv values (per_head == 1); query head h pairs
 *             with KV head h / (H / Hkv).  Read on the device, in stream order.
 *   Hkv       number of KV heads (H % Hkv == 0 when per_head == 1).
 *   descale   = the smallest power of two at or above
 *             fl(fl(absmax / 448) * fl(fl(softmax_scale * log2 e) * dk)), divided
 *             by fl(fl(softmax_scale * log2 e) * dk), then moved one ulp at a time
 *             (at most 16) until c is within 4 ulps of that power of two; so
 *             absmax / 448 <= descale < 2 * absmax / 448 up to a few ulps.  A zero
 *             or non-finite absmax (or dk), or no such descale, keeps the plain
 *             quantize_e4m3 descale.  Codes as in quantize_e4m3, of x / descale.
 * Other arguments, limits and errors as for quantize_e4m3 (softmax_scale must be
 * finite and positive).  Four kernels are enqueued.
 */
int quantize_e4m3_q_pow2(const float* x, uint8_t* out, float* descale,
                         int B, int N, int H, int d, int per_head,
                         const float* k_descale, int Hkv, float softmax_scale,
                         void* stream);

/*
 * Q, K and V quantised in one call: K and V as quantize_e4m3, Q as
 * quantize_e4m3_q_pow2 against K's descales (q_pow2 == 1) or as quantize_e4m3
 * (q_pow2 == 0); codes and descales are bit-identical to those separate calls.
 * Four kernels are enqueued instead of twelve (each pass runs over the three
 * tensors in one launch), which saves the short launches' start-up and tail
 * costs (the per-tensor scale factors: kongchang.com "ZYFA 的性能与精度数据").
 *   q           DEVICE float32 (B, Nq, Hq, d_qk); k (B, Nk, Hkv, d_qk); v
 *               (B, Nk, Hkv, d_v); all contiguous and 16-byte aligned.
 *   q_out, k_out, v_out  DEVICE uint8 codes of the same shapes, 4-byte aligned.
 *               q_out may be NULL: then only Q's descales are computed, for
 *               attn_fwd_causal_fp8_qf32, which encodes float32 Q itself.
 *   q_descale, k_descale, v_descale  DEVICE float32: 1 value each (per_head ==
 *               0), else Hq, Hkv and Hkv values; used as scratch during the
 *               call.
 *   softmax_scale  as for quantize_e4m3_q_pow2 (read only when q_pow2 == 1).
 * d_qk and d_v must be multiples of 4, Hq and Hkv at most 65535, Hq % Hkv == 0
 * with q_pow2 and per_head, each tensor below 2^31 elements.  Invalid
 * arguments return ATTN_E_INVAL / ATTN_E_ALIGN before any launch.
 */
int quantize_e4m3_qkv(const float* q, const float* k, const float* v,
                      uint8_t* q_out, uint8_t* k_out, uint8_t* v_out,
                      float* q_descale, float* k_descale, float* v_descale,
                      int B, int Nq, int Nk, int Hq, int Hkv, int d_qk, int d_v,
                      int per_head, int q_pow2, float softmax_scale, void* stream);

/*
 * quantize_e4m3 of the Hadamard-rotated tensor, the FP8 pre-step for Q and K
 * (spke.com "ZYFAのFP8アテンションの精度はどのくらいか?": most of the FP8
 * error comes from quantising Q, K and V, and a Hadamard rotation of Q and K
 * roughly halves that input error).  Each block of hb channels of every
 * (b, n, h) row, hb = the largest power of two dividing d and at most 128
 * (128 for d = 128, 64 for d = 192), is multiplied by H / sqrt(hb), H the
 * Sylvester Hadamard matrix of order hb.  That matrix is orthogonal and
 * symmetric, so rotating both Q and K leaves every score Q.K unchanged while
 * outlier channels are spread over the block; feed the codes and descales to
 * attn_fwd_causal_fp8 as usual (V is not rotated).
 *   The rotated values are the float32 results of radix-2 butterflies on the
 *   unnormalised block (stage half-sizes 1, 2, 4, ... in that order; the element
 *   with the stage bit clear becomes a + b, its partner a - b); codes are
 *   round-to-nearest-even e4m3 of value / (absmax / 448) as in quantize_e4m3,
 *   and descale = (absmax / 448) * float32(1 / sqrt(hb)), so code * descale is
 *   the normalised rotated value.  Arguments, limits and errors as for
 *   quantize_e4m3.  Four kernels are enqueued.
 *   Whether the rotation lowers the score error depends on the data: with
 *   synthetic outlier channels shared by Q and K it cuts the FP8 score error
 *   several-fold; with outliers on different channels of Q and K it raises it,
 *   since e4m3 keeps a relative precision per element and the rotation mixes
 *   every channel into each.
 */
int quantize_e4m3_hadamard(const float* x, uint8_t* out, float* descale,
                           int B, int N, int H, int d, int per_head, void* stream);

/*
 * Outlier channels.  gfx950's FP8 matrix instructions add each run of 8
 * consecutive channel products after truncating every product toward zero to
 * 13 bits below the run's largest exponent sum (measured through this library).  One
 * channel whose Q or K magnitude is far above the others (the outlier
 * channels of real activations) then swamps the small products of its run:
 * on such inputs the scores, and the LSE, move by up to about 0.1-0.3 instead
 * of the rounding of the inputs (the pages name the FP8 error of Q and K as
 * the one that matters, spke.com "ZYFAのFP8アテンションの精度はどのくらいか?").
 * Permuting the channels of Q and K the same way leaves every score
 * unchanged, so the pair below takes those channels out of the FP8 products:
 * quantize_e4m3_qk_outliers stores each KV head's ATTN_OUTLIER_CHANNELS
 * largest-product channels last and writes them also as bf16 side arrays, and
 * attn_fwd_causal_fp8_outliers multiplies those last channels of every Q and K
 * row on the BF16 matrix instructions from the side arrays (exact products,
 * float32 sums) and the other channels on the FP8 ones from the codes.
 */
#define ATTN_OUTLIER_CHANNELS 32

/*
 * e4m3 quantisation of Q (B, N, Hq, d) and K (B, N, Hkv, d), float32, with
 * each KV head's largest-product channels stored last in every Q and K row.
 *   Channel absmax: max |x| over all (b, n) of one head (NaN ignored).  The
 *   importance of channel c for KV head g is the float32 product of the
 *   largest Q absmax of c among g's query heads and K's absmax of c (0 when
 *   either is 0).  The ATTN_OUTLIER_CHANNELS channels of largest importance
 *   (ties: the lower channel) are stored last in ascending channel order,
 *   after the other channels in ascending order.
 *   q_out, k_out  DEVICE uint8 codes (same shapes), 4-byte aligned: stored
 *             position j of a row of head h (KV head g = h / (Hq / Hkv) for Q)
 *             holds the code of channel perm[g * d + j]; the codes themselves
 *             are quantize_e4m3's (x / descale rounded to nearest even).
 *   q_exact, k_exact  DEVICE bf16 side arrays (B, N, Hq, ATTN_OUTLIER_CHANNELS)
 *             and (B, N, Hkv, ATTN_OUTLIER_CHANNELS), 16-byte aligned: for the
 *             last ATTN_OUTLIER_CHANNELS stored positions, the bf16 (round to
 *             nearest even) of the float32 quotient x / descale, i.e. the same
 *             channels in descale units with 8 instead of 4 significant bits.
 *   q_descale, k_descale  DEVICE float32 outputs, Hq / Hkv values (per_head)
 *             or 1 each: quantize_e4m3's descales; with q_pow2 = 1, Q's is
 *             the one quantize_e4m3_q_pow2 would choose against K's.
 *   perm      DEVICE uint8 output (Hkv, d), 4-byte aligned.
 *   workspace DEVICE scratch of workspace_bytes >=
 *             quantize_e4m3_qk_outliers_workspace_bytes(Hq, Hkv, d) bytes,
 *             4-byte aligned; its contents on entry do not matter.
 *   q, k      DEVICE float32, 16-byte aligned.
 *   d         a multiple of 4 in [ATTN_OUTLIER_CHANNELS, 256]; Hq % Hkv == 0;
 *             softmax_scale finite and > 0 when q_pow2 (else unused).
 * Codes and descales are bit-identical across runs.  Six kernels are
 * enqueued.  Invalid arguments return ATTN_E_INVAL / ATTN_E_ALIGN before any
 * launch.
 */
int quantize_e4m3_qk_outliers(const float* q, const float* k,
                              uint8_t* q_out, uint8_t* k_out, void* q_exact, void* k_exact,
                              float* q_descale, float* k_descale, uint8_t* perm,
                              void* workspace, size_t workspace_bytes,
                              int B, int N, int Hq, int Hkv, int d, int per_head,
                              int q_pow2, float softmax_scale, void* stream);

/* Bytes of workspace quantize_e4m3_qk_outliers needs: (Hq + Hkv) * d * 4. */
size_t quantize_e4m3_qk_outliers_workspace_bytes(int Hq, int Hkv, int d);

/*
 * quantize_e4m3_qk_outliers without the workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the per-channel accumulators live in
 * a fixed scratch array of ATTN_NOALLOC_SCRATCH_WORDS 32-bit words per device,
 * part of the library's device code (each GPU the library runs on holds its own
 * copy, 256 KiB, until the process ends).  The call allocates nothing.
 *   (Hq + Hkv) * d > ATTN_NOALLOC_SCRATCH_WORDS returns ATTN_E_TOO_LARGE before
 *   any launch; other arguments, results and errors as for
 *   quantize_e4m3_qk_outliers (bit-identical outputs).
 *   The scratch is cleared by the call's first kernel, so earlier calls leave
 *   nothing behind that matters; but every call on one GPU shares it, so calls
 *   that overlap on one GPU (other streams, other threads) race and give wrong
 *   results: serialise them.  The first call on each device looks the array's
 *   address up (hipGetSymbolAddress) and keeps it.
 */
#define ATTN_NOALLOC_SCRATCH_WORDS 65536
int quantize_e4m3_qk_outliers_noalloc(const float* q, const float* k,
                                      uint8_t* q_out, uint8_t* k_out,
                                      void* q_exact, void* k_exact,
                                      float* q_descale, float* k_descale, uint8_t* perm,
                                      int B, int N, int Hq, int Hkv, int d, int per_head,
                                      int q_pow2, float softmax_scale, void* stream);

/*
 * attn_fwd_causal_fp8 and attn_fwd_causal_offset_fp8 with the last
 * ATTN_OUTLIER_CHANNELS channels of every Q and K row taken from bf16 side
 * arrays and multiplied on the BF16 matrix instructions (exact products,
 * float32 sums) instead of the FP8 ones: channel c < d_qk - 32 of a Q row has
 * the value e4m3(q[c]) * q_descale, channel d_qk - 32 + i the value
 * bf16(q_exact[i]) * q_descale (K alike); the codes of the last 32 channels
 * are not read.  Feed them the outputs of quantize_e4m3_qk_outliers.
 *   q_exact (B, N, Hq, 32), k_exact (B, N, Hkv, 32)  DEVICE bf16, 16-byte
 *             aligned (offset form: Nq rows for q_exact, Nk for k_exact).
 * d_qk must be 128 (else ATTN_E_UNSUPPORTED).  lse may be NULL (then the
 * probabilities take the fast path, as for attn_fwd_causal_fp8).  Everything
 * else as for those entry points.  The extra work per key tile is 8 BF16
 * matrix instructions of 32x32x16 (a quarter of the tile's Q.K^T time) and a
 * 64-byte side row per key copied with the tile.
 */
int attn_fwd_causal_fp8_outliers(const uint8_t* q, const uint8_t* k, const uint8_t* v,
                                 const void* q_exact, const void* k_exact,
                                 const float* q_descale, const float* k_descale,
                                 const float* v_descale, int descale_per_head,
                                 void* o, float* lse,
                                 int B, int Hq, int Hkv, int N, int d_qk, int d_v,
                                 float softmax_scale, void* stream);

int attn_fwd_causal_offset_fp8_outliers(const uint8_t* q, const uint8_t* k,
                                        const uint8_t* v, const void* q_exact,
                                        const void* k_exact, const float* q_descale,
                                        const float* k_descale, const float* v_descale,
                                        int descale_per_head, void* o, float* lse,
                                        int B, int Hq, int Hkv, int Nq, int Nk,
                                        int q_offset, int d_qk, int d_v,
                                        float softmax_scale, void* stream);

/* Static, NUL-terminated name of a status code; never NULL. */
const char* attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* LIBATTN_ATTN_H */
