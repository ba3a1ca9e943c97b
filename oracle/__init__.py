"""CPU fp64 oracle for causal prefill attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check in the repository's entry module and the
CPU-baseline leg of the benchmark may import this package.  The product path
(the HIP library and its Python binding) never imports, calls or links it, and
this package shares no code with that path: it is a plain, slow restatement of
what the path computes, written from the method's description, so that the
GPU results can be checked against it.

Contents
--------
formats    -- exact decoders for bf16 and OCP e4m3fn codes, a round-to-nearest-
              even saturating e4m3 encoder, absmax quantisation, and the same
              after a block Hadamard rotation (float32 butterflies), and Q
              quantisation with a descale that makes the FP8 softmax constant a
              power of two; joint Q/K quantisation that stores each KV group's
              largest-product channels last (scores unchanged) with those channels
              also as bf16 side arrays; a round-to-nearest-even bf16 encoder.
attention  -- the plain definition of causal softmax attention in float64
              (whole-row softmax, no online/tiled evaluation), over all rows or
              over sampled (b, h, i) rows; the same with Nq queries over Nk keys
              and a query offset; the merge of two partial attentions.

Every function is pinned by the `-m "not gpu"` tests against library routines
(torch's float8/bfloat16 casts, torch's scaled_dot_product_attention in fp64),
closed forms (equal scores, row 0, hard-max limit), invariants (causality,
rows of P summing to one, GQA == repeated-KV MHA) and brute-force loops on tiny
inputs.  No function here is "parity unpinned".
"""
from .formats import (bf16_decode, e4m3_decode, e4m3_encode, quantize_e4m3,
                      absmax_descale, encode_with_descale, E4M3_MAX, hadamard_block,
                      hadamard_unnormalised_fp32, quantize_e4m3_hadamard,
                      quantize_e4m3_q_pow2, pow2_q_descale_one, OUTLIER_CHANNELS,
                      channel_absmax, outlier_permutation, quantize_e4m3_qk_outliers,
                      bf16_encode, decode_qk_outliers)
from .attention import (causal_attention, causal_attention_rows, kv_head_of,
                        merge_partials, offset_attention, visible_keys)

__all__ = ["bf16_decode", "e4m3_decode", "e4m3_encode", "quantize_e4m3", "absmax_descale",
           "encode_with_descale", "E4M3_MAX", "hadamard_block", "hadamard_unnormalised_fp32",
           "quantize_e4m3_hadamard", "quantize_e4m3_q_pow2", "pow2_q_descale_one",
           "OUTLIER_CHANNELS", "channel_absmax", "outlier_permutation",
           "quantize_e4m3_qk_outliers", "bf16_encode", "decode_qk_outliers",
           "causal_attention", "causal_attention_rows", "kv_head_of", "visible_keys",
           "offset_attention", "merge_partials"]
