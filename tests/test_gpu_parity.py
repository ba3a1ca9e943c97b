"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Small and mid sizes compare every output element; the full 16K/32K workloads
compare sampled rows (the oracle computes them one by one) in the same launch
configuration the benchmark times.  Also: quantize_e4m3 bit-exact against the
oracle's encoder, run-to-run byte identity, causality under perturbation of
later keys, GQA == MHA with repeated K/V, and the equal-scores closed form.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_harness import (DEV, ROUNDED_LSE_BOUND, ElemBoundMiss, LseGateMiss, abs_v, bf16_bytes, check,
                         gpu_quantize, note, run_bf16, run_fp8)

import bf16_causal_prefill_amd as ba

pytestmark = pytest.mark.gpu

W = workloads.CONFIGS


def _small_cases():
    g = W["tiny"]
    return {
        "tiny": W["tiny"],
        "mid_gqa": W["mid_gqa"],
        "ragged_gqa_n300_b2": g.with_(name="ragged", B=2, Hq=8, Hkv=2, N=300, seed=21),
        "n1": g.with_(name="n1", N=1, seed=22),
        "n33": g.with_(name="n33", Hq=4, Hkv=1, N=33, seed=23),
        "n65_b3": g.with_(name="n65", B=3, N=65, seed=24),
        "mistral_n1024": W["mistral16k"].with_(N=1024, seed=25),
        "mla_n700": W["mla16k"].with_(N=700, Hq=4, Hkv=4, seed=26),
        "mla_n256_per_tensor": W["mla16k"].with_(N=256, Hq=2, Hkv=2, fp8_per_head=False, seed=27),
    }


SMALL = _small_cases()


def _oracle_bf16(x, w):
    qu, ku, vu = (bf16_bytes(x[n]) for n in "qkv")
    dec = [oracle.bf16_decode(a) for a in (qu, ku, vu)]
    return (qu, ku, vu), dec


def _fp8_inputs(x, w):
    """GPU-quantised device codes + oracle-quantised host codes; asserts equality."""
    dev, host = [], []
    for n in "qkv":
        codes_d, ds_d = gpu_quantize(x[n], w.fp8_per_head)
        codes_h, ds_h = oracle.quantize_e4m3(x[n], w.fp8_per_head)
        cd = codes_d.cpu().numpy()
        assert np.array_equal(cd, codes_h), f"quantize_e4m3({n}) codes differ from the oracle"
        assert np.array_equal(ds_d.cpu().numpy().view(np.uint32), ds_h.view(np.uint32)), n
        dev.append((codes_d, ds_d))
        host.append(oracle.e4m3_decode(codes_h) * (ds_h[None, None, :, None].astype(np.float64)
                                                   if w.fp8_per_head else float(ds_h[0])))
    return dev, host


@pytest.mark.parametrize("case", list(SMALL))
def test_bf16_parity_full(case):
    w = SMALL[case]
    note(f"case bf16 {case}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} d={w.d_qk}/{w.d_v}")
    x = workloads.generate(w)
    (qu, ku, vu), (q, k, v) = _oracle_bf16(x, w)
    out = run_bf16(qu, ku, vu, w.softmax_scale)[0]
    ro, rl = oracle.causal_attention(q, k, v, w.softmax_scale)
    check(case, "bf16", out.o, ro, out.lse, rl)


# The plain FP8 path on the outlier-channel recipe: its LSE misses the 1e-2 gate.  The
# FP8 matrix instruction sums each run of 8 products after aligning them to the largest,
# truncating about 12 bits below it (test_fp8_matrix_accumulation_model), and an x20
# outlier channel of Q or K makes that largest product large against the rest of its
# run.  Measured worst LSE errors: 0.115 (absmax Q scale) and 0.23 (power-of-two Q
# scale) at N=1024, 0.015 on the sampled 16K rows; the same score errors move single O
# elements past the per-element bound, whose score term assumes accurate scores.  These cases stay here, xfail and
# strict (they must keep failing for that reason, and an unexpected pass is reported);
# the outlier-channel path (quantize_e4m3_qk_outliers with the exact-channel attention)
# is the one that meets the gate on this recipe.
PLAIN_FP8_LSE_MISS = pytest.mark.xfail(
    strict=True, raises=(LseGateMiss, ElemBoundMiss),
    reason="plain FP8 path on x20 outlier channels: the FP8 matrix instruction's grouped "
           "truncation moves the scores, so the LSE (measured 0.115 at N=1024) and the O "
           "elements next to it leave their bounds")


def _xfail_outliers(cases, recipe_of):
    return [pytest.param(c, marks=PLAIN_FP8_LSE_MISS) if recipe_of(c) == "mistral" else c
            for c in cases]


@pytest.mark.parametrize("case", _xfail_outliers(list(SMALL), lambda c: SMALL[c].recipe))
def test_fp8_parity_full(case):
    w = SMALL[case]
    note(f"case fp8 {case}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} d={w.d_qk}/{w.d_v} "
         f"per_head={w.fp8_per_head}")
    x = workloads.generate(w)
    dev, (q, k, v) = _fp8_inputs(x, w)
    (qc, qd), (kc, kd), (vc, vd) = dev
    out = run_fp8(qc, kc, vc, qd, kd, vd, w.fp8_per_head, w.softmax_scale)[0]
    ro, rl = oracle.causal_attention(q, k, v, w.softmax_scale)
    check(case, "fp8", out.o, ro, out.lse, rl, fp8_path="exact",
          ref_abs_o=abs_v(oracle.causal_attention, q, k, v, w.softmax_scale))


@pytest.mark.parametrize("prec", ["bf16", "fp8"])
def test_without_lse(prec):
    """lse=NULL skips the LSE work.  BF16: O is byte-identical to the LSE run.
    FP8: without the LSE the kernel writes the probabilities with the one-FMA
    e4m3 code and normalises by the row sum of the rounded codes (a different,
    cheaper approximation than the LSE run's exact exponentials), so O is checked
    against the oracle on its own, within the FP8 tolerance."""
    w = SMALL["ragged_gqa_n300_b2"]
    x = workloads.generate(w)
    if prec == "bf16":
        (qu, ku, vu), _ = _oracle_bf16(x, w)
        a = run_bf16(qu, ku, vu, w.softmax_scale, want_lse=True)[0]
        b = run_bf16(qu, ku, vu, w.softmax_scale, want_lse=False)[0]
        assert a.o_bytes == b.o_bytes
    else:
        for case in ("ragged_gqa_n300_b2", "mistral_n1024", "mla_n700"):
            w = SMALL[case]
            x = workloads.generate(w)
            dev, (q, k, v) = _fp8_inputs(x, w)
            (qc, qd), (kc, kd), (vc, vd) = dev
            b = run_fp8(qc, kc, vc, qd, kd, vd, w.fp8_per_head, w.softmax_scale,
                        want_lse=False)[0]
            ro, _ = oracle.causal_attention(q, k, v, w.softmax_scale)
            check(case + "/no-lse", "fp8", b.o, ro, fp8_path="lean",
                  ref_abs_o=abs_v(oracle.causal_attention, q, k, v, w.softmax_scale))


@pytest.mark.parametrize("name", ["tiny", "mid_gqa"])
@pytest.mark.parametrize("prec", ["bf16", "fp8", "fp8_nolse"])
def test_deterministic_repeats(prec, name):
    """100 runs of the same call give byte-identical O and LSE (the pages report
    bit-identical outputs over repeated runs; spke.com "ZYFAのFP8アテンションの精度は
    どのくらいか?")."""
    w = W[name]
    x = workloads.generate(w)
    if prec == "bf16":
        (qu, ku, vu), _ = _oracle_bf16(x, w)
        run_bf16(qu, ku, vu, w.softmax_scale, repeats=100)
    else:
        dev, _ = _fp8_inputs(x, w)
        (qc, qd), (kc, kd), (vc, vd) = dev
        run_fp8(qc, kc, vc, qd, kd, vd, w.fp8_per_head, w.softmax_scale,
                want_lse=prec == "fp8", repeats=100)


@pytest.mark.parametrize("prec", ["bf16", "fp8"])
def test_causality_under_perturbation(prec):
    """Rewriting K/V rows >= c leaves O and LSE rows < c byte-identical."""
    w = W["tiny"].with_(B=1, Hq=4, Hkv=2, N=520, seed=31)
    x = workloads.generate(w)
    rng = np.random.default_rng(99)
    for c in (1, 64, 257, 519):
        y = {n: a.copy() for n, a in x.items()}
        y["k"][:, c:] = rng.standard_normal(y["k"][:, c:].shape).astype(np.float32) * 0.5
        y["v"][:, c:] = rng.standard_normal(y["v"][:, c:].shape).astype(np.float32) * 0.5
        if prec == "bf16":
            (qu, ku, vu), _ = _oracle_bf16(x, w)
            (qu2, ku2, vu2), _ = _oracle_bf16(y, w)
            a = run_bf16(qu, ku, vu, w.softmax_scale)[0]
            b = run_bf16(qu2, ku2, vu2, w.softmax_scale)[0]
        else:
            # quantise the unperturbed draw, then rewrite later codes only, so the
            # descales (and so every earlier input value) stay the same
            dev, _ = _fp8_inputs(x, w)
            (qc, qd), (kc, kd), (vc, vd) = dev
            kc2, vc2 = kc.clone(), vc.clone()
            for t in (kc2, vc2):   # random finite codes (never 0x7F / 0xFF)
                r = rng.integers(0, 0x7F, size=t[:, c:].shape) | (rng.integers(0, 2, size=t[:, c:].shape) << 7)
                t[:, c:] = torch.from_numpy(r.astype(np.uint8)).to(t.device)
            a = run_fp8(qc, kc, vc, qd, kd, vd, False, w.softmax_scale)[0]
            b = run_fp8(qc, kc2, vc2, qd, kd, vd, False, w.softmax_scale)[0]
        assert np.array_equal(a.o[:, :c], b.o[:, :c]), c
        assert np.array_equal(a.lse[:, :, :c], b.lse[:, :, :c]), c
        assert not np.array_equal(a.o[:, c:], b.o[:, c:]), c


@pytest.mark.parametrize("prec", ["bf16", "fp8"])
def test_gqa_equals_repeated_mha(prec):
    w = W["tiny"].with_(B=2, Hq=8, Hkv=2, N=200, seed=32)
    x = workloads.generate(w)
    G = w.Hq // w.Hkv
    xr = {"q": x["q"], "k": np.ascontiguousarray(np.repeat(x["k"], G, axis=2)),
          "v": np.ascontiguousarray(np.repeat(x["v"], G, axis=2))}
    if prec == "bf16":
        a = run_bf16(*_oracle_bf16(x, w)[0], w.softmax_scale)[0]
        b = run_bf16(*_oracle_bf16(xr, w)[0], w.softmax_scale)[0]
    else:
        wr = w.with_(Hkv=w.Hq)
        (qc, qd), (kc, kd), (vc, vd) = _fp8_inputs(x, w.with_(fp8_per_head=False))[0]
        a = run_fp8(qc, kc, vc, qd, kd, vd, False, w.softmax_scale)[0]
        (qc, qd), (kc, kd), (vc, vd) = _fp8_inputs(xr, wr.with_(fp8_per_head=False))[0]
        b = run_fp8(qc, kc, vc, qd, kd, vd, False, w.softmax_scale)[0]
    assert a.o_bytes == b.o_bytes and a.lse_bytes == b.lse_bytes


@pytest.mark.parametrize("prec", ["bf16", "fp8"])
def test_equal_scores_mean_of_v(prec):
    """Q = 0: O_i = mean(V_0..V_i) and LSE_i = ln(i+1)."""
    w = W["tiny"].with_(B=1, Hq=2, Hkv=1, N=300, seed=33)
    x = workloads.generate(w)
    x["q"][:] = 0.0
    if prec == "bf16":
        (qu, ku, vu), (_, _, v) = _oracle_bf16(x, w)
        out = run_bf16(qu, ku, vu, w.softmax_scale)[0]
    else:
        dev, (_, _, v) = _fp8_inputs(x, w)
        (qc, qd), (kc, kd), (vc, vd) = dev
        out = run_fp8(qc, kc, vc, qd, kd, vd, False, w.softmax_scale)[0]
    mean = np.cumsum(v[0, :, 0], axis=0) / np.arange(1, w.N + 1)[:, None]
    for h in range(w.Hq):
        err = np.max(np.abs(out.o[0, :, h] - mean))
        assert err < 2e-2, err
        assert np.max(np.abs(out.lse[0, h] - np.log(np.arange(1, w.N + 1)))) < 1e-4


# ---- full-size workloads, sampled rows -------------------------------------------

FULL = ["mistral16k", "gauss32k", "mla16k", "mla32k"]


def _sample_rows(w, n_rand=48, seed=7):
    rng = np.random.default_rng(seed)
    N = w.N
    fixed_i = [0, 1, 63, 64, 255, 256, N // 2, N - 257, N - 256, N - 65, N - 1]
    rows = []
    for b in range(w.B):
        for h in sorted({0, w.Hq - 1, w.Hq // 2}):
            rows += [(b, h, i) for i in fixed_i]
    rows += [(int(rng.integers(w.B)), int(rng.integers(w.Hq)), int(rng.integers(N)))
             for _ in range(n_rand)]
    return rows


FULL_CASES = [(p, n) for p in ("bf16", "fp8") for n in FULL] + \
    [("fp8_nolse", n) for n in ("gauss32k", "mla32k")] + \
    [("fp8_rounded_lse", n) for n in ("gauss32k", "mla32k")]


def _full_case_id(c):
    return f"{c[0]}-{c[1]}"


@pytest.mark.parametrize(
    "prec,name",
    [pytest.param(*c, marks=PLAIN_FP8_LSE_MISS, id=_full_case_id(c))
     if c == ("fp8", "mistral16k") else pytest.param(*c, id=_full_case_id(c))
     for c in FULL_CASES])
def test_full_size_sampled_rows(prec, name):
    """The full workloads in the launch configuration bench.py times, 10 byte-identical
    runs, every output finite, sampled rows against the oracle.  fp8_nolse is the Lean P
    kernel (no LSE), fp8_rounded_lse the same kernel writing the LSE of its rounded row
    sums (checked against its own bound, ROUNDED_LSE_BOUND)."""
    w = W[name]
    note(f"case full {prec} {name}: N={w.N} Hq={w.Hq} Hkv={w.Hkv} d={w.d_qk}/{w.d_v}")
    x = workloads.generate(w)
    rows = _sample_rows(w)
    bb = np.array([r[0] for r in rows])
    hh = np.array([r[1] for r in rows])
    ii = np.array([r[2] for r in rows])
    if prec == "bf16":
        (qu, ku, vu), (q, k, v) = _oracle_bf16(x, w)
        out = run_bf16(qu, ku, vu, w.softmax_scale, repeats=10)[0]
    elif prec == "fp8_rounded_lse":
        dev, (q, k, v) = _fp8_inputs(x, w)
        (qc, qd), (kc, kd), (vc, vd) = dev
        out = _run_rounded_lse(qc, kc, vc, qd, kd, vd, w, repeats=10)
    else:
        dev, (q, k, v) = _fp8_inputs(x, w)
        (qc, qd), (kc, kd), (vc, vd) = dev
        out = run_fp8(qc, kc, vc, qd, kd, vd, w.fp8_per_head, w.softmax_scale,
                      want_lse=prec == "fp8", repeats=10)[0]
    ro, rl = oracle.causal_attention_rows(q, k, v, w.softmax_scale, rows)
    go = out.o[bb, ii, hh]
    assert np.all(np.isfinite(out.o))
    gl = None
    if out.lse is not None:
        assert np.all(np.isfinite(out.lse))
        gl = out.lse[bb, hh, ii]
    heads = [(b, h) for b, h, _ in rows]
    if prec == "bf16":
        check(f"{name}/rows", prec, go, ro, gl, rl, row_heads=heads)
        return
    ra = abs_v(oracle.causal_attention_rows, q, k, v, w.softmax_scale, rows)
    path = "exact" if prec == "fp8" else "lean"
    if prec == "fp8_rounded_lse":
        check(f"{name}/rows/{prec}", "fp8", go, ro, ref_abs_o=ra, fp8_path=path, row_heads=heads)
        err = float(np.max(np.abs(gl - rl)))
        note(f"  rounded-sum LSE max |error| {err:.4f} (bound {ROUNDED_LSE_BOUND:.4f})")
        assert err <= ROUNDED_LSE_BOUND
    else:
        check(f"{name}/rows/{prec}", "fp8", go, ro, gl, rl if gl is not None else None,
              ref_abs_o=ra, fp8_path=path, row_heads=heads)




def _run_rounded_lse(qc, kc, vc, qd, kd, vd, w, repeats=1):
    """attn_fwd_causal_offset_fp8_rounded_lse with Nq = Nk = N, q_offset = 0 (the
    plain causal case); O must be byte-identical to the lse = NULL call."""
    from gpu_harness import _repeat
    B, N, Hq, _ = qc.shape
    out = _repeat(lambda o, lse: ba.attn_fwd_causal_offset_fp8_rounded_lse(
        qc, kc, vc, qd, kd, vd, o, lse, q_offset=0, softmax_scale=w.softmax_scale,
        descale_per_head=int(w.fp8_per_head)), B, N, Hq, vc.shape[3], True, repeats,
        "fp8/rounded-lse")[0]
    plain = run_fp8(qc, kc, vc, qd, kd, vd, w.fp8_per_head, w.softmax_scale, want_lse=False)[0]
    assert plain.o_bytes == out.o_bytes, "rounded-LSE O differs from the lse = NULL call"
    return out


def test_fp8_matrix_accumulation_model():
    """Pins the grouped accumulation of the FP8 matrix instruction, through the C ABI.  With N = 1 the LSE of row 0 is its single score q.k (scale 1, unit
    descales).  q = [256, 1 x 15, 0...], k = [64, 1 x 15, 0...]: the exact dot product
    is 16384 + 15 = 16399.  The 7 unit products that share the 8-channel group of the
    2^14 product fall below 2^(14-12) and are dropped; the 8 in the next group are
    kept, so the hardware gives 16392."""
    dev = "cuda:0"
    qc = np.zeros((1, 1, 1, 128), np.uint8)
    kc = np.zeros((1, 1, 1, 128), np.uint8)
    qc[..., 0], kc[..., 0] = 0x78, 0x68          # e4m3 256 and 64
    qc[..., 1:16], kc[..., 1:16] = 0x38, 0x38    # e4m3 1.0
    vc = np.full((1, 1, 1, 128), 0x38, np.uint8)
    one = torch.ones(1, device=dev)
    t = lambda a: torch.from_numpy(a).to(dev)
    out = run_fp8(t(qc), t(kc), t(vc), one, one, one, False, 1.0)[0]
    lse0 = float(out.lse[0, 0, 0])
    note(f"fp8 accumulation pin: lse0={lse0} (exact 16399, grouped model 16392)")
    assert abs(lse0 - 16392.0) < 0.5
    assert np.all(out.o == 1.0)


# Products of one run of 8 channels next to a 2^14 product (256 * 64 at the run's first
# channel, unit descales, scale 1, N = 1 so that the LSE is the score): each smaller
# product is truncated toward zero to a multiple of 2 = 2^(8 + 6 - 13).  (channel values of
# Q and K for channels 1..7; the score the hardware gives)
ROUNDING_CASES = {
    "ones": ((1.0, 1.0), 16384.0),             # 1 -> 0
    "minus_ones": ((1.0, -1.0), 16384.0),      # -1 -> 0 (toward zero, not down)
    "threes": ((1.5, 2.0), 16384.0 + 7 * 2),   # 3 -> 2
    "minus_threes": ((-1.5, 2.0), 16384.0 - 7 * 2),
    "twos": ((1.0, 2.0), 16384.0 + 7 * 2),     # multiples of 2 are kept
    "fours": ((2.0, 2.0), 16384.0 + 7 * 4),
    "minus_halves": ((-0.5, 1.0), 16384.0),
}
_E4M3 = {0.5: 0x30, 1.0: 0x38, 1.5: 0x3C, 2.0: 0x40}
# 240 * 120 = 28800 = 3.52 * 2^13: the window is set by the exponent sum 7 + 6 = 13 of
# the factors, not by the product's own exponent 14, so the 1.5 products keep 1.


def test_fp8_matrix_accumulation_rounding():
    """The rounding of the grouped FP8 accumulation, through the C ABI: toward zero (a
    -1 next to the 2^14 product is dropped, not rounded down to -2) to a multiple of
    2^(E - 13), E the run's largest exponent sum of the factors (3 becomes 2 next to
    256 * 64; 1.5 becomes 1 next to 240 * 120, whose exponent sum is 13).  The oracle
    tests model the FP8 accumulation this way."""
    names = sorted(ROUNDING_CASES) + ["exponent_sum"]
    B = len(names)
    qc = np.zeros((B, 1, 1, 128), np.uint8)
    kc = np.zeros((B, 1, 1, 128), np.uint8)
    code = lambda x: _E4M3[abs(x)] | (0x80 if x < 0 else 0)
    for b, n in enumerate(names):
        if n == "exponent_sum":
            qc[b, 0, 0, 0], kc[b, 0, 0, 0] = 0x77, 0x6F          # 240 * 120
            qc[b, 0, 0, 1:8], kc[b, 0, 0, 1:8] = code(1.5), code(1.0)
            continue
        (a, c), _ = ROUNDING_CASES[n]
        qc[b, 0, 0, 0], kc[b, 0, 0, 0] = 0x78, 0x68
        qc[b, 0, 0, 1:8], kc[b, 0, 0, 1:8] = code(a), code(c)
    vc = np.full((B, 1, 1, 128), 0x38, np.uint8)
    one = torch.ones(1, device=DEV)
    t = lambda a: torch.from_numpy(a).to(DEV)
    out = run_fp8(t(qc), t(kc), t(vc), one, one, one, False, 1.0)[0]
    for b, n in enumerate(names):
        want = 28800.0 + 7 * 1.0 if n == "exponent_sum" else ROUNDING_CASES[n][1]
        got = float(out.lse[b, 0, 0])
        note(f"  {n}: {got} (model {want})")
        assert abs(got - want) < 0.5, n


# ---- FP8 with a power-of-two softmax constant ------------------------------------------
# When scale * log2(e) * dq * dk is (within 4 ulps) a power of two, the FP8 kernel with
# the LSE applies it through the Q operand's matrix-instruction scale and starts the
# first k-step from minus the running max, so the scores leave the matrix instruction as
# exponent arguments.  quantize_e4m3_q_pow2 picks such a Q descale (at or above
# absmax/448, by less than 2x).

def _pow2_fp8_inputs(x, w):
    """K and V quantised as usual, Q by quantize_e4m3_q_pow2 against K's descales, all on
    the GPU and each asserted bit-identical to the oracle; returns device (codes,
    descale) pairs and the oracle's decoded float64 tensors."""
    host_c, host_d = {}, {}
    for n in "kv":
        host_c[n], host_d[n] = oracle.quantize_e4m3(x[n], w.fp8_per_head)
    host_c["q"], host_d["q"] = oracle.quantize_e4m3_q_pow2(x["q"], w.fp8_per_head, host_d["k"],
                                                           w.softmax_scale)
    dev = {}
    for n in "kv":
        dev[n] = gpu_quantize(x[n], w.fp8_per_head)
    qx = torch.from_numpy(x["q"]).to("cuda:0")
    qc = torch.empty(x["q"].shape, device="cuda:0", dtype=torch.uint8)
    qd = torch.empty((w.Hq if w.fp8_per_head else 1,), device="cuda:0", dtype=torch.float32)
    ba.quantize_e4m3_q_pow2(qx, qc, qd, dev["k"][1], w.softmax_scale, w.fp8_per_head)
    torch.cuda.synchronize()
    dev["q"] = (qc, qd)
    for n in "qkv":
        assert np.array_equal(dev[n][0].cpu().numpy(), host_c[n]), n
        assert np.array_equal(dev[n][1].cpu().numpy().view(np.uint32), host_d[n].view(np.uint32)), n
    bc = (lambda d: d[None, None, :, None].astype(np.float64)) if w.fp8_per_head else \
        (lambda d: float(d[0]))
    host = [oracle.e4m3_decode(host_c[n]) * bc(host_d[n]) for n in "qkv"]
    return [dev[n] for n in "qkv"], host


@pytest.mark.parametrize("case", _xfail_outliers(list(SMALL), lambda c: SMALL[c].recipe))
def test_fp8_pow2_softmax_constant(case):
    w = SMALL[case]
    note(f"case fp8 pow2 {case}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} d={w.d_qk}/{w.d_v}")
    x = workloads.generate(w)
    dev, (q, k, v) = _pow2_fp8_inputs(x, w)
    (qc, qd), (kc, kd), (vc, vd) = dev
    out = run_fp8(qc, kc, vc, qd, kd, vd, w.fp8_per_head, w.softmax_scale, repeats=2)[0]
    ro, rl = oracle.causal_attention(q, k, v, w.softmax_scale)
    check(f"{case}/pow2", "fp8", out.o, ro, out.lse, rl, fp8_path="exact",
          ref_abs_o=abs_v(oracle.causal_attention, q, k, v, w.softmax_scale))


@pytest.mark.parametrize("name", _xfail_outliers(FULL, lambda n: W[n].recipe))
def test_fp8_pow2_full_size_sampled_rows(name):
    w = W[name]
    note(f"case fp8 pow2 full {name}: N={w.N} Hq={w.Hq} Hkv={w.Hkv} d={w.d_qk}/{w.d_v}")
    x = workloads.generate(w)
    rows = _sample_rows(w)
    dev, (q, k, v) = _pow2_fp8_inputs(x, w)
    (qc, qd), (kc, kd), (vc, vd) = dev
    out = run_fp8(qc, kc, vc, qd, kd, vd, w.fp8_per_head, w.softmax_scale)[0]
    ro, rl = oracle.causal_attention_rows(q, k, v, w.softmax_scale, rows)
    bb, hh, ii = (np.array([r[j] for r in rows]) for j in range(3))
    go, gl = out.o[bb, ii, hh], out.lse[bb, hh, ii]
    assert np.all(np.isfinite(out.o)) and np.all(np.isfinite(out.lse))
    check(f"{name}/pow2/rows", "fp8", go, ro, gl, rl, fp8_path="exact",
          ref_abs_o=abs_v(oracle.causal_attention_rows, q, k, v, w.softmax_scale, rows),
          row_heads=[(b, h) for b, h, _ in rows])
