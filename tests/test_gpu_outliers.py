"""GPU tests of the outlier-channel path: quantize_e4m3_qk_outliers (bit-exact against
the oracle's quantize_e4m3_qk_outliers: codes, descales, permutation) and the FP8
attention that multiplies the last 32 channels of every Q and K row exactly
(attn_fwd_causal_fp8_outliers / attn_fwd_causal_offset_fp8_outliers), against the
fp64 oracle on the decoded inputs, with the plain spec gates: FP8 relative
Frobenius <= 6e-2 (also per head, per row and per element) and LSE max-abs <= 1e-2,
including the outlier-channel recipe where the plain FP8 path misses the LSE gate.
"""
import numpy as np
import pytest
import torch

import bf16_causal_prefill_amd as ba
import oracle
import workloads
from gpu_harness import DEV, _repeat, abs_v, check, gpu_quantize, note

pytestmark = pytest.mark.gpu

W = workloads.CONFIGS


def _bc(ds, per_head):
    return ds[None, None, :, None].astype(np.float64) if per_head else float(ds[0])


T = ba.OUTLIER_CHANNELS


def _u16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def outlier_inputs(x, per_head, pow2_scale=None):
    """Q and K through the library's quantize_e4m3_qk_outliers, V through quantize_e4m3,
    each asserted bit-identical to the oracle (codes, bf16 side arrays, descales,
    permutation); returns device (codes, descale) for q, k, v, the device side arrays
    (q_exact, k_exact), the device permutation and the oracle's decoded float64 q, k, v
    (side values for the last 32 channels)."""
    q, k = x["q"], x["k"]
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    qc_h, kc_h, qx_h, kx_h, qd_h, kd_h, perm_h = oracle.quantize_e4m3_qk_outliers(
        q, k, per_head, q_pow2_scale=pow2_scale)
    qo = torch.empty(q.shape, device=DEV, dtype=torch.uint8)
    ko = torch.empty(k.shape, device=DEV, dtype=torch.uint8)
    qx = torch.empty((B, N, Hq, T), device=DEV, dtype=torch.bfloat16)
    kx = torch.empty((B, N, Hkv, T), device=DEV, dtype=torch.bfloat16)
    qd = torch.empty((Hq if per_head else 1,), device=DEV, dtype=torch.float32)
    kd = torch.empty((Hkv if per_head else 1,), device=DEV, dtype=torch.float32)
    perm = torch.empty((Hkv, d), device=DEV, dtype=torch.uint8)
    ba.quantize_e4m3_qk_outliers(torch.from_numpy(q).to(DEV), torch.from_numpy(k).to(DEV), qo, ko,
                                 qx, kx, qd, kd, perm, per_head, q_pow2=pow2_scale is not None,
                                 softmax_scale=pow2_scale)
    torch.cuda.synchronize()
    assert np.array_equal(perm.cpu().numpy(), perm_h.astype(np.uint8)), "permutation differs"
    assert np.array_equal(qd.cpu().numpy().view(np.uint32), qd_h.view(np.uint32)), "q descale"
    assert np.array_equal(kd.cpu().numpy().view(np.uint32), kd_h.view(np.uint32)), "k descale"
    assert np.array_equal(qo.cpu().numpy(), qc_h), "q codes differ from the oracle"
    assert np.array_equal(ko.cpu().numpy(), kc_h), "k codes differ from the oracle"
    assert np.array_equal(_u16(qx), qx_h), "q side array differs from the oracle"
    assert np.array_equal(_u16(kx), kx_h), "k side array differs from the oracle"
    vc, vd = gpu_quantize(x["v"], per_head)
    vc_h, vd_h = oracle.quantize_e4m3(x["v"], per_head)
    assert np.array_equal(vc.cpu().numpy(), vc_h)
    dec = [oracle.decode_qk_outliers(qc_h, qx_h, qd_h, per_head),
           oracle.decode_qk_outliers(kc_h, kx_h, kd_h, per_head),
           oracle.e4m3_decode(vc_h) * _bc(vd_h, per_head)]
    return [(qo, qd), (ko, kd), (vc, vd)], (qx, kx), perm, dec


def run_outliers(dev, exact, per_head, scale, want_lse=True, repeats=1):
    (qc, qd), (kc, kd), (vc, vd) = dev
    qx, kx = exact
    B, N, Hq, _ = qc.shape
    return _repeat(lambda o, lse: ba.attn_fwd_causal_fp8_outliers(
        qc, kc, vc, qx, kx, qd, kd, vd, o, lse, softmax_scale=scale,
        descale_per_head=int(per_head)),
        B, N, Hq, vc.shape[3], want_lse, repeats,
        "fp8 outliers" + ("" if want_lse else "/no-lse"))[0]


# ---- the quantiser -----------------------------------------------------------------------

QUANT_CASES = {
    "mistral_n300_per_head": (W["mistral16k"].with_(N=300, seed=71), True, False),
    "mistral_n300_per_tensor": (W["mistral16k"].with_(N=300, seed=72), False, False),
    "mistral_n300_pow2": (W["mistral16k"].with_(N=300, seed=73), True, True),
    "mistral_b2_n65_gqa2": (W["mistral16k"].with_(B=2, N=65, Hq=4, Hkv=2, seed=74), True, False),
    "mla_d192": (W["mla16k"].with_(N=200, Hq=4, Hkv=4, seed=75), True, False),
    "gauss_tiny": (W["tiny"], False, True),
}


@pytest.mark.parametrize("case", sorted(QUANT_CASES))
def test_outlier_quantiser_bit_exact(case):
    w, per_head, pow2 = QUANT_CASES[case]
    note(f"outlier quantiser {case}: B={w.B} N={w.N} Hq={w.Hq} Hkv={w.Hkv} d={w.d_qk}")
    x = workloads.generate(w)
    outlier_inputs(x, per_head, w.softmax_scale if pow2 else None)


def test_outlier_quantiser_zero_and_tied_channels():
    """All-zero Q: every importance is 0, ties go to the lower channel, so channels
    0..31 are stored last; the descale of an all-zero tensor is 1."""
    rng = np.random.default_rng(77)
    x = {"q": np.zeros((1, 40, 4, 128), np.float32),
         "k": rng.standard_normal((1, 40, 2, 128)).astype(np.float32),
         "v": rng.standard_normal((1, 40, 2, 128)).astype(np.float32)}
    dev, _, perm, _ = outlier_inputs(x, True)
    p = perm.cpu().numpy()
    assert np.array_equal(p[0], np.r_[np.arange(32, 128), np.arange(32)])
    assert np.all(dev[0][1].cpu().numpy() == 1.0)


# ---- the attention with exact channels ---------------------------------------------------

def test_exact_channels_accumulate_exactly():
    """N = 1 (LSE = the score), scale 1, unit descales.  A 2^14 product with seven 1.0
    products in its run of 8 channels: in the FP8 channels (codes) the ones fall below
    the run's 13-bit window and are dropped (16384); in the last 32 channels, taken from
    the bf16 side arrays and multiplied on the BF16 pipe, they are kept (16391).  The
    codes of the last 32 channels are not read: they hold 448s here."""
    q = np.zeros((2, 1, 1, 128), np.uint8)
    k = np.zeros((2, 1, 1, 128), np.uint8)
    q[..., 96:] = k[..., 96:] = 0x7E                      # ignored codes (448)
    qx = np.zeros((2, 1, 1, 32), np.uint16)
    kx = np.zeros((2, 1, 1, 32), np.uint16)
    q[0, 0, 0, 0], k[0, 0, 0, 0] = 0x78, 0x68              # FP8 run: 256 * 64
    q[0, 0, 0, 1:8], k[0, 0, 0, 1:8] = 0x38, 0x38          # 1.0 * 1.0
    qx[1, 0, 0, 0], kx[1, 0, 0, 0] = 0x4380, 0x4280        # exact run: bf16 256 * 64
    qx[1, 0, 0, 1:8], kx[1, 0, 0, 1:8] = 0x3F80, 0x3F80    # bf16 1.0 * 1.0
    v = np.full((2, 1, 1, 128), 0x38, np.uint8)
    one = torch.ones(1, device=DEV)
    t = lambda a: torch.from_numpy(a).to(DEV)
    tb = lambda a: torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    dev = [(t(q), one), (t(k), one), (t(v), one)]
    out = run_outliers(dev, (tb(qx), tb(kx)), False, 1.0)
    got = out.lse[:, 0, 0]
    note(f"exact channels: FP8 run {got[0]}, exact run {got[1]} (16384, 16391)")
    assert abs(got[0] - 16384.0) < 0.5 and abs(got[1] - 16391.0) < 0.5
    assert np.all(out.o == 1.0)


SMALL = {
    "mistral_n1024": W["mistral16k"].with_(N=1024, seed=25),
    "mistral_n2048_s5": W["mistral16k"].with_(N=2048, seed=5),
    "mistral_ragged_n300_b2": W["mistral16k"].with_(B=2, N=300, Hq=8, Hkv=2, seed=78),
    "mistral_n33": W["mistral16k"].with_(N=33, Hq=4, Hkv=1, seed=79),
    "mistral_n1": W["mistral16k"].with_(N=1, Hq=4, Hkv=2, seed=80),
    "gauss_tiny": W["tiny"],
    "gauss_mid_gqa": W["mid_gqa"],
}


@pytest.mark.parametrize("want_lse,pow2", [(True, False), (True, True), (False, False)],
                         ids=["lse-absmax_q", "lse-pow2_q", "nolse"])
@pytest.mark.parametrize("case", sorted(SMALL))
def test_outlier_attention_parity(case, want_lse, pow2):
    """Every output element against the oracle, plain gates (LSE max-abs 1e-2).  The
    power-of-two Q descale only changes the LSE path, so it runs with the LSE."""
    w = SMALL[case]
    note(f"outliers {case} lse={want_lse} pow2={pow2}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N}")
    x = workloads.generate(w)
    dev, ex, _, (q, k, v) = outlier_inputs(x, w.fp8_per_head, w.softmax_scale if pow2 else None)
    out = run_outliers(dev, ex, w.fp8_per_head, w.softmax_scale, want_lse=want_lse)
    ro, rl = oracle.causal_attention(q, k, v, w.softmax_scale)
    check(f"{case}/outliers", "fp8", out.o, ro, out.lse, rl if want_lse else None,
          fp8_path="exact" if want_lse else "lean",
          ref_abs_o=abs_v(oracle.causal_attention, q, k, v, w.softmax_scale))


def test_outlier_attention_on_plain_codes():
    """The exact-channel kernel on plain quantize_e4m3 codes with side arrays holding the
    e4m3 values of their last 32 channels (exact in bf16): the same attention as the
    plain kernel computes, within the FP8 checks (Gaussian inputs)."""
    w = W["mid_gqa"].with_(N=700, seed=81)
    x = workloads.generate(w)
    dev, host, side = [], [], []
    for n in "qkv":
        c, d = gpu_quantize(x[n], True)
        ch, dh = oracle.quantize_e4m3(x[n], True)
        assert np.array_equal(c.cpu().numpy(), ch)
        dev.append((c, d))
        host.append(oracle.e4m3_decode(ch) * _bc(dh, True))
        if n != "v":
            vals = oracle.e4m3_decode(np.ascontiguousarray(ch[..., -T:])).astype(np.float32)
            side.append(torch.from_numpy(oracle.bf16_encode(vals).view(np.int16)).to(DEV)
                        .view(torch.bfloat16))
    out = run_outliers(dev, tuple(side), True, w.softmax_scale)
    ro, rl = oracle.causal_attention(*host, w.softmax_scale)
    check("plain codes/outliers", "fp8", out.o, ro, out.lse, rl, fp8_path="exact",
          ref_abs_o=abs_v(oracle.causal_attention, *host, w.softmax_scale))


@pytest.mark.parametrize("mode", ["absmax_q", "pow2_q", "nolse"])
def test_outlier_attention_full_size_mistral16k(mode):
    """The Mistral-shaped 16K workload in full: 10 byte-identical runs, sampled rows
    against the oracle with the plain gates."""
    w = W["mistral16k"]
    note(f"outliers full mistral16k {mode}")
    x = workloads.generate(w)
    dev, ex, _, (q, k, v) = outlier_inputs(x, True, w.softmax_scale if mode == "pow2_q" else None)
    out = run_outliers(dev, ex, True, w.softmax_scale, want_lse=mode != "nolse", repeats=10)
    rng = np.random.default_rng(7)
    N = w.N
    rows = [(0, h, i) for h in (0, 13, 31) for i in (0, 1, 63, 64, 255, 256, N // 2, N - 1)]
    rows += [(0, int(rng.integers(w.Hq)), int(rng.integers(N))) for _ in range(64)]
    ro, rl = oracle.causal_attention_rows(q, k, v, w.softmax_scale, rows)
    bb, hh, ii = (np.array([r[j] for r in rows]) for j in range(3))
    assert np.all(np.isfinite(out.o))
    gl = None
    if out.lse is not None:
        assert np.all(np.isfinite(out.lse))
        gl = out.lse[bb, hh, ii]
    check(f"mistral16k/rows/outliers/{mode}", "fp8", out.o[bb, ii, hh], ro, gl,
          rl if gl is not None else None, fp8_path="lean" if mode == "nolse" else "exact",
          ref_abs_o=abs_v(oracle.causal_attention_rows, q, k, v, w.softmax_scale, rows),
          row_heads=[(b, h) for b, h, _ in rows])


OFFSET = {   # name: (B, Nq, Nk, q_offset, Hq, Hkv)
    "chunk_tail": (1, 64, 600, 536, 4, 2),
    "all_visible": (2, 100, 77, 77, 4, 4),
    "q_longer": (1, 257, 129, 5, 2, 1),
}


@pytest.mark.parametrize("case", sorted(OFFSET))
def test_outlier_offset_attention(case):
    B, Nq, Nk, off, Hq, Hkv = OFFSET[case]
    note(f"outliers offset {case}: B={B} Nq={Nq} Nk={Nk} q_offset={off}")
    w = W["mistral16k"].with_(B=B, N=max(Nq, Nk), Hq=Hq, Hkv=Hkv, seed=82)
    x = workloads.generate(w)
    # the queries are the last Nq positions' rows, the keys the first Nk
    x = {"q": np.ascontiguousarray(x["q"][:, -Nq:]), "k": np.ascontiguousarray(x["k"][:, :Nk]),
         "v": np.ascontiguousarray(x["v"][:, :Nk])}
    if Nq != Nk:
        # the joint quantiser wants one N: quantise the padded pair, then slice
        n = max(Nq, Nk)
        pad = lambda a: np.concatenate([a, np.zeros((B, n - a.shape[1]) + a.shape[2:], np.float32)], 1)
        dev, ex, _, dec = outlier_inputs({"q": pad(x["q"]), "k": pad(x["k"]), "v": pad(x["v"])},
                                         True)
        dev = [(dev[0][0][:, :Nq].contiguous(), dev[0][1]), (dev[1][0][:, :Nk].contiguous(), dev[1][1]),
               (dev[2][0][:, :Nk].contiguous(), dev[2][1])]
        ex = (ex[0][:, :Nq].contiguous(), ex[1][:, :Nk].contiguous())
        dec = [dec[0][:, :Nq], dec[1][:, :Nk], dec[2][:, :Nk]]
    else:
        dev, ex, _, dec = outlier_inputs(x, True)
    (qc, qd), (kc, kd), (vc, vd) = dev
    scale = w.softmax_scale
    o = torch.full((B, Nq, Hq, 128), float("nan"), device=DEV, dtype=torch.bfloat16)
    lse = torch.full((B, Hq, Nq), float("nan"), device=DEV, dtype=torch.float32)
    ba.attn_fwd_causal_offset_fp8_outliers(qc, kc, vc, ex[0], ex[1], qd, kd, vd, o, lse,
                                           q_offset=off, softmax_scale=scale, descale_per_head=1)
    torch.cuda.synchronize()
    ro, rl = oracle.offset_attention(*dec, scale, off)
    check(f"offset {case}/outliers", "fp8", o.float().cpu().numpy().astype(np.float64), ro,
          lse.cpu().numpy().astype(np.float64), rl, fp8_path="exact",
          ref_abs_o=abs_v(oracle.offset_attention, *dec, scale, off))


def test_outlier_attention_deterministic():
    w = W["mistral16k"].with_(N=4096, seed=83)
    x = workloads.generate(w)
    dev, ex, _, _ = outlier_inputs(x, True)
    run_outliers(dev, ex, True, w.softmax_scale, repeats=100)
    run_outliers(dev, ex, True, w.softmax_scale, want_lse=False, repeats=100)
