"""Seeded random sweep of the attention entry points against the fp64 oracle, through
the C ABI: shapes (B, Nq, Nk, q_offset, GQA ratio, head dims), scales (per tensor or per
head), softmax scale and input magnitudes are drawn from a fixed seed, so each case is
reproducible by its id.  Every case runs one kernel variant and compares every output
element with oracle.offset_attention on the same bf16 bytes or e4m3 codes, with the
same gates as the fixed-shape tests (gpu_harness.check): BF16, FP8 with the exact LSE
(absmax or power-of-two Q scale), FP8 without the LSE (Lean P), the rounded-sum LSE,
and the exact-channel path after the joint Q/K quantiser.

Inputs: Q and K i.i.d. normal times a per-channel log-normal spread (sigma 0.3) and a
global magnitude in [0.25, 4] (BF16) or [0.5, 2] (FP8), in the exact-channel cases with
four outlier channels per head twenty times larger (the Mistral-shaped recipe); V
i.i.d. N(0, 1).  The plain
FP8 kernel is not run on outlier channels (its LSE misses the gate there; see the
strict xfails of test_gpu_parity.py).
"""
import numpy as np
import pytest
import torch

import bf16_causal_prefill_amd as ba
import oracle
from gpu_harness import (DEV, ROUNDED_LSE_BOUND, abs_v, bf16_bytes, check, gpu_quantize, note,
                         to_dev_u16_as_bf16)

pytestmark = pytest.mark.gpu

VARIANTS = ["bf16", "fp8_lse", "fp8_lse_pow2", "fp8_lean", "fp8_rounded", "fp8_exact_channels",
            "fp8_exact_channels_nolse"]
N_PER_VARIANT = 8


def _case(variant: str, i: int) -> dict:
    """The i-th random case of a variant (seeded by both)."""
    rng = np.random.default_rng(1000 * VARIANTS.index(variant) + i)
    mla = variant in ("bf16", "fp8_lse", "fp8_lean") and rng.random() < 0.3
    dqk = 192 if mla else 128
    hkv = int(rng.choice([1, 2, 4]))
    g = 1 if mla else int(rng.choice([1, 2, 4]))
    nk = int(rng.integers(1, 700))
    kind = rng.random()
    if kind < 0.4:                        # square causal
        nq, off = nk, 0
    elif kind < 0.8:                      # a chunk of the last queries
        nq = int(rng.integers(1, nk + 1))
        off = nk - nq
    else:                                 # anything, including more queries than keys
        nq = int(rng.integers(1, 700))
        off = int(rng.integers(0, nk + 50))
    # FP8: logits of standard deviation up to about 6; beyond that the softmax follows
    # one score, whose FP8 accumulation error (grouped truncation, about 2e-3 of the
    # product magnitudes) then reaches the LSE undiluted
    smax, mmax = (2.0, 4.0) if variant == "bf16" else (1.5, 2.0)
    return dict(B=int(rng.integers(1, 3)), Nq=nq, Nk=nk, off=off, Hq=hkv * g, Hkv=hkv, dqk=dqk,
                dv=128, per_head=bool(rng.random() < 0.6),
                scale=float(rng.uniform(0.5, smax) / np.sqrt(dqk)),
                mag=float(np.exp(rng.uniform(np.log(1.0 / mmax), np.log(mmax)))),
                outliers=variant.startswith("fp8_exact"), seed=int(rng.integers(1 << 30)))


def _inputs(c: dict):
    rng = np.random.default_rng(c["seed"])

    def qk(n, H, d):
        spread = np.exp(rng.normal(0.0, 0.3, (H, d))).astype(np.float32)
        if c["outliers"]:
            for h in range(H):
                spread[h, rng.choice(d, 4, replace=False)] *= 20.0
        x = rng.standard_normal((c["B"], n, H, d), dtype=np.float32)
        return (x * spread[None, None] * np.float32(c["mag"])).astype(np.float32)
    # Q's and K's outlier channels are drawn independently; the joint quantiser finds
    # them from the absmax either way.  V stays N(0, 1), the scale the BF16 max-abs
    # gate of 2e-2 is stated for (bf16 rounding of an output of magnitude 8 is 2^-5).
    q, k = qk(c["Nq"], c["Hq"], c["dqk"]), qk(c["Nk"], c["Hkv"], c["dqk"])
    return q, k, rng.standard_normal((c["B"], c["Nk"], c["Hkv"], c["dv"]), dtype=np.float32)


def _out(c, want_lse=True):
    o = torch.full((c["B"], c["Nq"], c["Hq"], c["dv"]), float("nan"), device=DEV,
                   dtype=torch.bfloat16)
    lse = (torch.full((c["B"], c["Hq"], c["Nq"]), float("nan"), device=DEV, dtype=torch.float32)
           if want_lse else None)
    return o, lse


def _host(o, lse):
    torch.cuda.synchronize()
    return (o.float().cpu().numpy().astype(np.float64),
            None if lse is None else lse.cpu().numpy().astype(np.float64))


def _bc(ds, per_head):
    return ds[None, None, :, None].astype(np.float64) if per_head else float(ds[0])


def _quantised(x, per_head):
    cd, dd = gpu_quantize(x, per_head)
    ch, dh = oracle.quantize_e4m3(x, per_head)
    assert np.array_equal(cd.cpu().numpy(), ch)
    assert np.array_equal(dd.cpu().numpy().view(np.uint32), dh.view(np.uint32))
    return (cd, dd), oracle.e4m3_decode(ch) * _bc(dh, per_head), dh


CASES = [(v, i) for v in VARIANTS for i in range(N_PER_VARIANT)]


@pytest.mark.parametrize("variant,i", CASES, ids=[f"{v}-{i}" for v, i in CASES])
def test_random_case(variant, i):
    c = _case(variant, i)
    note(f"random {variant}-{i}: " + " ".join(f"{k}={v}" for k, v in c.items()))
    q, k, v = _inputs(c)
    off, s, ph = c["off"], c["scale"], c["per_head"]
    if variant == "bf16":
        qu, ku, vu = (bf16_bytes(a) for a in (q, k, v))
        o, lse = _out(c)
        ba.attn_fwd_causal_offset_bf16(*(to_dev_u16_as_bf16(a) for a in (qu, ku, vu)), o, lse,
                                       q_offset=off, softmax_scale=s)
        go, gl = _host(o, lse)
        ro, rl = oracle.offset_attention(*(oracle.bf16_decode(a) for a in (qu, ku, vu)), s, off)
        check(f"random-{variant}-{i}", "bf16", go, ro, gl, rl)
        return

    if variant.startswith("fp8_exact"):
        T = ba.OUTLIER_CHANNELS
        want_lse = variant == "fp8_exact_channels"
        # the joint quantiser takes one N: both sides quantise Q and K zero-padded to the
        # longer of the two (zeros leave every absmax unchanged), then keep the real rows
        n, B = max(c["Nq"], c["Nk"]), c["B"]
        pad = lambda a: np.concatenate(
            [a, np.zeros((B, n - a.shape[1]) + a.shape[2:], np.float32)], axis=1)
        qp, kp = pad(q), pad(k)
        qc_h, kc_h, qx_h, kx_h, qd_h, kd_h, perm_h = oracle.quantize_e4m3_qk_outliers(qp, kp, ph)
        qo = torch.empty(qp.shape, device=DEV, dtype=torch.uint8)
        ko = torch.empty(kp.shape, device=DEV, dtype=torch.uint8)
        qx = torch.empty((B, n, c["Hq"], T), device=DEV, dtype=torch.bfloat16)
        kx = torch.empty((B, n, c["Hkv"], T), device=DEV, dtype=torch.bfloat16)
        qd = torch.empty((c["Hq"] if ph else 1,), device=DEV, dtype=torch.float32)
        kd = torch.empty((c["Hkv"] if ph else 1,), device=DEV, dtype=torch.float32)
        perm = torch.empty((c["Hkv"], c["dqk"]), device=DEV, dtype=torch.uint8)
        ba.quantize_e4m3_qk_outliers(torch.from_numpy(qp).to(DEV), torch.from_numpy(kp).to(DEV),
                                     qo, ko, qx, kx, qd, kd, perm, ph)
        torch.cuda.synchronize()
        assert np.array_equal(qo.cpu().numpy(), qc_h) and np.array_equal(ko.cpu().numpy(), kc_h)
        assert np.array_equal(perm.cpu().numpy(), perm_h.astype(np.uint8))
        Nq, Nk = c["Nq"], c["Nk"]
        qo, qx = qo[:, :Nq].contiguous(), qx[:, :Nq].contiguous()
        ko, kx = ko[:, :Nk].contiguous(), kx[:, :Nk].contiguous()
        qc_h, qx_h = qc_h[:, :Nq], qx_h[:, :Nq]
        kc_h, kx_h = kc_h[:, :Nk], kx_h[:, :Nk]
        (vc, vd), vdec, _ = _quantised(v, ph)
        o, lse = _out(c, want_lse)
        ba.attn_fwd_causal_offset_fp8_outliers(qo, ko, vc, qx, kx, qd, kd, vd, o, lse,
                                               q_offset=off, softmax_scale=s,
                                               descale_per_head=int(ph))
        go, gl = _host(o, lse)
        qdec = oracle.decode_qk_outliers(qc_h, qx_h, qd_h, ph)
        kdec = oracle.decode_qk_outliers(kc_h, kx_h, kd_h, ph)
        ro, rl = oracle.offset_attention(qdec, kdec, vdec, s, off)
        check(f"random-{variant}-{i}", "fp8", go, ro, gl, rl if want_lse else None,
              fp8_path="exact" if want_lse else "lean",
              ref_abs_o=abs_v(oracle.offset_attention, qdec, kdec, vdec, s, off))
        return

    (kc, kd), kdec, kd_h = _quantised(k, ph)
    (vc, vd), vdec, _ = _quantised(v, ph)
    if variant == "fp8_lse_pow2":
        ch, dh = oracle.quantize_e4m3_q_pow2(q, ph, kd_h, s)
        qc = torch.empty(q.shape, device=DEV, dtype=torch.uint8)
        qd = torch.empty((c["Hq"] if ph else 1,), device=DEV, dtype=torch.float32)
        ba.quantize_e4m3_q_pow2(torch.from_numpy(q).to(DEV), qc, qd, kd, s, ph)
        torch.cuda.synchronize()
        assert np.array_equal(qc.cpu().numpy(), ch)
        assert np.array_equal(qd.cpu().numpy().view(np.uint32), dh.view(np.uint32))
        qdec = oracle.e4m3_decode(ch) * _bc(dh, ph)
    else:
        (qc, qd), qdec, _ = _quantised(q, ph)
    ro, rl = oracle.offset_attention(qdec, kdec, vdec, s, off)
    ra = abs_v(oracle.offset_attention, qdec, kdec, vdec, s, off)
    args = (qc, kc, vc, qd, kd, vd)
    if variant == "fp8_rounded":
        o, lse = _out(c)
        ba.attn_fwd_causal_offset_fp8_rounded_lse(*args, o, lse, q_offset=off, softmax_scale=s,
                                                  descale_per_head=int(ph))
        go, gl = _host(o, lse)
        check(f"random-{variant}-{i}", "fp8", go, ro, fp8_path="lean", ref_abs_o=ra)
        err = float(np.max(np.abs(gl - rl)))
        note(f"  rounded-sum LSE max |error| {err:.4f} (bound {ROUNDED_LSE_BOUND:.4f})")
        assert np.all(np.isfinite(gl)) and err <= ROUNDED_LSE_BOUND
        return
    want_lse = variant != "fp8_lean"
    o, lse = _out(c, want_lse)
    ba.attn_fwd_causal_offset_fp8(*args, o, lse, q_offset=off, softmax_scale=s,
                                  descale_per_head=int(ph))
    go, gl = _host(o, lse)
    check(f"random-{variant}-{i}", "fp8", go, ro, gl, rl if want_lse else None,
          fp8_path="exact" if want_lse else "lean", ref_abs_o=ra)
