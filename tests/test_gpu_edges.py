"""GPU edge cases against the fp64 oracle, through the C ABI.

* quantize_e4m3 on degenerate tensors: all zeros (descale 1), one all-zero head in
  per-head mode, exact rounding ties between neighbouring e4m3 values, signed zeros
  and values below half the smallest subnormal, NaN elements (no part in the absmax,
  code 0x7F) and an infinity (infinite descale): bit-exact codes and descales.
* Extreme score patterns: scores that rise along the key axis by more than the lazy
  rescale threshold in every key tile (the running max moves on every tile), and
  scores that fall so steeply that most probabilities underflow (rows dominated by
  their first keys, block exponents at their cap, probabilities flushed to zero).
* The largest launch the entry points accept: B*N*Hq*d one batch short of 2^31
  elements (they reject 2^31 and above), inputs drawn on the device, outputs
  compared on sampled rows.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_harness import DEV, abs_v, bf16_bytes, check, gpu_quantize, note, run_bf16, run_fp8

import bf16_causal_prefill_amd as ba

pytestmark = pytest.mark.gpu


# ---- quantize_e4m3 on degenerate inputs ------------------------------------------------

def _e4m3_grid() -> np.ndarray:
    """Every finite non-negative e4m3 value, the midpoints between neighbours (exact
    in float32; round-to-nearest-even ties), values just off each midpoint, and values
    at and below half the smallest subnormal 2^-9."""
    vals = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8)).astype(np.float32)
    mids = ((vals[:-1].astype(np.float64) + vals[1:]) / 2).astype(np.float32)
    up = np.nextafter(mids, np.float32(np.inf))
    down = np.nextafter(mids, np.float32(0))
    tiny = np.array([2.0 ** -10, 2.0 ** -11, 1e-30, 1e-40, 0.0], np.float32)
    g = np.concatenate([vals, mids, up, down, tiny]).astype(np.float32)
    return np.concatenate([g, -g])


QZ_CASES = ["zeros_tensor", "zeros_one_head", "ties_tensor", "ties_head", "nan_tensor",
            "nan_head", "inf_tensor", "inf_head"]


@pytest.mark.parametrize("case", QZ_CASES)
def test_quantize_degenerate(case):
    note(f"case quantize {case}")
    rng = np.random.default_rng(41)
    if case == "zeros_tensor":
        x, per_head = np.zeros((2, 33, 3, 128), np.float32), False
    elif case == "zeros_one_head":
        x, per_head = rng.standard_normal((1, 70, 4, 128)).astype(np.float32), True
        x[:, :, 2, :] = 0.0
    elif case.startswith("ties"):
        g = _e4m3_grid()
        # 2 * 1024 grid slots; absmax is exactly 448 in every head, so the descale is
        # exactly 1 and the quotients are the grid values themselves
        n = 2 * 8 * 128
        x = np.resize(g, n).reshape(1, 2, 8, 128).astype(np.float32)
        x[0, 0, :, 0] = 448.0
        x = np.concatenate([x, x[:, :, ::-1, ::-1]], axis=1)   # (1, 4, 8, 128)
        per_head = case == "ties_head"
    elif case.startswith("nan"):
        # NaN elements leave the absmax as if absent and encode to 0x7F; in per-head
        # mode head 3 holds nothing but NaN (descale 1)
        x = rng.standard_normal((2, 40, 4, 128)).astype(np.float32)
        x[0, 5, 1, 7] = np.nan
        x[1, 39, 0, 127] = -np.nan
        x[:, :, 3, :] = np.nan
        per_head = case == "nan_head"
    elif case.startswith("inf"):
        # an infinity makes the descale infinite: finite elements encode to signed
        # zeros, the infinity itself (inf / inf) to 0x7F
        x = rng.standard_normal((1, 40, 4, 128)).astype(np.float32)
        x[0, 11, 2, 64] = -np.inf
        per_head = case == "inf_head"
    else:
        raise ValueError(case)
    codes_d, ds_d = gpu_quantize(x, per_head)
    codes_h, ds_h = oracle.quantize_e4m3(x, per_head)
    assert np.array_equal(ds_d.cpu().numpy().view(np.uint32), ds_h.view(np.uint32))
    assert np.array_equal(codes_d.cpu().numpy(), codes_h)
    if case.startswith("zeros"):
        zero_heads = [0, 1, 2] if case == "zeros_tensor" else [2]
        for h in zero_heads:
            assert np.all(codes_h[:, :, h, :] == 0)
        assert ds_h[zero_heads[-1] if per_head else 0] == 1.0
    elif case.startswith("ties"):
        assert np.all(ds_h == 1.0)
    elif case.startswith("nan"):
        assert np.all(codes_h[np.isnan(x)] == 0x7F)
        assert np.all(np.isfinite(ds_h)) and (not per_head or ds_h[3] == 1.0)
    else:
        assert np.isinf(ds_h[2 if per_head else 0])


@pytest.mark.parametrize("per_head", [False, True])
@pytest.mark.parametrize("shape", [(1, 300, 8, 128, 2), (2, 77, 4, 192, 4), (1, 16, 6, 8, 3)])
def test_quantize_q_pow2_bit_exact(shape, per_head):
    """quantize_e4m3_q_pow2 against the oracle's rule: descales bit-identical (also for
    an all-zero head), codes bit-identical; K's descales come from the oracle."""
    B, N, H, d, Hkv = shape
    note(f"case quantize_q_pow2 {shape} per_head={per_head}")
    rng = np.random.default_rng(sum(shape) + per_head)
    x = (rng.standard_normal((B, N, H, d)) * rng.uniform(1e-3, 40, H)[None, None, :, None]
         ).astype(np.float32)
    if per_head:
        x[:, :, 1, :] = 0.0
    k = rng.standard_normal((B, N, Hkv, d)).astype(np.float32) * np.float32(3.0)
    _, kd = oracle.quantize_e4m3(k, per_head)
    scale = 1.0 / np.sqrt(d)
    ch, dh = oracle.quantize_e4m3_q_pow2(x, per_head, kd, scale)
    xd = torch.from_numpy(x).to(DEV)
    codes = torch.empty(x.shape, device=DEV, dtype=torch.uint8)
    ds = torch.empty(H if per_head else 1, device=DEV, dtype=torch.float32)
    ba.quantize_e4m3_q_pow2(xd, codes, ds, torch.from_numpy(kd).to(DEV), scale, per_head)
    torch.cuda.synchronize()
    assert np.array_equal(ds.cpu().numpy().view(np.uint32), dh.view(np.uint32))
    assert np.array_equal(codes.cpu().numpy(), ch)


# (B, Nq, Nk, Hq, Hkv, d_qk, d_v): GQA, Nq != Nk, the MLA dims, a ragged row count,
# more heads than one quantiser workgroup's columns
QKV_SHAPES = {"gqa": (1, 300, 300, 8, 2, 128, 128), "chunk": (2, 77, 130, 4, 4, 128, 128),
              "mla": (1, 65, 65, 4, 4, 192, 128), "tiny": (1, 3, 5, 6, 3, 8, 4),
              "wide": (1, 40, 40, 64, 8, 128, 128)}


@pytest.mark.parametrize("q_pow2", [False, True], ids=["absmax_q", "pow2_q"])
@pytest.mark.parametrize("per_head", [False, True], ids=["per_tensor", "per_head"])
@pytest.mark.parametrize("shape", list(QKV_SHAPES))
def test_quantize_qkv_bit_exact(shape, per_head, q_pow2):
    """quantize_e4m3_qkv: codes and descales bit-identical to the three separate calls
    and to the oracle's quantisers (Q with the power-of-two rule against the oracle's K
    descales, or plain absmax), with an all-zero head and NaN elements in Q, an all-zero
    V head, and very different magnitudes per head."""
    B, Nq, Nk, Hq, Hkv, dqk, dv = QKV_SHAPES[shape]
    note(f"case quantize_qkv {shape} per_head={per_head} q_pow2={q_pow2}")
    rng = np.random.default_rng(Nq * 7 + Hq + per_head + 2 * q_pow2)
    mag = lambda H: rng.uniform(1e-3, 40, H)[None, None, :, None]
    q = (rng.standard_normal((B, Nq, Hq, dqk)) * mag(Hq)).astype(np.float32)
    k = (rng.standard_normal((B, Nk, Hkv, dqk)) * mag(Hkv)).astype(np.float32)
    v = (rng.standard_normal((B, Nk, Hkv, dv)) * mag(Hkv)).astype(np.float32)
    q[:, :, Hq - 1, :] = 0.0
    q[0, 0, 0, :3] = np.nan
    v[:, :, 0, :] = 0.0
    scale = 1.0 / np.sqrt(dqk)
    kc_h, kd_h = oracle.quantize_e4m3(k, per_head)
    vc_h, vd_h = oracle.quantize_e4m3(v, per_head)
    if q_pow2:
        qc_h, qd_h = oracle.quantize_e4m3_q_pow2(q, per_head, kd_h, scale)
    else:
        qc_h, qd_h = oracle.quantize_e4m3(q, per_head)
    dev = {n: torch.from_numpy(a).to(DEV) for n, a in (("q", q), ("k", k), ("v", v))}
    ns = {"q": Hq if per_head else 1, "k": Hkv if per_head else 1, "v": Hkv if per_head else 1}
    fused = {n: (torch.empty(dev[n].shape, device=DEV, dtype=torch.uint8),
                 torch.full((ns[n],), float("nan"), device=DEV)) for n in "qkv"}
    ba.quantize_e4m3_qkv(dev["q"], dev["k"], dev["v"], fused["q"][0], fused["k"][0],
                         fused["v"][0], fused["q"][1], fused["k"][1], fused["v"][1], per_head,
                         q_pow2=q_pow2, softmax_scale=scale)
    sep = {n: (torch.empty(dev[n].shape, device=DEV, dtype=torch.uint8),
               torch.empty((ns[n],), device=DEV)) for n in "qkv"}
    for n in "kv":
        ba.quantize_e4m3(dev[n], sep[n][0], sep[n][1], per_head)
    if q_pow2:
        ba.quantize_e4m3_q_pow2(dev["q"], sep["q"][0], sep["q"][1], sep["k"][1], scale, per_head)
    else:
        ba.quantize_e4m3(dev["q"], sep["q"][0], sep["q"][1], per_head)
    torch.cuda.synchronize()
    for n, (ch, dh) in (("q", (qc_h, qd_h)), ("k", (kc_h, kd_h)), ("v", (vc_h, vd_h))):
        fc, fd = (t.cpu().numpy() for t in fused[n])
        sc, sd = (t.cpu().numpy() for t in sep[n])
        assert np.array_equal(fd.view(np.uint32), sd.view(np.uint32)), n
        assert np.array_equal(fc, sc), n
        assert np.array_equal(fd.view(np.uint32), dh.view(np.uint32)), n
        assert np.array_equal(fc, ch), n


# ---- extreme score patterns ------------------------------------------------------------

def _slope_inputs(N: int, slope_log2: float, seed: int):
    """Q = a e_0 for every query, K_j = b_j e_0, V ~ N(0, 1): the score of key j is
    (linear in j) so that, in log2 units after the softmax scale, it changes by
    slope_log2 per key.  One nonzero channel keeps every score an exact product."""
    B, Hq, Hkv, d = 1, 4, 2, 128
    scale = 1.0 / np.sqrt(d)
    c = scale * np.log2(np.e)
    a = 16.0
    rng = np.random.default_rng(seed)
    q = np.zeros((B, N, Hq, d), np.float32)
    k = np.zeros((B, N, Hkv, d), np.float32)
    q[..., 0] = a
    k[..., 0] = (slope_log2 / (c * a) * np.arange(N, dtype=np.float64))[None, :, None]
    v = rng.standard_normal((B, N, Hkv, d)).astype(np.float32)
    return {"q": q, "k": k, "v": v}, scale


SLOPES = {"rising": 0.1, "falling": -0.75}


@pytest.mark.parametrize("pattern", list(SLOPES))
@pytest.mark.parametrize("prec", ["bf16", "fp8", "fp8_nolse"])
def test_extreme_score_slopes(pattern, prec):
    """rising: the row max grows by 12.8 (log2) per 128-key tile, above the rescale
    threshold of 8, so every tile rescales; falling: scores drop by 96 per tile, so
    from the second tile on every probability underflows.  fp8_nolse is the FP8 call
    without the LSE (the linear-code probabilities and their row sums)."""
    N = 1000
    x, scale = _slope_inputs(N, SLOPES[pattern], seed=43)
    note(f"case slope {pattern} {prec}: N={N}")
    if prec == "bf16":
        qu, ku, vu = (bf16_bytes(x[n]) for n in "qkv")
        q, k, v = (oracle.bf16_decode(a) for a in (qu, ku, vu))
        out = run_bf16(qu, ku, vu, scale)[0]
    else:
        dev, host = [], []
        for n in "qkv":
            cd, dd = gpu_quantize(x[n], False)
            ch, dh = oracle.quantize_e4m3(x[n], False)
            assert np.array_equal(cd.cpu().numpy(), ch)
            dev.append((cd, dd))
            host.append(oracle.e4m3_decode(ch) * float(dh[0]))
        q, k, v = host
        (qc, qd), (kc, kd), (vc, vd) = dev
        out = run_fp8(qc, kc, vc, qd, kd, vd, False, scale, want_lse=prec == "fp8")[0]
    ro, rl = oracle.causal_attention(q, k, v, scale)
    ra = abs_v(oracle.causal_attention, q, k, v, scale) if prec != "bf16" else None
    if prec == "fp8_nolse":
        check(f"slope_{pattern}", "fp8", out.o, ro, ref_abs_o=ra, fp8_path="lean")
    else:
        check(f"slope_{pattern}", prec, out.o, ro, out.lse, rl, ref_abs_o=ra, fp8_path="exact")


# ---- the largest accepted launch ---------------------------------------------------------

# B*N*Hq*d = 1023 * 512 * 32 * 128 = 2^31 - 2^21 elements per Q / O tensor (the entry
# points reject 2^31 and above); 65472 workgroups.
MAX_SHAPE = dict(B=1023, N=512, Hq=32, Hkv=8, d=128)


def _max_rows(rng):
    B, N, Hq = MAX_SHAPE["B"], MAX_SHAPE["N"], MAX_SHAPE["Hq"]
    rows = [(b, h, i) for b in (0, B // 2, B - 1) for h in (0, Hq - 1) for i in (0, 255, 256, N - 1)]
    rows += [(int(rng.integers(B)), int(rng.integers(Hq)), int(rng.integers(N))) for _ in range(24)]
    return rows


def _oracle_rows_from_device(tensors, decoders, scale, rows):
    """Oracle rows from per-batch slices copied off the device (the oracle never sees
    the whole multi-GiB tensors); decoders map a device slice to float64 values."""
    q, k, v = tensors
    ro = np.empty((len(rows), v.shape[3]))
    ra = np.empty((len(rows), v.shape[3]))
    rl = np.empty(len(rows))
    by_b = {}
    for r, (b, h, i) in enumerate(rows):
        by_b.setdefault(b, []).append(r)
    for b, idx in by_b.items():
        qb, kb, vb = (dec(t[b:b + 1]) for dec, t in zip(decoders, tensors))
        sub = [(0, rows[r][1], rows[r][2]) for r in idx]
        o1, l1 = oracle.causal_attention_rows(qb, kb, vb, scale, sub)
        ro[idx], rl[idx] = o1, l1
        ra[idx] = abs_v(oracle.causal_attention_rows, qb, kb, vb, scale, sub)
    return ro, rl, ra


@pytest.mark.parametrize("prec", ["bf16", "fp8"])
def test_largest_launch_sampled_rows(prec):
    B, N, Hq, Hkv, d = (MAX_SHAPE[k] for k in ("B", "N", "Hq", "Hkv", "d"))
    assert B * N * Hq * d < 2 ** 31 <= (B + 1) * N * Hq * d
    note(f"case largest launch {prec}: B={B} N={N} Hq={Hq} Hkv={Hkv} d={d}")
    scale = 1.0 / np.sqrt(d)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(47)
    dt = torch.bfloat16 if prec == "bf16" else torch.float8_e4m3fn

    def draw(H):   # N(0, 1) drawn per batch on the device, stored in the kernel's dtype
        t = torch.empty((B, N, H, d), device=DEV, dtype=dt)
        for b in range(B):
            t[b] = torch.randn((N, H, d), device=DEV, generator=gen).to(dt)
        return t

    q, k, v = draw(Hq), draw(Hkv), draw(Hkv)
    o = torch.full((B, N, Hq, d), float("nan"), device=DEV, dtype=torch.bfloat16)
    lse = torch.full((B, Hq, N), float("nan"), device=DEV, dtype=torch.float32)
    if prec == "bf16":
        ba.attn_fwd_causal_bf16(q, k, v, o, lse, softmax_scale=scale)
        tensors = (q, k, v)
        dec = lambda t: oracle.bf16_decode(t.view(torch.int16).cpu().numpy().view(np.uint16))
        decoders = (dec, dec, dec)
    else:
        # per-tensor descales 1/2 (q), 1 (k) and 2 (v) on the drawn codes
        descales = (0.5, 1.0, 2.0)
        tensors = tuple(t.view(torch.uint8) for t in (q, k, v))
        dq, dk, dv = (torch.full((1,), s, device=DEV) for s in descales)
        ba.attn_fwd_causal_fp8(*tensors, dq, dk, dv, o, lse, softmax_scale=scale,
                               descale_per_head=0)
        decoders = tuple((lambda t, s=s: oracle.e4m3_decode(t.cpu().numpy()) * s)
                         for s in descales)
    torch.cuda.synchronize()
    rows = _max_rows(np.random.default_rng(49))
    ro, rl, ra = _oracle_rows_from_device(tensors, decoders, scale, rows)
    bb = torch.tensor([r[0] for r in rows], device=DEV)
    hh = torch.tensor([r[1] for r in rows], device=DEV)
    ii = torch.tensor([r[2] for r in rows], device=DEV)
    go = o[bb, ii, hh].float().cpu().numpy().astype(np.float64)
    gl = lse[bb, hh, ii].cpu().numpy().astype(np.float64)
    # every output element was written (the buffers started as NaN)
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    check("largest_launch/rows", prec, go, ro, gl, rl, ref_abs_o=ra, fp8_path="exact",
          row_heads=[(b, h) for b, h, _ in rows])
