"""GPU parity of the extensions past the pages' Nq == Nk scope, through the C ABI:
causal attention of Nq queries over Nk keys with a query offset (chunked prefill,
a KV prefix seen in full), the merge of two partial attentions, and the
flash_attn_func-style wrapper.  References: oracle.offset_attention and
oracle.merge_partials (fp64, CPU), plus byte identity with the plain entry points
where the computation is the same.
"""
import zlib

import numpy as np
import pytest
import torch

import bf16_causal_prefill_amd as ba
import oracle
from gpu_harness import (DEV, ROUNDED_LSE_BOUND, abs_v, bf16_bytes, check, gpu_quantize, note,
                         to_dev_u16_as_bf16)

pytestmark = pytest.mark.gpu

# name: (B, Nq, Nk, q_offset, Hq, Hkv, d_qk, per_head); key j visible to query i iff
# j <= i + q_offset
CASES = {
    "chunk_tail": (1, 64, 300, 236, 4, 2, 128, True),     # the last 64 of 300 positions
    "square": (2, 300, 300, 0, 4, 2, 128, False),         # the plain causal case
    "all_visible": (2, 100, 77, 77, 4, 4, 128, True),     # every key visible
    "q_longer": (1, 257, 129, 5, 2, 1, 128, False),       # more queries than keys
    "mla_chunk": (1, 33, 700, 667, 2, 2, 192, True),
    "offset_past_nk": (1, 40, 1000, 5000, 2, 1, 128, False),
    "one_query": (1, 1, 513, 512, 8, 2, 128, True),
}


def _draw(name, B, Nq, Nk, Hq, Hkv, dqk, dv=128):
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    q = rng.standard_normal((B, Nq, Hq, dqk), dtype=np.float32)
    k = rng.standard_normal((B, Nk, Hkv, dqk), dtype=np.float32)
    v = rng.standard_normal((B, Nk, Hkv, dv), dtype=np.float32)
    return q, k, v


def _empty_out(B, Nq, Hq, dv=128, want_lse=True):
    o = torch.full((B, Nq, Hq, dv), float("nan"), device=DEV, dtype=torch.bfloat16)
    lse = torch.full((B, Hq, Nq), float("nan"), device=DEV, dtype=torch.float32) if want_lse else None
    return o, lse


def _host(o, lse):
    return (o.float().cpu().numpy().astype(np.float64),
            None if lse is None else lse.cpu().numpy().astype(np.float64))


@pytest.mark.parametrize("case", sorted(CASES))
def test_offset_bf16(case):
    B, Nq, Nk, off, Hq, Hkv, dqk, _ = CASES[case]
    note(f"offset bf16 {case}: B={B} Nq={Nq} Nk={Nk} q_offset={off} Hq={Hq} Hkv={Hkv} d={dqk}")
    q, k, v = _draw(case, B, Nq, Nk, Hq, Hkv, dqk)
    qu, ku, vu = (bf16_bytes(a) for a in (q, k, v))
    scale = 1.0 / np.sqrt(dqk)
    o, lse = _empty_out(B, Nq, Hq)
    ba.attn_fwd_causal_offset_bf16(*(to_dev_u16_as_bf16(a) for a in (qu, ku, vu)), o, lse,
                                   q_offset=off, softmax_scale=scale)
    torch.cuda.synchronize()
    go, gl = _host(o, lse)
    ro, rl = oracle.offset_attention(*(oracle.bf16_decode(a) for a in (qu, ku, vu)), scale, off)
    check(case, "bf16", go, ro, gl, rl)


@pytest.mark.parametrize("want_lse", [True, False], ids=["lse", "nolse"])
@pytest.mark.parametrize("case", sorted(CASES))
def test_offset_fp8(case, want_lse):
    B, Nq, Nk, off, Hq, Hkv, dqk, per_head = CASES[case]
    note(f"offset fp8 {case} lse={want_lse}: B={B} Nq={Nq} Nk={Nk} q_offset={off}")
    q, k, v = _draw(case, B, Nq, Nk, Hq, Hkv, dqk)
    scale = 1.0 / np.sqrt(dqk)
    dev, dec = [], []
    for x in (q, k, v):
        cd, dd = gpu_quantize(x, per_head)
        ch, dh = oracle.quantize_e4m3(x, per_head)
        assert np.array_equal(cd.cpu().numpy(), ch)
        dev.append((cd, dd))
        dec.append(oracle.e4m3_decode(ch) * (dh[None, None, :, None].astype(np.float64)
                                             if per_head else float(dh[0])))
    o, lse = _empty_out(B, Nq, Hq, want_lse=want_lse)
    ba.attn_fwd_causal_offset_fp8(dev[0][0], dev[1][0], dev[2][0], dev[0][1], dev[1][1],
                                  dev[2][1], o, lse, q_offset=off, softmax_scale=scale,
                                  descale_per_head=int(per_head))
    torch.cuda.synchronize()
    go, gl = _host(o, lse)
    ro, rl = oracle.offset_attention(*dec, scale, off)
    check(case, "fp8", go, ro, gl, rl if want_lse else None, fp8_path="exact" if want_lse else "lean",
          ref_abs_o=abs_v(oracle.offset_attention, *dec, scale, off))


@pytest.mark.parametrize("case", sorted(CASES))
def test_offset_fp8_pow2_q_scale(case):
    """The offset entry point with the LSE on Q quantised by quantize_e4m3_q_pow2 (the
    power-of-two softmax constant path, whose first tile sets the running max)."""
    B, Nq, Nk, off, Hq, Hkv, dqk, per_head = CASES[case]
    note(f"offset fp8 pow2 {case}: B={B} Nq={Nq} Nk={Nk} q_offset={off}")
    q, k, v = _draw(case, B, Nq, Nk, Hq, Hkv, dqk)
    scale = 1.0 / np.sqrt(dqk)
    dev, dec, host_ds = {}, {}, {}
    bc = (lambda d: d[None, None, :, None].astype(np.float64)) if per_head else \
        (lambda d: float(d[0]))
    for n, x in (("k", k), ("v", v)):
        cd, dd = gpu_quantize(x, per_head)
        ch, dh = oracle.quantize_e4m3(x, per_head)
        assert np.array_equal(cd.cpu().numpy(), ch)
        assert np.array_equal(dd.cpu().numpy().view(np.uint32), dh.view(np.uint32))
        dev[n], dec[n], host_ds[n] = (cd, dd), oracle.e4m3_decode(ch) * bc(dh), dh
    ch, dh = oracle.quantize_e4m3_q_pow2(q, per_head, host_ds["k"], scale)
    qc = torch.empty(q.shape, device=DEV, dtype=torch.uint8)
    qd = torch.empty((Hq if per_head else 1,), device=DEV, dtype=torch.float32)
    ba.quantize_e4m3_q_pow2(torch.from_numpy(q).to(DEV), qc, qd, dev["k"][1], scale, per_head)
    torch.cuda.synchronize()
    assert np.array_equal(qc.cpu().numpy(), ch)
    assert np.array_equal(qd.cpu().numpy().view(np.uint32), dh.view(np.uint32))
    dec["q"] = oracle.e4m3_decode(ch) * bc(dh)
    o, lse = _empty_out(B, Nq, Hq)
    ba.attn_fwd_causal_offset_fp8(qc, dev["k"][0], dev["v"][0], qd, dev["k"][1], dev["v"][1],
                                  o, lse, q_offset=off, softmax_scale=scale,
                                  descale_per_head=int(per_head))
    torch.cuda.synchronize()
    go, gl = _host(o, lse)
    ro, rl = oracle.offset_attention(dec["q"], dec["k"], dec["v"], scale, off)
    check(f"{case}/pow2", "fp8", go, ro, gl, rl, fp8_path="exact",
          ref_abs_o=abs_v(oracle.offset_attention, dec["q"], dec["k"], dec["v"], scale, off))


@pytest.mark.parametrize("prec", ["bf16", "fp8"])
def test_offset_zero_square_is_plain_causal(prec):
    """Nq == Nk with q_offset 0 runs the same kernel as the plain entry point: the
    outputs are byte-identical."""
    B, N, Hq, Hkv = 1, 333, 4, 2
    q, k, v = _draw("square-identity", B, N, N, Hq, Hkv, 128)
    o1, l1 = _empty_out(B, N, Hq)
    o2, l2 = _empty_out(B, N, Hq)
    if prec == "bf16":
        t = [to_dev_u16_as_bf16(bf16_bytes(a)) for a in (q, k, v)]
        ba.attn_fwd_causal_bf16(*t, o1, l1)
        ba.attn_fwd_causal_offset_bf16(*t, o2, l2, q_offset=0)
    else:
        dv = [gpu_quantize(a, True) for a in (q, k, v)]
        args = (dv[0][0], dv[1][0], dv[2][0], dv[0][1], dv[1][1], dv[2][1])
        ba.attn_fwd_causal_fp8(*args, o1, l1)
        ba.attn_fwd_causal_offset_fp8(*args, o2, l2, q_offset=0)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_merge_against_oracle():
    """Random partials (bf16 O, fp32 LSE with some empty partials) merged on the GPU,
    out of place and in place, against the fp64 merge of the same values."""
    rng = np.random.default_rng(31)
    B, N, Hq, dv = 2, 77, 6, 128
    oa = rng.standard_normal((B, N, Hq, dv), dtype=np.float32)
    ob = rng.standard_normal((B, N, Hq, dv), dtype=np.float32)
    la = (3.0 * rng.standard_normal((B, Hq, N))).astype(np.float32)
    lb = (3.0 * rng.standard_normal((B, Hq, N))).astype(np.float32)
    la[0, 1, :5] = -np.inf                    # partial a empty for these rows
    lb[1, 2, 7:9] = -np.inf                   # partial b empty
    la[1, 3, 10] = lb[1, 3, 10] = -np.inf     # both empty
    oau, obu = bf16_bytes(oa), bf16_bytes(ob)
    ro, rl = oracle.merge_partials(oracle.bf16_decode(oau), la, oracle.bf16_decode(obu), lb)
    for inplace in (False, True):
        da, db = to_dev_u16_as_bf16(oau), to_dev_u16_as_bf16(obu)
        dla, dlb = torch.from_numpy(la).to(DEV), torch.from_numpy(lb).to(DEV)
        if inplace:
            o, lse = da, dla
        else:
            o, lse = _empty_out(B, N, Hq)
        ba.attn_merge_partials(da, dla, db, dlb, o, lse)
        torch.cuda.synchronize()
        go, gl = _host(o, lse)
        fin = np.isfinite(rl)
        assert np.array_equal(fin, np.isfinite(gl))
        assert np.max(np.abs(gl[fin] - rl[fin])) < 1e-5
        # bf16 rounding of the fp32 result: half an ulp (2^-8 relative) plus fp32 slack
        err = np.abs(go - ro)
        assert np.all(err <= 2.0 ** -8 * np.abs(ro) + 1e-6), float(err.max())
        note(f"merge inplace={inplace}: max abs err {err.max():.3e}")


@pytest.mark.parametrize("prec", ["bf16", "fp8"])
def test_split_keys_and_merge_equals_causal(prec):
    """Queries P..N-1: attention to the prefix 0..P-1 (all visible) merged with the
    causal attention to P..N-1 equals causal attention over 0..N-1 (the oracle's rows),
    within the precision's tolerance."""
    B, N, P, Hq, Hkv = 1, 700, 300, 4, 2
    q, k, v = _draw(f"split-{prec}", B, N, N, Hq, Hkv, 128)
    scale = 1.0 / np.sqrt(128)
    nq = N - P
    oa, la = _empty_out(B, nq, Hq)
    ob, lb = _empty_out(B, nq, Hq)
    if prec == "bf16":
        qu, ku, vu = (bf16_bytes(a) for a in (q, k, v))
        tq = to_dev_u16_as_bf16(np.ascontiguousarray(qu[:, P:]))
        tk0 = to_dev_u16_as_bf16(np.ascontiguousarray(ku[:, :P]))
        tv0 = to_dev_u16_as_bf16(np.ascontiguousarray(vu[:, :P]))
        tk1 = to_dev_u16_as_bf16(np.ascontiguousarray(ku[:, P:]))
        tv1 = to_dev_u16_as_bf16(np.ascontiguousarray(vu[:, P:]))
        ba.attn_fwd_causal_offset_bf16(tq, tk0, tv0, oa, la, q_offset=P, softmax_scale=scale)
        ba.attn_fwd_causal_offset_bf16(tq, tk1, tv1, ob, lb, q_offset=0, softmax_scale=scale)
        dec = [oracle.bf16_decode(a) for a in (qu, ku, vu)]
    else:
        # per-tensor scales of the whole tensors, so both chunks use the same codes
        cods = [gpu_quantize(a, False) for a in (q, k, v)]
        host = [oracle.quantize_e4m3(a, False) for a in (q, k, v)]
        for (cd, _), (ch, _) in zip(cods, host):
            assert np.array_equal(cd.cpu().numpy(), ch)
        (cq, dq), (ck, dk), (cv, dvs) = cods
        sl = lambda t, a, b: t[:, a:b].contiguous()
        ba.attn_fwd_causal_offset_fp8(sl(cq, P, N), sl(ck, 0, P), sl(cv, 0, P), dq, dk, dvs,
                                      oa, la, q_offset=P, softmax_scale=scale)
        ba.attn_fwd_causal_offset_fp8(sl(cq, P, N), sl(ck, P, N), sl(cv, P, N), dq, dk, dvs,
                                      ob, lb, q_offset=0, softmax_scale=scale)
        dec = [oracle.e4m3_decode(ch) * float(dh[0]) for ch, dh in host]
    ba.attn_merge_partials(oa, la, ob, lb, oa, la)      # in place into partial a
    torch.cuda.synchronize()
    go, gl = _host(oa, la)
    ro, rl = oracle.causal_attention(*dec, scale)
    ra = abs_v(oracle.causal_attention, *dec, scale)[:, P:] if prec == "fp8" else None
    check(f"split-merge-{prec}", prec, go, ro[:, P:], gl, rl[:, :, P:], ref_abs_o=ra,
          fp8_path="exact")


def test_flash_attn_func_bf16_matches_entry_point():
    B, N, Hq, Hkv = 2, 190, 4, 2
    q, k, v = (to_dev_u16_as_bf16(bf16_bytes(a)) for a in _draw("fa-bf16", B, N, N, Hq, Hkv, 128))
    o1, l1 = _empty_out(B, N, Hq)
    ba.attn_fwd_causal_bf16(q, k, v, o1, l1)
    o2, l2 = ba.flash_attn_func(q, k, v, causal=True, return_lse=True)
    o3 = ba.flash_attn_func(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16))
    assert torch.equal(l1, l2)


def test_flash_attn_func_fp8_matches_entry_point():
    B, N, Hq, Hkv = 1, 260, 4, 1
    x = _draw("fa-fp8", B, N, N, Hq, Hkv, 128)
    dv = [gpu_quantize(a, True) for a in x]
    (cq, dq), (ck, dk), (cv, dvs) = dv
    o1, l1 = _empty_out(B, N, Hq)
    ba.attn_fwd_causal_fp8(cq, ck, cv, dq, dk, dvs, o1, l1)
    o2, l2 = ba.flash_attn_func(cq, ck, cv, return_lse=True, q_descale=dq, k_descale=dk,
                                v_descale=dvs)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)
    if hasattr(torch, "float8_e4m3fn"):
        f8 = [t.view(torch.float8_e4m3fn) for t in (cq, ck, cv)]
        o3, l3 = ba.flash_attn_func(*f8, return_lse=True, q_descale=dq, k_descale=dk,
                                    v_descale=dvs)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o3.view(torch.int16))
        assert torch.equal(l1, l3)
    # without the LSE the FP8 kernel takes its other probability path (one-FMA codes);
    # the wrapper must select the same one
    o4, _ = _empty_out(B, N, Hq, want_lse=False)
    ba.attn_fwd_causal_fp8(cq, ck, cv, dq, dk, dvs, o4, None)
    o5 = ba.flash_attn_func(cq, ck, cv, q_descale=dq, k_descale=dk, v_descale=dvs)
    torch.cuda.synchronize()
    assert torch.equal(o4.view(torch.int16), o5.view(torch.int16))


def test_flash_attn_func_non_causal_and_rectangular():
    """causal=False: every key visible; causal=True with Nq < Nk: bottom-right diagonal."""
    B, Nq, Nk, Hq, Hkv = 1, 50, 130, 4, 2
    q, k, v = _draw("fa-rect", B, Nq, Nk, Hq, Hkv, 128)
    qu, ku, vu = (bf16_bytes(a) for a in (q, k, v))
    tq, tk, tv = (to_dev_u16_as_bf16(a) for a in (qu, ku, vu))
    dec = [oracle.bf16_decode(a) for a in (qu, ku, vu)]
    scale = 1.0 / np.sqrt(128)
    for causal, off in ((False, Nk), (True, Nk - Nq)):
        o, lse = ba.flash_attn_func(tq, tk, tv, causal=causal, return_lse=True)
        torch.cuda.synchronize()
        go, gl = _host(o, lse)
        ro, rl = oracle.offset_attention(*dec, scale, off)
        check(f"flash_attn_func causal={causal}", "bf16", go, ro, gl, rl)


# ---- the rounded-row-sum LSE (consistent with O on the fast FP8 path) -------------------

def _fp8_inputs(name, B, Nq, Nk, Hq, Hkv, dqk, per_head):
    q, k, v = _draw(name, B, Nq, Nk, Hq, Hkv, dqk)
    dev, dec = [], []
    for x in (q, k, v):
        cd, dd = gpu_quantize(x, per_head)
        ch, dh = oracle.quantize_e4m3(x, per_head)
        assert np.array_equal(cd.cpu().numpy(), ch)
        dev.append((cd, dd))
        dec.append(oracle.e4m3_decode(ch) * (dh[None, None, :, None].astype(np.float64)
                                             if per_head else float(dh[0])))
    return dev, dec


@pytest.mark.parametrize("case", ["square", "chunk_tail", "mla_chunk", "q_longer"])
def test_rounded_lse(case):
    """O is byte-identical to the lse == NULL call; the LSE is within the rounding bound
    of the oracle's exact LSE."""
    B, Nq, Nk, off, Hq, Hkv, dqk, per_head = CASES[case]
    note(f"rounded lse {case}: B={B} Nq={Nq} Nk={Nk} q_offset={off}")
    dev, dec = _fp8_inputs("rounded-" + case, B, Nq, Nk, Hq, Hkv, dqk, per_head)
    args = (dev[0][0], dev[1][0], dev[2][0], dev[0][1], dev[1][1], dev[2][1])
    scale = 1.0 / np.sqrt(dqk)
    o1, _ = _empty_out(B, Nq, Hq, want_lse=False)
    o2, l2 = _empty_out(B, Nq, Hq)
    ba.attn_fwd_causal_offset_fp8(*args, o1, None, q_offset=off, softmax_scale=scale,
                                  descale_per_head=int(per_head))
    ba.attn_fwd_causal_offset_fp8_rounded_lse(*args, o2, l2, q_offset=off, softmax_scale=scale,
                                              descale_per_head=int(per_head))
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    ro, rl = oracle.offset_attention(*dec, scale, off)
    go, gl = _host(o2, l2)
    check(case, "fp8", go, ro, fp8_path="lean", ref_abs_o=abs_v(oracle.offset_attention, *dec, scale, off))
    err = float(np.max(np.abs(gl - rl)))
    note(f"  rounded LSE max |error| {err:.4f} (bound {ROUNDED_LSE_BOUND:.4f})")
    assert np.all(np.isfinite(gl)) and err <= ROUNDED_LSE_BOUND


def test_rounded_lse_merge_of_split_keys():
    """The consistent LSE merges: a KV prefix seen in full plus the causal chunk, both on
    the fast path with rounded LSEs, merged, match attention over all keys (oracle)."""
    B, N, P, Hq, Hkv, dqk = 1, 500, 300, 4, 2, 128
    note(f"rounded lse merge: N={N} prefix={P}")
    dev, dec = _fp8_inputs("rounded-merge", B, N, N, Hq, Hkv, dqk, True)
    scale = 1.0 / np.sqrt(dqk)
    qc = dev[0][0][:, P:].contiguous()
    kp, vp = dev[1][0][:, :P].contiguous(), dev[2][0][:, :P].contiguous()
    kc, vc = dev[1][0][:, P:].contiguous(), dev[2][0][:, P:].contiguous()
    ds = (dev[0][1], dev[1][1], dev[2][1])
    oa, la = _empty_out(B, N - P, Hq)
    ob, lb = _empty_out(B, N - P, Hq)
    ba.attn_fwd_causal_offset_fp8_rounded_lse(qc, kp, vp, *ds, oa, la, q_offset=P,
                                              softmax_scale=scale, descale_per_head=1)
    ba.attn_fwd_causal_offset_fp8_rounded_lse(qc, kc, vc, *ds, ob, lb, q_offset=0,
                                              softmax_scale=scale, descale_per_head=1)
    om, lm = _empty_out(B, N - P, Hq)
    ba.attn_merge_partials(oa, la, ob, lb, om, lm)
    torch.cuda.synchronize()
    ro, rl = oracle.offset_attention(dec[0][:, P:], dec[1], dec[2], scale, P)
    go, gl = _host(om, lm)
    check("rounded merge", "fp8", go, ro, fp8_path="lean",
          ref_abs_o=abs_v(oracle.offset_attention, dec[0][:, P:], dec[1], dec[2], scale, P))
    assert float(np.max(np.abs(gl - rl))) <= ROUNDED_LSE_BOUND
