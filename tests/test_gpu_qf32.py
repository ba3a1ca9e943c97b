"""attn_fwd_causal_fp8_qf32: the FP8 attention on float32 Q, which the kernel encodes as it
loads each row (with the quantisers' encoder and Q's descales).  Every case runs the same
inputs both ways, quantise Q then attn_fwd_causal_fp8 on its codes, and float32 Q straight
into attn_fwd_causal_fp8_qf32, and requires byte-identical O and LSE (NaN payloads
included); the descales come from quantize_e4m3_qkv with q_out = None (Q's descales only),
whose descales and K/V codes must equal the separate quantisers'.  One case per shape is
also compared with the fp64 oracle, and the full 32K workloads (gauss32k, mla32k) are
compared byte for byte with the codes step over every workgroup of the launch.

Cases: d_qk 128 with GQA and d_qk 192 (the MLA shape), a ragged N, per-tensor and per-head
descales, Q's descale from quantize_e4m3_q_pow2 (the power-of-two softmax constant) and
from plain absmax, with and without the LSE; Q holds an all-zero row, a head scaled by 30
and, in the per-head cases, a NaN element (byte identity then covers that row's output as
well)."""
import numpy as np
import pytest
import torch

import bf16_causal_prefill_amd as ba
import oracle
from gpu_harness import DEV, abs_v, check, note

pytestmark = pytest.mark.gpu

# name: B, N, Hq, Hkv, d_qk, d_v
SHAPES = {"gqa_ragged": (1, 700, 8, 2, 128, 128), "mla": (1, 300, 4, 4, 192, 128),
          "batch": (2, 257, 4, 1, 128, 128)}


def _inputs(B, N, Hq, Hkv, dqk, dv, seed, with_nan):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, N, Hq, dqk)).astype(np.float32)
    k = rng.standard_normal((B, N, Hkv, dqk)).astype(np.float32)
    v = rng.standard_normal((B, N, Hkv, dv)).astype(np.float32)
    q[:, 3, :, :] = 0.0
    q[:, :, Hq - 1, :] *= np.float32(30.0)
    if with_nan:
        q[0, 5, 0, 7] = np.nan
    return q, k, v


@pytest.mark.parametrize("want_lse", [True, False], ids=["lse", "nolse"])
@pytest.mark.parametrize("q_pow2", [True, False], ids=["pow2_q", "absmax_q"])
@pytest.mark.parametrize("per_head", [True, False], ids=["per_head", "per_tensor"])
@pytest.mark.parametrize("shape", list(SHAPES))
def test_qf32_byte_identical(shape, per_head, q_pow2, want_lse):
    B, N, Hq, Hkv, dqk, dv = SHAPES[shape]
    with_nan = per_head
    note(f"qf32 {shape} per_head={per_head} q_pow2={q_pow2} lse={want_lse} nan={with_nan}")
    q, k, v = _inputs(B, N, Hq, Hkv, dqk, dv, 5000 + list(SHAPES).index(shape), with_nan)
    scale = 1.0 / np.sqrt(dqk)
    dev = {n: torch.from_numpy(a).to(DEV) for n, a in (("q", q), ("k", k), ("v", v))}
    ns = {"q": Hq if per_head else 1, "k": Hkv if per_head else 1, "v": Hkv if per_head else 1}
    # descales and K/V codes of the one-call quantiser without Q's codes ...
    codes = {n: torch.empty(dev[n].shape, device=DEV, dtype=torch.uint8) for n in "kv"}
    ds = {n: torch.empty((ns[n],), device=DEV) for n in "qkv"}
    ba.quantize_e4m3_qkv(dev["q"], dev["k"], dev["v"], None, codes["k"], codes["v"], ds["q"],
                         ds["k"], ds["v"], per_head, q_pow2=q_pow2, softmax_scale=scale)
    # ... equal the separate quantisers'
    sep = {n: (torch.empty(dev[n].shape, device=DEV, dtype=torch.uint8),
               torch.empty((ns[n],), device=DEV)) for n in "qkv"}
    for n in "kv":
        ba.quantize_e4m3(dev[n], sep[n][0], sep[n][1], per_head)
    if q_pow2:
        ba.quantize_e4m3_q_pow2(dev["q"], sep["q"][0], sep["q"][1], sep["k"][1], scale, per_head)
    else:
        ba.quantize_e4m3(dev["q"], sep["q"][0], sep["q"][1], per_head)
    torch.cuda.synchronize()
    for n in "qkv":
        assert torch.equal(ds[n].view(torch.int32), sep[n][1].view(torch.int32)), n
    for n in "kv":
        assert torch.equal(codes[n], sep[n][0]), n

    def outputs():
        o = torch.full((B, N, Hq, dv), float("nan"), device=DEV, dtype=torch.bfloat16)
        lse = (torch.full((B, Hq, N), float("nan"), device=DEV, dtype=torch.float32)
               if want_lse else None)
        return o, lse
    o_ref, lse_ref = outputs()
    ba.attn_fwd_causal_fp8(sep["q"][0], codes["k"], codes["v"], ds["q"], ds["k"], ds["v"], o_ref,
                           lse_ref, softmax_scale=scale, descale_per_head=int(per_head))
    o_new, lse_new = outputs()
    ba.attn_fwd_causal_fp8_qf32(dev["q"], codes["k"], codes["v"], ds["q"], ds["k"], ds["v"],
                                o_new, lse_new, softmax_scale=scale, descale_per_head=int(per_head))
    torch.cuda.synchronize()
    assert torch.equal(o_ref.view(torch.int16), o_new.view(torch.int16)), "O differs"
    if want_lse:
        assert torch.equal(lse_ref.view(torch.int32), lse_new.view(torch.int32)), "LSE differs"
    note("  byte-identical to quantising Q first")
    if with_nan or not (q_pow2 and want_lse):
        return
    # the oracle on the same codes (NaN-free cases with the LSE)
    qc_h, qd_h = oracle.quantize_e4m3_q_pow2(q, per_head, oracle.quantize_e4m3(k, per_head)[1],
                                             scale)
    kc_h, kd_h = oracle.quantize_e4m3(k, per_head)
    vc_h, vd_h = oracle.quantize_e4m3(v, per_head)
    bc = (lambda d: d[None, None, :, None].astype(np.float64)) if per_head else \
        (lambda d: float(d[0]))
    qd_, kd_, vd_ = (oracle.e4m3_decode(c) * bc(d) for c, d in
                     ((qc_h, qd_h), (kc_h, kd_h), (vc_h, vd_h)))
    ro, rl = oracle.causal_attention(qd_, kd_, vd_, scale)
    check(f"qf32-{shape}", "fp8", o_new.float().cpu().numpy().astype(np.float64), ro,
          lse_new.cpu().numpy().astype(np.float64), rl, fp8_path="exact",
          ref_abs_o=abs_v(oracle.causal_attention, qd_, kd_, vd_, scale))


@pytest.mark.parametrize("name", ["gauss32k", "mla32k"])
def test_qf32_full_size_byte_identical(name):
    """The full 32K workloads (d_qk 128 with GQA, per-tensor descales; the MLA shape,
    per-head): the float32-Q step (quantize_e4m3_qkv with Q's descales only, then
    attn_fwd_causal_fp8_qf32) gives O and LSE byte-identical to the codes step, over every
    workgroup of the launch."""
    import workloads
    w = workloads.get(name)
    note(f"qf32 full {name}: N={w.N} Hq={w.Hq} Hkv={w.Hkv} d={w.d_qk}/{w.d_v}")
    x = workloads.generate(w)
    xd = {n: torch.from_numpy(x[n]).to(DEV) for n in "qkv"}
    del x
    ph = w.fp8_per_head
    ns = {"q": w.Hq if ph else 1, "k": w.Hkv if ph else 1, "v": w.Hkv if ph else 1}
    codes = {n: torch.empty(xd[n].shape, device=DEV, dtype=torch.uint8) for n in "qkv"}
    ds = {n: torch.empty((ns[n],), device=DEV) for n in "qkv"}
    ba.quantize_e4m3_qkv(xd["q"], xd["k"], xd["v"], codes["q"], codes["k"], codes["v"], ds["q"],
                         ds["k"], ds["v"], ph, q_pow2=True, softmax_scale=w.softmax_scale)
    outs = []
    for qf32 in (False, True):
        o = torch.full((w.B, w.N, w.Hq, w.d_v), float("nan"), device=DEV, dtype=torch.bfloat16)
        lse = torch.full((w.B, w.Hq, w.N), float("nan"), device=DEV, dtype=torch.float32)
        if qf32:
            dq = torch.full_like(ds["q"], float("nan"))
            ba.quantize_e4m3_qkv(xd["q"], xd["k"], xd["v"], None, codes["k"], codes["v"], dq,
                                 ds["k"], ds["v"], ph, q_pow2=True, softmax_scale=w.softmax_scale)
            assert torch.equal(dq.view(torch.int32), ds["q"].view(torch.int32))
            ba.attn_fwd_causal_fp8_qf32(xd["q"], codes["k"], codes["v"], dq, ds["k"], ds["v"],
                                        o, lse, softmax_scale=w.softmax_scale,
                                        descale_per_head=int(ph))
        else:
            ba.attn_fwd_causal_fp8(codes["q"], codes["k"], codes["v"], ds["q"], ds["k"], ds["v"],
                                   o, lse, softmax_scale=w.softmax_scale, descale_per_head=int(ph))
        torch.cuda.synchronize()
        outs.append((o, lse))
    (o0, l0), (o1, l1) = outs
    assert not torch.isnan(o0.float()).any() and not torch.isnan(l0).any()
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16)), "O differs"
    assert torch.equal(l0.view(torch.int32), l1.view(torch.int32)), "LSE differs"
    note("  byte-identical at full size")


@pytest.mark.parametrize("case", ["inf_element", "tiny_values", "all_zero"])
@pytest.mark.parametrize("per_head", [True, False], ids=["per_head", "per_tensor"])
def test_qf32_descale_edges(case, per_head):
    """Descales outside the branch-free encoder's range take the kernel's per-element
    encoder: an infinity in Q (descale +inf: finite values encode to signed zeros, the
    infinity to 0x7F), Q scaled by 1e-30 (descales near 2^-108), and an all-zero Q
    (descale 1).  Byte identity with quantising Q first, absmax Q descales."""
    B, N, Hq, Hkv, dqk, dv = 1, 300, 4, 2, 128, 128
    note(f"qf32 edge {case} per_head={per_head}")
    q, k, v = _inputs(B, N, Hq, Hkv, dqk, dv, 5100, False)
    if case == "inf_element":
        q[0, 7, 1, 3] = np.inf
    elif case == "tiny_values":
        q *= np.float32(1e-30)
    else:
        q[:] = 0.0
    scale = 1.0 / np.sqrt(dqk)
    dev = {n: torch.from_numpy(a).to(DEV) for n, a in (("q", q), ("k", k), ("v", v))}
    nh = {"q": Hq if per_head else 1, "k": Hkv if per_head else 1, "v": Hkv if per_head else 1}
    codes = {n: torch.empty(dev[n].shape, device=DEV, dtype=torch.uint8) for n in "qkv"}
    ds = {n: torch.empty((nh[n],), device=DEV) for n in "qkv"}
    for n in "qkv":
        ba.quantize_e4m3(dev[n], codes[n], ds[n], per_head)
    outs = []
    for qf32 in (False, True):
        o = torch.full((B, N, Hq, dv), float("nan"), device=DEV, dtype=torch.bfloat16)
        lse = torch.full((B, Hq, N), float("nan"), device=DEV, dtype=torch.float32)
        call = ba.attn_fwd_causal_fp8_qf32 if qf32 else ba.attn_fwd_causal_fp8
        call(dev["q"] if qf32 else codes["q"], codes["k"], codes["v"], ds["q"], ds["k"], ds["v"],
             o, lse, softmax_scale=scale, descale_per_head=int(per_head))
        torch.cuda.synchronize()
        outs.append((o, lse))
    (o0, l0), (o1, l1) = outs
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16)), "O differs"
    assert torch.equal(l0.view(torch.int32), l1.view(torch.int32)), "LSE differs"
    dq = ds["q"].cpu().numpy()
    if case == "tiny_values":
        assert np.all(dq < 2.0 ** -100), dq          # the per-element encoder's range
    elif case == "inf_element":
        assert np.isinf(dq).any()
    else:
        assert np.all(dq == 1.0)
