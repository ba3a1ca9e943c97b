"""The workgroup -> (batch, head, query tile) map: with B*Hkv a multiple of 8 the launcher
trades tiles between the XCDs of each pair and, for the FP8 kernels, rotates them over
each XCD's shader engines; every (batch, head, query tile) must still be computed exactly
once, by the same arithmetic.  Each case runs a batched launch where those apply (at
least 6 items per CU of an XCD) and the same work one batch element at a time (B = 1:
too few items for the exchange, a different map), into NaN-filled outputs, and requires
byte-identical O and LSE: a tile computed twice or not at all, or for the wrong head or
batch, cannot give that."""
import numpy as np
import pytest
import torch

import bf16_causal_prefill_amd as ba
from gpu_harness import DEV, note

pytestmark = pytest.mark.gpu

# name: B, Hq, Hkv, N, d_qk, d_v (items per XCD = B*Hkv/8 * Hq/Hkv * ceil(N/256))
CASES = {
    "gqa_b8_n2048": (8, 32, 8, 2048, 128, 128),      # 4 items per row, 256 per XCD
    "heads_b2_n24576": (2, 8, 8, 24576, 128, 128),   # 2 items per row, 192 per XCD
    "mla_b8_n4096": (8, 16, 16, 4096, 192, 128),     # 16 items per row, 256 per XCD
}


def _run(kind, q, k, v, ds, o, lse, scale):
    if kind == "bf16":
        ba.attn_fwd_causal_bf16(q, k, v, o, lse, softmax_scale=scale)
    else:
        ba.attn_fwd_causal_fp8(q, k, v, ds["q"], ds["k"], ds["v"], o, lse, softmax_scale=scale,
                               descale_per_head=1)


@pytest.mark.parametrize("kind", ["fp8_lse", "fp8_nolse", "bf16"])
@pytest.mark.parametrize("case", list(CASES))
def test_batched_map_equals_per_batch_launches(case, kind):
    B, Hq, Hkv, N, dqk, dv = CASES[case]
    note(f"tile map {case} {kind}: B={B} Hq={Hq} Hkv={Hkv} N={N} d={dqk}/{dv}")
    g = torch.Generator(device="cpu").manual_seed(7000 + list(CASES).index(case))
    xf = {n: torch.randn((B, N, H, d), generator=g, dtype=torch.float32)
          for n, H, d in (("q", Hq, dqk), ("k", Hkv, dqk), ("v", Hkv, dv))}
    scale = 1.0 / float(np.sqrt(dqk))
    ds = {}
    if kind == "bf16":
        x = {n: t.to(DEV).to(torch.bfloat16) for n, t in xf.items()}
    else:
        x = {}
        for n, t in xf.items():
            td = t.to(DEV)
            x[n] = torch.empty(td.shape, device=DEV, dtype=torch.uint8)
            ds[n] = torch.empty((td.shape[2],), device=DEV)
            ba.quantize_e4m3(td, x[n], ds[n], True)
            del td
    want_lse = kind != "fp8_nolse"

    def outputs(b):
        o = torch.full((b, N, Hq, dv), float("nan"), device=DEV, dtype=torch.bfloat16)
        lse = torch.full((b, Hq, N), float("nan"), device=DEV) if want_lse else None
        return o, lse

    o_all, lse_all = outputs(B)
    _run(kind, x["q"], x["k"], x["v"], ds, o_all, lse_all, scale)
    torch.cuda.synchronize()
    assert not torch.isnan(o_all.float()).any(), "a tile was not written"
    for b in range(B):
        o_b, lse_b = outputs(1)
        _run(kind, x["q"][b:b + 1], x["k"][b:b + 1], x["v"][b:b + 1], ds, o_b, lse_b, scale)
        torch.cuda.synchronize()
        assert torch.equal(o_b.view(torch.int16), o_all[b:b + 1].view(torch.int16)), \
            f"O of batch {b} differs"
        if want_lse:
            assert torch.equal(lse_b.view(torch.int32), lse_all[b:b + 1].view(torch.int32)), \
                f"LSE of batch {b} differs"
    note("  batched launch byte-identical to per-batch launches")


@pytest.mark.parametrize("kind", ["fp8_lse", "fp8_nolse", "bf16"])
def test_batched_map_with_query_offset(kind):
    """Chunked prefill (the last 4096 queries over 16384 keys, B = 8): every item sees
    most of the keys, so the weights the exchange plan trades are nearly equal; batched
    launch byte-identical to per-batch launches as above."""
    B, Hq, Hkv, Nq, Nk, d = 8, 32, 8, 4096, 16384, 128
    note(f"tile map offset {kind}: B={B} Nq={Nq} Nk={Nk}")
    g = torch.Generator(device="cpu").manual_seed(7100)
    xf = {"q": torch.randn((B, Nq, Hq, d), generator=g),
          "k": torch.randn((B, Nk, Hkv, d), generator=g),
          "v": torch.randn((B, Nk, Hkv, d), generator=g)}
    scale = 1.0 / float(np.sqrt(d))
    ds = {}
    if kind == "bf16":
        x = {n: t.to(DEV).to(torch.bfloat16) for n, t in xf.items()}
    else:
        x = {}
        for n, t in xf.items():
            td = t.to(DEV)
            x[n] = torch.empty(td.shape, device=DEV, dtype=torch.uint8)
            ds[n] = torch.empty((td.shape[2],), device=DEV)
            ba.quantize_e4m3(td, x[n], ds[n], True)
            del td
    want_lse = kind != "fp8_nolse"

    def run(sl, b):
        o = torch.full((b, Nq, Hq, d), float("nan"), device=DEV, dtype=torch.bfloat16)
        lse = torch.full((b, Hq, Nq), float("nan"), device=DEV) if want_lse else None
        if kind == "bf16":
            ba.attn_fwd_causal_offset_bf16(x["q"][sl], x["k"][sl], x["v"][sl], o, lse,
                                           q_offset=Nk - Nq, softmax_scale=scale)
        else:
            ba.attn_fwd_causal_offset_fp8(x["q"][sl], x["k"][sl], x["v"][sl], ds["q"], ds["k"],
                                          ds["v"], o, lse, q_offset=Nk - Nq,
                                          softmax_scale=scale, descale_per_head=1)
        torch.cuda.synchronize()
        return o, lse

    o_all, lse_all = run(slice(0, B), B)
    assert not torch.isnan(o_all.float()).any(), "a tile was not written"
    for b in range(B):
        o_b, lse_b = run(slice(b, b + 1), 1)
        assert torch.equal(o_b.view(torch.int16), o_all[b:b + 1].view(torch.int16)), b
        if want_lse:
            assert torch.equal(lse_b.view(torch.int32), lse_all[b:b + 1].view(torch.int32)), b
