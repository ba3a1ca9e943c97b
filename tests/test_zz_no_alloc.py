"""The allocation-free joint quantiser (quantize_e4m3_qk_outliers_noalloc), through the
C ABI: its outputs (codes, descales, permutation) are bit-identical to those of
quantize_e4m3_qk_outliers with a workspace, on consecutive calls of different sizes
(the scratch array keeps the previous call's contents), and to the oracle's."""
import numpy as np
import pytest
import torch

import bf16_causal_prefill_amd as ba
import oracle
import workloads
from gpu_harness import DEV, note

pytestmark = pytest.mark.gpu


def _outputs(x, per_head):
    q, k = x["q"], x["k"]
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    T = ba.OUTLIER_CHANNELS
    return (torch.empty(q.shape, device=DEV, dtype=torch.uint8),
            torch.empty(k.shape, device=DEV, dtype=torch.uint8),
            torch.empty((B, N, Hq, T), device=DEV, dtype=torch.bfloat16),
            torch.empty((B, N, Hkv, T), device=DEV, dtype=torch.bfloat16),
            torch.empty((Hq if per_head else 1,), device=DEV, dtype=torch.float32),
            torch.empty((Hkv if per_head else 1,), device=DEV, dtype=torch.float32),
            torch.empty((Hkv, d), device=DEV, dtype=torch.uint8))


def _host(outs):
    return [(t.view(torch.int16) if t.dtype == torch.bfloat16 else t).cpu().numpy()
            for t in outs]


CALLS = [   # consecutive calls on one device: a larger one, then smaller ones
    (workloads.CONFIGS["mistral16k"].with_(N=512, seed=91), True, True),
    (workloads.CONFIGS["mistral16k"].with_(B=2, N=65, Hq=4, Hkv=1, seed=92), True, False),
    (workloads.CONFIGS["mla16k"].with_(N=40, Hq=2, Hkv=2, seed=93), False, False),
]


def test_noalloc_matches_workspace_entry_point():
    for n, (w, per_head, pow2) in enumerate(CALLS):
        note(f"noalloc call {n}: B={w.B} N={w.N} Hq={w.Hq} Hkv={w.Hkv} d={w.d_qk} "
             f"per_head={per_head} pow2={pow2}")
        x = workloads.generate(w)
        q, k = (torch.from_numpy(x[t]).to(DEV) for t in "qk")
        scale = w.softmax_scale
        a = _outputs(x, per_head)
        ba.quantize_e4m3_qk_outliers_noalloc(q, k, *a, per_head, q_pow2=pow2, softmax_scale=scale)
        b = _outputs(x, per_head)
        ba.quantize_e4m3_qk_outliers(q, k, *b, per_head, q_pow2=pow2, softmax_scale=scale)
        torch.cuda.synchronize()
        ha, hb = _host(a), _host(b)
        names = ("q codes", "k codes", "q side", "k side", "q descale", "k descale", "perm")
        for name, u, v in zip(names, ha, hb):
            assert np.array_equal(u.view(np.uint8), v.view(np.uint8)), f"call {n}: {name}"
        qc, kc, qx, kx, qd, kd, perm = oracle.quantize_e4m3_qk_outliers(
            x["q"], x["k"], per_head, q_pow2_scale=scale if pow2 else None)
        assert np.array_equal(ha[0], qc) and np.array_equal(ha[1], kc), f"call {n}: oracle codes"
        assert np.array_equal(ha[2].view(np.uint16), qx), f"call {n}: q side"
        assert np.array_equal(ha[3].view(np.uint16), kx), f"call {n}: k side"
        assert np.array_equal(ha[4].view(np.uint32), qd.view(np.uint32)), f"call {n}"
        assert np.array_equal(ha[5].view(np.uint32), kd.view(np.uint32)), f"call {n}"
        assert np.array_equal(ha[6], perm.astype(np.uint8)), f"call {n}: perm"


def test_noalloc_rejects_sizes_beyond_its_scratch():
    w = ba.NOALLOC_SCRATCH_WORDS
    Hq = Hkv = w // 128        # (Hq + Hkv) * 128 = 2 * words
    q = torch.zeros((1, 1, Hq, 128), device=DEV)
    k = torch.zeros((1, 1, Hkv, 128), device=DEV)
    outs = (torch.empty(q.shape, device=DEV, dtype=torch.uint8),
            torch.empty(k.shape, device=DEV, dtype=torch.uint8),
            torch.empty((1, 1, Hq, 32), device=DEV, dtype=torch.bfloat16),
            torch.empty((1, 1, Hkv, 32), device=DEV, dtype=torch.bfloat16),
            torch.empty((Hq,), device=DEV), torch.empty((Hkv,), device=DEV),
            torch.empty((Hkv, 128), device=DEV, dtype=torch.uint8))
    with pytest.raises(ba.AttnError) as e:
        ba.quantize_e4m3_qk_outliers_noalloc(q, k, *outs, True)
    assert e.value.status == ba.ATTN_E_TOO_LARGE
