"""GPU parity of the Hadamard pre-step (quantize_e4m3_hadamard) through the C ABI:
codes and descales bit-identical to oracle.quantize_e4m3_hadamard, and FP8 causal
attention on rotated Q and K against the fp64 oracle, both on the decoded rotated
inputs (the kernel's own parity) and on the unrotated float32 inputs (the rotation
leaves every score unchanged, so only the quantisation error remains).
"""
import zlib

import numpy as np
import pytest
import torch

import bf16_causal_prefill_amd as ba
import oracle
from gpu_harness import DEV, FP8_REL_FRO, abs_v, check, gpu_quantize, note, rel_fro, run_fp8

pytestmark = pytest.mark.gpu

# (B, N, H, d, per_head): every Hadamard block size (4 .. 128 channels, so every
# cross-lane butterfly stage), ragged row counts, per-tensor and per-head descales.
QCASES = [
    (2, 77, 4, 128, True),
    (1, 300, 3, 192, False),
    (1, 33, 2, 8, True),
    (1, 5, 1, 4, False),
    (1, 65, 5, 12, True),
    (3, 1000, 2, 128, False),
    (1, 129, 3, 16, True),       # block of 16 channels
    (2, 70, 2, 32, False),       # 32
    (1, 90, 5, 96, True),        # 32 (96 = 3 x 32)
    (1, 257, 2, 64, False),      # 64
]


def _rotate_on_gpu(x: np.ndarray, per_head: bool):
    xd = torch.from_numpy(x).to(DEV)
    codes = torch.empty(x.shape, device=DEV, dtype=torch.uint8)
    ds = torch.empty((x.shape[2] if per_head else 1,), device=DEV, dtype=torch.float32)
    ba.quantize_e4m3_hadamard(xd, codes, ds, per_head)
    torch.cuda.synchronize()
    return codes, ds


@pytest.mark.parametrize("case", QCASES, ids=lambda c: "B{}_N{}_H{}_d{}_{}".format(
    *c[:4], "head" if c[4] else "tensor"))
def test_quantize_hadamard_bit_exact(case):
    B, N, H, d, per_head = case
    note(f"quantize_e4m3_hadamard B={B} N={N} H={H} d={d} per_head={per_head}")
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()))
    x = rng.standard_normal((B, N, H, d), dtype=np.float32) * np.exp(
        rng.standard_normal(d)).astype(np.float32)
    codes, ds = _rotate_on_gpu(x, per_head)
    ch, dh = oracle.quantize_e4m3_hadamard(x, per_head)
    assert np.array_equal(codes.cpu().numpy(), ch), "codes differ from the oracle"
    assert np.array_equal(ds.cpu().numpy().view(np.uint32), dh.view(np.uint32)), \
        "descales differ from the oracle"


def _outlier_draw(seed, B, N, Hq, Hkv, d):
    """Q and K with per-channel scales ~ LogNormal(0, 0.5) and four channels x20 shared by
    Q and K (the case the rotation is for); V standard normal."""
    rng = np.random.default_rng(seed)
    out = rng.choice(d, 4, replace=False)
    sq = np.exp(0.5 * rng.standard_normal(d))
    sk = np.exp(0.5 * rng.standard_normal(d))
    sq[out] *= 20
    sk[out] *= 20
    q = (rng.standard_normal((B, N, Hq, d)) * sq / np.sqrt(d)).astype(np.float32)
    k = (rng.standard_normal((B, N, Hkv, d)) * sk / np.sqrt(d)).astype(np.float32)
    v = rng.standard_normal((B, N, Hkv, 128), dtype=np.float32)
    return q, k, v


@pytest.mark.parametrize("d", [128, 192])
def test_fp8_attention_on_rotated_qk(d):
    B, N, Hq, Hkv, per_head = 1, 700, 4, 2, True
    note(f"fp8 attention on Hadamard-rotated Q/K: N={N} Hq={Hq} Hkv={Hkv} d={d}")
    q, k, v = _outlier_draw(97 + d, B, N, Hq, Hkv, d)
    scale = 1.0 / np.sqrt(d)
    rq, rk = _rotate_on_gpu(q, per_head), _rotate_on_gpu(k, per_head)
    pv = gpu_quantize(v, per_head)
    (cq, dq), (ck, dk) = (oracle.quantize_e4m3_hadamard(a, per_head) for a in (q, k))
    cv, dv = oracle.quantize_e4m3(v, per_head)
    assert np.array_equal(rq[0].cpu().numpy(), cq) and np.array_equal(rk[0].cpu().numpy(), ck)
    dec = [oracle.e4m3_decode(c) * s[None, None, :, None].astype(np.float64)
           for c, s in ((cq, dq), (ck, dk), (cv, dv))]
    g = run_fp8(rq[0], rk[0], pv[0], rq[1], rk[1], pv[1], per_head, scale)[0]
    ro, rl = oracle.causal_attention(*dec, scale)
    check(f"rotated d={d}", "fp8", g.o, ro, g.lse, rl, fp8_path="exact",
          ref_abs_o=abs_v(oracle.causal_attention, *dec, scale))
    # Against the unrotated float32 inputs: the rotation is orthogonal, so what is left
    # is the quantisation error of Q, K and V.
    fo, _ = oracle.causal_attention(q, k, v, scale)
    err = rel_fro(g.o, fo)
    note(f"  rel-Fro error against the unrotated float32 inputs: {err:.4f}")
    assert err <= FP8_REL_FRO
