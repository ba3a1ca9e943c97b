"""Shared plumbing of the GPU parity tests: build inputs, run the HIP path
through the C ABI, run the oracle on the same bytes, compare.

Independence: the HIP path sees only device tensors; the oracle sees only host
numpy arrays.  For BF16 both consume the same bf16 bytes (torch's CPU cast of
the float32 draw).  For FP8 each side quantises the float32 draw itself (the
library's quantize_e4m3 on the GPU, oracle.quantize_e4m3 on the CPU); the
tests require those codes and descales to be bit-identical, so both attention
computations then run on the same e4m3 inputs.
"""
from __future__ import annotations

import dataclasses
import sys

import numpy as np
import torch

import bf16_causal_prefill_amd as ba
import oracle
import workloads

DEV = "cuda:0"

# Tolerances (the numeric contract of the path).
BF16_REL_FRO = 1e-2
BF16_MAX_ABS = 2e-2
FP8_REL_FRO = 6e-2
LSE_MAX_ABS = 1e-2

# The gfx950 FP8 matrix instructions add the products of each run of 8 consecutive
# k-elements after aligning them to the largest one's exponent, keeping at least
# FP8_ALIGN_BITS fraction bits below it and truncating the rest (measured through the
# C ABI in test_fp8_matrix_accumulation_model).  One score q.k then differs from the
# exact sum by less than 7 * 2^-FP8_ALIGN_BITS * max|q_c k_c| per group of 8 channels.
FP8_ALIGN_BITS = 12


def fp8_score_error_bound(q_dec, k_dec, scale: float, rows) -> np.ndarray:
    """Worst-case |LSE_i - exact| from the grouped accumulation of the FP8 Q.K^T
    products, for each (b, h, i) in rows: scale * max_{j<=i} sum over 8-channel
    groups of 7 * 2^-12 * max_c |q_ic k_jc|.  LSE is 1-Lipschitz in the max norm of
    the scores, so this bounds the LSE error the accumulation alone can cause."""
    Hq, Hkv = q_dec.shape[2], k_dec.shape[2]
    out = np.empty(len(rows))
    for r, (b, h, i) in enumerate(rows):
        g = h // (Hq // Hkv)
        prod = np.abs(np.asarray(q_dec[b, i, h, :], dtype=np.float64)[None, :] *
                      np.asarray(k_dec[b, : i + 1, g, :], dtype=np.float64))
        d = prod.shape[1]
        grp = prod.reshape(i + 1, d // 8, 8).max(axis=2).sum(axis=1)
        out[r] = scale * 7.0 * 2.0 ** -FP8_ALIGN_BITS * float(grp.max())
    return out


def note(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def bf16_bytes(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), rounded by torch's CPU cast."""
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def to_dev_u16_as_bf16(u16: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(u16.view(np.int16)).to(DEV).view(torch.bfloat16)


@dataclasses.dataclass
class GpuOut:
    o: np.ndarray            # float64 (B, N, Hq, dv)
    lse: np.ndarray | None   # float64 (B, Hq, N)
    o_bytes: bytes
    lse_bytes: bytes | None


def run_bf16(qu, ku, vu, scale, want_lse=True, repeats=1):
    """Run the BF16 entry point on bf16 bytes; returns the list of outputs."""
    q, k, v = (to_dev_u16_as_bf16(a) for a in (qu, ku, vu))
    B, N, Hq, _ = qu.shape
    dv = vu.shape[3]
    outs = []
    for _ in range(repeats):
        o = torch.full((B, N, Hq, dv), float("nan"), device=DEV, dtype=torch.bfloat16)
        lse = torch.full((B, Hq, N), float("nan"), device=DEV, dtype=torch.float32) if want_lse else None
        ba.attn_fwd_causal_bf16(q, k, v, o, lse, softmax_scale=scale)
        torch.cuda.synchronize()
        outs.append(_collect(o, lse))
    return outs


def gpu_quantize(x: np.ndarray, per_head: bool):
    """Quantise on the GPU with the library; returns device codes, device descale."""
    xd = torch.from_numpy(x).to(DEV)
    codes = torch.empty(x.shape, device=DEV, dtype=torch.uint8)
    ds = torch.empty((x.shape[2] if per_head else 1,), device=DEV, dtype=torch.float32)
    ba.quantize_e4m3(xd, codes, ds, per_head)
    torch.cuda.synchronize()
    return codes, ds


def run_fp8(qc, kc, vc, qd, kd, vd, per_head, scale, want_lse=True, repeats=1):
    B, N, Hq, _ = qc.shape
    dv = vc.shape[3]
    outs = []
    for _ in range(repeats):
        o = torch.full((B, N, Hq, dv), float("nan"), device=DEV, dtype=torch.bfloat16)
        lse = torch.full((B, Hq, N), float("nan"), device=DEV, dtype=torch.float32) if want_lse else None
        ba.attn_fwd_causal_fp8(qc, kc, vc, qd, kd, vd, o, lse, softmax_scale=scale,
                               descale_per_head=int(per_head))
        torch.cuda.synchronize()
        outs.append(_collect(o, lse))
    return outs


def _collect(o, lse) -> GpuOut:
    oc = o.float().cpu().numpy().astype(np.float64)
    ob = o.view(torch.int16).cpu().numpy().tobytes()
    if lse is None:
        return GpuOut(oc, None, ob, None)
    lc = lse.cpu().numpy()
    return GpuOut(oc, lc.astype(np.float64), ob, lc.tobytes())


def rel_fro(a: np.ndarray, ref: np.ndarray) -> float:
    return float(np.linalg.norm((a - ref).ravel()) / np.linalg.norm(ref.ravel()))


def check(name: str, prec: str, o, ref_o, lse=None, ref_lse=None, lse_bound=None) -> dict:
    """Compare with the tolerances for `prec`; returns the metrics, raises on failure.

    lse_bound: optional callable mapping flat indices of lse (rows whose error
    exceeds LSE_MAX_ABS) to extra allowed error per row (fp8_score_error_bound);
    used only for FP8 on workloads with outlier channels, where the FP8 matrix
    instruction's accumulation alone can move the scores by more than 1e-2."""
    assert np.all(np.isfinite(o)), f"{name}: non-finite output"
    m = {"rel_fro": rel_fro(o, ref_o), "max_abs": float(np.max(np.abs(o - ref_o)))}
    if lse is not None:
        assert np.all(np.isfinite(lse)), f"{name}: non-finite lse"
        m["lse_max_abs"] = float(np.max(np.abs(lse - ref_lse)))
    note(f"[{name} {prec}] " + " ".join(f"{k}={v:.3e}" for k, v in m.items()))
    if prec == "bf16":
        assert m["rel_fro"] <= BF16_REL_FRO, m
        assert m["max_abs"] <= BF16_MAX_ABS, m
    else:
        assert m["rel_fro"] <= FP8_REL_FRO, m
    if lse is not None:
        err = np.abs(lse - ref_lse).ravel()
        over = np.nonzero(err > LSE_MAX_ABS)[0]
        if len(over) and lse_bound is not None:
            extra = lse_bound(over)
            m["lse_rows_over_1e-2"] = int(len(over))
            m["lse_worst_excess_over_bound"] = float(np.max(err[over] - LSE_MAX_ABS - extra))
            note(f"[{name} {prec}] {len(over)} rows above {LSE_MAX_ABS}: worst error "
                 f"{err[over].max():.3e}, largest allowed by the accumulation bound "
                 f"{(LSE_MAX_ABS + extra).max():.3e}")
            assert np.all(err[over] <= LSE_MAX_ABS + extra), m
        else:
            assert m["lse_max_abs"] <= LSE_MAX_ABS, m
    return m


def inputs(w: workloads.Workload):
    return workloads.generate(w)

