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
import json
import os
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

# Finer-grained FP8 output checks (beyond the whole-tensor figure):
# - relative Frobenius error of every (batch, head) slice, against the same 6e-2;
# - a per-element bound from how the probabilities are rounded.  On the exact path
#   (LSE requested) each probability is an e4m3 round-to-nearest of the exact one,
#   within a factor 1 +- 2^-4, and O is divided by the exact sum, so
#   |O_ic - O*_ic| <= 2^-4 * sum_j w_ij |v_jc|.  On the Lean P path (no LSE, or the
#   rounded-sum LSE) each code is within a factor [0.917, 1.061] of the exact
#   probability (test_oracle_formats.test_lean_code_ratio_bound) and O is divided by
#   the sum of the same rounded values, so every weight is off by at most a factor
#   1.061 / 0.917 and |O_ic - O*_ic| <= 0.157 * sum_j w_ij |v_jc|.  Added: the bf16
#   rounding of O (2^-8 relative), 0.01 * sum_j w_ij |v_jc| for the FP8 score error, and
#   2e-3 of the mean of sum_j w_ij |v_jc| for probabilities below e4m3's normal range.
#   sum_j w_ij |v_jc| is the oracle's attention with |V| in place of V (ref_abs_o);
# - a per-row relative error ||O_i - O*_i|| / ||O*_i|| <= 0.25.  Independent rounding
#   errors of the probabilities average to a few percent of ||O*_i|| in every row; an
#   output row that belongs to another query, head or key range is off by about
#   sqrt(2) and fails.
FP8_HEAD_REL_FRO = 6e-2
BF16_HEAD_REL_FRO = 1e-2
FP8_P_EPS = {"exact": 2.0 ** -4, "lean": 1.061 / 0.917 - 1.0}
FP8_SCORE_EPS = 0.01
FP8_ROW_REL = 0.25

# The LSE of the rounded-probability row sum (attn_fwd_causal_offset_fp8_rounded_lse):
# each rounded probability is within a factor [0.917, 1.061] of the exact one
# (test_oracle_formats.test_lean_code_ratio_bound derives it from the code rule), so the
# row sum and its log are within ln(1/0.917) = 0.0866 of the exact ones; plus 1e-2 for
# the scores.
ROUNDED_LSE_BOUND = 0.0866 + 1e-2


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


def _same(a, b) -> bool:
    """Byte equality of two device tensors (NaN payloads included)."""
    if a is None:
        return b is None
    return bool(torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                            b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)))


def _repeat(launch, B, N, Hq, dv, want_lse, repeats, what):
    """Runs `launch(o, lse)` `repeats` times into fresh NaN-filled buffers; every run
    after the first must give byte-identical O and LSE (compared on the device, stopping
    at the first mismatch).  Returns [the first run's outputs]."""
    first = None
    for r in range(repeats):
        o = torch.full((B, N, Hq, dv), float("nan"), device=DEV, dtype=torch.bfloat16)
        lse = torch.full((B, Hq, N), float("nan"), device=DEV, dtype=torch.float32) if want_lse else None
        launch(o, lse)
        torch.cuda.synchronize()
        if first is None:
            first = (o, lse)
        else:
            assert _same(first[0], o) and _same(first[1], lse), \
                f"{what}: run {r} differs from run 0 (of {repeats} repeats)"
    if repeats > 1:
        note(f"  {what}: {repeats} runs byte-identical")
    return [_collect(*first)]


def run_bf16(qu, ku, vu, scale, want_lse=True, repeats=1):
    """Run the BF16 entry point on bf16 bytes; returns [outputs] (repeats > 1: every
    repeat checked byte-identical to the first)."""
    q, k, v = (to_dev_u16_as_bf16(a) for a in (qu, ku, vu))
    B, N, Hq, _ = qu.shape
    dv = vu.shape[3]
    return _repeat(lambda o, lse: ba.attn_fwd_causal_bf16(q, k, v, o, lse, softmax_scale=scale),
                   B, N, Hq, dv, want_lse, repeats, "bf16")


def gpu_quantize(x: np.ndarray, per_head: bool):
    """Quantise on the GPU with the library; returns device codes, device descale."""
    xd = torch.from_numpy(x).to(DEV)
    codes = torch.empty(x.shape, device=DEV, dtype=torch.uint8)
    ds = torch.empty((x.shape[2] if per_head else 1,), device=DEV, dtype=torch.float32)
    ba.quantize_e4m3(xd, codes, ds, per_head)
    torch.cuda.synchronize()
    return codes, ds


def run_fp8(qc, kc, vc, qd, kd, vd, per_head, scale, want_lse=True, repeats=1):
    """Run the FP8 entry point on device codes; returns [outputs] (repeats > 1: every
    repeat checked byte-identical to the first)."""
    B, N, Hq, _ = qc.shape
    dv = vc.shape[3]
    return _repeat(lambda o, lse: ba.attn_fwd_causal_fp8(qc, kc, vc, qd, kd, vd, o, lse,
                                                         softmax_scale=scale,
                                                         descale_per_head=int(per_head)),
                   B, N, Hq, dv, want_lse, repeats, "fp8" + ("" if want_lse else "/no-lse"))


def _collect(o, lse) -> GpuOut:
    oc = o.float().cpu().numpy().astype(np.float64)
    ob = o.view(torch.int16).cpu().numpy().tobytes()
    if lse is None:
        return GpuOut(oc, None, ob, None)
    lc = lse.cpu().numpy()
    return GpuOut(oc, lc.astype(np.float64), ob, lc.tobytes())


def rel_fro(a: np.ndarray, ref: np.ndarray) -> float:
    return float(np.linalg.norm((a - ref).ravel()) / np.linalg.norm(ref.ravel()))


class LseGateMiss(AssertionError):
    """The LSE error exceeds LSE_MAX_ABS (raised after every O check has passed, so an
    expected LSE miss cannot hide an O failure)."""


class ElemBoundMiss(AssertionError):
    """An FP8 output element is outside the per-element bound (whose score term assumes
    the scores are accurate to about 1e-2)."""


def _head_slices(o, row_heads):
    """(b, h) -> index of that head's rows: o is (B, N, Hq, dv), or (R, dv) with
    row_heads[r] = (b, h) of row r."""
    if o.ndim == 4:
        return {(b, h): (b, slice(None), h) for b in range(o.shape[0]) for h in range(o.shape[2])}
    groups: dict = {}
    for r, bh in enumerate(row_heads):
        groups.setdefault((int(bh[0]), int(bh[1])), []).append(r)
    return {bh: (np.array(idx),) for bh, idx in groups.items()}


def check(name: str, prec: str, o, ref_o, lse=None, ref_lse=None, *, ref_abs_o=None,
          fp8_path=None, row_heads=None) -> dict:
    """Compare with the tolerances for `prec`; returns the metrics, raises on failure.

    o / ref_o: (B, N, Hq, dv) outputs, or (R, dv) sampled rows with row_heads[r] = (b, h).
    FP8 needs ref_abs_o (the oracle's attention on |V|, same shape as ref_o) and
    fp8_path, "exact" (the LSE call) or "lean" (no LSE, or the rounded-sum LSE), which
    select the per-element bound above."""
    o = np.asarray(o)
    ref_o = np.asarray(ref_o)
    assert np.all(np.isfinite(o)), f"{name}: non-finite output"
    if o.ndim != 4 and row_heads is None:
        row_heads = [(0, 0)] * o.shape[0]
    m = {"rel_fro": rel_fro(o, ref_o), "max_abs": float(np.max(np.abs(o - ref_o)))}
    heads = {bh: rel_fro(o[ix], ref_o[ix]) for bh, ix in _head_slices(o, row_heads).items()}
    worst_head = max(heads, key=heads.get)
    m["head_rel_fro"] = heads[worst_head]
    flat, flat_ref = o.reshape(-1, o.shape[-1]), ref_o.reshape(-1, ref_o.shape[-1])
    row_err = np.linalg.norm(flat - flat_ref, axis=1) / np.maximum(
        np.linalg.norm(flat_ref, axis=1), 1e-30)
    m["row_rel"] = float(row_err.max())
    if lse is not None:
        assert np.all(np.isfinite(lse)), f"{name}: non-finite lse"
        m["lse_max_abs"] = float(np.max(np.abs(lse - ref_lse)))
    if prec != "bf16":
        assert fp8_path in FP8_P_EPS, f"{name}: fp8_path must be one of {list(FP8_P_EPS)}"
        assert ref_abs_o is not None, f"{name}: the FP8 element bound needs ref_abs_o"
        ra = np.asarray(ref_abs_o)
        tol = ((FP8_P_EPS[fp8_path] + FP8_SCORE_EPS) * ra + 2.0 ** -8 * np.abs(ref_o)
               + 2e-3 * float(np.mean(ra)))
        m["elem_err_over_bound"] = float(np.max(np.abs(o - ref_o) / tol))
    note(f"[{name} {prec}] " + " ".join(f"{k}={v:.3e}" for k, v in m.items()) +
         f" (worst head {worst_head}, worst row {int(np.argmax(row_err))})")
    if os.environ.get("ATTN_TEST_METRICS"):
        with open(os.environ["ATTN_TEST_METRICS"], "a") as f:
            f.write(json.dumps({"name": name, "prec": prec, "path": fp8_path, **m}) + "\n")
    if prec == "bf16":
        assert m["rel_fro"] <= BF16_REL_FRO, m
        assert m["max_abs"] <= BF16_MAX_ABS, m
        assert m["head_rel_fro"] <= BF16_HEAD_REL_FRO, m
    else:
        assert m["rel_fro"] <= FP8_REL_FRO, m
        assert m["head_rel_fro"] <= FP8_HEAD_REL_FRO, m
        assert m["row_rel"] <= FP8_ROW_REL, m
        if not m["elem_err_over_bound"] <= 1.0:
            raise ElemBoundMiss(f"{name}: {m}")
    if lse is not None and not m["lse_max_abs"] <= LSE_MAX_ABS:
        raise LseGateMiss(f"{name}: LSE max |error| {m['lse_max_abs']:.4f} > {LSE_MAX_ABS}")
    return m


def abs_v(fn, q, k, v, *args, **kw):
    """The oracle attention `fn` with |V| in place of V: sum_j w_ij |v_jc|, the scale of
    the FP8 per-element bound (same rows and shape as fn's O)."""
    return fn(q, k, np.abs(v), *args, **kw)[0]


def inputs(w: workloads.Workload):
    return workloads.generate(w)

