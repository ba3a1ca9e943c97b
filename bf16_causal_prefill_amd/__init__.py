"""Python binding of libattn (causal prefill attention for MI355X / gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/attn.h.  The functions take torch
tensors that already live on the GPU (torch provides device memory and the
stream), read their shapes and raw pointers, and call the entry point of the
same name.  A non-zero status raises AttnError.  If libattn.so has not been
built, loading raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = ["AttnError", "load_library", "attn_fwd_causal_bf16", "attn_fwd_causal_fp8",
           "attn_fwd_causal_offset_bf16", "attn_fwd_causal_offset_fp8",
           "attn_fwd_causal_offset_fp8_rounded_lse", "attn_merge_partials",
           "quantize_e4m3", "quantize_e4m3_hadamard", "quantize_e4m3_q_pow2",
           "attn_status_string", "flash_attn_func",
           "LIB_PATH",
           "EXPORTED_SYMBOLS"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")
EXPORTED_SYMBOLS = ("attn_fwd_causal_bf16", "attn_fwd_causal_fp8",
                    "attn_fwd_causal_offset_bf16", "attn_fwd_causal_offset_fp8",
                    "attn_merge_partials", "quantize_e4m3", "quantize_e4m3_hadamard",
                    "attn_fwd_causal_offset_fp8_rounded_lse", "quantize_e4m3_q_pow2",
                    "attn_status_string")

ATTN_OK = 0
ATTN_E_INVAL = -1
ATTN_E_UNSUPPORTED = -2
ATTN_E_ALIGN = -3
ATTN_E_NODEVICE = -4
ATTN_E_LAUNCH = -5

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {attn_status_string(status)} (status {status})")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libattn.so once and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m bf16_causal_prefill_amd.build`")
    L = ctypes.CDLL(path)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    L.attn_fwd_causal_bf16.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    L.attn_fwd_causal_bf16.restype = i
    L.attn_fwd_causal_fp8.argtypes = [vp, vp, vp, vp, vp, vp, i, vp, vp,
                                      i, i, i, i, i, i, f, vp]
    L.attn_fwd_causal_fp8.restype = i
    L.attn_fwd_causal_offset_bf16.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f,
                                              vp]
    L.attn_fwd_causal_offset_bf16.restype = i
    L.attn_fwd_causal_offset_fp8.argtypes = [vp, vp, vp, vp, vp, vp, i, vp, vp,
                                             i, i, i, i, i, i, i, i, f, vp]
    L.attn_fwd_causal_offset_fp8.restype = i
    L.attn_fwd_causal_offset_fp8_rounded_lse.argtypes = [vp, vp, vp, vp, vp, vp, i, vp, vp,
                                                         i, i, i, i, i, i, i, i, f, vp]
    L.attn_fwd_causal_offset_fp8_rounded_lse.restype = i
    L.attn_merge_partials.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, vp]
    L.attn_merge_partials.restype = i
    L.quantize_e4m3.argtypes = [vp, vp, vp, i, i, i, i, i, vp]
    L.quantize_e4m3_q_pow2.argtypes = [vp, vp, vp, i, i, i, i, i, vp, i, f, vp]
    L.quantize_e4m3_q_pow2.restype = i
    L.quantize_e4m3.restype = i
    L.quantize_e4m3_hadamard.argtypes = [vp, vp, vp, i, i, i, i, i, vp]
    L.quantize_e4m3_hadamard.restype = i
    L.attn_status_string.argtypes = [i]
    L.attn_status_string.restype = ctypes.c_char_p
    _lib = L
    return L


def attn_status_string(status: int) -> str:
    return load_library().attn_status_string(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(getattr(stream, "cuda_stream", stream))


def _check(status: int, where: str) -> None:
    if status != ATTN_OK:
        raise AttnError(status, where)


def _dims(q, k, v):
    B, N, Hq, dqk = q.shape
    Hkv = k.shape[2]
    dv = v.shape[3]
    return int(B), int(Hq), int(Hkv), int(N), int(dqk), int(dv)


def attn_fwd_causal_bf16(q, k, v, o, lse=None, softmax_scale=None, stream=None) -> None:
    """q (B,N,Hq,dqk), k (B,N,Hkv,dqk), v (B,N,Hkv,dv) bf16 -> o (B,N,Hq,dv) bf16,
    lse (B,Hq,N) float32 or None.  Tensors must be contiguous on the GPU."""
    B, Hq, Hkv, N, dqk, dv = _dims(q, k, v)
    scale = 1.0 / math.sqrt(dqk) if softmax_scale is None else float(softmax_scale)
    st = load_library().attn_fwd_causal_bf16(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                             B, Hq, Hkv, N, dqk, dv, scale, _stream(stream))
    _check(st, "attn_fwd_causal_bf16")


def attn_fwd_causal_fp8(q, k, v, q_descale, k_descale, v_descale, o, lse=None,
                        softmax_scale=None, descale_per_head=None, stream=None) -> None:
    """q/k/v uint8 e4m3fn codes; *_descale float32 device tensors of 1 element
    (per tensor) or Hq / Hkv elements (per head)."""
    B, Hq, Hkv, N, dqk, dv = _dims(q, k, v)
    scale = 1.0 / math.sqrt(dqk) if softmax_scale is None else float(softmax_scale)
    if descale_per_head is None:
        descale_per_head = int(q_descale.numel() > 1)
    st = load_library().attn_fwd_causal_fp8(
        _ptr(q), _ptr(k), _ptr(v), _ptr(q_descale), _ptr(k_descale), _ptr(v_descale),
        int(descale_per_head), _ptr(o), _ptr(lse), B, Hq, Hkv, N, dqk, dv, scale,
        _stream(stream))
    _check(st, "attn_fwd_causal_fp8")


def quantize_e4m3(x, out, descale, per_head: bool, stream=None) -> None:
    """x float32 (B,N,H,d) -> out uint8 codes, descale float32 (H,) or (1,)."""
    B, N, H, d = (int(s) for s in x.shape)
    st = load_library().quantize_e4m3(_ptr(x), _ptr(out), _ptr(descale), B, N, H, d,
                                      int(bool(per_head)), _stream(stream))
    _check(st, "quantize_e4m3")


def quantize_e4m3_q_pow2(x, out, descale, k_descale, softmax_scale: float, per_head: bool,
                         stream=None) -> None:
    """quantize_e4m3 of Q with the descale that makes the FP8 softmax constant (with K's
    descales k_descale, (Hkv,) or (1,)) a power of two."""
    B, N, H, d = (int(s) for s in x.shape)
    Hkv = int(k_descale.numel()) if per_head else 1
    st = load_library().quantize_e4m3_q_pow2(_ptr(x), _ptr(out), _ptr(descale), B, N, H, d,
                                             int(bool(per_head)), _ptr(k_descale), Hkv,
                                             float(softmax_scale), _stream(stream))
    _check(st, "quantize_e4m3_q_pow2")


def quantize_e4m3_hadamard(x, out, descale, per_head: bool, stream=None) -> None:
    """quantize_e4m3 of x rotated by H/sqrt(hb) per block of hb channels (for Q and K);
    code * descale is the rotated value."""
    B, N, H, d = (int(s) for s in x.shape)
    st = load_library().quantize_e4m3_hadamard(_ptr(x), _ptr(out), _ptr(descale), B, N, H, d,
                                               int(bool(per_head)), _stream(stream))
    _check(st, "quantize_e4m3_hadamard")


def _dims_qk(q, k, v):
    B, Nq, Hq, dqk = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    dv = v.shape[3]
    return int(B), int(Hq), int(Hkv), int(Nq), int(Nk), int(dqk), int(dv)


def attn_fwd_causal_offset_bf16(q, k, v, o, lse=None, q_offset=None, softmax_scale=None,
                                stream=None) -> None:
    """q (B,Nq,Hq,dqk), k (B,Nk,Hkv,dqk), v (B,Nk,Hkv,dv) bf16 -> o (B,Nq,Hq,dv) bf16,
    lse (B,Hq,Nq) float32 or None.  Key j is visible to query i iff j <= i + q_offset
    (default Nk - Nq: the queries are the last Nq of the Nk positions)."""
    B, Hq, Hkv, Nq, Nk, dqk, dv = _dims_qk(q, k, v)
    off = Nk - Nq if q_offset is None else int(q_offset)
    scale = 1.0 / math.sqrt(dqk) if softmax_scale is None else float(softmax_scale)
    st = load_library().attn_fwd_causal_offset_bf16(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, off, dqk, dv, scale,
        _stream(stream))
    _check(st, "attn_fwd_causal_offset_bf16")


def attn_fwd_causal_offset_fp8(q, k, v, q_descale, k_descale, v_descale, o, lse=None,
                               q_offset=None, softmax_scale=None, descale_per_head=None,
                               stream=None) -> None:
    """FP8 codes version of attn_fwd_causal_offset_bf16 (descales as for
    attn_fwd_causal_fp8)."""
    B, Hq, Hkv, Nq, Nk, dqk, dv = _dims_qk(q, k, v)
    off = Nk - Nq if q_offset is None else int(q_offset)
    scale = 1.0 / math.sqrt(dqk) if softmax_scale is None else float(softmax_scale)
    if descale_per_head is None:
        descale_per_head = int(q_descale.numel() > 1)
    st = load_library().attn_fwd_causal_offset_fp8(
        _ptr(q), _ptr(k), _ptr(v), _ptr(q_descale), _ptr(k_descale), _ptr(v_descale),
        int(descale_per_head), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, off, dqk, dv, scale,
        _stream(stream))
    _check(st, "attn_fwd_causal_offset_fp8")


def attn_fwd_causal_offset_fp8_rounded_lse(q, k, v, q_descale, k_descale, v_descale, o, lse,
                                           q_offset=None, softmax_scale=None,
                                           descale_per_head=None, stream=None) -> None:
    """attn_fwd_causal_offset_fp8 on the rounded-probability path, also writing the LSE
    of the rounded row sum that normalises O (consistent with O, not the exact LSE)."""
    B, Hq, Hkv, Nq, Nk, dqk, dv = _dims_qk(q, k, v)
    off = Nk - Nq if q_offset is None else int(q_offset)
    scale = 1.0 / math.sqrt(dqk) if softmax_scale is None else float(softmax_scale)
    if descale_per_head is None:
        descale_per_head = int(q_descale.numel() > 1)
    st = load_library().attn_fwd_causal_offset_fp8_rounded_lse(
        _ptr(q), _ptr(k), _ptr(v), _ptr(q_descale), _ptr(k_descale), _ptr(v_descale),
        int(descale_per_head), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, off, dqk, dv, scale,
        _stream(stream))
    _check(st, "attn_fwd_causal_offset_fp8_rounded_lse")


def attn_merge_partials(o_a, lse_a, o_b, lse_b, o, lse=None, stream=None) -> None:
    """Merge two partial attentions (bf16 o (B,N,Hq,dv), float32 lse (B,Hq,N)) of the
    same queries over disjoint key sets into o / lse (which may alias the inputs)."""
    B, N, Hq, dv = (int(x) for x in o_a.shape)
    st = load_library().attn_merge_partials(_ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b),
                                            _ptr(o), _ptr(lse), B, N, Hq, dv, _stream(stream))
    _check(st, "attn_merge_partials")


def flash_attn_func(q, k, v, softmax_scale=None, causal=True, return_lse=False,
                    q_descale=None, k_descale=None, v_descale=None, stream=None):
    """flash_attn_func-style call: torch tensors in, a new o (B,Nq,Hq,dv) bf16 out (and
    lse (B,Hq,Nq) float32 when return_lse).  q (B,Nq,Hq,dqk), k (B,Nk,Hkv,dqk),
    v (B,Nk,Hkv,dv), contiguous on the GPU.  bf16 inputs run the BF16 kernel; e4m3fn
    inputs (torch.float8_e4m3fn or uint8 codes) run the FP8 kernel, with float32 descale
    tensors on the device (1 or H values each; default 1.0).  causal=True aligns the
    causal diagonal to the bottom-right when Nq != Nk (query i sees keys
    j <= i + Nk - Nq), causal=False lets every query see every key.  Only the output
    buffers are allocated here (by torch); all arithmetic runs in the library."""
    import torch
    for t in (q, k, v):
        if not (t.is_cuda and t.is_contiguous()):
            raise ValueError("flash_attn_func: q, k, v must be contiguous GPU tensors")
    B, Nq, Hq, _ = q.shape
    Nk, dv = k.shape[1], v.shape[3]
    off = (Nk - Nq) if causal else Nk
    if off < 0:
        raise ValueError("flash_attn_func: causal attention needs Nk >= Nq")
    o = torch.empty((B, Nq, Hq, dv), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device) if return_lse else None
    fp8_types = (torch.uint8,) + ((torch.float8_e4m3fn,) if hasattr(torch, "float8_e4m3fn") else ())
    if q.dtype == torch.bfloat16:
        attn_fwd_causal_offset_bf16(q, k, v, o, lse, q_offset=off, softmax_scale=softmax_scale,
                                    stream=stream)
    elif q.dtype in fp8_types:
        one = None
        if q_descale is None or k_descale is None or v_descale is None:
            one = torch.ones(1, dtype=torch.float32, device=q.device)
        qd = one if q_descale is None else q_descale
        kd = one if k_descale is None else k_descale
        vd = one if v_descale is None else v_descale
        Hkv = k.shape[2]
        per_head = int(qd.numel() > 1 or kd.numel() > 1 or vd.numel() > 1)
        want = (Hq, Hkv, Hkv) if per_head else (1, 1, 1)
        if (qd.numel(), kd.numel(), vd.numel()) != want:
            raise ValueError(f"flash_attn_func: descales need {want} elements "
                             f"(per {'head' if per_head else 'tensor'})")
        attn_fwd_causal_offset_fp8(q, k, v, qd, kd, vd, o, lse, q_offset=off,
                                   softmax_scale=softmax_scale, descale_per_head=per_head,
                                   stream=stream)
    else:
        raise TypeError(f"flash_attn_func: unsupported dtype {q.dtype}")
    return (o, lse) if return_lse else o
