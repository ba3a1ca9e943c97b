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
           "quantize_e4m3", "attn_status_string", "LIB_PATH", "EXPORTED_SYMBOLS"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")
EXPORTED_SYMBOLS = ("attn_fwd_causal_bf16", "attn_fwd_causal_fp8", "quantize_e4m3",
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
    L.quantize_e4m3.argtypes = [vp, vp, vp, i, i, i, i, i, vp]
    L.quantize_e4m3.restype = i
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
