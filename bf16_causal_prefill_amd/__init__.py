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
           "attn_fwd_causal_fp8_qf32",
           "attn_fwd_causal_offset_bf16", "attn_fwd_causal_offset_fp8",
           "attn_fwd_causal_offset_fp8_rounded_lse", "attn_merge_partials",
           "quantize_e4m3", "quantize_e4m3_hadamard", "quantize_e4m3_q_pow2", "quantize_e4m3_qkv",
           "attn_status_string", "flash_attn_func", "quantize_e4m3_qk_outliers",
           "quantize_e4m3_qk_outliers_workspace_bytes", "attn_fwd_causal_fp8_outliers",
           "attn_fwd_causal_offset_fp8_outliers", "OUTLIER_CHANNELS",
           "quantize_e4m3_qk_outliers_noalloc", "NOALLOC_SCRATCH_WORDS",
           "LIB_PATH", "PHASE_TIMERS_LIB_PATH", "attn_phase_timers_set",
           "EXPORTED_SYMBOLS"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")
# The measurement build with phase timers (bf16_causal_prefill_amd.build --phase-timers).
PHASE_TIMERS_LIB_PATH = os.path.join(os.path.dirname(LIB_PATH), "libattn_phase_timers.so")
EXPORTED_SYMBOLS = ("attn_fwd_causal_bf16", "attn_fwd_causal_fp8",
                    "attn_fwd_causal_offset_bf16", "attn_fwd_causal_offset_fp8",
                    "attn_merge_partials", "quantize_e4m3", "quantize_e4m3_hadamard",
                    "attn_fwd_causal_offset_fp8_rounded_lse", "quantize_e4m3_q_pow2",
                    "attn_status_string", "quantize_e4m3_qk_outliers",
                    "quantize_e4m3_qk_outliers_workspace_bytes", "attn_fwd_causal_fp8_outliers",
                    "attn_fwd_causal_offset_fp8_outliers",
                    "quantize_e4m3_qk_outliers_noalloc", "quantize_e4m3_qkv",
                    "attn_fwd_causal_fp8_qf32")

# Channels per Q/K row that the *_outliers entry points multiply exactly (stored last).
OUTLIER_CHANNELS = 32
# 32-bit words of the fixed scratch of quantize_e4m3_qk_outliers_noalloc.
NOALLOC_SCRATCH_WORDS = 65536

ATTN_OK = 0
ATTN_E_INVAL = -1
ATTN_E_UNSUPPORTED = -2
ATTN_E_ALIGN = -3
ATTN_E_NODEVICE = -4
ATTN_E_LAUNCH = -5
ATTN_E_TOO_LARGE = -6

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
    L.attn_fwd_causal_fp8_qf32.argtypes = L.attn_fwd_causal_fp8.argtypes
    L.attn_fwd_causal_fp8_qf32.restype = i
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
    L.quantize_e4m3_qkv.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i,
                                    i, f, vp]
    L.quantize_e4m3_qkv.restype = i
    L.quantize_e4m3_hadamard.argtypes = [vp, vp, vp, i, i, i, i, i, vp]
    L.quantize_e4m3_hadamard.restype = i
    L.quantize_e4m3_qk_outliers.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                            ctypes.c_size_t, i, i, i, i, i, i, i, f, vp]
    L.quantize_e4m3_qk_outliers.restype = i
    L.quantize_e4m3_qk_outliers_workspace_bytes.argtypes = [i, i, i]
    L.quantize_e4m3_qk_outliers_workspace_bytes.restype = ctypes.c_size_t
    L.quantize_e4m3_qk_outliers_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                                    i, i, i, i, i, i, i, f, vp]
    L.quantize_e4m3_qk_outliers_noalloc.restype = i
    L.attn_fwd_causal_fp8_outliers.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, vp, vp,
                                               i, i, i, i, i, i, f, vp]
    L.attn_fwd_causal_fp8_outliers.restype = i
    L.attn_fwd_causal_offset_fp8_outliers.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, vp,
                                                      vp, i, i, i, i, i, i, i, i, f, vp]
    L.attn_fwd_causal_offset_fp8_outliers.restype = i
    L.attn_status_string.argtypes = [i]
    L.attn_status_string.restype = ctypes.c_char_p
    if hasattr(L, "attn_phase_timers_set"):          # the measurement build only
        L.attn_phase_timers_set.argtypes = [vp, ctypes.c_size_t]
        L.attn_phase_timers_set.restype = i
    _lib = L
    return L


def attn_phase_timers_set(buf=None) -> None:
    """Measurement build (PHASE_TIMERS_LIB_PATH loaded first) only: record the attention
    kernels' phase timers into buf, a contiguous int64 CUDA tensor (8 waves x 10 words
    per recorded workgroup, include/attn_phase_timers.h), or stop with None."""
    L = load_library()
    if not hasattr(L, "attn_phase_timers_set"):
        raise RuntimeError("the loaded library is not the phase-timer build")
    if buf is not None:
        import torch
        if not (buf.is_cuda and buf.dtype == torch.int64 and buf.is_contiguous()):
            raise ValueError("buf must be a contiguous int64 CUDA tensor")
    nbytes = 0 if buf is None else buf.numel() * 8
    _check(L.attn_phase_timers_set(_ptr(buf), nbytes), "attn_phase_timers_set")


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


# ---- argument checks -----------------------------------------------------------------
# Every wrapper checks dtypes, shapes, devices and contiguity before the library is
# called, so a tensor that does not match what the kernels will index (a K/V with fewer
# rows than Q, a descale with fewer values than heads, an output of the wrong size) is
# reported as ValueError instead of being read or written past its end on the device.
# Shapes and dtypes are checked first, then the device and the memory layout.

def _dtypes(kind):
    import torch
    if kind == "bf16":
        return (torch.bfloat16,)
    if kind == "e4m3":
        return (torch.uint8,) + ((torch.float8_e4m3fn,) if hasattr(torch, "float8_e4m3fn") else ())
    return (torch.float32,)


def _want(t, name, kind, shape):
    """t must be a tensor of one of `kind`'s dtypes with exactly `shape`."""
    if t is None:
        raise ValueError(f"{name} is required")
    if not hasattr(t, "data_ptr") or not hasattr(t, "shape"):
        raise ValueError(f"{name} must be a torch tensor")
    if t.dtype not in _dtypes(kind):
        raise ValueError(f"{name}: dtype {t.dtype}, expected {kind}")
    if tuple(int(x) for x in t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")


def _on_gpu(device, **tensors):
    """Every given tensor is a contiguous tensor on `device` (a CUDA/HIP device)."""
    for name, t in tensors.items():
        if t is None:
            continue
        if not getattr(t, "is_cuda", False):
            raise ValueError(f"{name} must be a GPU tensor")
        if device is not None and t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def _rank4(t, name):
    if t is None or not hasattr(t, "shape") or len(t.shape) != 4:
        raise ValueError(f"{name} must be a 4-d (B, N, H, d) tensor")
    return tuple(int(x) for x in t.shape)


def _attn_shapes(q, k, v, kind, same_n, q_kind=None):
    """(B, Hq, Hkv, Nq, Nk, dqk, dv) of q (B,Nq,Hq,dqk), k (B,Nk,Hkv,dqk), v (B,Nk,Hkv,dv);
    q of dtype q_kind when given, else kind."""
    B, Nq, Hq, dqk = _rank4(q, "q")
    _, Nk, Hkv, _ = _rank4(k, "k")
    dv = _rank4(v, "v")[3]
    _want(q, "q", q_kind or kind, (B, Nq, Hq, dqk))
    _want(k, "k", kind, (B, Nk, Hkv, dqk))
    _want(v, "v", kind, (B, Nk, Hkv, dv))
    if same_n and Nk != Nq:
        raise ValueError(f"k/v have {Nk} rows, q has {Nq}")
    if Hkv < 1 or Hq % Hkv:
        raise ValueError(f"Hq={Hq} is not a multiple of Hkv={Hkv}")
    return B, Hq, Hkv, Nq, Nk, dqk, dv


def _outputs(o, lse, B, Nq, Hq, dv, lse_required=False):
    _want(o, "o", "bf16", (B, Nq, Hq, dv))
    if lse is not None or lse_required:
        _want(lse, "lse", "f32", (B, Hq, Nq))


def _descales(q_descale, k_descale, v_descale, Hq, Hkv, per_head):
    """Per-head choice (inferred from the sizes when per_head is None) and the check that
    all three descales hold 1 value (per tensor) or Hq / Hkv / Hkv values (per head)."""
    for n, t in (("q_descale", q_descale), ("k_descale", k_descale), ("v_descale", v_descale)):
        if t is None or not hasattr(t, "numel"):
            raise ValueError(f"{n} is required")
        if t.dtype not in _dtypes("f32"):
            raise ValueError(f"{n}: dtype {t.dtype}, expected float32")
    if per_head is None:
        per_head = int(q_descale.numel() > 1 or k_descale.numel() > 1 or v_descale.numel() > 1)
    per_head = int(bool(per_head))
    want = (Hq, Hkv, Hkv) if per_head else (1, 1, 1)
    got = (q_descale.numel(), k_descale.numel(), v_descale.numel())
    if got != want:
        raise ValueError(f"descales hold {got} values, expected {want} "
                         f"(per {'head' if per_head else 'tensor'})")
    return per_head


def attn_fwd_causal_bf16(q, k, v, o, lse=None, softmax_scale=None, stream=None) -> None:
    """q (B,N,Hq,dqk), k (B,N,Hkv,dqk), v (B,N,Hkv,dv) bf16 -> o (B,N,Hq,dv) bf16,
    lse (B,Hq,N) float32 or None.  Tensors must be contiguous on the GPU."""
    B, Hq, Hkv, N, _, dqk, dv = _attn_shapes(q, k, v, "bf16", same_n=True)
    _outputs(o, lse, B, N, Hq, dv)
    _on_gpu(q.device, q=q, k=k, v=v, o=o, lse=lse)
    scale = 1.0 / math.sqrt(dqk) if softmax_scale is None else float(softmax_scale)
    st = load_library().attn_fwd_causal_bf16(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                             B, Hq, Hkv, N, dqk, dv, scale, _stream(stream))
    _check(st, "attn_fwd_causal_bf16")


def attn_fwd_causal_fp8(q, k, v, q_descale, k_descale, v_descale, o, lse=None,
                        softmax_scale=None, descale_per_head=None, stream=None) -> None:
    """q/k/v uint8 e4m3fn codes; *_descale float32 device tensors of 1 element
    (per tensor) or Hq / Hkv elements (per head)."""
    B, Hq, Hkv, N, _, dqk, dv = _attn_shapes(q, k, v, "e4m3", same_n=True)
    _outputs(o, lse, B, N, Hq, dv)
    descale_per_head = _descales(q_descale, k_descale, v_descale, Hq, Hkv, descale_per_head)
    _on_gpu(q.device, q=q, k=k, v=v, o=o, lse=lse, q_descale=q_descale, k_descale=k_descale,
            v_descale=v_descale)
    scale = 1.0 / math.sqrt(dqk) if softmax_scale is None else float(softmax_scale)
    st = load_library().attn_fwd_causal_fp8(
        _ptr(q), _ptr(k), _ptr(v), _ptr(q_descale), _ptr(k_descale), _ptr(v_descale),
        int(descale_per_head), _ptr(o), _ptr(lse), B, Hq, Hkv, N, dqk, dv, scale,
        _stream(stream))
    _check(st, "attn_fwd_causal_fp8")


def attn_fwd_causal_fp8_qf32(q, k, v, q_descale, k_descale, v_descale, o, lse=None,
                             softmax_scale=None, descale_per_head=None, stream=None) -> None:
    """attn_fwd_causal_fp8 with q float32 (B,N,Hq,dqk), encoded by the kernel with
    q_descale exactly as quantize_e4m3 / quantize_e4m3_q_pow2 encode it (outputs
    byte-identical to quantising q and calling attn_fwd_causal_fp8); k, v e4m3 codes."""
    B, Hq, Hkv, N, _, dqk, dv = _attn_shapes(q, k, v, "e4m3", same_n=True, q_kind="f32")
    _outputs(o, lse, B, N, Hq, dv)
    descale_per_head = _descales(q_descale, k_descale, v_descale, Hq, Hkv, descale_per_head)
    _on_gpu(q.device, q=q, k=k, v=v, o=o, lse=lse, q_descale=q_descale, k_descale=k_descale,
            v_descale=v_descale)
    scale = 1.0 / math.sqrt(dqk) if softmax_scale is None else float(softmax_scale)
    st = load_library().attn_fwd_causal_fp8_qf32(
        _ptr(q), _ptr(k), _ptr(v), _ptr(q_descale), _ptr(k_descale), _ptr(v_descale),
        int(descale_per_head), _ptr(o), _ptr(lse), B, Hq, Hkv, N, dqk, dv, scale,
        _stream(stream))
    _check(st, "attn_fwd_causal_fp8_qf32")


def _quant_args(x, out, descale, per_head, k_descale=None):
    """Checks of the quantisers' arguments (k_descale: quantize_e4m3_q_pow2's);
    returns (B, N, H, d, Hkv)."""
    B, N, H, d = _rank4(x, "x")
    _want(x, "x", "f32", (B, N, H, d))
    _want(out, "out", "e4m3", (B, N, H, d))
    _want(descale, "descale", "f32", (H if per_head else 1,))
    Hkv = 1
    if k_descale is not None:
        if not hasattr(k_descale, "numel") or k_descale.dtype not in _dtypes("f32"):
            raise ValueError("k_descale must be a float32 tensor")
        Hkv = int(k_descale.numel()) if per_head else 1
        if not per_head and k_descale.numel() != 1:
            raise ValueError("k_descale must hold 1 value with per-tensor scales")
        if Hkv < 1 or H % Hkv:
            raise ValueError(f"H={H} is not a multiple of the {Hkv} KV-head descales")
    _on_gpu(x.device, x=x, out=out, descale=descale, k_descale=k_descale)
    return B, N, H, d, Hkv


def quantize_e4m3(x, out, descale, per_head: bool, stream=None) -> None:
    """x float32 (B,N,H,d) -> out uint8 codes, descale float32 (H,) or (1,)."""
    B, N, H, d, _ = _quant_args(x, out, descale, per_head)
    st = load_library().quantize_e4m3(_ptr(x), _ptr(out), _ptr(descale), B, N, H, d,
                                      int(bool(per_head)), _stream(stream))
    _check(st, "quantize_e4m3")


def quantize_e4m3_q_pow2(x, out, descale, k_descale, softmax_scale: float, per_head: bool,
                         stream=None) -> None:
    """quantize_e4m3 of Q with the descale that makes the FP8 softmax constant (with K's
    descales k_descale, (Hkv,) or (1,)) a power of two."""
    if k_descale is None:
        raise ValueError("k_descale is required")
    B, N, H, d, Hkv = _quant_args(x, out, descale, per_head, k_descale)
    st = load_library().quantize_e4m3_q_pow2(_ptr(x), _ptr(out), _ptr(descale), B, N, H, d,
                                             int(bool(per_head)), _ptr(k_descale), Hkv,
                                             float(softmax_scale), _stream(stream))
    _check(st, "quantize_e4m3_q_pow2")


def quantize_e4m3_qkv(q, k, v, q_out, k_out, v_out, q_descale, k_descale, v_descale,
                      per_head: bool, q_pow2: bool = False, softmax_scale=None,
                      stream=None) -> None:
    """Q, K and V in one call (four kernels): K and V as quantize_e4m3, Q as
    quantize_e4m3_q_pow2 against K's descales (q_pow2) or as quantize_e4m3; codes and
    descales bit-identical to those calls (q_out None: Q's descales only, for
    attn_fwd_causal_fp8_qf32).  q (B,Nq,Hq,dqk), k (B,Nk,Hkv,dqk),
    v (B,Nk,Hkv,dv) float32; outputs uint8 of the same shapes and float32 descales of
    (Hq,) / (Hkv,) / (Hkv,) values (per_head) or (1,)."""
    B, Nq, Hq, dqk = _rank4(q, "q")
    _, Nk, Hkv, _ = _rank4(k, "k")
    dv = _rank4(v, "v")[3]
    _want(q, "q", "f32", (B, Nq, Hq, dqk))
    _want(k, "k", "f32", (B, Nk, Hkv, dqk))
    _want(v, "v", "f32", (B, Nk, Hkv, dv))
    if q_out is not None:
        _want(q_out, "q_out", "e4m3", (B, Nq, Hq, dqk))
    _want(k_out, "k_out", "e4m3", (B, Nk, Hkv, dqk))
    _want(v_out, "v_out", "e4m3", (B, Nk, Hkv, dv))
    _want(q_descale, "q_descale", "f32", (Hq if per_head else 1,))
    _want(k_descale, "k_descale", "f32", (Hkv if per_head else 1,))
    _want(v_descale, "v_descale", "f32", (Hkv if per_head else 1,))
    if q_pow2 and per_head and Hq % Hkv:
        raise ValueError(f"Hq={Hq} is not a multiple of Hkv={Hkv}")
    _on_gpu(q.device, q=q, k=k, v=v, q_out=q_out, k_out=k_out, v_out=v_out,
            q_descale=q_descale, k_descale=k_descale, v_descale=v_descale)
    scale = 1.0 / math.sqrt(dqk) if softmax_scale is None else float(softmax_scale)
    st = load_library().quantize_e4m3_qkv(
        _ptr(q), _ptr(k), _ptr(v), _ptr(q_out), _ptr(k_out), _ptr(v_out), _ptr(q_descale),
        _ptr(k_descale), _ptr(v_descale), B, Nq, Nk, Hq, Hkv, dqk, dv, int(bool(per_head)),
        int(bool(q_pow2)), scale, _stream(stream))
    _check(st, "quantize_e4m3_qkv")


def quantize_e4m3_hadamard(x, out, descale, per_head: bool, stream=None) -> None:
    """quantize_e4m3 of x rotated by H/sqrt(hb) per block of hb channels (for Q and K);
    code * descale is the rotated value."""
    B, N, H, d, _ = _quant_args(x, out, descale, per_head)
    st = load_library().quantize_e4m3_hadamard(_ptr(x), _ptr(out), _ptr(descale), B, N, H, d,
                                               int(bool(per_head)), _stream(stream))
    _check(st, "quantize_e4m3_hadamard")


def attn_fwd_causal_offset_bf16(q, k, v, o, lse=None, q_offset=None, softmax_scale=None,
                                stream=None) -> None:
    """q (B,Nq,Hq,dqk), k (B,Nk,Hkv,dqk), v (B,Nk,Hkv,dv) bf16 -> o (B,Nq,Hq,dv) bf16,
    lse (B,Hq,Nq) float32 or None.  Key j is visible to query i iff j <= i + q_offset
    (default Nk - Nq: the queries are the last Nq of the Nk positions)."""
    B, Hq, Hkv, Nq, Nk, dqk, dv = _attn_shapes(q, k, v, "bf16", same_n=False)
    _outputs(o, lse, B, Nq, Hq, dv)
    _on_gpu(q.device, q=q, k=k, v=v, o=o, lse=lse)
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
    B, Hq, Hkv, Nq, Nk, dqk, dv = _attn_shapes(q, k, v, "e4m3", same_n=False)
    _outputs(o, lse, B, Nq, Hq, dv, lse_required=False)
    descale_per_head = _descales(q_descale, k_descale, v_descale, Hq, Hkv, descale_per_head)
    _on_gpu(q.device, q=q, k=k, v=v, o=o, lse=lse, q_descale=q_descale, k_descale=k_descale,
            v_descale=v_descale)
    off = Nk - Nq if q_offset is None else int(q_offset)
    scale = 1.0 / math.sqrt(dqk) if softmax_scale is None else float(softmax_scale)
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
    B, Hq, Hkv, Nq, Nk, dqk, dv = _attn_shapes(q, k, v, "e4m3", same_n=False)
    _outputs(o, lse, B, Nq, Hq, dv, lse_required=True)
    descale_per_head = _descales(q_descale, k_descale, v_descale, Hq, Hkv, descale_per_head)
    _on_gpu(q.device, q=q, k=k, v=v, o=o, lse=lse, q_descale=q_descale, k_descale=k_descale,
            v_descale=v_descale)
    off = Nk - Nq if q_offset is None else int(q_offset)
    scale = 1.0 / math.sqrt(dqk) if softmax_scale is None else float(softmax_scale)
    st = load_library().attn_fwd_causal_offset_fp8_rounded_lse(
        _ptr(q), _ptr(k), _ptr(v), _ptr(q_descale), _ptr(k_descale), _ptr(v_descale),
        int(descale_per_head), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, off, dqk, dv, scale,
        _stream(stream))
    _check(st, "attn_fwd_causal_offset_fp8_rounded_lse")


def _exact_args(q_exact, k_exact, B, Nq, Nk, Hq, Hkv):
    _want(q_exact, "q_exact", "bf16", (B, Nq, Hq, OUTLIER_CHANNELS))
    _want(k_exact, "k_exact", "bf16", (B, Nk, Hkv, OUTLIER_CHANNELS))


def attn_fwd_causal_fp8_outliers(q, k, v, q_exact, k_exact, q_descale, k_descale, v_descale, o,
                                 lse=None, softmax_scale=None, descale_per_head=None,
                                 stream=None) -> None:
    """attn_fwd_causal_fp8 with the last OUTLIER_CHANNELS channels of every Q and K row
    taken from the bf16 side arrays q_exact (B,N,Hq,32) / k_exact (B,N,Hkv,32) and
    multiplied exactly (the outputs of quantize_e4m3_qk_outliers); d_qk must be 128."""
    B, Hq, Hkv, N, _, dqk, dv = _attn_shapes(q, k, v, "e4m3", same_n=True)
    _outputs(o, lse, B, N, Hq, dv)
    _exact_args(q_exact, k_exact, B, N, N, Hq, Hkv)
    descale_per_head = _descales(q_descale, k_descale, v_descale, Hq, Hkv, descale_per_head)
    _on_gpu(q.device, q=q, k=k, v=v, o=o, lse=lse, q_descale=q_descale, k_descale=k_descale,
            v_descale=v_descale, q_exact=q_exact, k_exact=k_exact)
    scale = 1.0 / math.sqrt(dqk) if softmax_scale is None else float(softmax_scale)
    st = load_library().attn_fwd_causal_fp8_outliers(
        _ptr(q), _ptr(k), _ptr(v), _ptr(q_exact), _ptr(k_exact),
        _ptr(q_descale), _ptr(k_descale), _ptr(v_descale),
        int(descale_per_head), _ptr(o), _ptr(lse), B, Hq, Hkv, N, dqk, dv, scale,
        _stream(stream))
    _check(st, "attn_fwd_causal_fp8_outliers")


def attn_fwd_causal_offset_fp8_outliers(q, k, v, q_exact, k_exact, q_descale, k_descale,
                                        v_descale, o, lse=None, q_offset=None,
                                        softmax_scale=None, descale_per_head=None,
                                        stream=None) -> None:
    """attn_fwd_causal_offset_fp8 with the exact channels of attn_fwd_causal_fp8_outliers
    (q_exact (B,Nq,Hq,32), k_exact (B,Nk,Hkv,32))."""
    B, Hq, Hkv, Nq, Nk, dqk, dv = _attn_shapes(q, k, v, "e4m3", same_n=False)
    _outputs(o, lse, B, Nq, Hq, dv)
    _exact_args(q_exact, k_exact, B, Nq, Nk, Hq, Hkv)
    descale_per_head = _descales(q_descale, k_descale, v_descale, Hq, Hkv, descale_per_head)
    _on_gpu(q.device, q=q, k=k, v=v, o=o, lse=lse, q_descale=q_descale, k_descale=k_descale,
            v_descale=v_descale, q_exact=q_exact, k_exact=k_exact)
    off = Nk - Nq if q_offset is None else int(q_offset)
    scale = 1.0 / math.sqrt(dqk) if softmax_scale is None else float(softmax_scale)
    st = load_library().attn_fwd_causal_offset_fp8_outliers(
        _ptr(q), _ptr(k), _ptr(v), _ptr(q_exact), _ptr(k_exact),
        _ptr(q_descale), _ptr(k_descale), _ptr(v_descale),
        int(descale_per_head), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, off, dqk, dv, scale,
        _stream(stream))
    _check(st, "attn_fwd_causal_offset_fp8_outliers")


def quantize_e4m3_qk_outliers_workspace_bytes(Hq: int, Hkv: int, d: int) -> int:
    return int(load_library().quantize_e4m3_qk_outliers_workspace_bytes(int(Hq), int(Hkv), int(d)))


def quantize_e4m3_qk_outliers(q, k, q_out, k_out, q_exact, k_exact, q_descale, k_descale, perm,
                              per_head: bool, q_pow2: bool = False, softmax_scale=None,
                              workspace=None, stream=None) -> None:
    """Joint e4m3 quantisation of q (B,N,Hq,d) and k (B,N,Hkv,d) float32 with each KV head's
    OUTLIER_CHANNELS largest-product channels stored last: q_out/k_out uint8 codes,
    q_exact (B,N,Hq,32) / k_exact (B,N,Hkv,32) bf16 side arrays of those last channels
    (x / descale), q_descale (Hq,)/(1,), k_descale (Hkv,)/(1,), perm uint8 (Hkv, d).  With q_pow2, Q's
    descale makes the FP8 softmax constant a power of two (softmax_scale, default
    1/sqrt(d)).  workspace: a device buffer of at least
    quantize_e4m3_qk_outliers_workspace_bytes(Hq, Hkv, d) bytes (allocated here when None)."""
    B, N, Hq, Hkv, d = _outlier_quant_args(q, k, q_out, k_out, q_exact, k_exact, q_descale,
                                           k_descale, perm, per_head)
    _on_gpu(q.device, workspace=workspace)
    need = quantize_e4m3_qk_outliers_workspace_bytes(Hq, Hkv, d)
    if workspace is None:
        import torch
        workspace = torch.empty(max(need, 4), dtype=torch.uint8, device=q.device)
    nbytes = int(workspace.numel() * workspace.element_size())
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    st = load_library().quantize_e4m3_qk_outliers(
        _ptr(q), _ptr(k), _ptr(q_out), _ptr(k_out), _ptr(q_exact), _ptr(k_exact),
        _ptr(q_descale), _ptr(k_descale), _ptr(perm), _ptr(workspace), nbytes, B, N, Hq, Hkv, d, int(bool(per_head)), int(bool(q_pow2)),
        scale, _stream(stream))
    _check(st, "quantize_e4m3_qk_outliers")


def quantize_e4m3_qk_outliers_noalloc(q, k, q_out, k_out, q_exact, k_exact, q_descale,
                                      k_descale, perm, per_head: bool, q_pow2: bool = False,
                                      softmax_scale=None, stream=None) -> None:
    """quantize_e4m3_qk_outliers with the library's fixed per-device scratch instead of a
    workspace (nothing is allocated; (Hq + Hkv) * d <= NOALLOC_SCRATCH_WORDS; calls that
    overlap on one GPU race)."""
    B, N, Hq, Hkv, d = _outlier_quant_args(q, k, q_out, k_out, q_exact, k_exact, q_descale,
                                           k_descale, perm, per_head)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    st = load_library().quantize_e4m3_qk_outliers_noalloc(
        _ptr(q), _ptr(k), _ptr(q_out), _ptr(k_out), _ptr(q_exact), _ptr(k_exact),
        _ptr(q_descale), _ptr(k_descale), _ptr(perm),
        B, N, Hq, Hkv, d, int(bool(per_head)), int(bool(q_pow2)), scale, _stream(stream))
    _check(st, "quantize_e4m3_qk_outliers_noalloc")


def _outlier_quant_args(q, k, q_out, k_out, q_exact, k_exact, q_descale, k_descale, perm,
                        per_head):
    """Checks of the joint quantisers' arguments; returns (B, N, Hq, Hkv, d)."""
    B, N, Hq, d = _rank4(q, "q")
    Hkv = _rank4(k, "k")[2]
    _want(q, "q", "f32", (B, N, Hq, d))
    _want(k, "k", "f32", (B, N, Hkv, d))
    _want(q_out, "q_out", "e4m3", (B, N, Hq, d))
    _want(k_out, "k_out", "e4m3", (B, N, Hkv, d))
    _exact_args(q_exact, k_exact, B, N, N, Hq, Hkv)
    _want(q_descale, "q_descale", "f32", (Hq if per_head else 1,))
    _want(k_descale, "k_descale", "f32", (Hkv if per_head else 1,))
    if perm is None or getattr(perm, "dtype", None) is None or str(perm.dtype) != "torch.uint8" \
            or tuple(perm.shape) != (Hkv, d):
        raise ValueError(f"perm must be a uint8 tensor of shape {(Hkv, d)}")
    if Hkv < 1 or Hq % Hkv:
        raise ValueError(f"Hq={Hq} is not a multiple of Hkv={Hkv}")
    _on_gpu(q.device, q=q, k=k, q_out=q_out, k_out=k_out, q_exact=q_exact, k_exact=k_exact,
            q_descale=q_descale, k_descale=k_descale, perm=perm)
    return B, N, Hq, Hkv, d


def attn_merge_partials(o_a, lse_a, o_b, lse_b, o, lse=None, stream=None) -> None:
    """Merge two partial attentions (bf16 o (B,N,Hq,dv), float32 lse (B,Hq,N)) of the
    same queries over disjoint key sets into o / lse (which may alias the inputs)."""
    B, N, Hq, dv = _rank4(o_a, "o_a")
    for n, t in (("o_a", o_a), ("o_b", o_b), ("o", o)):
        _want(t, n, "bf16", (B, N, Hq, dv))
    for n, t in (("lse_a", lse_a), ("lse_b", lse_b)) + ((("lse", lse),) if lse is not None else ()):
        _want(t, n, "f32", (B, Hq, N))
    _on_gpu(o_a.device, o_a=o_a, lse_a=lse_a, o_b=o_b, lse_b=lse_b, o=o, lse=lse)
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
