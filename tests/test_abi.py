"""The C-ABI library: it loads, exports every entry point include/attn.h
declares, and rejects invalid arguments with the documented status codes
before touching a device (CPU only; no kernel is launched)."""
import ctypes
import os
import re

import pytest

import bf16_causal_prefill_amd as ba

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

A16 = 0x10000          # an aligned, never-dereferenced stand-in pointer value


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    lib = ba.load_library()
    declared = _declared_functions()
    assert set(declared) == set(ba.EXPORTED_SYMBOLS)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5):
        s = ba.attn_status_string(code)
        assert s and s != "unknown status"
    assert ba.attn_status_string(12345) == "unknown status"


def _bf16(lib, **kw):
    a = dict(q=A16, k=A16, v=A16, o=A16, lse=None, B=1, Hq=2, Hkv=2, N=16, dqk=128, dv=128,
             scale=0.1)
    a.update(kw)
    vp = ctypes.c_void_p
    return lib.attn_fwd_causal_bf16(vp(a["q"]), vp(a["k"]), vp(a["v"]), vp(a["o"]),
                                    vp(a["lse"]), a["B"], a["Hq"], a["Hkv"], a["N"],
                                    a["dqk"], a["dv"], a["scale"], None)


def _fp8(lib, **kw):
    a = dict(q=A16, k=A16, v=A16, qd=A16, kd=A16, vd=A16, ph=0, o=A16, lse=None, B=1, Hq=2,
             Hkv=2, N=16, dqk=128, dv=128, scale=0.1)
    a.update(kw)
    vp = ctypes.c_void_p
    return lib.attn_fwd_causal_fp8(vp(a["q"]), vp(a["k"]), vp(a["v"]), vp(a["qd"]),
                                   vp(a["kd"]), vp(a["vd"]), a["ph"], vp(a["o"]),
                                   vp(a["lse"]), a["B"], a["Hq"], a["Hkv"], a["N"],
                                   a["dqk"], a["dv"], a["scale"], None)


BAD_ARGS = [
    (dict(B=0), ba.ATTN_E_INVAL), (dict(N=0), ba.ATTN_E_INVAL), (dict(Hq=0), ba.ATTN_E_INVAL),
    (dict(Hkv=0), ba.ATTN_E_INVAL), (dict(Hq=6, Hkv=4), ba.ATTN_E_INVAL),
    (dict(scale=0.0), ba.ATTN_E_INVAL), (dict(scale=-1.0), ba.ATTN_E_INVAL),
    (dict(scale=float("nan")), ba.ATTN_E_INVAL), (dict(scale=float("inf")), ba.ATTN_E_INVAL),
    (dict(dqk=64, dv=64), ba.ATTN_E_UNSUPPORTED), (dict(dqk=192, dv=192), ba.ATTN_E_UNSUPPORTED),
    (dict(dqk=128, dv=192), ba.ATTN_E_UNSUPPORTED),
    (dict(q=None), ba.ATTN_E_INVAL), (dict(o=None), ba.ATTN_E_INVAL),
    (dict(q=A16 + 8), ba.ATTN_E_ALIGN), (dict(v=A16 + 2), ba.ATTN_E_ALIGN),
    (dict(lse=A16 + 2), ba.ATTN_E_ALIGN),
    (dict(B=1 << 20, N=1 << 20), ba.ATTN_E_INVAL),
]


@pytest.mark.parametrize("kw,code", BAD_ARGS, ids=[str(k) for k, _ in BAD_ARGS])
def test_bf16_rejects(kw, code):
    assert _bf16(ba.load_library(), **kw) == code


@pytest.mark.parametrize("kw,code", BAD_ARGS + [
    (dict(qd=None), ba.ATTN_E_INVAL), (dict(vd=None), ba.ATTN_E_INVAL),
    (dict(ph=2), ba.ATTN_E_INVAL), (dict(kd=A16 + 1), ba.ATTN_E_ALIGN)],
    ids=lambda x: str(x))
def test_fp8_rejects(kw, code):
    assert _fp8(ba.load_library(), **kw) == code


@pytest.mark.parametrize("name", ["quantize_e4m3", "quantize_e4m3_hadamard"])
def test_quantize_rejects(name):
    fn = getattr(ba.load_library(), name)
    vp = ctypes.c_void_p
    q = lambda x=A16, o=A16, d_=A16, B=1, N=4, H=2, d=8, ph=0: fn(
        vp(x), vp(o), vp(d_), B, N, H, d, ph, None)
    assert q(x=None) == ba.ATTN_E_INVAL
    assert q(d=6) == ba.ATTN_E_INVAL
    assert q(N=0) == ba.ATTN_E_INVAL
    assert q(ph=3) == ba.ATTN_E_INVAL
    assert q(H=70000) == ba.ATTN_E_INVAL
    assert q(x=A16 + 4) == ba.ATTN_E_ALIGN
    assert q(o=A16 + 1) == ba.ATTN_E_ALIGN


def test_quantize_q_pow2_rejects():
    fn = ba.load_library().quantize_e4m3_q_pow2
    vp = ctypes.c_void_p
    q = lambda x=A16, o=A16, d_=A16, B=1, N=4, H=4, d=8, ph=1, kd=A16, Hkv=2, s=0.1: fn(
        vp(x), vp(o), vp(d_), B, N, H, d, ph, vp(kd), Hkv, s, None)
    assert q(kd=None) == ba.ATTN_E_INVAL
    assert q(x=None) == ba.ATTN_E_INVAL
    assert q(d=6) == ba.ATTN_E_INVAL
    assert q(Hkv=0) == ba.ATTN_E_INVAL
    assert q(Hkv=3) == ba.ATTN_E_INVAL            # H % Hkv != 0 with per-head scales
    assert q(s=0.0) == ba.ATTN_E_INVAL
    assert q(s=float("nan")) == ba.ATTN_E_INVAL
    assert q(ph=2) == ba.ATTN_E_INVAL
    assert q(kd=A16 + 2) == ba.ATTN_E_ALIGN
    assert q(x=A16 + 4) == ba.ATTN_E_ALIGN


def _no_device():
    import torch
    return torch.cuda.device_count() == 0


@pytest.mark.skipif(not _no_device(), reason="only meaningful on a machine without a GPU")
def test_valid_call_without_device_reports_nodevice():
    lib = ba.load_library()
    assert _bf16(lib) == ba.ATTN_E_NODEVICE
    assert _fp8(lib) == ba.ATTN_E_NODEVICE
    assert lib.quantize_e4m3(ctypes.c_void_p(A16), ctypes.c_void_p(A16), ctypes.c_void_p(A16),
                             1, 4, 2, 8, 0, None) == ba.ATTN_E_NODEVICE
    assert lib.quantize_e4m3_hadamard(ctypes.c_void_p(A16), ctypes.c_void_p(A16),
                                      ctypes.c_void_p(A16), 1, 4, 2, 8, 0,
                                      None) == ba.ATTN_E_NODEVICE


def test_rounded_lse_entry_requires_lse_and_validates():
    """attn_fwd_causal_offset_fp8_rounded_lse rejects a NULL lse and bad arguments before
    touching a device."""
    lib = ba.load_library()
    vp = ctypes.c_void_p

    def call(lse=A16, B=1, q=A16, Nq=16, Nk=16, off=0, dqk=128):
        return lib.attn_fwd_causal_offset_fp8_rounded_lse(
            vp(q), vp(A16), vp(A16), vp(A16), vp(A16), vp(A16), 0, vp(A16), vp(lse), B, 2, 2,
            Nq, Nk, off, dqk, 128, ctypes.c_float(0.1), None)
    assert call(lse=None) == ba.ATTN_E_INVAL
    assert call(B=0) == ba.ATTN_E_INVAL
    assert call(off=-1) == ba.ATTN_E_INVAL
    assert call(q=None) == ba.ATTN_E_INVAL
    assert call(dqk=64) == ba.ATTN_E_UNSUPPORTED
    assert call(q=A16 + 4) == ba.ATTN_E_ALIGN
