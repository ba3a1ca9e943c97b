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


TIMERS_HEADER = os.path.join(ROOT, "include", "attn_phase_timers.h")


def _declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    lib = ba.load_library()
    declared = _declared_functions()
    assert set(declared) == set(ba.EXPORTED_SYMBOLS)
    for name in declared:
        assert hasattr(lib, name), name
    # the phase-timer entry point belongs to the measurement build only
    for name in _declared_functions(TIMERS_HEADER):
        assert not hasattr(lib, name), name


@pytest.mark.skipif(not os.path.exists(ba.PHASE_TIMERS_LIB_PATH),
                    reason="libattn_phase_timers.so not built (build.py --phase-timers)")
def test_phase_timer_build_exports_and_validates():
    """The measurement build exports include/attn.h's entry points plus
    include/attn_phase_timers.h's, and its setter checks alignment and size."""
    lib = ctypes.CDLL(ba.PHASE_TIMERS_LIB_PATH)
    declared = _declared_functions(TIMERS_HEADER)
    assert declared == ["attn_phase_timers_set"]
    for name in _declared_functions() + declared:
        assert hasattr(lib, name), name
    fn = lib.attn_phase_timers_set
    fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    fn.restype = ctypes.c_int
    assert fn(ctypes.c_void_p(A16 + 4), 4096) == ba.ATTN_E_ALIGN
    assert fn(ctypes.c_void_p(A16), 8 * 10 * 8 - 8) == ba.ATTN_E_INVAL
    assert fn(ctypes.c_void_p(A16), 8 * 10 * 8) == ba.ATTN_OK
    assert fn(None, 0) == ba.ATTN_OK


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5, -6):
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


def test_quantize_qkv_rejects():
    fn = ba.load_library().quantize_e4m3_qkv
    vp = ctypes.c_void_p

    def q(q=A16, k=A16, v=A16, qo=A16, ko=A16, vo=A16, qd=A16, kd=A16, vd=A16, B=1, Nq=4, Nk=4,
          Hq=4, Hkv=2, dqk=8, dv=8, ph=1, p2=1, s=0.1):
        return fn(vp(q), vp(k), vp(v), vp(qo), vp(ko), vp(vo), vp(qd), vp(kd), vp(vd), B, Nq, Nk,
                  Hq, Hkv, dqk, dv, ph, p2, s, None)
    for name in ("q", "k", "v", "ko", "vo", "qd", "kd", "vd"):
        assert q(**{name: None}) == ba.ATTN_E_INVAL, name
    assert q(Nk=0) == ba.ATTN_E_INVAL
    assert q(dqk=6) == ba.ATTN_E_INVAL
    assert q(dv=2) == ba.ATTN_E_INVAL
    assert q(Hkv=3) == ba.ATTN_E_INVAL            # Hq % Hkv != 0 with pow2 and per-head
    assert q(p2=2) == ba.ATTN_E_INVAL
    assert q(ph=2) == ba.ATTN_E_INVAL
    assert q(s=0.0) == ba.ATTN_E_INVAL
    assert q(Hq=70000, Hkv=70000) == ba.ATTN_E_INVAL
    assert q(B=1, Nq=1 << 20, Hq=32, dqk=128) == ba.ATTN_E_INVAL   # 2^32 elements
    assert q(v=A16 + 4) == ba.ATTN_E_ALIGN
    assert q(vo=A16 + 2) == ba.ATTN_E_ALIGN
    assert q(kd=A16 + 1) == ba.ATTN_E_ALIGN
    if _no_device():
        assert q() == ba.ATTN_E_NODEVICE
        assert q(Hkv=3, p2=0) == ba.ATTN_E_NODEVICE   # no pairing without the pow2 Q scale
        assert q(s=0.0, p2=0) == ba.ATTN_E_NODEVICE   # the scale is not read then
        assert q(qo=None) == ba.ATTN_E_NODEVICE       # Q's descales only
        assert q(qo=None, q=A16 + 4) == ba.ATTN_E_ALIGN


def test_fp8_qf32_entry_validates():
    """The float32-Q entry point shares the FP8 checks (shape, scale, alignment,
    descales) and takes the same argument list."""
    lib = ba.load_library()
    vp = ctypes.c_void_p

    def call(**kw):
        a = dict(q=A16, k=A16, v=A16, qd=A16, kd=A16, vd=A16, ph=0, o=A16, lse=None, B=1, Hq=2,
                 Hkv=2, N=16, dqk=128, dv=128, scale=0.1)
        a.update(kw)
        return lib.attn_fwd_causal_fp8_qf32(vp(a["q"]), vp(a["k"]), vp(a["v"]), vp(a["qd"]),
                                            vp(a["kd"]), vp(a["vd"]), a["ph"], vp(a["o"]),
                                            vp(a["lse"]), a["B"], a["Hq"], a["Hkv"], a["N"],
                                            a["dqk"], a["dv"], a["scale"], None)
    assert call(q=None) == ba.ATTN_E_INVAL
    assert call(qd=None) == ba.ATTN_E_INVAL
    assert call(Hq=3) == ba.ATTN_E_INVAL
    assert call(scale=-1.0) == ba.ATTN_E_INVAL
    assert call(dqk=64) == ba.ATTN_E_UNSUPPORTED
    assert call(q=A16 + 8) == ba.ATTN_E_ALIGN
    assert call(ph=2) == ba.ATTN_E_INVAL
    if _no_device():
        assert call() == ba.ATTN_E_NODEVICE


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


# ---- the Python binding's argument checks (CPU tensors; the library is never called) ----

@pytest.fixture
def no_library(monkeypatch):
    """Any call into the library fails the test: the checks must come first."""
    def boom(*a, **k):
        raise AssertionError("the library was called before the arguments were checked")
    monkeypatch.setattr(ba, "load_library", boom)


def _t(shape, dtype):
    import torch
    return torch.zeros(shape, dtype=dtype)


def _fp8_args(B=1, Nq=8, Nk=8, Hq=4, Hkv=2, d=128, dv=128, nq=4, nk=2, nv=2, lse=True):
    import torch
    return dict(q=_t((B, Nq, Hq, d), torch.uint8), k=_t((B, Nk, Hkv, d), torch.uint8),
                v=_t((B, Nk, Hkv, dv), torch.uint8), q_descale=_t((nq,), torch.float32),
                k_descale=_t((nk,), torch.float32), v_descale=_t((nv,), torch.float32),
                o=_t((B, Nq, Hq, dv), torch.bfloat16),
                lse=_t((B, Hq, Nq), torch.float32) if lse else None)


FP8_BAD = {
    "k_fewer_rows": (dict(Nk=4), "rows"),
    "k_descale_one_value_per_head_q": (dict(nk=1), "descales"),
    "v_descale_short": (dict(nv=1), "descales"),
    "q_descale_short": (dict(nq=2), "descales"),
    "heads_not_multiple": (dict(Hq=3, Hkv=2, nq=3), "multiple"),
}


@pytest.mark.parametrize("case", sorted(FP8_BAD))
def test_binding_rejects_fp8_mismatch(no_library, case):
    kw, msg = FP8_BAD[case]
    with pytest.raises(ValueError, match=msg):
        ba.attn_fwd_causal_fp8(**_fp8_args(**kw))


def test_binding_rejects_fp8_wrong_outputs(no_library):
    import torch
    a = _fp8_args()
    with pytest.raises(ValueError, match="o: shape"):
        ba.attn_fwd_causal_fp8(**dict(a, o=_t((1, 8, 4, 64), torch.bfloat16)))
    with pytest.raises(ValueError, match="o: dtype"):
        ba.attn_fwd_causal_fp8(**dict(a, o=_t((1, 8, 4, 128), torch.float32)))
    with pytest.raises(ValueError, match="lse: shape"):
        ba.attn_fwd_causal_fp8(**dict(a, lse=_t((1, 8, 4), torch.float32)))
    with pytest.raises(ValueError, match="q: dtype"):
        ba.attn_fwd_causal_fp8(**dict(a, q=_t((1, 8, 4, 128), torch.bfloat16)))
    with pytest.raises(ValueError, match="q_descale: dtype"):
        ba.attn_fwd_causal_fp8(**dict(a, q_descale=_t((4,), torch.float64)))


def test_binding_rejects_cpu_and_noncontiguous(no_library):
    import torch
    with pytest.raises(ValueError, match="GPU tensor"):
        ba.attn_fwd_causal_fp8(**_fp8_args())
    q = _t((1, 8, 4, 128), torch.bfloat16)
    k = _t((1, 8, 2, 128), torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        ba.attn_fwd_causal_bf16(q, k, k.clone(), _t((1, 8, 4, 128), torch.bfloat16))
    with pytest.raises(ValueError, match="rows"):
        ba.attn_fwd_causal_bf16(q, k[:, :4], k[:, :4].clone(), _t((1, 8, 4, 128), torch.bfloat16))


def test_binding_rejects_offset_and_rounded(no_library):
    a = _fp8_args(Nq=4, Nk=8)
    with pytest.raises(ValueError, match="lse is required"):
        ba.attn_fwd_causal_offset_fp8_rounded_lse(**dict(a, lse=None))
    with pytest.raises(ValueError, match="v: shape"):
        b = _fp8_args(Nq=4, Nk=8)
        b["v"] = b["v"][:, :5].clone()
        ba.attn_fwd_causal_offset_fp8(**b)
    with pytest.raises(ValueError, match="GPU tensor"):
        ba.attn_fwd_causal_offset_fp8(**a)


def test_binding_rejects_quantize_mismatch(no_library):
    import torch
    x = _t((1, 4, 3, 8), torch.float32)
    out = _t((1, 4, 3, 8), torch.uint8)
    with pytest.raises(ValueError, match="descale: shape"):
        ba.quantize_e4m3(x, out, _t((1,), torch.float32), per_head=True)
    with pytest.raises(ValueError, match="descale: shape"):
        ba.quantize_e4m3_hadamard(x, out, _t((3,), torch.float32), per_head=False)
    with pytest.raises(ValueError, match="out: shape"):
        ba.quantize_e4m3(x, _t((1, 4, 3, 4), torch.uint8), _t((3,), torch.float32), True)
    with pytest.raises(ValueError, match="x: dtype"):
        ba.quantize_e4m3(x.double(), out, _t((3,), torch.float32), True)
    with pytest.raises(ValueError, match="multiple"):
        ba.quantize_e4m3_q_pow2(x, out, _t((3,), torch.float32), _t((2,), torch.float32),
                                0.1, per_head=True)
    with pytest.raises(ValueError, match="GPU tensor"):
        ba.quantize_e4m3(x, out, _t((3,), torch.float32), True)
    k = _t((1, 4, 1, 8), torch.float32)
    v = _t((1, 4, 1, 4), torch.float32)
    qkv = dict(q=x, k=k, v=v, q_out=out, k_out=_t((1, 4, 1, 8), torch.uint8),
               v_out=_t((1, 4, 1, 4), torch.uint8), q_descale=_t((3,), torch.float32),
               k_descale=_t((1,), torch.float32), v_descale=_t((1,), torch.float32),
               per_head=True)
    with pytest.raises(ValueError, match="v_out: shape"):
        ba.quantize_e4m3_qkv(**{**qkv, "v_out": _t((1, 4, 1, 8), torch.uint8)})
    with pytest.raises(ValueError, match="k_descale: shape"):
        ba.quantize_e4m3_qkv(**{**qkv, "k_descale": _t((2,), torch.float32)})
    with pytest.raises(ValueError, match="k: shape"):
        ba.quantize_e4m3_qkv(**{**qkv, "k": _t((1, 4, 1, 4), torch.float32)})
    with pytest.raises(ValueError, match="GPU tensor"):
        ba.quantize_e4m3_qkv(**qkv, q_pow2=True)
    with pytest.raises(ValueError, match="GPU tensor"):
        ba.quantize_e4m3_qkv(**{**qkv, "q_out": None})     # Q's descales only: accepted
    q8, k8 = _t((1, 8, 4, 128), torch.uint8), _t((1, 8, 2, 128), torch.uint8)
    d4, d2 = _t((4,), torch.float32), _t((2,), torch.float32)
    o = _t((1, 8, 4, 128), torch.bfloat16)
    with pytest.raises(ValueError, match="q: dtype"):
        ba.attn_fwd_causal_fp8_qf32(q8, k8, k8.clone(), d4, d2, d2.clone(), o)
    with pytest.raises(ValueError, match="GPU tensor"):
        ba.attn_fwd_causal_fp8_qf32(_t((1, 8, 4, 128), torch.float32), k8, k8.clone(), d4, d2,
                                    d2.clone(), o)


def test_binding_rejects_merge_mismatch(no_library):
    import torch
    o = _t((1, 8, 4, 128), torch.bfloat16)
    l = _t((1, 4, 8), torch.float32)
    with pytest.raises(ValueError, match="o_b: shape"):
        ba.attn_merge_partials(o, l, _t((1, 7, 4, 128), torch.bfloat16), l, o.clone())
    with pytest.raises(ValueError, match="lse_b: shape"):
        ba.attn_merge_partials(o, l, o.clone(), _t((1, 4, 7), torch.float32), o.clone())
    with pytest.raises(ValueError, match="GPU tensor"):
        ba.attn_merge_partials(o, l, o.clone(), l.clone(), o.clone())


def test_outlier_entry_points_validate():
    """The exact-channel attention accepts only d_qk 128; the joint quantiser checks its
    sizes, flags, workspace size and alignment before touching a device."""
    lib = ba.load_library()
    vp = ctypes.c_void_p
    f = ctypes.c_float

    def attn(dqk=128, B=1, q=A16, qx=A16, kx=A16):
        return lib.attn_fwd_causal_fp8_outliers(vp(q), vp(A16), vp(A16), vp(qx), vp(kx),
                                                vp(A16), vp(A16), vp(A16), 0, vp(A16),
                                                vp(None), B, 2, 2, 16, dqk, 128, f(0.1), None)
    assert attn(dqk=192) == ba.ATTN_E_UNSUPPORTED
    assert attn(B=0) == ba.ATTN_E_INVAL
    assert attn(qx=None) == ba.ATTN_E_INVAL
    assert attn(kx=None) == ba.ATTN_E_INVAL
    assert attn(q=A16 + 4) == ba.ATTN_E_ALIGN
    assert attn(kx=A16 + 8) == ba.ATTN_E_ALIGN
    assert lib.attn_fwd_causal_offset_fp8_outliers(
        vp(A16), vp(A16), vp(A16), vp(A16), vp(A16), vp(A16), vp(A16), vp(A16), 0, vp(A16),
        vp(None), 1, 2, 2, 16, 16, -1, 128, 128, f(0.1), None) == ba.ATTN_E_INVAL

    assert lib.quantize_e4m3_qk_outliers_workspace_bytes(32, 8, 128) == 40 * 128 * 4
    assert lib.quantize_e4m3_qk_outliers_workspace_bytes(0, 8, 128) == 0

    def qz(B=1, N=4, Hq=4, Hkv=2, d=128, ph=1, p2=0, s=0.1, ws_bytes=None, q=A16, perm=A16,
           ws=A16, qx=A16):
        wb = lib.quantize_e4m3_qk_outliers_workspace_bytes(max(Hq, 1), max(Hkv, 1), max(d, 1)) \
            if ws_bytes is None else ws_bytes
        return lib.quantize_e4m3_qk_outliers(vp(q), vp(A16), vp(A16), vp(A16), vp(qx), vp(A16),
                                             vp(A16), vp(A16), vp(perm), vp(ws), wb, B, N, Hq,
                                             Hkv, d, ph, p2, f(s), None)
    assert qz(q=None) == ba.ATTN_E_INVAL
    assert qz(ws=None) == ba.ATTN_E_INVAL
    assert qz(qx=None) == ba.ATTN_E_INVAL
    assert qz(qx=A16 + 4) == ba.ATTN_E_ALIGN
    assert qz(Hq=3) == ba.ATTN_E_INVAL            # Hq % Hkv
    assert qz(d=28) == ba.ATTN_E_INVAL            # fewer channels than the exact block
    assert qz(d=260) == ba.ATTN_E_INVAL
    assert qz(d=130) == ba.ATTN_E_INVAL
    assert qz(ph=2) == ba.ATTN_E_INVAL
    assert qz(p2=1, s=0.0) == ba.ATTN_E_INVAL
    assert qz(ws_bytes=100) == ba.ATTN_E_INVAL
    assert qz(q=A16 + 4) == ba.ATTN_E_ALIGN
    assert qz(perm=A16 + 2) == ba.ATTN_E_ALIGN
    if _no_device():
        assert qz() == ba.ATTN_E_NODEVICE
        assert qz(p2=1) == ba.ATTN_E_NODEVICE
        assert attn() == ba.ATTN_E_NODEVICE


def test_binding_rejects_outlier_quantiser_mismatch(no_library):
    import torch
    q = _t((1, 4, 4, 128), torch.float32)
    k = _t((1, 4, 2, 128), torch.float32)
    a = dict(q=q, k=k, q_out=_t((1, 4, 4, 128), torch.uint8), k_out=_t((1, 4, 2, 128), torch.uint8),
             q_exact=_t((1, 4, 4, 32), torch.bfloat16), k_exact=_t((1, 4, 2, 32), torch.bfloat16),
             q_descale=_t((4,), torch.float32), k_descale=_t((2,), torch.float32),
             perm=_t((2, 128), torch.uint8), per_head=True)
    with pytest.raises(ValueError, match="perm"):
        ba.quantize_e4m3_qk_outliers(**dict(a, perm=_t((4, 128), torch.uint8)))
    with pytest.raises(ValueError, match="k_descale: shape"):
        ba.quantize_e4m3_qk_outliers(**dict(a, k_descale=_t((1,), torch.float32)))
    with pytest.raises(ValueError, match="k_out: shape"):
        ba.quantize_e4m3_qk_outliers(**dict(a, k_out=_t((1, 4, 4, 128), torch.uint8)))
    with pytest.raises(ValueError, match="k_exact: shape"):
        ba.quantize_e4m3_qk_outliers(**dict(a, k_exact=_t((1, 4, 2, 16), torch.bfloat16)))
    with pytest.raises(ValueError, match="q_exact: dtype"):
        ba.quantize_e4m3_qk_outliers(**dict(a, q_exact=_t((1, 4, 4, 32), torch.float32)))
    with pytest.raises(ValueError, match="GPU tensor"):
        ba.quantize_e4m3_qk_outliers(**a)


def test_noalloc_quantiser_validates_and_bounds_its_scratch():
    """quantize_e4m3_qk_outliers_noalloc: the same argument checks as the workspace
    form, and (Hq + Hkv) * d beyond its fixed scratch is ATTN_E_TOO_LARGE, all before
    any HIP call."""
    lib = ba.load_library()
    vp = ctypes.c_void_p

    def qz(B=1, N=4, Hq=4, Hkv=2, d=128, ph=1, p2=0, s=0.1, q=A16, perm=A16):
        return lib.quantize_e4m3_qk_outliers_noalloc(vp(q), vp(A16), vp(A16), vp(A16), vp(A16),
                                                     vp(A16), vp(A16), vp(A16), vp(perm), B, N,
                                                     Hq, Hkv, d, ph, p2, ctypes.c_float(s), None)
    assert qz(q=None) == ba.ATTN_E_INVAL
    assert qz(Hq=3) == ba.ATTN_E_INVAL
    assert qz(d=28) == ba.ATTN_E_INVAL
    assert qz(p2=1, s=float("nan")) == ba.ATTN_E_INVAL
    assert qz(perm=A16 + 1) == ba.ATTN_E_ALIGN
    words = ba.NOALLOC_SCRATCH_WORDS
    assert qz(Hq=words // 128, Hkv=words // 128, d=128) == ba.ATTN_E_TOO_LARGE
    assert qz(Hq=256, Hkv=4, d=256) == ba.ATTN_E_TOO_LARGE       # 260 * 256 > 65536
    assert "scratch" in ba.attn_status_string(ba.ATTN_E_TOO_LARGE)
    if _no_device():
        assert qz() == ba.ATTN_E_NODEVICE
        assert qz(Hq=256, Hkv=256, d=128) == ba.ATTN_E_NODEVICE   # exactly at the limit
