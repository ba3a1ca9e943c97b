"""Number formats for the oracle (test infrastructure only).

bf16: 1 sign, 8 exponent, 7 mantissa bits; a bf16 code is the upper half of
the float32 with the same value (the BF16 description on kongchang.com, "ZYFA
的性能与精度数据": 8 exponent and 7 mantissa bits).

e4m3: 1 sign, 4 exponent, 3 mantissa bits (same section).  The variant is OCP
E4M3FN (exponent bias 7, no infinities, codes 0x7F/0xFF are NaN, largest
finite value 448 = code 0x7E), the variant gfx950's matrix instructions
consume.  Read as an integer, the code of a power of two grows by 8 per
doubling (the-ai.news "Drie technieken om de bottleneck te omzeilen";
spke.com "Lean P"), which the tests pin.

Quantisation maps each tensor (or each head) into the e4m3 range with one
scale factor, accumulation staying in higher precision (kongchang.com "ZYFA
的性能与精度数据": per-tensor or per-head scaling factors).  The reading used
here: descale = absmax / 448 computed in float32, code = round-to-nearest-even
of the float32 quotient x / descale, saturating at +-448.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E4M3_BIAS = 7
_MIN_NORMAL_EXP = 1 - E4M3_BIAS          # -6
_MANT_BITS = 3


def bf16_decode(u16: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values."""
    u16 = np.asarray(u16, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """OCP e4m3fn codes (uint8) -> exact float64 values (NaN for 0x7F/0xFF).

    Field decoding: exponent field e, mantissa field m;
    e == 0: subnormal, value = m * 2^(1 - bias - 3);  else (1 + m/8) * 2^(e - bias).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    sub = m.astype(np.float64) * 2.0 ** (_MIN_NORMAL_EXP - _MANT_BITS)
    nrm = (1.0 + m / 8.0) * np.exp2((e - E4M3_BIAS).astype(np.float64))
    val = sign * np.where(e == 0, sub, nrm)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """float32 values -> e4m3fn codes, round to nearest (ties to even),
    saturating finite overflow to +-448; NaN -> 0x7F.

    Works on the value, not the bit pattern: find the binade 2^e of |x|
    (clamped to the smallest normal binade 2^-6, below which the spacing is
    the subnormal step 2^-9), round |x| / spacing to the nearest integer with
    ties to even, rescale, clamp at 448, then write the fields.
    """
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    a = np.abs(x)
    finite = np.isfinite(a)
    a_f = np.where(finite, a, 0.0)
    _, ex = np.frexp(a_f)                      # a = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex - 1, _MIN_NORMAL_EXP)    # binade exponent, clamped
    spacing = np.exp2((e - _MANT_BITS).astype(np.float64))
    r = np.rint(a_f / spacing) * spacing       # np.rint rounds half to even
    r = np.minimum(r, E4M3_MAX)
    r = np.where(np.isinf(a), E4M3_MAX, r)
    # fields of the rounded value
    _, er = np.frexp(np.where(r > 0, r, 1.0))
    er = er - 1
    is_sub = r < 2.0 ** _MIN_NORMAL_EXP
    sub_code = np.rint(r / 2.0 ** (_MIN_NORMAL_EXP - _MANT_BITS))
    mant = np.rint((r / np.exp2(er.astype(np.float64)) - 1.0) * 8.0)
    nrm_code = (er + E4M3_BIAS) * 8 + mant
    code = np.where(is_sub, sub_code, nrm_code).astype(np.int64)
    code = code | np.where(np.signbit(x), 0x80, 0)
    code = np.where(np.isnan(x), 0x7F, code)
    return code.astype(np.uint8)


def absmax_descale(x: np.ndarray, per_head: bool) -> np.ndarray:
    """descale of a (B, N, H, d) float32 tensor: float32(absmax) / float32(448)
    per head ((H,)) or per tensor ((1,)); 1 where the absmax is 0.

    A NaN element has no magnitude and takes no part in the absmax (it encodes
    to 0x7F whatever the descale); an infinity does, giving an infinite descale."""
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 4:
        raise ValueError("expected (B, N, H, d)")
    a = np.abs(x)
    a = np.where(np.isnan(a), np.float32(0.0), a)
    if per_head:
        amax = np.max(a, axis=(0, 1, 3)).astype(np.float32)
    else:
        amax = np.array([np.max(a)], dtype=np.float32)
    descale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    return np.where(amax > 0, descale, np.float32(1.0)).astype(np.float32)


_LOG2E_F32 = np.float32(1.4426950408889634)


def _near_pow2(c: np.float32) -> bool:
    """c within 4 ulps of a power of two (mantissa field at most 4 above or below)."""
    b = int(np.float32(c).view(np.uint32))
    e, man = (b >> 23) & 0xFF, b & 0x7FFFFF
    return 0 < e < 0xFF and (man <= 4 or man >= 0x7FFFFC)


def pow2_q_descale_one(amax: np.float32, dk: np.float32, scale: float) -> np.float32:
    """One Q descale for which the FP8 softmax constant, evaluated in float32 as
    c = fl(fl(scale * log2 e) * fl(dq * dk)), lies within 4 ulps of a power of two:
    the power of two is the smallest at or above fl(fl(amax / 448) * fl(fl(scale *
    log2 e) * dk)), dq starts at fl(target / fl(fl(scale * log2 e) * dk)) and moves one
    ulp at a time (at most 16) towards the target until c is there.  An all-zero (or
    non-finite) absmax, or no such dq, gives the plain absmax descale."""
    amax, dk = np.float32(amax), np.float32(dk)
    plain = np.float32(amax / np.float32(E4M3_MAX)) if amax > 0 else np.float32(1.0)
    if not (np.isfinite(amax) and amax > 0 and np.isfinite(dk) and dk > 0):
        return plain
    sl = np.float32(np.float32(scale) * _LOG2E_F32)
    a = np.float32(sl * dk)
    tmin = np.float32(np.float32(amax / np.float32(E4M3_MAX)) * a)
    if not (np.isfinite(tmin) and tmin > 0):
        return plain
    b = int(tmin.view(np.uint32))
    exp = (b >> 23) & 0xFF
    if exp == 0 or exp >= 0xFE:
        return plain
    target = tmin if (b & 0x7FFFFF) == 0 else np.uint32((exp + 1) << 23).view(np.float32)
    target = np.float32(target)
    d = np.float32(target / a)
    for _ in range(16):
        c = np.float32(sl * np.float32(d * dk))
        if _near_pow2(c) and abs(float(c) / float(target) - 1.0) < 2.0 ** -20:
            return d
        d = np.nextafter(d, np.float32(np.inf) if c < target else np.float32(0))
    return plain


def quantize_e4m3_q_pow2(x: np.ndarray, per_head: bool, k_descale: np.ndarray,
                         softmax_scale: float) -> tuple[np.ndarray, np.ndarray]:
    """Quantisation of Q whose descales make the FP8 softmax constant a power of two
    (reading: any descale at or above absmax / 448 keeps every value in range; this one
    lets the kernel apply the constant through the matrix instruction's power-of-two
    operand scale).  k_descale: K's descales, one (per tensor) or Hkv (per head);
    query head h pairs with KV head h / (H / Hkv).  Codes are the e4m3 rounding of
    x / descale, as in quantize_e4m3."""
    x = np.asarray(x, dtype=np.float32)
    H = x.shape[2]
    a = np.abs(x)
    a = np.where(np.isnan(a), np.float32(0.0), a)
    amax = (np.max(a, axis=(0, 1, 3)) if per_head else np.array([np.max(a)])).astype(np.float32)
    kd = np.asarray(k_descale, dtype=np.float32).ravel()
    if per_head:
        g = H // len(kd)
        descale = np.array([pow2_q_descale_one(amax[h], kd[h // g], softmax_scale)
                            for h in range(H)], dtype=np.float32)
        ds = descale[None, None, :, None]
    else:
        descale = np.array([pow2_q_descale_one(amax[0], kd[0], softmax_scale)], np.float32)
        ds = descale[0]
    return encode_with_descale(x, ds), descale


def encode_with_descale(x: np.ndarray, descale) -> np.ndarray:
    """e4m3 codes of the float32 quotient x / descale (descale broadcast
    against x; float32 / float32 is correctly rounded)."""
    with np.errstate(invalid="ignore"):     # inf / inf is NaN, encoded as 0x7F
        qv = (np.asarray(x, dtype=np.float32) / np.asarray(descale, dtype=np.float32)).astype(np.float32)
    return e4m3_encode(qv)


def quantize_e4m3(x: np.ndarray, per_head: bool) -> tuple[np.ndarray, np.ndarray]:
    """Absmax quantisation of a (B, N, H, d) float32 tensor.

    Returns (codes uint8 (B,N,H,d), descale float32 of shape (H,) if per_head
    else (1,)).  descale = float32(absmax) / float32(448) (float32 division);
    an all-zero tensor/head gets descale 1.  Each code is the e4m3 rounding of
    the float32 quotient x / descale, so code * descale reproduces x to within
    e4m3's half-spacing.
    """
    descale = absmax_descale(x, per_head)
    ds = descale[None, None, :, None] if per_head else descale[0]
    return encode_with_descale(x, ds), descale


# ---- Hadamard rotation before quantisation -----------------------------------------
# Rotating Q and K by the same orthogonal matrix leaves every score unchanged while
# spreading outlier channels, which roughly halves the FP8 input error (spke.com
# "ZYFAのFP8アテンションの精度はどのくらいか?").  Reading used here: each block of hb
# channels (hb = the largest power of two dividing d, at most 128) is multiplied by
# H / sqrt(hb), H the Sylvester Hadamard matrix (H_1 = [1], H_2n = [[H_n, H_n],
# [H_n, -H_n]]); the unnormalised product is evaluated in float32 by radix-2
# butterflies with stage half-sizes 1, 2, 4, ... (the element with the stage bit clear
# becomes a + b, its partner a - b), and the 1/sqrt(hb) goes into the descale.


def hadamard_block(d: int) -> int:
    """Largest power of two dividing d, at most 128 (d a multiple of 4)."""
    hb = 4
    while hb < 128 and d % (2 * hb) == 0:
        hb *= 2
    return hb


def hadamard_unnormalised_fp32(x: np.ndarray, hb: int) -> np.ndarray:
    """x (..., d) float32 -> each block of hb channels times the Sylvester Hadamard
    matrix of order hb, as float32 butterflies (stage half-sizes 1, 2, 4, ...)."""
    x = np.asarray(x, dtype=np.float32)
    d = x.shape[-1]
    y = x.reshape(x.shape[:-1] + (d // hb, hb)).copy()
    h = 1
    while h < hb:
        z = y.reshape(y.shape[:-1] + (hb // (2 * h), 2, h))
        a = z[..., 0, :].copy()
        b = z[..., 1, :].copy()
        z[..., 0, :] = a + b                       # float32 arithmetic
        z[..., 1, :] = a - b
        y = z.reshape(y.shape)
        h *= 2
    return y.reshape(x.shape)


def quantize_e4m3_hadamard(x: np.ndarray, per_head: bool) -> tuple[np.ndarray, np.ndarray]:
    """Codes and descale of the Hadamard-rotated (B, N, H, d) float32 tensor: the
    codes quantise the unnormalised float32 rotation with its own absmax descale, and
    the returned descale is that descale times float32(1/sqrt(hb)), so
    code * descale is the normalised rotated value."""
    x = np.asarray(x, dtype=np.float32)
    hb = hadamard_block(x.shape[-1])
    xu = hadamard_unnormalised_fp32(x, hb)
    codes, ds = quantize_e4m3(xu, per_head)
    post = np.float32(1.0 / np.sqrt(float(hb)))
    return codes, (ds * post).astype(np.float32)


# ---- Q/K quantisation with the large-product channels moved to the end of the row ----
# Not on the pages.  The pages name the FP8 error of Q and K as the one that matters
# (spke.com "ZYFAのFP8アテンションの精度はどのくらいか?"); on the device the FP8 matrix
# instruction adds up runs of 8 channel products after truncating them to 13 bits below
# the largest, so a channel with a large Q or K magnitude swamps the small products that
# share its run.  Permuting the channels of Q and K the same way leaves every score Q.K
# unchanged, so the quantiser may store them in any common order: this one moves, per KV
# head, the n_split channels with the largest product bound to the end of every Q and K
# row, and also writes those channels as bf16 side arrays, which the attention multiplies
# exactly (in bf16) instead of as e4m3 codes.  Reading used here:
#   * channel absmax: max |x| over all (b, n) of one head, NaN elements ignored;
#   * importance of channel c for KV head g: fl32(max over the query heads h of g of
#     amax_q[h, c]) * amax_k[g, c], in float32, and 0 when either factor is 0;
#   * the n_split channels of largest importance (ties: the lower channel first) go
#     last, in ascending channel order, after the other channels in ascending order;
#   * codes and descales are those of quantize_e4m3 (or quantize_e4m3_q_pow2 for Q)
#     of the unpermuted tensor, the codes then permuted: stored position j of a row of
#     head h holds channel perm[g(h), j];
#   * side arrays: for the last n_split stored positions, bf16 (round to nearest even) of
#     the float32 quotient x / descale, so side value * descale is the channel's value;
#     the attention reads those channels from the side arrays and not from the codes.

OUTLIER_CHANNELS = 32
_BF16_NAN = np.uint16(0x7FC0)


def bf16_encode(x: np.ndarray) -> np.ndarray:
    """float32 values -> bf16 bit patterns (uint16), round to nearest even on the value
    (overflow past the largest bf16 goes to infinity), NaN -> 0x7FC0.

    Written on values: the bf16 neighbours of |x| are the float32 values whose low 16
    bits are zero; take the nearer, ties to the one whose bf16 mantissa is even."""
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x).astype(np.float64)
    u = np.abs(x).view(np.uint32).astype(np.int64)
    lo = (u >> 16) << 16                                   # truncated neighbour (bits)
    lo_v = lo.astype(np.uint32).view(np.float32).astype(np.float64)
    hi = lo + (1 << 16)
    with np.errstate(over="ignore"):
        hi_v = np.where(hi >= 0x7F800000, np.inf,
                        np.minimum(hi, 0x7F7F0000).astype(np.uint32).view(np.float32).astype(np.float64))
    with np.errstate(invalid="ignore"):      # inf - inf for infinite |x|, overridden below
        d_lo, d_hi = a - lo_v, hi_v - a
    even_lo = ((lo >> 16) & 1) == 0
    up = (d_hi < d_lo) | ((d_hi == d_lo) & ~even_lo)
    bits = np.where(up, hi >> 16, lo >> 16)
    bits = np.where(np.isinf(a), 0x7F80, bits)
    bits = bits | np.where(np.signbit(x), 0x8000, 0)
    bits = np.where(np.isnan(x), int(_BF16_NAN), bits)
    return bits.astype(np.uint16)


def channel_absmax(x: np.ndarray) -> np.ndarray:
    """(B, N, H, d) float32 -> (H, d) float32: max |x| over batch and position, NaN
    elements taking no part (an all-NaN or all-zero channel gives 0)."""
    a = np.abs(np.asarray(x, dtype=np.float32))
    a = np.where(np.isnan(a), np.float32(0.0), a)
    return np.max(a, axis=(0, 1)).astype(np.float32)


def outlier_permutation(amax_q: np.ndarray, amax_k: np.ndarray, n_split: int) -> np.ndarray:
    """(Hq, d), (Hkv, d) channel absmax -> (Hkv, d) int64 permutation: row g lists the
    source channel of every stored position, the n_split channels of largest importance
    last (see the reading above)."""
    amax_q = np.asarray(amax_q, np.float32)
    amax_k = np.asarray(amax_k, np.float32)
    Hq, d = amax_q.shape
    Hkv = amax_k.shape[0]
    if Hq % Hkv or not 0 < n_split <= d:
        raise ValueError("need Hq % Hkv == 0 and 0 < n_split <= d")
    G = Hq // Hkv
    perm = np.empty((Hkv, d), dtype=np.int64)
    for g in range(Hkv):
        aq = np.max(amax_q[g * G:(g + 1) * G], axis=0).astype(np.float32)
        ak = amax_k[g]
        with np.errstate(invalid="ignore"):      # 0 * inf, replaced by 0 below
            prod = (aq * ak).astype(np.float32)
        imp = np.where((aq == 0) | (ak == 0), np.float32(0.0), prod)
        order = sorted(range(d), key=lambda c: (-float(imp[c]), c))
        chosen = set(order[:n_split])
        perm[g] = [c for c in range(d) if c not in chosen] + sorted(chosen)
    return perm


def quantize_e4m3_qk_outliers(q: np.ndarray, k: np.ndarray, per_head: bool,
                              n_split: int = OUTLIER_CHANNELS,
                              q_pow2_scale: float | None = None):
    """Codes of Q (B, N, Hq, d) and K (B, N, Hkv, d) with each KV group's n_split
    largest-product channels stored last, plus those channels as bf16 side arrays.
    Returns (q_codes, k_codes, q_exact, k_exact, q_descale, k_descale, perm): codes
    uint8 in the permuted channel order; q_exact (B, N, Hq, n_split) and k_exact
    (B, N, Hkv, n_split) bf16 bit patterns (uint16) of x / descale for the last n_split
    stored channels; descales as quantize_e4m3 gives them (Q's as quantize_e4m3_q_pow2
    with softmax scale q_pow2_scale when that is given); perm (Hkv, d)."""
    q = np.asarray(q, dtype=np.float32)
    k = np.asarray(k, dtype=np.float32)
    Hq, Hkv = q.shape[2], k.shape[2]
    perm = outlier_permutation(channel_absmax(q), channel_absmax(k), n_split)
    kc, kd = quantize_e4m3(k, per_head)
    if q_pow2_scale is None:
        qc, qd = quantize_e4m3(q, per_head)
    else:
        qc, qd = quantize_e4m3_q_pow2(q, per_head, kd, q_pow2_scale)
    G = Hq // Hkv
    qp = np.stack([qc[:, :, h, perm[h // G]] for h in range(Hq)], axis=2)
    kp = np.stack([kc[:, :, g, perm[g]] for g in range(Hkv)], axis=2)

    def side(x, ds, heads_perm):
        out = []
        for h, pr in enumerate(heads_perm):
            d_h = np.float32(ds[h] if per_head else ds[0])
            with np.errstate(invalid="ignore", divide="ignore", over="ignore"):
                quo = (x[:, :, h, pr[-n_split:]] / d_h).astype(np.float32)
            out.append(bf16_encode(quo))
        return np.ascontiguousarray(np.stack(out, axis=2))
    qx = side(q, qd, [perm[h // G] for h in range(Hq)])
    kx = side(k, kd, [perm[g] for g in range(Hkv)])
    return (np.ascontiguousarray(qp), np.ascontiguousarray(kp), qx, kx, qd, kd, perm)


def decode_qk_outliers(codes: np.ndarray, exact: np.ndarray, descale: np.ndarray,
                       per_head: bool) -> np.ndarray:
    """float64 values the exact-channel attention computes with: the e4m3 codes times
    the descale for the first d - n_split stored channels, the bf16 side values times
    the descale for the last n_split (whose codes are not read)."""
    n_split = exact.shape[-1]
    ds = (np.asarray(descale, np.float64)[None, None, :, None] if per_head
          else float(np.asarray(descale)[0]))
    v = e4m3_decode(codes) * ds
    v[..., -n_split:] = bf16_decode(exact) * ds
    return v
