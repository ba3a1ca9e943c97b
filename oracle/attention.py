"""Plain fp64 causal attention (test infrastructure only).

What is computed (the definition, not the tiled method): for every batch b,
query head h and query i, scores s_ij = scale * <Q[b,i,h,:], K[b,j,g,:]> for the
keys j the causal mask leaves visible (j <= i), weights w_ij = softmax_j(s_ij),
output O[b,i,h,:] = sum_j w_ij V[b,j,g,:] and log-sum-exp
LSE[b,h,i] = log sum_j exp(s_ij).

Sources: attention turns the QK^T scores into probabilities with a softmax and
multiplies them by V (the-ai.news "Waarom presteert FP8 minder goed op de
MI355X?"; spke.com "なぜMI355XではFP8注意機構の性能が低いのか?"); the kernels
compute the causal forward (prefill) pass (ai-daily-news.org "Qué cubren los
kernels"; spke.com "TL;DR"); FlashAttention's tiles and online softmax give
the same result as the whole-row softmax without storing the score matrix
(kongchang.com "为什么 prefill attention 值得单独优化"), which is why the oracle
can use the whole-row form.

Readings where the pages are silent:
* causal alignment: Nq == Nk == N, key j visible to query i iff j <= i;
* grouped KV heads: query head h reads KV head floor(h / (Hq / Hkv));
* LSE: natural log over the scaled scores, shape (B, Hq, N).

Beyond the pages (their kernels stop at Nq == Nk and leave variable-length work
for later, ai-daily-news.org "Qué cubren los kernels"): offset_attention lets Nq
queries attend Nk keys with key j visible to query i iff j <= i + q_offset, and
merge_partials combines two partial attentions over disjoint key sets.

Inputs are float64 arrays of already-decoded values (bf16 or e4m3 codes times
their descale), in the (B, N, H, d) layout.
"""
from __future__ import annotations

import numpy as np


def kv_head_of(h: int, Hq: int, Hkv: int) -> int:
    """KV head read by query head h: consecutive groups of Hq/Hkv heads."""
    return h // (Hq // Hkv)


def visible_keys(i: int, q_offset: int = 0, n_keys: int | None = None) -> int:
    """Number of keys query i may attend to: keys 0..i + q_offset, at most n_keys."""
    n = i + q_offset + 1
    return n if n_keys is None else min(n, n_keys)


def _rows(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
          i_abs: np.ndarray, q_offset: int = 0) -> tuple[np.ndarray, np.ndarray]:
    """Whole-row softmax attention for a block of query rows.

    q_rows (R, dqk), k (Nk, dqk), v (Nk, dv), i_abs (R,) query indices; row r sees
    keys 0 .. min(i_abs[r] + q_offset, Nk - 1).
    """
    lim = np.array([visible_keys(int(i), q_offset, k.shape[0]) for i in i_abs])
    nk = int(lim.max())
    s = scale * (q_rows @ k[:nk].T)                           # (R, nk)
    mask = np.arange(nk)[None, :] < lim[:, None]
    s = np.where(mask, s, -np.inf)
    m = np.max(s, axis=1, keepdims=True)
    e = np.exp(s - m)
    l = np.sum(e, axis=1, keepdims=True)
    o = (e @ v[:nk]) / l
    lse = m[:, 0] + np.log(l[:, 0])
    return o, lse


def causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                     block: int = 512) -> tuple[np.ndarray, np.ndarray]:
    """All outputs.  q (B,N,Hq,dqk), k (B,N,Hkv,dqk), v (B,N,Hkv,dv), float64.

    Returns O (B,N,Hq,dv) float64 and LSE (B,Hq,N) float64.  Query rows are
    processed in blocks only to bound memory; each row's softmax is taken over
    its whole visible key range at once.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, N, Hq, _ = q.shape
    Hkv = k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    o = np.empty((B, N, Hq, v.shape[3]), dtype=np.float64)
    lse = np.empty((B, Hq, N), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            kk = np.ascontiguousarray(k[b, :, g, :])
            vv = np.ascontiguousarray(v[b, :, g, :])
            for i0 in range(0, N, block):
                i1 = min(N, i0 + block)
                ob, lb = _rows(q[b, i0:i1, h, :], kk, vv, scale, np.arange(i0, i1))
                o[b, i0:i1, h, :] = ob
                lse[b, h, i0:i1] = lb
    return o, lse


def causal_attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                          rows) -> tuple[np.ndarray, np.ndarray]:
    """Outputs for sampled rows only: rows is an iterable of (b, h, i).

    q, k, v may be any arrays indexable as x[b, i, h, :] whose values convert
    to float64 exactly; returns O (R, dv) and LSE (R,) in the order of `rows`.
    Each row costs O(i * d), so this is usable at the full 16K/32K sizes.
    """
    rows = [(int(b), int(h), int(i)) for (b, h, i) in rows]
    Hq = q.shape[2]
    Hkv = k.shape[2]
    dv = v.shape[3]
    out_o = np.empty((len(rows), dv), dtype=np.float64)
    out_l = np.empty((len(rows),), dtype=np.float64)
    by_head: dict[tuple[int, int], list[int]] = {}
    for r, (b, h, i) in enumerate(rows):
        by_head.setdefault((b, h), []).append(r)
    for (b, h), idx in by_head.items():
        g = kv_head_of(h, Hq, Hkv)
        i_abs = np.array([rows[r][2] for r in idx])
        nk = max(visible_keys(int(i)) for i in i_abs)
        kk = np.asarray(k[b, :nk, g, :], dtype=np.float64)
        vv = np.asarray(v[b, :nk, g, :], dtype=np.float64)
        qr = np.stack([np.asarray(q[b, i, h, :], dtype=np.float64) for i in i_abs])
        ob, lb = _rows(qr, kk, vv, scale, i_abs)
        out_o[idx] = ob
        out_l[idx] = lb
    return out_o, out_l


def offset_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                     q_offset: int, block: int = 512) -> tuple[np.ndarray, np.ndarray]:
    """Nq queries over Nk keys, key j visible to query i iff j <= i + q_offset.

    q (B,Nq,Hq,dqk), k (B,Nk,Hkv,dqk), v (B,Nk,Hkv,dv), float64; q_offset >= 0 (so
    every query sees key 0).  Returns O (B,Nq,Hq,dv) and LSE (B,Hq,Nq), float64.
    causal_attention is the case Nq == Nk, q_offset == 0.
    """
    if q_offset < 0:
        raise ValueError("q_offset must be >= 0")
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Nq, Hq, _ = q.shape
    Hkv = k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    o = np.empty((B, Nq, Hq, v.shape[3]), dtype=np.float64)
    lse = np.empty((B, Hq, Nq), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            kk = np.ascontiguousarray(k[b, :, g, :])
            vv = np.ascontiguousarray(v[b, :, g, :])
            for i0 in range(0, Nq, block):
                i1 = min(Nq, i0 + block)
                ob, lb = _rows(q[b, i0:i1, h, :], kk, vv, scale, np.arange(i0, i1), q_offset)
                o[b, i0:i1, h, :] = ob
                lse[b, h, i0:i1] = lb
    return o, lse


def merge_partials(o_a: np.ndarray, lse_a: np.ndarray, o_b: np.ndarray,
                   lse_b: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Attention over the union of two disjoint key sets from the two partial
    attentions over each: o (B,N,Hq,dv), lse (B,Hq,N).  Each partial's softmax is
    normalised over its own keys, so partial X contributes with weight
    exp(lse_X) / (exp(lse_a) + exp(lse_b)) and the union's LSE is the log of that
    denominator.  A partial with LSE -inf (no keys) contributes nothing."""
    la = np.asarray(lse_a, dtype=np.float64)
    lb = np.asarray(lse_b, dtype=np.float64)
    m = np.maximum(la, lb)
    safe = np.where(np.isfinite(m), m, 0.0)
    wa = np.exp(la - safe)
    wb = np.exp(lb - safe)
    den = wa + wb
    with np.errstate(divide="ignore", invalid="ignore"):
        lse = np.where(den > 0, safe + np.log(np.where(den > 0, den, 1.0)), -np.inf)
        fa = np.where(den > 0, wa / np.where(den > 0, den, 1.0), 0.0)
        fb = np.where(den > 0, wb / np.where(den > 0, den, 1.0), 0.0)
    # weights are per (b, h, n); O is (b, n, h, :)
    fa = np.transpose(fa, (0, 2, 1))[..., None]
    fb = np.transpose(fb, (0, 2, 1))[..., None]
    o = fa * np.asarray(o_a, dtype=np.float64) + fb * np.asarray(o_b, dtype=np.float64)
    return o, lse
