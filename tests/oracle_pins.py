"""Pins for the attention oracle: each returns None or raises AssertionError.

Every pin checks the oracle against something other than itself: a brute-force
loop on tiny inputs, torch's scaled_dot_product_attention in float64 (a library
routine), closed forms (equal scores give the mean of V, row 0 sees only key
0, a huge scale turns softmax into a hard max) and invariants (rows of P sum to
one, a query never depends on later keys, GQA equals MHA with repeated K/V).
The mutation tests plant mistakes in the oracle and require that at least one
pin fails for each.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def pin_bruteforce():
    """Pure-Python loops with math.exp on a tiny GQA problem, 1e-12."""
    rng = np.random.default_rng(11)
    B, N, Hq, Hkv, d, dv = 2, 9, 4, 2, 5, 3
    q, k, v = _rand(rng, B, N, Hq, d), _rand(rng, B, N, Hkv, d), _rand(rng, B, N, Hkv, dv)
    scale = 0.7
    o, lse = oracle.causal_attention(q, k, v, scale, block=4)
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            for i in range(N):
                sc = [scale * sum(q[b, i, h, c] * k[b, j, g, c] for c in range(d))
                      for j in range(i + 1)]
                mx = max(sc)
                ex = [math.exp(s - mx) for s in sc]
                tot = sum(ex)
                for c in range(dv):
                    ref = sum(ex[j] * v[b, j, g, c] for j in range(i + 1)) / tot
                    assert abs(o[b, i, h, c] - ref) < 1e-12
                assert abs(lse[b, h, i] - (mx + math.log(tot))) < 1e-12


def _sdpa(q, k, v, scale):
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3)
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, is_causal=True, scale=scale, enable_gqa=True)
    return out.permute(0, 2, 1, 3).numpy()


def pin_sdpa():
    """torch SDPA (causal, GQA, fp64, CPU) on d=128 GQA and MLA-shaped inputs."""
    rng = np.random.default_rng(12)
    for (B, N, Hq, Hkv, d, dv) in [(1, 256, 2, 2, 128, 128), (2, 300, 8, 2, 64, 32),
                                   (1, 130, 4, 4, 192, 128)]:
        q, k, v = _rand(rng, B, N, Hq, d), _rand(rng, B, N, Hkv, d), _rand(rng, B, N, Hkv, dv)
        scale = 1.0 / math.sqrt(d)
        o, _ = oracle.causal_attention(q, k, v, scale, block=64)
        ref = _sdpa(q, k, v, scale)
        assert np.max(np.abs(o - ref)) < 1e-12


def pin_equal_scores():
    """Q = 0: every visible key gets weight 1/(i+1); O_i = mean(V_0..V_i),
    LSE_i = ln(i+1)."""
    rng = np.random.default_rng(13)
    B, N, Hq, Hkv, d, dv = 1, 70, 4, 2, 16, 8
    q = np.zeros((B, N, Hq, d))
    k, v = _rand(rng, B, N, Hkv, d), _rand(rng, B, N, Hkv, dv)
    o, lse = oracle.causal_attention(q, k, v, 0.3, block=32)
    csum = np.cumsum(v, axis=1) / np.arange(1, N + 1)[None, :, None, None]
    for h in range(Hq):
        assert np.max(np.abs(o[:, :, h] - csum[:, :, h // 2])) < 1e-12
        assert np.max(np.abs(lse[:, h] - np.log(np.arange(1, N + 1))[None])) < 1e-12


def pin_row_zero():
    """Query 0 sees only key 0: O_0 = V_0, LSE_0 = s_00."""
    rng = np.random.default_rng(14)
    B, N, Hq, Hkv, d, dv = 2, 40, 6, 3, 16, 8
    q, k, v = _rand(rng, B, N, Hq, d), _rand(rng, B, N, Hkv, d), _rand(rng, B, N, Hkv, dv)
    o, lse = oracle.causal_attention(q, k, v, 0.25, block=16)
    for b in range(B):
        for h in range(Hq):
            g = h // 2
            assert np.max(np.abs(o[b, 0, h] - v[b, 0, g])) < 1e-12
            assert abs(lse[b, h, 0] - 0.25 * float(q[b, 0, h] @ k[b, 0, g])) < 1e-12


def pin_hardmax():
    """A huge scale makes softmax a hard max: O_i = V at argmax_j<=i q.k_j
    and LSE_i - scale*max_j q.k_j -> 0."""
    rng = np.random.default_rng(15)
    B, N, Hq, Hkv, d, dv = 1, 50, 2, 1, 8, 4
    q, k, v = _rand(rng, B, N, Hq, d), _rand(rng, B, N, Hkv, d), _rand(rng, B, N, Hkv, dv)
    scale = 1e4
    o, lse = oracle.causal_attention(q, k, v, scale, block=16)
    for h in range(Hq):
        for i in range(N):
            dots = k[0, : i + 1, 0] @ q[0, i, h]
            j = int(np.argmax(dots))
            srt = np.sort(dots)
            if i > 0 and srt[-1] - srt[-2] < 1e-2:
                continue  # near-tie: the limit is not reached at this scale
            assert np.max(np.abs(o[0, i, h] - v[0, j, 0])) < 1e-9
            assert abs(lse[0, h, i] - scale * dots[j]) < 1e-6


def pin_rows_sum_to_one():
    """V = 1 gives O = 1 for every row (rows of P sum to one)."""
    rng = np.random.default_rng(16)
    B, N, Hq, Hkv, d = 2, 64, 4, 4, 32
    q, k = 3 * _rand(rng, B, N, Hq, d), _rand(rng, B, N, Hkv, d)
    v = np.ones((B, N, Hkv, 5))
    o, _ = oracle.causal_attention(q, k, v, 0.5, block=16)
    assert np.max(np.abs(o - 1.0)) < 1e-12


def pin_causality():
    """Changing K/V rows >= c leaves O and LSE of rows < c bit-identical,
    and changes some row >= c."""
    rng = np.random.default_rng(17)
    B, N, Hq, Hkv, d, dv = 1, 48, 2, 1, 16, 16
    q, k, v = _rand(rng, B, N, Hq, d), _rand(rng, B, N, Hkv, d), _rand(rng, B, N, Hkv, dv)
    o1, l1 = oracle.causal_attention(q, k, v, 0.3, block=48)
    for c in (1, 17, 47):
        k2, v2 = k.copy(), v.copy()
        k2[:, c:] = _rand(rng, B, N - c, Hkv, d)
        v2[:, c:] = _rand(rng, B, N - c, Hkv, dv)
        o2, l2 = oracle.causal_attention(q, k2, v2, 0.3, block=48)
        assert np.array_equal(o1[:, :c], o2[:, :c])
        assert np.array_equal(l1[:, :, :c], l2[:, :, :c])
        assert not np.array_equal(o1[:, c:], o2[:, c:])


def pin_gqa_equals_repeated_mha():
    """Hq/Hkv query heads per KV head == MHA with each KV head repeated."""
    rng = np.random.default_rng(18)
    B, N, Hq, Hkv, d, dv = 1, 33, 8, 2, 16, 8
    q, k, v = _rand(rng, B, N, Hq, d), _rand(rng, B, N, Hkv, d), _rand(rng, B, N, Hkv, dv)
    o, lse = oracle.causal_attention(q, k, v, 0.3, block=16)
    kr, vr = np.repeat(k, Hq // Hkv, axis=2), np.repeat(v, Hq // Hkv, axis=2)
    for h in range(Hq):   # each head alone against its repeated KV head, as MHA
        oh, lh = oracle.causal_attention(q[:, :, h:h + 1], kr[:, :, h:h + 1],
                                         vr[:, :, h:h + 1], 0.3, block=16)
        assert np.array_equal(oh[:, :, 0], o[:, :, h])
        assert np.array_equal(lh[:, 0], lse[:, h])


def pin_rows_match_full():
    """The sampled-row oracle gives the full oracle's rows."""
    rng = np.random.default_rng(19)
    B, N, Hq, Hkv, d, dv = 2, 90, 4, 2, 16, 8
    q, k, v = _rand(rng, B, N, Hq, d), _rand(rng, B, N, Hkv, d), _rand(rng, B, N, Hkv, dv)
    o, lse = oracle.causal_attention(q, k, v, 0.3, block=32)
    rows = [(0, 0, 0), (1, 3, 89), (0, 2, 31), (1, 1, 32), (0, 3, 64)]
    ro, rl = oracle.causal_attention_rows(q, k, v, 0.3, rows)
    for r, (b, h, i) in enumerate(rows):
        assert np.max(np.abs(ro[r] - o[b, i, h])) < 1e-13
        assert abs(rl[r] - lse[b, h, i]) < 1e-13


def pin_offset_bruteforce():
    """Nq queries over Nk keys with a query offset: pure-Python loops, 1e-12.
    Covers chunked prefill (q_offset = Nk - Nq), Nq > Nk, and every key visible."""
    rng = np.random.default_rng(21)
    B, Hq, Hkv, d, dv = 1, 4, 2, 5, 3
    scale = 0.6
    for Nq, Nk, off in [(4, 11, 7), (9, 5, 0), (6, 8, 2), (5, 6, 9), (7, 7, 0)]:
        q, k, v = _rand(rng, B, Nq, Hq, d), _rand(rng, B, Nk, Hkv, d), _rand(rng, B, Nk, Hkv, dv)
        o, lse = oracle.offset_attention(q, k, v, scale, off, block=3)
        for h in range(Hq):
            g = h // (Hq // Hkv)
            for i in range(Nq):
                keys = [j for j in range(Nk) if j <= i + off]
                sc = [scale * sum(q[0, i, h, c] * k[0, j, g, c] for c in range(d)) for j in keys]
                mx = max(sc)
                ex = [math.exp(x - mx) for x in sc]
                tot = sum(ex)
                for c in range(dv):
                    ref = sum(e * v[0, j, g, c] for e, j in zip(ex, keys)) / tot
                    assert abs(o[0, i, h, c] - ref) < 1e-12
                assert abs(lse[0, h, i] - (mx + math.log(tot))) < 1e-12


def pin_offset_chunk_identity():
    """The last Nq rows of causal attention over N positions are the offset attention
    of those queries over all N keys with q_offset = N - Nq."""
    rng = np.random.default_rng(22)
    B, N, Hq, Hkv, d, dv = 2, 70, 4, 2, 16, 8
    q, k, v = _rand(rng, B, N, Hq, d), _rand(rng, B, N, Hkv, d), _rand(rng, B, N, Hkv, dv)
    o, lse = oracle.causal_attention(q, k, v, 0.4, block=32)
    for nq in (1, 23, 70):
        oo, ll = oracle.offset_attention(q[:, N - nq:], k, v, 0.4, N - nq, block=16)
        assert np.max(np.abs(oo - o[:, N - nq:])) < 1e-12
        assert np.max(np.abs(ll - lse[:, :, N - nq:])) < 1e-12


def _sdpa_full(q, k, v, scale):
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3)
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, is_causal=False, scale=scale, enable_gqa=True)
    return out.permute(0, 2, 1, 3).numpy()


def pin_offset_all_visible_sdpa():
    """q_offset >= Nk - 1 leaves every key visible: torch SDPA without a mask (fp64),
    and the LSE against torch.logsumexp of the unmasked scores."""
    rng = np.random.default_rng(23)
    B, Nq, Nk, Hq, Hkv, d, dv = 1, 40, 57, 4, 2, 32, 16
    q, k, v = _rand(rng, B, Nq, Hq, d), _rand(rng, B, Nk, Hkv, d), _rand(rng, B, Nk, Hkv, dv)
    for off in (Nk - 1, Nk + 5):
        o, lse = oracle.offset_attention(q, k, v, 0.2, off)
        assert np.max(np.abs(o - _sdpa_full(q, k, v, 0.2))) < 1e-12
        tk = torch.from_numpy(k).repeat_interleave(Hq // Hkv, dim=2)
        s = 0.2 * torch.einsum("bihc,bjhc->bhij", torch.from_numpy(q), tk)
        assert np.max(np.abs(lse - torch.logsumexp(s, dim=-1).numpy())) < 1e-12


def pin_merge_split():
    """Splitting the keys of causal attention at P and merging the two partials (all of
    keys 0..P-1, then keys P.. causally) gives the causal attention of rows P.."""
    rng = np.random.default_rng(24)
    B, N, Hq, Hkv, d, dv = 2, 60, 4, 2, 8, 8
    q, k, v = _rand(rng, B, N, Hq, d), _rand(rng, B, N, Hkv, d), _rand(rng, B, N, Hkv, dv)
    o, lse = oracle.causal_attention(q, k, v, 0.5)
    for p in (1, 17, 59):
        oa, la = oracle.offset_attention(q[:, p:], k[:, :p], v[:, :p], 0.5, p)
        ob, lb = oracle.offset_attention(q[:, p:], k[:, p:], v[:, p:], 0.5, 0)
        om, lm = oracle.merge_partials(oa, la, ob, lb)
        assert np.max(np.abs(om - o[:, p:])) < 1e-12
        assert np.max(np.abs(lm - lse[:, :, p:])) < 1e-12


def pin_merge_closed_forms():
    """An empty partial (LSE -inf) leaves the other unchanged; two identical partials
    give the same O and LSE + ln 2; both empty give O = 0, LSE = -inf."""
    rng = np.random.default_rng(25)
    o1 = _rand(rng, 1, 5, 3, 4)
    l1 = _rand(rng, 1, 3, 5)
    empty = np.full_like(l1, -np.inf)
    om, lm = oracle.merge_partials(o1, l1, _rand(rng, 1, 5, 3, 4), empty)
    assert np.array_equal(om, o1) and np.array_equal(lm, l1)
    om, lm = oracle.merge_partials(o1, l1, o1, l1)
    assert np.max(np.abs(om - o1)) < 1e-15 and np.max(np.abs(lm - (l1 + math.log(2)))) < 1e-14
    om, lm = oracle.merge_partials(o1, empty, o1, empty)
    assert np.all(om == 0) and np.all(lm == -np.inf)


ALL_PINS = [pin_bruteforce, pin_sdpa, pin_equal_scores, pin_row_zero, pin_hardmax,
            pin_rows_sum_to_one, pin_causality, pin_gqa_equals_repeated_mha,
            pin_rows_match_full, pin_offset_bruteforce, pin_offset_chunk_identity,
            pin_offset_all_visible_sdpa, pin_merge_split, pin_merge_closed_forms]
