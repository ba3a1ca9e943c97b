"""The oracle's joint Q/K quantisation that stores each KV group's largest-product
channels last (oracle.quantize_e4m3_qk_outliers), pinned on the CPU:

* a hand-worked example whose answer depends on every part of the rule (K's magnitude
  counts, the maximum over the group's query heads and not their sum, ties to the
  lower channel, both parts in ascending order);
* brute force over random tensors: the stored-last set is exactly the top of the
  importance order, and the rest is a permutation;
* the codes are quantize_e4m3's (quantize_e4m3_q_pow2's for Q) permuted, with
  bit-identical descales, so every decoded score Q.K is unchanged;
* the bf16 side arrays of the last 32 stored channels are torch's bf16 cast of the
  float32 quotient x / descale (the bf16 encoder itself is pinned against that cast),
  and the decoded values differ from the codes' only by the finer rounding;
* what the permutation is for, on a model of the FP8 matrix instruction's grouped
  accumulation (the model itself is pinned on the GPU by the accumulation tests in
  test_gpu_parity.py): without the exact channels the LSE of outlier-channel inputs
  moves by far more than 1e-2, with them it stays well inside.
"""
import numpy as np
import pytest

import oracle
import workloads
from oracle import formats


def _with_absmax(amax_per_head, n=3, seed=0):
    """(1, n, H, d) float32 whose per-(head, channel) absmax is amax_per_head (H, d):
    row 0 holds the maxima (signs alternating), the other rows smaller values."""
    a = np.asarray(amax_per_head, np.float32)
    rng = np.random.default_rng(seed)
    x = (rng.uniform(-0.5, 0.5, size=(1, n) + a.shape) * a).astype(np.float32)
    sign = np.where(np.arange(a.shape[-1]) % 2 == 0, 1.0, -1.0).astype(np.float32)
    x[0, 0] = a * sign
    return x


def test_hand_example():
    """Hq = 2 query heads on one KV head, d = 8, n_split = 2.
    Q absmax: head 0 [1, 1, 9, 1, 4, 1, 1, 1], head 1 [1, 1, 1, 1, 4, 1, 1, 7]
    K absmax:        [1, 8, 1, 1, 1, 1, 1, 1]
    importance = max over heads of Q x K = [1, 8, 9, 1, 4, 1, 1, 7]:
    stored last are channels 2 (9) and 1 (8), in ascending order, after 0, 3..7.
    A rule that ignored K would pick 2 and 7; one that summed the heads (channel 4
    sums to 8, ties channel 1 and wins nothing, but 4 + 4 > 7) would differ on the
    next example; see test_hand_example_sum_vs_max."""
    q = _with_absmax([[1, 1, 9, 1, 4, 1, 1, 1], [1, 1, 1, 1, 4, 1, 1, 7]])
    k = _with_absmax([[1, 8, 1, 1, 1, 1, 1, 1]])
    perm = oracle.outlier_permutation(oracle.channel_absmax(q), oracle.channel_absmax(k), 2)
    assert perm.tolist() == [[0, 3, 4, 5, 6, 7, 1, 2]]


def test_hand_example_sum_vs_max():
    """Channel 4 has Q absmax 4 in both heads: its importance is max(4, 4) * 1 = 4, not
    8, so channel 7 (7) is chosen with channel 2 (9); ties at importance 1 do not enter."""
    q = _with_absmax([[1, 1, 9, 1, 4, 1, 1, 1], [1, 1, 1, 1, 4, 1, 1, 7]])
    k = _with_absmax([[1, 1, 1, 1, 1, 1, 1, 1]])
    perm = oracle.outlier_permutation(oracle.channel_absmax(q), oracle.channel_absmax(k), 2)
    assert perm.tolist() == [[0, 1, 3, 4, 5, 6, 2, 7]]


def test_ties_go_to_the_lower_channel():
    q = _with_absmax([[2, 3, 3, 3, 1, 3]])
    k = _with_absmax([[1, 1, 1, 1, 1, 1]])
    perm = oracle.outlier_permutation(oracle.channel_absmax(q), oracle.channel_absmax(k), 2)
    assert perm.tolist() == [[0, 3, 4, 5, 1, 2]]


def test_zero_infinite_and_nan_channels():
    """An all-zero channel has importance 0 whatever the other factor (no 0 * inf);
    an infinite absmax ranks first; NaN elements take no part in the absmax."""
    q = _with_absmax([[0, 1, 1, 1, 1, np.inf]])
    k = _with_absmax([[np.inf, 1, 2, 1, 1, 1]])
    q[0, 1, 0, 3] = np.nan
    am_q, am_k = oracle.channel_absmax(q), oracle.channel_absmax(k)
    assert am_q[0, 3] == 1.0 and am_q[0, 0] == 0.0
    perm = oracle.outlier_permutation(am_q, am_k, 2)
    assert perm.tolist() == [[0, 1, 3, 4, 2, 5]]


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_selection(seed):
    rng = np.random.default_rng(100 + seed)
    Hq, Hkv, d, T = [(4, 2, 16, 4), (6, 3, 12, 5), (2, 2, 8, 8), (8, 1, 24, 1),
                     (4, 4, 16, 3), (3, 1, 32, 32)][seed]
    am_q = rng.choice(np.float32([0, 0.5, 1, 2, 3, 7.5]), size=(Hq, d)).astype(np.float32)
    am_k = rng.choice(np.float32([0, 1, 2, 4]), size=(Hkv, d)).astype(np.float32)
    perm = oracle.outlier_permutation(am_q, am_k, T)
    G = Hq // Hkv
    for g in range(Hkv):
        assert sorted(perm[g].tolist()) == list(range(d))
        imp = [float(np.float32(max(am_q[h, c] for h in range(g * G, (g + 1) * G)) * am_k[g, c]))
               for c in range(d)]
        best = sorted(range(d), key=lambda c: (-imp[c], c))[:T]
        assert sorted(best) == perm[g, d - T:].tolist()
        assert perm[g, : d - T].tolist() == sorted(set(range(d)) - set(best))


def test_bf16_encoder_matches_torch_cast():
    import torch
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(200000).astype(np.float32) * s
                        for s in (1e-38, 1e-20, 1e-3, 1.0, 1e3, 1e30)] +
                       [np.float32([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, 3.39e38,
                                    -3.39e38, 1.00390625, 1.01171875, 1.0078125])])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_encode(x), ref)
    assert oracle.bf16_encode(np.float32([np.nan]))[0] == 0x7FC0


@pytest.mark.parametrize("per_head,pow2", [(True, False), (False, False), (True, True)])
def test_codes_are_plain_codes_permuted(per_head, pow2):
    import torch
    w = workloads.CONFIGS["mistral16k"].with_(N=96, Hq=8, Hkv=2, seed=61)
    x = workloads.generate(w)
    scale = w.softmax_scale if pow2 else None
    qc, kc, qx, kx, qd, kd, perm = oracle.quantize_e4m3_qk_outliers(x["q"], x["k"], per_head,
                                                                    q_pow2_scale=scale)
    kc0, kd0 = oracle.quantize_e4m3(x["k"], per_head)
    if pow2:
        qc0, qd0 = oracle.quantize_e4m3_q_pow2(x["q"], per_head, kd0, scale)
    else:
        qc0, qd0 = oracle.quantize_e4m3(x["q"], per_head)
    assert np.array_equal(qd.view(np.uint32), qd0.view(np.uint32))
    assert np.array_equal(kd.view(np.uint32), kd0.view(np.uint32))
    G = w.Hq // w.Hkv
    T = oracle.OUTLIER_CHANNELS
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(
        torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for h in range(w.Hq):
        assert np.array_equal(qc[:, :, h], qc0[:, :, h][..., perm[h // G]])
        ds = np.float32(qd[h] if per_head else qd[0])
        assert np.array_equal(qx[:, :, h], bf(x["q"][:, :, h][..., perm[h // G][-T:]] / ds))
    for g in range(w.Hkv):
        assert np.array_equal(kc[:, :, g], kc0[:, :, g][..., perm[g]])
        ds = np.float32(kd[g] if per_head else kd[0])
        assert np.array_equal(kx[:, :, g], bf(x["k"][:, :, g][..., perm[g][-T:]] / ds))
    # a common permutation of Q's and K's channels leaves every score unchanged
    bq = lambda c, d_: oracle.e4m3_decode(c) * (d_[None, None, :, None].astype(np.float64)
                                                 if per_head else float(d_[0]))
    s_perm = np.einsum("bihc,bjhc->bhij", bq(qc, qd), np.repeat(bq(kc, kd), G, axis=2))
    s_plain = np.einsum("bihc,bjhc->bhij", bq(qc0, qd0), np.repeat(bq(kc0, kd0), G, axis=2))
    assert np.allclose(s_perm, s_plain, rtol=1e-12, atol=1e-12 * np.abs(s_plain).max())
    # the side arrays hold the same channels more finely: decoded values within half an
    # e4m3 step of the codes' values, and within half a bf16 step of x
    vq = oracle.decode_qk_outliers(qc, qx, qd, per_head)
    cq = bq(qc, qd)
    xs = np.stack([x["q"][:, :, h][..., perm[h // G]] for h in range(w.Hq)], axis=2)
    assert np.array_equal(vq[..., :-T], cq[..., :-T])
    assert np.all(np.abs(vq[..., -T:] - xs[..., -T:]) <= 2.0 ** -8 * np.abs(xs[..., -T:]) + 1e-30)
    assert np.all(np.abs(vq[..., -T:] - cq[..., -T:]) <=
                  2.0 ** -4 * np.abs(xs[..., -T:]) + 2.0 ** -8 * np.abs(xs[..., -T:]) +
                  2.0 ** -10 * (qd.max() if per_head else qd[0]))
    # the outlier channels of the recipe end up among the stored-last ones
    sq = formats.channel_absmax(x["q"])
    for g in range(w.Hkv):
        top_q = set(np.argsort(-sq[g * G:(g + 1) * G].max(axis=0), kind="stable")[:4].tolist())
        assert top_q <= set(perm[g, -T:].tolist())


# ---- the grouped accumulation of the FP8 matrix instruction, modelled ------------------
# Measured through the C ABI (test_gpu_parity.py, accumulation tests): each run of 8
# consecutive channel products is added after truncating every product toward zero to
# a multiple of 2^(E - 13), E the largest exponent sum e_q + e_k of the run's e4m3
# factor pairs (subnormals count as exponent -6).

def _e4m3_exponent(codes):
    e = (np.asarray(codes, np.int64) >> 3) & 0xF
    return np.where(e == 0, -6, e - 7)


def _grouped_dot(q, K, eq, eK):
    """q (d,), K (M, d) e4m3 values with exponents eq, eK -> the modelled FP8 dots."""
    p = q[None, :] * K
    M, d = p.shape
    pg = p.reshape(M, d // 8, 8)
    es = (eq[None, :] + eK).reshape(M, d // 8, 8)
    E = np.max(np.where(pg != 0, es, -100), axis=2, keepdims=True)
    ulp = np.exp2(E - 13.0)
    return (np.trunc(pg / ulp) * ulp).sum(axis=(1, 2))


def test_grouped_accumulation_model_reproduces_the_measured_cases():
    """The model gives the scores the GPU gave in the accumulation tests."""
    code = {1.0: 0x38, 1.5: 0x3C, 2.0: 0x40, 256.0: 0x78, 64.0: 0x68, 240.0: 0x77,
            120.0: 0x6F, 0.5: 0x30}
    cases = [((256, 64), (1.0, 1.0), 16384.0), ((256, 64), (1.0, -1.0), 16384.0),
             ((256, 64), (1.5, 2.0), 16398.0), ((256, 64), (-1.5, 2.0), 16370.0),
             ((256, 64), (2.0, 2.0), 16412.0), ((256, 64), (-0.5, 1.0), 16384.0),
             ((240, 120), (1.5, 1.0), 28807.0)]
    for (a0, b0), (a, b), want in cases:
        qc = np.zeros(8, np.uint8)
        kc = np.zeros((1, 8), np.uint8)
        qc[0], kc[0, 0] = code[a0], code[b0]
        qc[1:] = code[abs(a)] | (0x80 if a < 0 else 0)
        kc[0, 1:] = code[abs(b)] | (0x80 if b < 0 else 0)
        got = _grouped_dot(oracle.e4m3_decode(qc), oracle.e4m3_decode(kc),
                           _e4m3_exponent(qc), _e4m3_exponent(kc))[0]
        assert got == want, (a0, b0, a, b, got, want)


def _modelled_lse_error(qc, kc, qd, kd, scale, n_exact, rows, qv=None, kv=None):
    """Worst |LSE| change over `rows` when the last n_exact stored channels are
    multiplied exactly and the rest through the modelled FP8 accumulation (qv, kv: the
    unscaled values, by default the codes' e4m3 values)."""
    if qv is None:
        qv, kv = oracle.e4m3_decode(qc), oracle.e4m3_decode(kc)
    qe, ke = _e4m3_exponent(qc), _e4m3_exponent(kc)
    G = qv.shape[2] // kv.shape[2]
    worst = 0.0
    d = qv.shape[3]
    split = np.arange(d) >= d - n_exact
    for h, i in rows:
        g = h // G
        K, q = kv[0, : i + 1, g], qv[0, i, h]
        sc = float(qd[h]) * float(kd[g]) * scale
        exact = np.logaddexp.reduce((K @ q) * sc)
        model = _grouped_dot(np.where(split, 0.0, q), K, qe[0, i, h], ke[0, : i + 1, g]) + \
            K[:, split] @ q[split]
        worst = max(worst, abs(np.logaddexp.reduce(model * sc) - exact))
    return worst


def test_exact_channels_keep_the_lse_inside_the_gate_on_outlier_inputs():
    w = workloads.CONFIGS["mistral16k"].with_(N=512, seed=25)
    x = workloads.generate(w)
    qc, kc, qx, kx, qd, kd, _ = oracle.quantize_e4m3_qk_outliers(x["q"], x["k"], True)
    one = np.ones_like(qd)
    qv = oracle.decode_qk_outliers(qc, qx, one, True)      # unscaled (code units)
    kv = oracle.decode_qk_outliers(kc, kx, np.ones_like(kd), True)
    rng = np.random.default_rng(3)
    rows = [(int(rng.integers(w.Hq)), int(rng.integers(w.N))) for _ in range(800)]
    plain = _modelled_lse_error(qc, kc, qd, kd, w.softmax_scale, 0, rows)
    split = _modelled_lse_error(qc, kc, qd, kd, w.softmax_scale, oracle.OUTLIER_CHANNELS, rows,
                                qv=qv, kv=kv)
    print(f"modelled worst LSE error: all channels FP8 {plain:.4f}, "
          f"last {oracle.OUTLIER_CHANNELS} exact {split:.5f}")
    assert plain > 1e-2
    assert split < 2.5e-3
