"""The oracle's joint Q/K quantisation that stores each KV group's largest-product
channels last (oracle.quantize_e4m3_qk_outliers), pinned on the CPU:

* a hand-worked example whose answer depends on every part of the rule (K's magnitude
  counts, the maximum over the group's query heads and not their sum, ties to the
  lower channel, both parts in ascending order);
* brute force over random tensors: the stored-last set is exactly the top of the
  importance order, and the rest is a permutation;
* the codes are quantize_e4m3's (quantize_e4m3_q_pow2's for Q) permuted, with
  bit-identical descales, so every decoded score Q.K is unchanged;
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


@pytest.mark.parametrize("per_head,pow2", [(True, False), (False, False), (True, True)])
def test_codes_are_plain_codes_permuted(per_head, pow2):
    w = workloads.CONFIGS["mistral16k"].with_(N=96, Hq=8, Hkv=2, seed=61)
    x = workloads.generate(w)
    scale = w.softmax_scale if pow2 else None
    qc, kc, qd, kd, perm = oracle.quantize_e4m3_qk_outliers(x["q"], x["k"], per_head,
                                                            q_pow2_scale=scale)
    kc0, kd0 = oracle.quantize_e4m3(x["k"], per_head)
    if pow2:
        qc0, qd0 = oracle.quantize_e4m3_q_pow2(x["q"], per_head, kd0, scale)
    else:
        qc0, qd0 = oracle.quantize_e4m3(x["q"], per_head)
    assert np.array_equal(qd.view(np.uint32), qd0.view(np.uint32))
    assert np.array_equal(kd.view(np.uint32), kd0.view(np.uint32))
    G = w.Hq // w.Hkv
    for h in range(w.Hq):
        assert np.array_equal(qc[:, :, h], qc0[:, :, h][..., perm[h // G]])
    for g in range(w.Hkv):
        assert np.array_equal(kc[:, :, g], kc0[:, :, g][..., perm[g]])
    # a common permutation of Q's and K's channels leaves every score unchanged
    bq = lambda c, d_: oracle.e4m3_decode(c) * (d_[None, None, :, None].astype(np.float64)
                                                 if per_head else float(d_[0]))
    s_perm = np.einsum("bihc,bjhc->bhij", bq(qc, qd), np.repeat(bq(kc, kd), G, axis=2))
    s_plain = np.einsum("bihc,bjhc->bhij", bq(qc0, qd0), np.repeat(bq(kc0, kd0), G, axis=2))
    assert np.allclose(s_perm, s_plain, rtol=1e-12, atol=1e-12 * np.abs(s_plain).max())
    # the outlier channels of the recipe end up among the stored-last ones
    sq = formats.channel_absmax(x["q"])
    for g in range(w.Hkv):
        top_q = set(np.argsort(-sq[g * G:(g + 1) * G].max(axis=0), kind="stable")[:4].tolist())
        assert top_q <= set(perm[g, -oracle.OUTLIER_CHANNELS:].tolist())


# ---- the grouped accumulation of the FP8 matrix instruction, modelled ------------------
# Measured through the C ABI (test_gpu_parity.py, accumulation tests): each run of 8
# consecutive channel products is added after truncating every product toward zero to
# a multiple of 2^(E - 13), E the exponent of the run's largest product.

def _grouped_dot(q, K):
    p = q[None, :] * K
    pg = p.reshape(p.shape[0], -1, 8)
    mx = np.max(np.abs(pg), axis=2, keepdims=True)
    E = np.floor(np.log2(np.where(mx > 0, mx, 1.0)))
    ulp = np.exp2(E - 13)
    return (np.trunc(pg / ulp) * ulp).sum(axis=(1, 2))


def _modelled_lse_error(qv, kv, qd, kd, scale, n_exact, rows):
    """Worst |LSE| change over `rows` when the last n_exact stored channels are
    multiplied exactly and the rest through the modelled FP8 accumulation."""
    G = qv.shape[2] // kv.shape[2]
    worst = 0.0
    d = qv.shape[3]
    split = np.arange(d) >= d - n_exact
    for h, i in rows:
        g = h // G
        K, q = kv[0, : i + 1, g], qv[0, i, h]
        sc = float(qd[h]) * float(kd[g]) * scale
        exact = np.logaddexp.reduce((K @ q) * sc)
        model = _grouped_dot(np.where(split, 0.0, q), K) + K[:, split] @ q[split]
        worst = max(worst, abs(np.logaddexp.reduce(model * sc) - exact))
    return worst


def test_exact_channels_keep_the_lse_inside_the_gate_on_outlier_inputs():
    w = workloads.CONFIGS["mistral16k"].with_(N=512, seed=25)
    x = workloads.generate(w)
    qc, kc, qd, kd, _ = oracle.quantize_e4m3_qk_outliers(x["q"], x["k"], True)
    qv, kv = oracle.e4m3_decode(qc), oracle.e4m3_decode(kc)
    rng = np.random.default_rng(3)
    rows = [(int(rng.integers(w.Hq)), int(rng.integers(w.N))) for _ in range(800)]
    plain = _modelled_lse_error(qv, kv, qd, kd, w.softmax_scale, 0, rows)
    split = _modelled_lse_error(qv, kv, qd, kd, w.softmax_scale, oracle.OUTLIER_CHANNELS, rows)
    print(f"modelled worst LSE error: all channels FP8 {plain:.4f}, "
          f"last {oracle.OUTLIER_CHANNELS} exact {split:.5f}")
    assert plain > 1e-2
    assert split < 2.5e-3
