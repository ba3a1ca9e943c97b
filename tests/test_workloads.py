"""Seeded synthetic inputs: reproducibility and the statistics each recipe states."""
import numpy as np

import workloads


def test_configs_shapes():
    assert set(workloads.CONFIGS) == {"tiny", "mid_gqa", "mistral16k", "gauss32k", "mla16k", "mla32k"}
    g = workloads.get("gauss32k")
    assert (g.B, g.Hq, g.Hkv, g.N, g.d_qk, g.d_v) == (1, 32, 8, 32768, 128, 128)
    m = workloads.get("mla32k")
    assert (m.Hq, m.Hkv, m.N, m.d_qk, m.d_v) == (16, 16, 32768, 192, 128)
    assert abs(workloads.causal_flops(g) - 4 * 32 * 32768 ** 2 * 128 / 2) < 1
    assert abs(workloads.causal_flops(m) - 2 * 16 * 32768 ** 2 * 320 / 2) < 1


def test_reproducible_and_shapes():
    w = workloads.get("tiny")
    a, b = workloads.generate(w), workloads.generate(w)
    for n in "qkv":
        assert a[n].dtype == np.float32 and np.array_equal(a[n], b[n])
    assert a["q"].shape == (1, 256, 2, 128)
    assert abs(a["q"].std() - 1) < 0.02


def test_mistral_recipe_outliers_and_rope_norm():
    w = workloads.get("mistral16k").with_(N=512)
    x = workloads.generate(w)
    q = x["q"]
    # RoPE is a rotation of channel pairs: per-token pair norms equal the
    # unrotated draw's; position 0 is unrotated.  Channel spread: a few
    # channels per head carry ~20x larger scale.
    std = q.std(axis=(0, 1))                 # (H, d), pairs mixed by RoPE
    pair = np.sqrt(std[:, :64] ** 2 + std[:, 64:] ** 2)
    big = (pair > 8).sum(axis=1)
    assert np.all(big >= 1) and np.all(big <= 4)


def test_mla_recipe_shared_rope_dims():
    w = workloads.get("mla16k").with_(N=64)
    x = workloads.generate(w)
    k = x["k"]
    assert k.shape == (1, 64, 16, 192)
    assert np.array_equal(k[:, :, 0, 128:], k[:, :, 7, 128:])       # shared across heads
    assert not np.array_equal(k[:, :, 0, :128], k[:, :, 7, :128])
