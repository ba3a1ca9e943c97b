"""Seeded synthetic inputs for causal prefill attention.

This module only draws input tensors.  It holds none of the attention
arithmetic, no quantisation and no rounding to a storage format: it returns
float32 numpy arrays in the (B, N, H, d) "BSHD" layout that both the HIP
library and the CPU oracle consume.  Casting to bf16 or quantising to e4m3 is
done by the caller (torch for the bf16 cast, the library or the oracle for
e4m3).

The workloads stand in for the ones the ZYFA write-ups measure:

* Gaussian inputs at 32K tokens, head dim 128 and the MLA shape (the
  Gaussian benchmark figures on the-ai.news "Reele winsten en
  nauwkeurigheid" and spke.com "ZYFAはどのくらい速いのか?").
* Captured Mistral-7B and DeepSeek-V2-Lite activations at 16K (same
  sections).  Those activations are not available; the "mistral16k" and
  "mla16k" recipes below are synthetic stand-ins with the head counts of
  those models, lognormal per-channel spread with outlier channels and RoPE.
"""
from __future__ import annotations

import dataclasses
import numpy as np

__all__ = ["Workload", "CONFIGS", "get", "generate", "causal_flops"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    d_qk: int
    d_v: int
    seed: int
    recipe: str            # "gauss", "mistral", "mla"
    fp8_per_head: bool     # e4m3 scale granularity: per head (True) or per tensor
    rope_theta: float = 0.0
    rope_dims: int = 0     # number of trailing dims of d_qk that carry RoPE (MLA)
    description: str = ""

    @property
    def softmax_scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d_qk))

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


CONFIGS: dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny", 1, 2, 2, 256, 128, 128, 0, "gauss", False,
                 description="B=1 Hq=Hkv=2 N=256 d=128, iid N(0,1), per-tensor e4m3 scale"),
        Workload("mid_gqa", 1, 32, 8, 4096, 128, 128, 1, "gauss", True,
                 description="B=1 Hq=32 Hkv=8 N=4096 d=128, iid N(0,1), per-head e4m3 scales"),
        Workload("mistral16k", 1, 32, 8, 16384, 128, 128, 2, "mistral", True, rope_theta=1e6,
                 description="B=1 Hq=32 Hkv=8 N=16384 d=128, lognormal channel std with 4 x20 "
                             "outlier channels per head, RoPE theta=1e6 on Q/K, V iid N(0,1), "
                             "per-head e4m3 scales"),
        Workload("gauss32k", 1, 32, 8, 32768, 128, 128, 3, "gauss", False,
                 description="B=1 Hq=32 Hkv=8 N=32768 d=128, iid N(0,1), per-tensor e4m3 scale"),
        Workload("mla16k", 1, 16, 16, 16384, 192, 128, 4, "mla", True, rope_theta=1e4, rope_dims=64,
                 description="B=1 H=16 N=16384 d_qk=192 (128 no-rope + 64 RoPE dims, K rope part "
                             "shared across heads) d_v=128, iid N(0,1), per-head e4m3 scales"),
        Workload("mla32k", 1, 16, 16, 32768, 192, 128, 5, "mla", True, rope_theta=1e4, rope_dims=64,
                 description="as mla16k at N=32768"),
    ]
}


def get(name: str) -> Workload:
    return CONFIGS[name]


def causal_flops(w: Workload) -> float:
    """Useful causal FLOPs: 2 products (QK^T over d_qk, PV over d_v), 2 flop per
    multiply-add, over the N^2/2 lower triangle.  For d_qk == d_v == d this is
    4*B*Hq*N^2*d/2."""
    return 2.0 * w.B * w.Hq * float(w.N) ** 2 * (w.d_qk + w.d_v) / 2.0


def _rope(x: np.ndarray, theta: float) -> np.ndarray:
    """Rotate-half rotary embedding over the last axis of x (B, N, H, dr),
    position = token index; pairs are (c, c + dr/2)."""
    B, N, H, dr = x.shape
    half = dr // 2
    inv_freq = theta ** (-np.arange(half, dtype=np.float64) * 2.0 / dr)
    ang = np.arange(N, dtype=np.float64)[:, None] * inv_freq[None, :]
    cos = np.cos(ang).astype(np.float32)[None, :, None, :]
    sin = np.sin(ang).astype(np.float32)[None, :, None, :]
    x1 = x[..., :half]
    x2 = x[..., half:]
    out = np.empty_like(x)
    out[..., :half] = x1 * cos - x2 * sin
    out[..., half:] = x2 * cos + x1 * sin
    return out


def _outlier_channels(rng: np.random.Generator, H: int, d: int, n_out: int = 4,
                      factor: float = 20.0) -> np.ndarray:
    """Per-head channel std: lognormal(0, 0.5), with n_out distinct channels
    per head multiplied by `factor`.  Returns (H, d) float32."""
    sig = rng.lognormal(mean=0.0, sigma=0.5, size=(H, d)).astype(np.float32)
    for h in range(H):
        idx = rng.choice(d, size=n_out, replace=False)
        sig[h, idx] *= factor
    return sig


def generate(w: Workload) -> dict[str, np.ndarray]:
    """Draw q (B,N,Hq,d_qk), k (B,N,Hkv,d_qk), v (B,N,Hkv,d_v) as float32.

    Draw order from numpy's PCG64 default_rng(seed): Q, K, V, then the
    recipe's extras.  Same seed and numpy version give the same bytes.
    """
    rng = np.random.default_rng(w.seed)
    B, N, Hq, Hkv, dqk, dv = w.B, w.N, w.Hq, w.Hkv, w.d_qk, w.d_v
    if w.recipe == "gauss":
        q = rng.standard_normal((B, N, Hq, dqk), dtype=np.float32)
        k = rng.standard_normal((B, N, Hkv, dqk), dtype=np.float32)
        v = rng.standard_normal((B, N, Hkv, dv), dtype=np.float32)
    elif w.recipe == "mistral":
        q = rng.standard_normal((B, N, Hq, dqk), dtype=np.float32)
        k = rng.standard_normal((B, N, Hkv, dqk), dtype=np.float32)
        v = rng.standard_normal((B, N, Hkv, dv), dtype=np.float32)
        q *= _outlier_channels(rng, Hq, dqk)[None, None]
        k *= _outlier_channels(rng, Hkv, dqk)[None, None]
        q = _rope(q, w.rope_theta)
        k = _rope(k, w.rope_theta)
    elif w.recipe == "mla":
        assert Hq == Hkv, "MLA recipe is written for Hq == Hkv"
        dr = w.rope_dims
        q = rng.standard_normal((B, N, Hq, dqk), dtype=np.float32)
        k = np.empty((B, N, Hkv, dqk), dtype=np.float32)
        k[..., : dqk - dr] = rng.standard_normal((B, N, Hkv, dqk - dr), dtype=np.float32)
        v = rng.standard_normal((B, N, Hkv, dv), dtype=np.float32)
        k_rope = rng.standard_normal((B, N, 1, dr), dtype=np.float32)
        q[..., dqk - dr:] = _rope(np.ascontiguousarray(q[..., dqk - dr:]), w.rope_theta)
        k[..., dqk - dr:] = _rope(k_rope, w.rope_theta)  # broadcast over heads
    else:
        raise ValueError(f"unknown recipe {w.recipe!r}")
    return {"q": np.ascontiguousarray(q), "k": np.ascontiguousarray(k),
            "v": np.ascontiguousarray(v)}
