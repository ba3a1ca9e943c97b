"""Plant mistakes in the oracle (on the CPU) and require a pin to catch each.

This shows the pins are strong enough that a plausible slip in the oracle --
an off-by-one causal mask, no mask, a wrong GQA head mapping, a dropped
scale, a missing max in the LSE, a wrong channel index, a wrong normaliser, an
ignored or doubled query offset, a merge that averages, swaps or drops the
log-sum of its weights -- cannot pass unnoticed.
"""
import numpy as np
import pytest

import oracle
import oracle.attention as att
from oracle_pins import ALL_PINS


def _mutant_rows(kind):
    def rows(q_rows, k, v, scale, i_abs, q_offset=0):
        nk = max(att.visible_keys(int(i), q_offset, k.shape[0]) for i in i_abs)
        if kind == "no_mask":
            nk = k.shape[0]
        if kind == "reversed_channels":
            s = scale * (q_rows @ k[:nk, ::-1].T)
        elif kind == "no_scale":
            s = q_rows @ k[:nk].T
        else:
            s = scale * (q_rows @ k[:nk].T)
        lim = np.array([att.visible_keys(int(i), q_offset, k.shape[0]) for i in i_abs])
        mask = np.arange(nk)[None, :] < lim[:, None]
        if kind != "no_mask":
            s = np.where(mask, s, -np.inf)
        m = np.max(s, axis=1, keepdims=True)
        e = np.exp(s - m)
        l = np.sum(e, axis=1, keepdims=True)
        if kind == "unnormalised":
            o = e @ v[:nk]
        elif kind == "square_weights":
            o = ((e ** 2) @ v[:nk]) / np.sum(e ** 2, axis=1, keepdims=True)
        else:
            o = (e @ v[:nk]) / l
        if kind == "lse_no_max":
            lse = np.log(l[:, 0])
        elif kind == "lse_log2":
            lse = m[:, 0] + np.log2(l[:, 0])
        else:
            lse = m[:, 0] + np.log(l[:, 0])
        return o, lse
    return rows


def _clamp(n, n_keys):
    return n if n_keys is None else min(n, n_keys)


def _merge_mutant(kind):
    real = att.merge_partials

    def merge(o_a, lse_a, o_b, lse_b):
        o, lse = real(o_a, lse_a, o_b, lse_b)
        if kind == "plain_average":
            o = 0.5 * (np.asarray(o_a) + np.asarray(o_b))
        elif kind == "lse_max_only":
            lse = np.maximum(lse_a, lse_b)
        elif kind == "swapped_weights":
            o, _ = real(o_b, lse_a, o_a, lse_b)
        return o, lse
    return merge


MUTANTS = {
    "mask_excludes_diagonal": ("visible_keys",
                               lambda i, q_offset=0, n_keys=None: _clamp(max(i + q_offset, 1), n_keys)),
    "mask_one_extra_key": ("visible_keys",
                           lambda i, q_offset=0, n_keys=None: _clamp(i + q_offset + 2, n_keys)),
    "offset_ignored": ("visible_keys", lambda i, q_offset=0, n_keys=None: _clamp(i + 1, n_keys)),
    "offset_doubled": ("visible_keys",
                       lambda i, q_offset=0, n_keys=None: _clamp(i + 2 * q_offset + 1, n_keys)),
    "merge_plain_average": ("merge_partials", _merge_mutant("plain_average")),
    "merge_lse_max_only": ("merge_partials", _merge_mutant("lse_max_only")),
    "merge_swapped_weights": ("merge_partials", _merge_mutant("swapped_weights")),
    "no_mask": ("_rows", _mutant_rows("no_mask")),
    "gqa_modulo": ("kv_head_of", lambda h, Hq, Hkv: h % Hkv),
    "gqa_always_zero": ("kv_head_of", lambda h, Hq, Hkv: 0),
    "channel_index_reversed": ("_rows", _mutant_rows("reversed_channels")),
    "dropped_scale": ("_rows", _mutant_rows("no_scale")),
    "unnormalised": ("_rows", _mutant_rows("unnormalised")),
    "squared_weights": ("_rows", _mutant_rows("square_weights")),
    "lse_without_max": ("_rows", _mutant_rows("lse_no_max")),
    "lse_base2": ("_rows", _mutant_rows("lse_log2")),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(att, attr, fn)
    if hasattr(oracle, attr):          # the package re-exports some functions
        monkeypatch.setattr(oracle, attr, fn)
    caught = []
    for pin in ALL_PINS:
        try:
            pin()
        except Exception:   # AssertionError, or a shape error the mistake causes
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
