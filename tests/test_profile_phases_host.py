"""Host logic of profile_phases.timeline(): synthetic phase-timer records (the layout of
include/attn_phase_timers.h) with hand-chosen real-time stamps and hardware ids, and the
figures worked out by hand.  Eight XCDs, one CU each (on shader engine x mod 4), two
workgroups per CU one after the other, 0.4 µs apart; the odd XCDs take 1.1 times as long
in every phase."""
import numpy as np
import pytest

import profile_phases as pp

WAVES, WORDS = pp.WAVES, pp.WORDS


def _records():
    rec = np.zeros((16, WAVES, WORDS), dtype=np.int64)
    for x in range(8):
        f = 1.1 if x % 2 else 1.0
        pro, loop, epi = round(250 * f), round(1800 * f), round(130 * f)   # ticks (10 ns)
        hw = (x % 4) << 13                                                  # engine x mod 4, CU 0
        t = 1000
        for k in range(2):
            wg = 2 * x + k
            rec[wg, :, 4] = t                     # start
            rec[wg, :, 5] = t + pro               # loop entry
            rec[wg, :, 6] = t + pro + loop        # loop exit
            rec[wg, :, 7] = t + pro + loop + epi  # stores issued
            rec[wg, :, 8] = 9                     # key tiles: 10 matrix phases
            rec[wg, :, 9] = hw | (x << 32)
            t = t + pro + loop + epi + 40         # next workgroup 0.4 µs later
    return rec


def test_timeline_figures():
    span_us = (1000 + 2 * (275 + 1980 + 143) + 40 - 1000) / 100.0
    tl = pp.timeline(_records(), span_us / 1e3)
    assert tl["workgroups"] == 16 and tl["cus"] == 8 and tl["pairs"] == 8
    assert tl["prologue"] == pytest.approx((2.5 + 2.75) / 2)
    assert tl["epilogue"] == pytest.approx((1.3 + 1.43) / 2)
    assert tl["tile"] == pytest.approx((1.8 + 1.98) / 2)
    assert tl["gap_mean"] == pytest.approx(0.4) and tl["gap_median"] == pytest.approx(0.4)
    assert tl["span_over_event_mhz"] == pytest.approx(100.0)
    even, odd = 2 * 21.8, 2 * 23.98                    # busy µs per CU
    assert tl["xcd_busy"] == pytest.approx([even, odd] * 4)
    assert tl["odd_over_even"] == pytest.approx(odd / even)
    assert tl["span_over_mean_xcd"] == pytest.approx(span_us / ((even + odd) / 2))
    assert tl["se_gap"] == pytest.approx([0.4] * 4)


def test_timeline_ignores_unused_records():
    rec = np.concatenate([_records(), np.zeros((5, WAVES, WORDS), dtype=np.int64)])
    assert pp.timeline(rec, 1.0)["workgroups"] == 16
