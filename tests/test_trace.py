"""Trace decoding and summary (host logic) on hand-built records."""

import ctypes

import numpy as np
import pytest

import tile_level_sync_amd as tls
from tile_level_sync_amd import trace


def _recs(rows):
    a = np.zeros(len(rows), dtype=trace.REC)
    for i, (item, wg, hw, ts, tr, te) in enumerate(rows):
        a[i] = (item, wg, hw, ts, tr, te)
    return a


def test_record_layout_matches_the_c_struct():
    assert trace.REC.itemsize == ctypes.sizeof(tls.chain_trace_rec) == 32
    for name in trace.REC.names:
        assert trace.REC.fields[name][1] == getattr(tls.chain_trace_rec, name).offset


def test_decode_skips_unwritten_records():
    a = _recs([(0, 0, 1, 10, 10, 20), (1, 1, 2, 12, 15, 30)])
    buf = np.zeros(4 * 32, dtype=np.uint8)
    buf[:64] = np.frombuffer(a.tobytes(), dtype=np.uint8)
    d = trace.decode(buf)
    assert len(d) == 2 and list(d["item"]) == [0, 1]


def test_summary_closed_form():
    # 1000 kHz clock: one tick = 1 us.  Two CUs over [0, 100):
    #   CU 1 runs producer 0 on [0, 40) and consumer 2 on [40, 100) (ready at 50);
    #   CU 2 runs producer 1 on [0, 30), then consumer 3 on [35, 80) (ready at 60).
    r = _recs([(0, 0, 1, 0, 0, 40), (2, 0, 1, 40, 50, 100),
               (1, 1, 2, 0, 0, 30), (3, 1, 2, 35, 60, 80)])
    s = trace.summarize(r, producer_items=2, clock_khz=1000)
    assert s["span_us"] == pytest.approx(100)
    assert s["busy_frac"] == pytest.approx((100 + 75) / 200)
    assert s["tail_idle_frac"] == pytest.approx((0 + 20) / 200)
    assert s["producer_phase_us"] == pytest.approx(40)
    assert s["consumer_wait_mean_us"] == pytest.approx((10 + 25) / 2)
    assert s["consumer_wait_max_us"] == pytest.approx(25)
    assert s["producer_consumer_gap_us"] == pytest.approx(35 - 40)
    # a third CU that ran nothing is idle for the whole span
    s3 = trace.summarize(r, producer_items=2, clock_khz=1000, n_cu=3)
    assert s3["tail_idle_frac"] == pytest.approx((0 + 20 + 100) / 300)


def test_overlapping_workgroups_on_one_cu_count_once():
    r = _recs([(0, 0, 7, 0, 0, 60), (1, 1, 7, 20, 20, 100)])
    s = trace.summarize(r, producer_items=2, clock_khz=1000)
    assert s["busy_frac"] == pytest.approx(1.0)
    assert s["tail_idle_frac"] == pytest.approx(0.0)
