"""Host-side decoding and summary of the task trace (no GPU: synthetic words)."""
import numpy as np

from persistent_megakernel_04_amd import trace


def _buf(entries_per_wg, records):
    """records: per workgroup, a list of (type, layer, coord, clocks[7]) -> uint32 [grid][cap][8]."""
    grid = len(records)
    buf = np.zeros((grid, entries_per_wg, 8), dtype=np.uint32)
    for w, recs in enumerate(records):
        buf[w, 0, 0] = len(recs)
        for i, (ty, layer, coord, clocks) in enumerate(recs, start=1):
            buf[w, i, 0] = ty | (layer << 8) | (coord << 16)
            buf[w, i, 1:8] = clocks
    return buf


def test_decode_fields_and_phases():
    # one workgroup, two tasks; clocks in 10 ns ticks
    recs = [[(1, 0, 3, [100, 150, 200, 300, 320, 330, 340]), (3, 0, 7, [400, 700, 710, 800, 805, 810, 900])]]
    rec = trace.decode(_buf(4, recs))
    assert list(rec["type"]) == [1, 3] and list(rec["coord"]) == [3, 7]
    # microseconds from the earliest take
    np.testing.assert_allclose(rec["t0"], [0.0, 3.0])
    np.testing.assert_allclose(rec["ready"] - rec["t0"], [0.5, 3.0])
    np.testing.assert_allclose(rec["t1"] - rec["t0"], [2.4, 5.0])


def test_decode_clock_wrap():
    # the 32-bit clock wraps between the two records
    top = (1 << 32) - 50
    recs = [[(1, 0, 0, [top] * 7), (2, 0, 0, [20] * 7)]]
    rec = trace.decode(_buf(4, recs))
    np.testing.assert_allclose(rec["t0"], [0.0, 0.7])


def test_sync_overhead():
    # workgroup 0: waits 0.5 + 3.0 us over a 8.0 us span with 0.6 us between its tasks
    recs = [[(1, 0, 0, [100, 150, 200, 300, 320, 330, 340]), (3, 0, 0, [400, 700, 710, 800, 805, 810, 900])],
            [(1, 0, 1, [100, 100, 200, 300, 320, 330, 900])]]
    rec = trace.decode(_buf(4, recs))
    s = trace.sync_overhead(rec)
    np.testing.assert_allclose(s["spin_total_us"], 3.5)
    np.testing.assert_allclose(s["wait_us"], 1.75)
    np.testing.assert_allclose(s["wait_frac"], 3.5 / 16.0)
    np.testing.assert_allclose(s["between_us"], 0.3)
    assert "event waits" in trace.summary(rec)
