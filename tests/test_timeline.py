"""The tile-timeline summary (sparsity_sharq_prepare_amd.timeline) on
hand-made records: phases per tile, tiles and gaps per workgroup."""
import numpy as np

from sparsity_sharq_prepare_amd.timeline import summarize


def rec(t0, t1, t2, t3, wg):
    return [t0, t1, t2, t3, 0, wg, 0, 0]


def test_summary_of_two_workgroups():
    # stamps in 10 ns units: workgroup 3 runs two tiles, workgroup 8 one;
    # unused records are zero rows
    r = np.array([rec(1000, 1100, 2100, 2300, 3),     # first-step wait 1 us, steps 10 us, epilogue 2 us
                  rec(2350, 2400, 3400, 3600, 3),     # gap 0.5 us after the first tile
                  rec(1000, 1300, 2300, 2400, 8),
                  [0] * 8, [0] * 8], dtype=np.uint64)
    s = summarize(r)
    assert s["records"] == 3 and s["workgroups"] == 2
    assert abs(s["span_us"] - 26.0) < 1e-9                   # 1000 -> 3600
    p = s["phases_us"]
    assert abs(p["steps"]["mean"] - 10.0) < 1e-9
    assert abs(p["first-step wait"]["mean"] - (1.0 + 0.5 + 3.0) / 3) < 1e-9
    assert abs(p["epilogue issue"]["mean"] - (2.0 + 2.0 + 1.0) / 3) < 1e-9
    assert abs(p["gap to the next tile"]["mean"] - 0.5) < 1e-9
    assert abs(p["first tile's first-step wait"]["mean"] - 2.0) < 1e-9   # (1 + 3) / 2
    assert s["tiles_per_workgroup"] == {1: 1, 2: 1}
    assert abs(s["workgroup_end_us"]["max"] - 26.0) < 1e-9


def test_batch_summary_reports_events_after_start():
    from sparsity_sharq_prepare_amd.timeline import summarize_batch
    # words: 0 start, 1 first chunk staged, 2 last chunk multiplied,
    # 3 stored, 4-5 ids, 6 first chunk multiplied, 7 second chunk staged
    r = np.array([[1000, 1200, 3000, 3100, 0, 0, 1500, 1400],
                  [1100, 1300, 3300, 3500, 0, 1, 1600, 1500],
                  [0] * 8], dtype=np.uint64)
    s = summarize_batch(r)
    assert s["records"] == 2
    p = s["phases_us"]
    assert abs(p["first chunk staged"]["mean"] - 2.0) < 1e-9
    assert abs(p["second chunk staged"]["mean"] - 4.0) < 1e-9
    assert abs(p["first chunk multiplied"]["mean"] - 5.0) < 1e-9
    assert abs(p["last chunk multiplied"]["mean"] - 21.0) < 1e-9
    assert abs(p["stored"]["mean"] - 22.5) < 1e-9
    assert abs(s["span_us"] - 25.0) < 1e-9
