"""Host logic of the segmented prefill: segment rows and the automatic segment length (no GPU)."""
import numpy as np

from gated_delta_rule_15_amd.long_context import auto_seg_len, plan_segments


def test_plan_rows_cover_every_sequence():
    cu = np.cumsum([0, 2000, 300, 64, 0, 1, 777])
    plan = plan_segments(cu, 256)
    rows = plan.rows
    assert rows[0] == 0 and rows[-1] == cu[-1]
    assert np.all(np.diff(rows) >= 0)
    for n, r in enumerate(plan.row_of_seq):
        a, b = int(cu[n]), int(cu[n + 1])
        assert rows[r.start] == a and rows[r.stop] == b
        cuts = rows[r.start:r.stop + 1]
        # every cut is a multiple of 64 from the sequence start, segments at most 256 long
        assert all((c - a) % 64 == 0 for c in cuts[:-1])
        assert np.all(np.diff(cuts) <= 256)
    assert plan.multi == [0, 1, 5]
    assert plan.n_rows == 8 + 2 + 1 + 1 + 1 + 4


def test_plan_rejects_bad_lengths():
    import pytest
    for bad in (0, 100, -64):
        with pytest.raises(ValueError):
            plan_segments([0, 10], bad)


def test_auto_segment_length():
    assert auto_seg_len([0, 4096], 12) == 704           # 6 segments x 12 heads ~ 256 / 4 units
    assert auto_seg_len(np.cumsum([0] + [4096] * 32), 12) == 4096  # enough units: no cut
    assert auto_seg_len([0, 256], 1) == 512              # short: at least 512 (no cut at 256)
    for lens, H in (([4096], 12), ([100000], 2), ([5, 9000, 30], 4)):
        s = auto_seg_len(np.cumsum([0] + lens), H)
        assert s % 64 == 0 and s >= 512


def test_plan_cuts_only_long_sequences():
    cu = np.cumsum([0, 70000, 30000, 65536, 200000])
    plan = plan_segments(cu, 32768, cut_longer_than=65536)
    assert plan.multi == [0, 3]                    # 70,000 and 200,000 are cut; 30,000 and 65,536 stay whole
    assert [len(r) for r in plan.row_of_seq] == [3, 1, 1, 7]
    assert plan.rows[1] - plan.rows[0] == 32768


def test_longest_first_order():
    from gated_delta_rule_15_amd.long_context import longest_first
    rows = np.cumsum([0, 100, 300, 300, 64, 0, 500])
    order = longest_first(rows)
    assert order.tolist() == [5, 1, 2, 0, 3, 4]
    assert sorted(order.tolist()) == list(range(6))
