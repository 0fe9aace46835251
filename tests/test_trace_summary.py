"""The kernel-trace summary's update launch time: four consecutive update
dispatches per launch, timed from the first start to the last end (the two
row parts overlap on two streams)."""

import pytest

from jagged_embedding_sparse_amd.trace_summary import update_spans


def _row(d, name, start, end):
    return {"Dispatch_Id": str(d), "Kernel_Name": name, "Start_Timestamp": str(start),
            "End_Timestamp": str(end)}


K = "void fs::(anonymous namespace)::{}<128, unsigned short>(fs::(anonymous namespace)::RUArgs)"


def test_update_spans_overlapping_parts():
    rows = [
        _row(1, "fs::(anonymous namespace)::k_lookup(...)", 0, 500),
        # launch 1: long rows + fix on one stream, short + medium on the other
        _row(2, K.format("k_long"), 1000, 9000), _row(3, K.format("k_fix"), 9000, 9500),
        _row(4, K.format("k_short"), 1100, 6000), _row(5, K.format("k_medium"), 6000, 8000),
        _row(6, "fs::(anonymous namespace)::k_seg_prep(...)", 9600, 9700),
        # launch 2: one stream, in order
        _row(7, K.format("k_short"), 20000, 21000), _row(8, K.format("k_medium"), 21000, 22000),
        _row(9, K.format("k_long"), 22000, 25000), _row(10, K.format("k_fix"), 25000, 26000),
    ]
    (s1, b1), (s2, b2) = update_spans(rows)
    assert s1 == pytest.approx(8.5) and b1 == pytest.approx((8000 + 500 + 4900 + 2000) / 1e3)
    assert s2 == pytest.approx(6.0) and b2 == pytest.approx(6.0)


def test_update_spans_rejects_a_group_out_of_step():
    rows = [_row(1, K.format("k_short"), 0, 1), _row(2, K.format("k_short"), 1, 2),
            _row(3, K.format("k_long"), 2, 3), _row(4, K.format("k_fix"), 3, 4)]
    with pytest.raises(ValueError):
        update_spans(rows)
