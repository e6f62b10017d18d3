"""Coverage invariants of a launch plan (test infrastructure only).

The plan's tiling is a performance choice, so it has no unique expected value
("parity unpinned" by design); what must hold is coverage, after the LoRazor
article's active-row idea (launch work only for rows that still hold an
adapter): every active row is covered by exactly one work item, every work item
lies inside one segment and carries that segment's adapter and rank, and no item
exceeds the row count of its variant.
"""
import numpy as np


def check_plan_coverage(seg, work, ranges):
    """seg: SegmentsRef-like; work: int array [n_work, 4] of
    (row0, nrows, adapter, rank); ranges: list of (variant, begin, count,
    rows_per_item).  Raises AssertionError on violation."""
    work = np.asarray(work).reshape(-1, 4)
    covered = np.zeros(seg.n_active, dtype=np.int64)
    seen = np.zeros(work.shape[0], dtype=np.int64)
    for (_variant, begin, count, mt) in ranges:
        for w in range(begin, begin + count):
            seen[w] += 1
            row0, nrows, adapter, rank = (int(t) for t in work[w])
            assert 1 <= nrows <= mt, (w, nrows, mt)
            s = int(np.searchsorted(seg.seg_start, row0, side="right")) - 1
            assert 0 <= s < seg.n_seg
            assert row0 + nrows <= int(seg.seg_start[s + 1]), (w, row0, nrows)
            assert adapter == int(seg.seg_adapter[s]) and rank == int(seg.seg_rank[s])
            covered[row0:row0 + nrows] += 1
    assert np.all(seen == 1), "every work item in exactly one range"
    assert np.all(covered == 1), "every active row in exactly one work item"
