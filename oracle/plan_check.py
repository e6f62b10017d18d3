"""Coverage invariants of a launch plan (test infrastructure only).

The plan's tiling is a performance choice, so it has no unique expected value
("parity unpinned" by design); what must hold is coverage, after the LoRazor
article's active-row idea (launch work only for rows that still hold an
adapter): every active row is covered by exactly one work item, every work item
lies inside one segment and carries that segment's adapter and rank, and no item
exceeds the row count of its variant.
"""
import numpy as np


def check_plan_coverage(seg, work, ranges, shrink, v_slices):
    """seg: SegmentsRef-like; work: int array [n_work, 8] of
    (row0, nrows, adapter, rank, kslice, nslices, 0, 0); ranges: list of
    (variant, begin, count, rows_per_item).  A shrink plan must cover every
    (active row, K slice) pair of the row's segment exactly once; an expand
    plan every active row exactly once, with the same slice count per segment.
    Returns {segment: nslices}.  Raises AssertionError on violation."""
    work = np.asarray(work).reshape(-1, 8)
    covered = np.zeros((seg.n_active, v_slices), dtype=np.int64)
    seen = np.zeros(work.shape[0], dtype=np.int64)
    seg_slices = {}
    for (_variant, begin, count, mt) in ranges:
        for w in range(begin, begin + count):
            seen[w] += 1
            row0, nrows, adapter, rank, kslice, nslices = (int(t) for t in work[w][:6])
            assert 1 <= nrows <= mt, (w, nrows, mt)
            s = int(np.searchsorted(seg.seg_start, row0, side="right")) - 1
            assert 0 <= s < seg.n_seg
            assert row0 + nrows <= int(seg.seg_start[s + 1]), (w, row0, nrows)
            assert adapter == int(seg.seg_adapter[s]) and rank == int(seg.seg_rank[s])
            assert 1 <= nslices <= v_slices and 0 <= kslice < nslices
            assert seg_slices.setdefault(s, nslices) == nslices, "one slice count per segment"
            if shrink:
                covered[row0:row0 + nrows, kslice] += 1
            else:
                assert kslice == 0
                covered[row0:row0 + nrows, 0] += 1
    assert np.all(seen == 1), "every work item in exactly one range"
    for s in range(seg.n_seg):
        lo, hi = int(seg.seg_start[s]), int(seg.seg_start[s + 1])
        ns = seg_slices[s] if shrink else 1
        assert np.all(covered[lo:hi, :ns] == 1), "each active row (and K slice) covered once"
        assert np.all(covered[lo:hi, ns:] == 0)
    return seg_slices
