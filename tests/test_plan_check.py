"""Pins of the oracle's plan-coverage checker (CPU only).

``oracle.check_plan_coverage`` states what every launch plan must satisfy
(LoRazor article, mechanism section: LoRA work is launched only for the rows
that still hold an adapter, each of them once): every active row is covered by
exactly one work item (per K slice, for a shrink plan), every item lies inside
one segment and carries that segment's adapter and rank, one segment has one
slice count, and no item holds more rows than its range allows.

A checker that accepted everything would make every coverage test pass, so
it is pinned here on plans written out by hand (no library call is involved):
the correct plans pass, and each plan with one planted mistake must raise.
"""
import copy

import numpy as np
import pytest

import oracle

# Batch: rows 0..9 -> adapters [2, 0, 2, -1, 0, 0, 5, 2, 5, -1], six adapters
# of ranks [8, 4, 16, 4, 4, 32].  By hand: adapter 0 holds rows 1, 4, 5;
# adapter 2 rows 0, 2, 7; adapter 5 rows 6, 8; rows 3 and 9 are released.
ROW_ADAPTER = [2, 0, 2, -1, 0, 0, 5, 2, 5, -1]
RANKS = [8, 4, 16, 4, 4, 32]
SEGS = oracle.SegmentsRef(
    row_index=np.array([1, 4, 5, 0, 2, 7, 6, 8], np.int32),
    seg_start=np.array([0, 3, 6, 8], np.int32),
    seg_adapter=np.array([0, 2, 5], np.int32),
    seg_rank=np.array([8, 16, 32], np.int32),
)

# (row0, nrows, adapter, rank, kslice, nslices, 0, 0); segment 1 is split
# into two K slices, the others are not.
EXPAND_WORK = [
    [0, 2, 0, 8, 0, 1, 0, 0],
    [2, 1, 0, 8, 0, 1, 0, 0],
    [3, 3, 2, 16, 0, 2, 0, 0],
    [6, 2, 5, 32, 0, 1, 0, 0],
]
EXPAND_RANGES = [(0, 0, 2, 2), (1, 2, 2, 4)]          # (variant, begin, count, rows_per_item)
SHRINK_WORK = [
    [0, 3, 0, 8, 0, 1, 0, 0],
    [3, 3, 2, 16, 0, 2, 0, 0],
    [3, 3, 2, 16, 1, 2, 0, 0],
    [6, 1, 5, 32, 0, 1, 0, 0],
    [7, 1, 5, 32, 0, 1, 0, 0],
]
SHRINK_RANGES = [(0, 0, 1, 4), (1, 1, 2, 4), (2, 3, 2, 1)]
V_SLICES = 2


def _check(work, ranges, shrink):
    return oracle.check_plan_coverage(SEGS, np.array(work, np.int64), ranges, shrink, V_SLICES)


def test_hand_segment_table_is_the_oracle_s():
    ref = oracle.build_segments_ref(ROW_ADAPTER, RANKS)
    for f in ("row_index", "seg_start", "seg_adapter", "seg_rank"):
        assert np.array_equal(getattr(ref, f), getattr(SEGS, f)), f


def test_correct_plans_pass():
    assert _check(EXPAND_WORK, EXPAND_RANGES, False) == {0: 1, 1: 2, 2: 1}
    assert _check(SHRINK_WORK, SHRINK_RANGES, True) == {0: 1, 1: 2, 2: 1}


def _mut(work, i, **kw):
    w = copy.deepcopy(work)
    for k, v in kw.items():
        w[i][("row0", "nrows", "adapter", "rank", "kslice", "nslices").index(k)] = v
    return w


# Each case: (name, work, ranges) with one planted mistake.
EXPAND_BAD = [
    ("duplicated item", EXPAND_WORK + [EXPAND_WORK[0]], [(0, 0, 2, 2), (1, 2, 2, 4), (2, 4, 1, 2)]),
    ("dropped row", EXPAND_WORK[:1] + EXPAND_WORK[2:], [(0, 0, 1, 2), (1, 1, 2, 4)]),
    ("item shortened: a row left out", _mut(EXPAND_WORK, 3, nrows=1), EXPAND_RANGES),
    ("item crosses a segment boundary", _mut(EXPAND_WORK, 1, nrows=2), EXPAND_RANGES),
    ("overlapping items", _mut(EXPAND_WORK, 1, row0=1), EXPAND_RANGES),
    ("wrong adapter", _mut(EXPAND_WORK, 3, adapter=4), EXPAND_RANGES),
    ("wrong rank", _mut(EXPAND_WORK, 3, rank=16), EXPAND_RANGES),
    ("mixed slice counts in one segment", _mut(EXPAND_WORK, 1, nslices=2), EXPAND_RANGES),
    ("more rows than the range allows", EXPAND_WORK, [(0, 0, 2, 1), (1, 2, 2, 4)]),
    ("item in no range", EXPAND_WORK, [(0, 0, 2, 2), (1, 2, 1, 4)]),
    ("item in two ranges", EXPAND_WORK, [(0, 0, 3, 4), (1, 2, 2, 4)]),
    ("expand item with a K slice", _mut(EXPAND_WORK, 2, kslice=1), EXPAND_RANGES),
    ("slice count above the plan's", _mut(_mut(EXPAND_WORK, 0, nslices=3), 1, nslices=3), EXPAND_RANGES),
    ("item past the active rows", _mut(EXPAND_WORK, 3, row0=7), EXPAND_RANGES),
    ("item before the first row", _mut(EXPAND_WORK, 0, row0=-1, nrows=3), EXPAND_RANGES),
    ("empty item", _mut(EXPAND_WORK, 1, nrows=0), EXPAND_RANGES),
]
SHRINK_BAD = [
    ("a K slice missing", SHRINK_WORK[:2] + SHRINK_WORK[3:], [(0, 0, 1, 4), (1, 1, 1, 4), (2, 2, 2, 1)]),
    ("a K slice twice", _mut(SHRINK_WORK, 2, kslice=0), SHRINK_RANGES),
    ("K slice past the slice count", _mut(_mut(SHRINK_WORK, 0, kslice=1), 0, nslices=1), SHRINK_RANGES),
    ("row covered in a slice its segment does not have", SHRINK_WORK + [[0, 3, 0, 8, 1, 1, 0, 0]],
     [(0, 0, 1, 4), (1, 1, 2, 4), (2, 3, 2, 1), (3, 5, 1, 4)]),
    ("dropped decode row", SHRINK_WORK[:4], [(0, 0, 1, 4), (1, 1, 2, 4), (2, 3, 1, 1)]),
    ("wrong adapter", _mut(SHRINK_WORK, 4, adapter=2), SHRINK_RANGES),
]


@pytest.mark.parametrize("name,work,ranges", EXPAND_BAD, ids=[c[0] for c in EXPAND_BAD])
def test_expand_plan_mistake_is_caught(name, work, ranges):
    with pytest.raises(AssertionError):
        _check(work, ranges, False)


@pytest.mark.parametrize("name,work,ranges", SHRINK_BAD, ids=[c[0] for c in SHRINK_BAD])
def test_shrink_plan_mistake_is_caught(name, work, ranges):
    with pytest.raises(AssertionError):
        _check(work, ranges, True)


def test_expand_plan_read_as_shrink_plan_is_caught():
    # segment 1's expand item covers slice 0 only: as a shrink plan slice 1 is missing
    with pytest.raises(AssertionError):
        _check(EXPAND_WORK, EXPAND_RANGES, True)
