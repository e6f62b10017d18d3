"""Segment metadata and dense row offsets, by definition (test infrastructure only).

Segment table (BEE-30060 page, Punica paragraph: SGMV groups the requests of a
batch by adapter identity; LoRazor article, mechanism section: only rows whose
adapter is still held get LoRA work):

* the active rows are those whose adapter id is >= 0 (-1 marks a released row);
* ``row_index`` lists the active rows ordered by (adapter id, row index);
* one segment per distinct adapter present, in ascending adapter id;
  ``seg_start`` holds the CSR offsets of the segments in ``row_index``,
  ``seg_adapter`` the adapter of each segment and ``seg_rank`` its rank.

Written as the sort-then-split definition; no counting or bucketing tricks.
"""
from dataclasses import dataclass

import numpy as np


class SegmentError(ValueError):
    """Raised for inputs the library must reject; ``kind`` names the error."""

    def __init__(self, kind, msg):
        super().__init__(msg)
        self.kind = kind


@dataclass
class SegmentsRef:
    row_index: np.ndarray    # int32 [n_active]
    seg_start: np.ndarray    # int32 [n_seg + 1]
    seg_adapter: np.ndarray  # int32 [n_seg]
    seg_rank: np.ndarray     # int32 [n_seg]

    @property
    def n_seg(self):
        return int(self.seg_adapter.shape[0])

    @property
    def n_active(self):
        return int(self.row_index.shape[0])


def build_segments_ref(row_adapter, adapter_rank, max_rank=128):
    row_adapter = [int(v) for v in np.asarray(row_adapter).reshape(-1)]
    adapter_rank = [int(v) for v in np.asarray(adapter_rank).reshape(-1)]
    n_ad = len(adapter_rank)
    for a in row_adapter:
        if a < -1 or a >= n_ad:
            raise SegmentError("adapter", f"adapter id {a} outside [-1, {n_ad})")
    for r in adapter_rank:
        if r < 1 or r > max_rank:
            raise SegmentError("rank", f"rank {r} outside [1, {max_rank}]")
    active = [i for i, a in enumerate(row_adapter) if a >= 0]
    order = sorted(active, key=lambda i: (row_adapter[i], i))
    seg_start, seg_adapter = [], []
    for p, i in enumerate(order):
        if p == 0 or row_adapter[i] != row_adapter[order[p - 1]]:
            seg_start.append(p)
            seg_adapter.append(row_adapter[i])
    seg_start.append(len(order))
    return SegmentsRef(
        np.array(order, dtype=np.int32),
        np.array(seg_start, dtype=np.int32),
        np.array(seg_adapter, dtype=np.int32),
        np.array([adapter_rank[a] for a in seg_adapter], dtype=np.int32),
    )


def dense_offsets_ref(adapter_rank, max_rank, row_len, chunk_len):
    """Row-offset table of the packed dense layout.

    Adapters are packed in id order, each adapter's rows j = 0..r_a-1 back to
    back, every row occupying ``ceil(row_len / 8) * 8`` elements (16-byte
    aligned); chunk c of a row starts ``c * chunk_len`` elements after the row.
    Slots j >= r_a hold -1.  Entry index: (a * max_rank + j) * chunks + c."""
    chunks = -(-row_len // chunk_len)
    stride = -(-row_len // 8) * 8
    n_ad = len(adapter_rank)
    off = np.full(n_ad * max_rank * chunks, -1, dtype=np.int64)
    row = 0
    for a in range(n_ad):
        for j in range(int(adapter_rank[a])):
            for c in range(chunks):
                off[(a * max_rank + j) * chunks + c] = row * stride + c * chunk_len
            row += 1
    return off
