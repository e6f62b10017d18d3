"""Device-resident batch metadata and call marshalling.

``Batch`` runs the library's segment builder and planner on the host, then
moves row_index and both work lists to the device in one pinned host->device
copy on the caller's stream.  ``Batch.prepare_shrink`` / ``prepare_expand`` /
``prepare_merge`` build the C argument structs once and return a callable that
only issues the library call, so a serving loop pays no per-call marshalling.
PyTorch only provides memory and streams here.
"""
import numpy as np
import torch

from . import (LORA_MAX_SLICES, LORA_OP_APPLY, LORA_OP_EXPAND, LORA_OP_SHRINK, WORK_INTS, call_apply,
               call_expand, call_merge, call_shrink, lora_apply_proj_t, lora_build_segments, lora_expand_proj_t,
               lora_launch_t, lora_merge_mat_t, lora_mixture_rows, lora_plan, lora_plan_info_t, lora_shrink_proj_t,
               make_rows)


def staging_layout(n_active, n_work_shrink, n_work_expand, n_work_apply=0):
    """Byte offsets of (row_index, shrink work, expand work, apply work) in the
    staging buffer, and its size in int32 elements: row_index is int32
    [n_active], each work item WORK_INTS int32.  (The first four results are
    kept in this order for callers that use only the shrink/expand lists.)"""
    ri = 0
    ws = 4 * n_active
    we = ws + 4 * WORK_INTS * n_work_shrink
    wa = we + 4 * WORK_INTS * n_work_expand
    n = max(1, n_active + WORK_INTS * (n_work_shrink + n_work_expand + n_work_apply))
    if n_work_apply:
        return ri, ws, we, n, wa
    return ri, ws, we, n


def stream_handle(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


class Rows:
    """A row table on the device: pool (bf16 bits) + row_off (int64), and
    optionally neg_from (int32 per adapter: rank rows from there on enter
    negated, the A side of a deLoRA composite table)."""

    def __init__(self, pool, row_off, n_adapters, max_rank, row_len, chunk_len, neg_from=None):
        assert pool.is_cuda and row_off.is_cuda and row_off.dtype == torch.int64
        assert neg_from is None or (neg_from.is_cuda and neg_from.dtype == torch.int32)
        self.pool, self.row_off, self.neg_from = pool, row_off, neg_from
        self.n_adapters, self.max_rank, self.row_len, self.chunk_len = n_adapters, max_rank, row_len, chunk_len

    def c(self):
        return make_rows(self.pool.data_ptr(), self.row_off.data_ptr(), self.n_adapters, self.max_rank,
                         self.row_len, self.chunk_len,
                         None if self.neg_from is None else self.neg_from.data_ptr())


class Batch:
    """Segments + shrink/expand plans of one batch, resident on the device.

    ``refresh(row_adapter)`` rebuilds everything for a new batch of at most
    ``n_rows_max`` rows, reusing the host arrays, the pinned staging buffer and
    the device buffer; the launch structs are updated in place, so callables
    from ``prepare_*`` stay valid across refreshes."""

    def __init__(self, n_rows_max, adapter_rank, d_in, d_out, device="cuda"):
        self.adapter_rank = np.ascontiguousarray(adapter_rank, dtype=np.int32)
        self.d_in, self.d_out = int(d_in), int(d_out)
        self.device = torch.device(device)
        n = max(1, int(n_rows_max))
        nseg = max(1, min(n, self.adapter_rank.shape[0]))
        self._seg_out = (np.empty(n, np.int32), np.empty(nseg + 1, np.int32), np.empty(nseg, np.int32),
                         np.empty(nseg, np.int32))
        self._ws = np.empty((LORA_MAX_SLICES * n, WORK_INTS), np.int32)
        self._we = np.empty((n, WORK_INTS), np.int32)
        self._wa = np.empty(((LORA_MAX_SLICES + 1) * n, WORK_INTS), np.int32)
        self.info_shrink, self.info_expand = lora_plan_info_t(), lora_plan_info_t()
        self.info_apply = lora_plan_info_t()
        self.shrink_launch, self.expand_launch = lora_launch_t(), lora_launch_t()
        self.apply_launch = lora_launch_t()
        self._copied = None          # event of the last staging copy
        self._host = self._dev = None
        self._alloc(staging_layout(n, 4 * n, n, 5 * n)[3])
        self.segs = None

    def _alloc(self, cap):
        if self._copied is not None:
            self._copied.synchronize()
        self._host = torch.empty(cap, dtype=torch.int32, pin_memory=True)
        self._hnp = self._host.numpy()
        self._dev = torch.empty(cap, dtype=torch.int32, device=self.device)
        self._copied = None

    def refresh(self, row_adapter, stream=None):
        segs = lora_build_segments(row_adapter, self.adapter_rank, out=self._seg_out)
        ws, info_s = lora_plan(LORA_OP_SHRINK, segs, self.d_in, self.d_out, work_out=self._ws,
                               info_out=self.info_shrink)
        we, info_e = lora_plan(LORA_OP_EXPAND, segs, self.d_in, self.d_out, work_out=self._we,
                               info_out=self.info_expand)
        wa, info_a = lora_plan(LORA_OP_APPLY, segs, self.d_in, self.d_out, work_out=self._wa,
                               info_out=self.info_apply)
        na, ns, ne, nap = segs.n_active, ws.shape[0], we.shape[0], wa.shape[0]
        o_ri, o_ws, o_we, n, o_wa = staging_layout(na, ns, ne, max(1, nap))
        if n > self._host.shape[0]:
            self._alloc(n)
        if self._copied is not None:
            self._copied.synchronize()   # the staging buffer may still be in flight
        h = self._hnp
        h[:na] = segs.row_index
        h[na:na + WORK_INTS * ns] = ws.reshape(-1)
        h[na + WORK_INTS * ns:na + WORK_INTS * (ns + ne)] = we.reshape(-1)
        h[na + WORK_INTS * (ns + ne):na + WORK_INTS * (ns + ne + nap)] = wa.reshape(-1)
        s = torch.cuda.current_stream() if stream is None else stream
        with torch.cuda.stream(s):
            self._dev[:n].copy_(self._host[:n], non_blocking=True)
            self._copied = torch.cuda.Event()
            self._copied.record(s)
        base = self._dev.data_ptr()
        self.segs, self.work_shrink, self.work_expand, self.work_apply = segs, ws, we, wa
        for L, info, off in ((self.shrink_launch, info_s, o_ws), (self.expand_launch, info_e, o_we),
                             (self.apply_launch, info_a, o_wa)):
            L.row_index = base + o_ri
            L.work = base + off
            L.info = info
        return self

    @property
    def n_active(self):
        return self.segs.n_active

    @property
    def v_slices(self):
        return self.info_shrink.v_slices

    def new_v(self, ldv, fill=None):
        """A v buffer for this batch: fp32 [v_slices, max(1, n_active), ldv]."""
        shape = (self.v_slices, max(1, self.n_active), ldv)
        if fill is None:
            return torch.empty(shape, dtype=torch.float32, device=self.device)
        return torch.full(shape, fill, dtype=torch.float32, device=self.device)

    def _check_v(self, v):
        assert v.dtype == torch.float32 and v.is_contiguous() and v.dim() == 3
        assert v.shape[0] >= self.v_slices and v.shape[1] == max(1, self.n_active), \
            "v buffer does not match the batch (v_slices, n_active)"

    def prepare_shrink(self, projs, stream=None):
        """projs: list of (x tensor bf16 [*, ldx], Rows A, v tensor fp32 [v_slices, n_active, ldv]).
        Returns fn() that runs the shrink for the batch's current plan."""
        arr = (lora_shrink_proj_t * len(projs))(*[
            lora_shrink_proj_t(x.data_ptr(), x.stride(0), x.shape[1], A.c(), v.data_ptr(), v.stride(1))
            for x, A, v in projs])
        vs = [v for _, _, v in projs]
        h = stream_handle(stream)

        def run():
            for v in vs:
                self._check_v(v)
            call_shrink(self.shrink_launch, arr, len(vs), h)
        run.keep = (projs, arr)
        return run

    def prepare_expand(self, projs, stream=None):
        """projs: list of (v tensor fp32 [v_slices, n_active, ldv], Rows B, y tensor fp32 [*, ldy], scale)."""
        arr = (lora_expand_proj_t * len(projs))(*[
            lora_expand_proj_t(v.data_ptr(), v.stride(1), B.c(), y.shape[1], y.data_ptr(), y.stride(0), float(s))
            for v, B, y, s in projs])
        vs = [v for v, _, _, _ in projs]
        h = stream_handle(stream)

        def run():
            for v in vs:
                self._check_v(v)
            call_expand(self.expand_launch, arr, len(vs), h)
        run.keep = (projs, arr)
        return run

    def prepare_apply(self, projs, stream=None):
        """projs: list of (x, Rows A, v, Rows B, y, scale) as for the shrink and the
        expand; v (fp32 [v_slices, n_active, ldv]) serves the segments that are
        not fused.  Returns fn() that runs lora_apply for the current plan."""
        arr = (lora_apply_proj_t * len(projs))(*[
            lora_apply_proj_t(x.data_ptr(), x.stride(0), x.shape[1], A.c(), v.data_ptr(), v.stride(1), B.c(),
                              y.shape[1], y.data_ptr(), y.stride(0), float(s))
            for x, A, v, B, y, s in projs])
        vs = [p[2] for p in projs]
        h = stream_handle(stream)

        def run():
            for v in vs:
                self._check_v(v)
            call_apply(self.apply_launch, arr, len(vs), h)
        run.keep = (projs, arr)
        return run

    def apply(self, projs, stream=None):
        self.prepare_apply(projs, stream)()

    def shrink(self, projs, stream=None):
        self.prepare_shrink(projs, stream)()

    def expand(self, projs, stream=None):
        self.prepare_expand(projs, stream)()


def merge_mats(mats):
    """mats: list of (W tensor bf16 [d_out, ldw], Rows A, Rows B, adapter, rank, scale)."""
    return (lora_merge_mat_t * len(mats))(*[
        lora_merge_mat_t(W.data_ptr(), W.stride(0), W.shape[0], W.shape[1], A.c(), B.c(), int(a), int(r), float(s))
        for W, A, B, a, r, s in mats])


def prepare_merge(mats, stream=None, unmerge=False):
    """Returns fn() that merges (or unmerges) the given matrices in one launch."""
    arr = merge_mats(mats)
    h = stream_handle(stream)

    def run():
        call_merge(arr, len(mats), h, unmerge=unmerge)
    run.keep = (mats, arr)
    return run


def merge(mats, stream=None):
    prepare_merge(mats, stream)()


def unmerge(mats, stream=None):
    prepare_merge(mats, stream, unmerge=True)()


def mixture_tables(rows_host, rank, merged, out_max_rank, device="cuda"):
    """deLoRA (VaLoRA section 4.4.2) tables for one projection while adapter
    `merged` is merged: rows_host = (A_row_off, B_row_off, max_rank, A_chunks,
    B_chunks) of the real adapters (host int64 arrays).  Returns
    (A_row_off, B_row_off, neg_from) on the device and the composite ranks
    (host), for Rows(..., max_rank=out_max_rank, neg_from=neg_from) on the A
    side and Rows(..., max_rank=out_max_rank) on the B side."""
    a_off, b_off, max_rank, a_chunks, b_chunks = rows_host
    ca, crank, neg = lora_mixture_rows(rank, merged, a_chunks, a_off, max_rank, out_max_rank)
    cb, _, _ = lora_mixture_rows(rank, merged, b_chunks, b_off, max_rank, out_max_rank)
    dev = torch.device(device)
    return (torch.from_numpy(ca).to(dev), torch.from_numpy(cb).to(dev), torch.from_numpy(neg).to(dev), crank)
