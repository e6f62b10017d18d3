"""Device-resident batch metadata and call marshalling.

``Batch`` has the library build the segment table and the plans on the host
and upload row_index and the work lists to the device in one pinned
host->device copy on the caller's stream, all in one call.  ``DeviceBatch``
builds them on the GPU from a device row -> adapter map instead.  ``Batch.prepare_shrink`` / ``prepare_expand`` /
``prepare_merge`` build the C argument structs once and return a callable that
only issues the library call, so a serving loop pays no per-call marshalling.
PyTorch only provides memory and streams here.
"""
import ctypes

import numpy as np
import torch

from . import _lib as _hip  # the HIP runtime the library is linked to (and torch uses)
from . import (LORA_ECAPACITY, LORA_OK, LORA_OP_APPLY, LORA_PREPARE_INLINE, LORA_OP_EXPAND, LORA_OP_SHRINK, WORK_INTS, LoraPool, Segments,
               batch_prepare, call_apply, call_expand, call_merge, call_shrink, check_status, lora_apply_proj_t,
               lora_batch_t, lora_device_header_t, lora_device_plan, lora_expand_proj_t, lora_launch_t,
               lora_merge_mat_t, lora_mixture_rows, lora_pool_scatter, lora_shrink_proj_t, make_rows)


class HipEvent:
    """A HIP event recorded without the system-scope memory fence
    (hipEventDisableSystemFence).  Recording a default event makes the GPU
    write back and invalidate its caches when the event completes, which
    idles it for microseconds and leaves the next kernel cold; an event that
    only orders the host against the stream (the staging copy) or measures
    time between launches on one stream needs no such fence.  ``timing``
    keeps the timestamp (hipEventElapsedTime)."""

    DISABLE_TIMING, DISABLE_SYSTEM_FENCE = 0x2, 0x20000000

    def __init__(self, timing=False):
        self._h = ctypes.c_void_p()
        flags = self.DISABLE_SYSTEM_FENCE | (0 if timing else self.DISABLE_TIMING)
        check_status(0 if _hip.hipEventCreateWithFlags(ctypes.byref(self._h), flags) == 0 else -6,
                     "hipEventCreateWithFlags")

    def record(self, stream=None):
        """stream: a torch stream, a raw hipStream_t handle, or None for the
        current torch stream."""
        if stream is None:
            stream = torch.cuda.current_stream()
        h = stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
        if _hip.hipEventRecord(self._h, h) != 0:
            raise RuntimeError("hipEventRecord failed")

    def synchronize(self):
        if _hip.hipEventSynchronize(self._h) != 0:
            raise RuntimeError("hipEventSynchronize failed")

    def query(self):
        """True once the recorded work has completed."""
        return _hip.hipEventQuery(self._h) == 0

    def wait(self, stream=None):
        """Make `stream` (torch stream or raw handle; None: current) wait for this event."""
        if stream is None:
            stream = torch.cuda.current_stream()
        h = stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
        if _hip.hipStreamWaitEvent(h, self._h, 0) != 0:
            raise RuntimeError("hipStreamWaitEvent failed")

    def elapsed_time(self, end):
        """Milliseconds from this event to `end` (both recorded and complete)."""
        ms = ctypes.c_float()
        if _hip.hipEventElapsedTime(ctypes.byref(ms), self._h, end._h) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        # at interpreter exit the module globals may already be gone
        if self._h and _hip is not None:
            _hip.hipEventDestroy(self._h)
        self._h = None


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
    """Segments + shrink/expand/apply plans of one batch, resident on the device.

    ``refresh(row_adapter)`` rebuilds everything for a new batch (the buffers
    are sized for ``n_rows_max`` rows and grow when a batch needs more) with one
    library call (lora_batch_prepare: segment
    table, the three plans, and their upload from a pinned staging buffer on
    the caller's stream), reusing the host arrays and both buffers; the launch
    structs live in the library's output struct and are updated in place, so
    callables from ``prepare_*`` stay valid across refreshes.

    ``inline=True`` plans the apply op only, with LORA_PREPARE_INLINE: a
    small all-fused plan (decode batches) is then not copied at all but
    handed to the kernel in its launch arguments; a larger plan is copied as
    usual.  The shrink and expand launches are then unavailable."""

    def __init__(self, n_rows_max, adapter_rank, d_in, d_out, device="cuda", inline=False):
        self.adapter_rank = np.ascontiguousarray(adapter_rank, dtype=np.int32)
        self.d_in, self.d_out = int(d_in), int(d_out)
        self.device = torch.device(device)
        n = max(1, int(n_rows_max))
        self._alloc_segs(max(1, min(n, self.adapter_rank.shape[0])))
        self._rank_ptr = self.adapter_rank.ctypes.data
        self._b = lora_batch_t()
        self._b_ref = ctypes.byref(self._b)
        self._launch = [self._b.launch[op] for op in (LORA_OP_SHRINK, LORA_OP_EXPAND, LORA_OP_APPLY)]
        self._copied = HipEvent()   # the last staging copy
        self._pending = False
        self._stream, self._stream_h = None, None
        self._n_active, self._v_slices, self._op_slices = 0, 1, [0, 0, 0]
        self._op_mask = ((1 << LORA_OP_APPLY) | LORA_PREPARE_INLINE) if inline else 7
        self._alloc(n + WORK_INTS * 10 * n)  # grown on demand

    def _alloc_segs(self, cap):
        self._seg_cap = cap
        self._seg = (np.empty(cap + 1, np.int32), np.empty(cap, np.int32), np.empty(cap, np.int32))
        self._seg_ptr = tuple(a.ctypes.data for a in self._seg)

    def _alloc(self, cap):
        if self._pending:
            self._copied.synchronize()
            self._pending = False
        self._host = torch.empty(cap, dtype=torch.int32, pin_memory=True)
        self._hnp = self._host.numpy()
        self._dev = torch.empty(cap, dtype=torch.int32, device=self.device)
        self._host_ptr, self._dev_ptr = self._host.data_ptr(), self._dev.data_ptr()

    def refresh(self, row_adapter, stream=None):
        ra = row_adapter
        if not (isinstance(ra, np.ndarray) and ra.dtype == np.int32 and ra.flags.c_contiguous):
            ra = np.ascontiguousarray(ra, dtype=np.int32)
        if stream is None:
            stream = torch.cuda.current_stream()
        if stream is not self._stream:
            self._stream, self._stream_h = stream, stream.cuda_stream
        if self._pending:
            self._copied.synchronize()   # the staging buffer may still be in flight
            self._pending = False
        while True:
            st = batch_prepare(ra.shape[0], ra.ctypes.data, self.adapter_rank.shape[0], self._rank_ptr,
                               self.d_in, self.d_out, self._op_mask, self._seg_cap, *self._seg_ptr, self._host_ptr,
                               self._host.shape[0], self._dev_ptr, self._stream_h, self._b_ref)
            if st != LORA_ECAPACITY:
                break
            if self._b.n_seg > self._seg_cap:
                self._alloc_segs(self._b.n_seg)
            elif self._b.n_staged > self._host.shape[0]:
                self._alloc(int(self._b.n_staged) * 2)
            else:
                break
        check_status(st, "lora_batch_prepare")
        # an inline plan stays on the host (lora_apply copies it into the
        # launch arguments), so nothing is in flight to wait for next time
        if not (self._op_mask & LORA_PREPARE_INLINE) or self._launch[LORA_OP_APPLY].work:
            self._copied.record(stream)
            self._pending = True
        self._n_active = self._b.n_active
        # v buffers from new_v serve every planned op (the library trusts the
        # size of v, so each call checks its own plan's slices below)
        self._op_slices = [self._launch[op].info.v_slices if self._launch[op].info.op == op else 0
                           for op in (LORA_OP_SHRINK, LORA_OP_EXPAND, LORA_OP_APPLY)]
        self._v_slices = max(1, *self._op_slices)
        return self

    @property
    def shrink_launch(self):
        return self._launch[LORA_OP_SHRINK]

    @property
    def expand_launch(self):
        return self._launch[LORA_OP_EXPAND]

    @property
    def apply_launch(self):
        return self._launch[LORA_OP_APPLY]

    @property
    def info_shrink(self):
        return self._launch[LORA_OP_SHRINK].info

    @property
    def info_expand(self):
        return self._launch[LORA_OP_EXPAND].info

    @property
    def info_apply(self):
        return self._launch[LORA_OP_APPLY].info

    @property
    def segs(self):
        """Host segment table of the current batch (views of reused arrays)."""
        ns, na = self._b.n_seg, self._b.n_active
        return Segments(self._hnp[:na], self._seg[0][:ns + 1], self._seg[1][:ns], self._seg[2][:ns])

    def _work(self, op):
        L = self._launch[op]
        off = (L.host_work - self._host_ptr) // 4
        return self._hnp[off:off + WORK_INTS * L.info.n_work].reshape(-1, WORK_INTS)

    @property
    def work_shrink(self):
        return self._work(LORA_OP_SHRINK)

    @property
    def work_expand(self):
        return self._work(LORA_OP_EXPAND)

    @property
    def work_apply(self):
        return self._work(LORA_OP_APPLY)

    @property
    def n_active(self):
        return self._n_active

    @property
    def v_slices(self):
        return self._v_slices

    def new_v(self, ldv, fill=None):
        """A v buffer for this batch: fp32 [v_slices, max(1, n_active), ldv]."""
        shape = (self.v_slices, max(1, self.n_active), ldv)
        if fill is None:
            return torch.empty(shape, dtype=torch.float32, device=self.device)
        return torch.full(shape, fill, dtype=torch.float32, device=self.device)

    @staticmethod
    def _v_shapes(vs):
        """(v_slices, rows) of each v buffer, after the checks that do not
        depend on the batch (the buffers' pointers are bound at prepare time)."""
        for v in vs:
            assert v.dtype == torch.float32 and v.is_contiguous() and v.dim() == 3
        return [(int(v.shape[0]), int(v.shape[1])) for v in vs]

    def _check_v(self, shapes, op):
        """The library trusts v's size: check it against the plan of `op`
        before every call (v_slices of that plan, n_active rows)."""
        rows = max(1, self._n_active)
        need = self._op_slices[op]
        for s0, s1 in shapes:
            if s0 < need or s1 != rows:
                raise AssertionError("v buffer does not match the batch's plan (v_slices, n_active)")

    def prepare_shrink(self, projs, stream=None):
        """projs: list of (x tensor bf16 [*, ldx], Rows A, v tensor fp32 [v_slices, n_active, ldv]).
        Returns fn() that runs the shrink for the batch's current plan."""
        arr = (lora_shrink_proj_t * len(projs))(*[
            lora_shrink_proj_t(x.data_ptr(), x.stride(0), x.shape[1], A.c(), v.data_ptr(), v.stride(1))
            for x, A, v in projs])
        vs = [v for _, _, v in projs]
        h = stream_handle(stream)

        shapes, n, L = self._v_shapes(vs), len(vs), self._launch[LORA_OP_SHRINK]

        def run():
            self._check_v(shapes, LORA_OP_SHRINK)
            call_shrink(L, arr, n, h)
        run.keep = (projs, arr)
        return run

    def prepare_expand(self, projs, stream=None):
        """projs: list of (v tensor fp32 [v_slices, n_active, ldv], Rows B, y tensor fp32 [*, ldy], scale)."""
        arr = (lora_expand_proj_t * len(projs))(*[
            lora_expand_proj_t(v.data_ptr(), v.stride(1), B.c(), y.shape[1], y.data_ptr(), y.stride(0), float(s))
            for v, B, y, s in projs])
        vs = [v for v, _, _, _ in projs]
        h = stream_handle(stream)

        shapes, n, L = self._v_shapes(vs), len(vs), self._launch[LORA_OP_EXPAND]

        def run():
            self._check_v(shapes, LORA_OP_EXPAND)
            call_expand(L, arr, n, h)
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

        shapes, n, L = self._v_shapes(vs), len(vs), self._launch[LORA_OP_APPLY]

        def run():
            self._check_v(shapes, LORA_OP_APPLY)
            call_apply(L, arr, n, h)
        run.keep = (projs, arr)
        return run

    def apply(self, projs, stream=None):
        self.prepare_apply(projs, stream)()

    def shrink(self, projs, stream=None):
        self.prepare_shrink(projs, stream)()

    def expand(self, projs, stream=None):
        self.prepare_expand(projs, stream)()


class DeviceBatch:
    """A batch whose segment table and apply plan are built on the GPU.

    The launch shapes come from bounds alone (lora_device_plan: rows,
    adapters, largest rank, d); ``build(row_adapter, adapter_rank)`` takes
    both maps as device int32 tensors and enqueues the builder kernel
    (lora_batch_build_device) on the stream: no host work per batch beyond
    that one call, and no copy.  The launch struct is the same for every
    build, so callables from ``prepare_apply`` stay valid.  v buffers are
    sized for the bounds: fp32 [v_slices, n_rows, ldv]."""

    def __init__(self, n_rows, n_adapters, max_rank, d_in, d_out, device="cuda"):
        _, self.plan = lora_device_plan(n_rows, n_adapters, max_rank, d_in, d_out)
        self.device = torch.device(device)
        self.workspace = torch.empty(self.plan.workspace_bytes, dtype=torch.uint8, device=self.device)
        assert self.workspace.data_ptr() % 256 == 0
        self._ws = self.workspace.data_ptr()
        self._plan_ref = ctypes.byref(self.plan)
        self._launch = lora_launch_t()
        self._launch_ref = ctypes.byref(self._launch)

    def prepare_build(self, row_adapter, adapter_rank, stream=None):
        """row_adapter: device int32 [n_rows]; adapter_rank: device int32
        [n_adapters].  Returns fn() that enqueues the builder for the maps'
        current contents (one library call)."""
        assert row_adapter.dtype == torch.int32 and row_adapter.is_contiguous()
        assert adapter_rank.dtype == torch.int32 and adapter_rank.is_contiguous()
        assert row_adapter.numel() == self.plan.n_rows and adapter_rank.numel() == self.plan.n_adapters
        args = (self._plan_ref, row_adapter.data_ptr(), adapter_rank.data_ptr(), self._ws, stream_handle(stream),
                self._launch_ref)
        call = _hip.lora_batch_build_device

        def run():
            st = call(*args)
            if st != LORA_OK:
                check_status(st, "lora_batch_build_device")
        run.keep = (row_adapter, adapter_rank)
        return run

    def build(self, row_adapter, adapter_rank, stream=None):
        """Enqueue the builder once (see prepare_build)."""
        self.prepare_build(row_adapter, adapter_rank, stream)()
        return self

    @property
    def apply_launch(self):
        return self._launch

    @property
    def info_apply(self):
        return self.plan.info

    @property
    def v_slices(self):
        return self.plan.info.v_slices

    def new_v(self, ldv, fill=None):
        shape = (self.v_slices, self.plan.n_rows, ldv)
        if fill is None:
            return torch.empty(shape, dtype=torch.float32, device=self.device)
        return torch.full(shape, fill, dtype=torch.float32, device=self.device)

    def header(self):
        """The builder's header (waits for the device): status, n_seg,
        n_active, n_work and the live count of every range."""
        h = lora_device_header_t()
        raw = self.workspace[:ctypes.sizeof(h)].cpu().numpy().tobytes()
        ctypes.memmove(ctypes.addressof(h), raw, len(raw))
        return h

    def read(self):
        """Everything the builder wrote (waits for the device): header,
        row_index [n_active], the segment table, and per range its live work
        items (int32 [live, WORK_INTS])."""
        h = self.header()
        ws = self.workspace.cpu().numpy()
        p = self.plan

        def ints(off, n):
            return ws[off:off + 4 * n].view(np.int32)
        segs = Segments(ints(p.off_row_index, h.n_active).copy(), ints(p.off_seg_start, h.n_seg + 1).copy(),
                        ints(p.off_seg_adapter, h.n_seg).copy(), ints(p.off_seg_rank, h.n_seg).copy())
        work = ints(p.off_work, WORK_INTS * p.work_capacity).reshape(-1, WORK_INTS)
        items = {r.variant: work[r.begin:r.begin + h.live[i]].copy()
                 for i, r in enumerate(p.info.ranges[:p.info.n_ranges])}
        return h, segs, items

    def prepare_apply(self, projs, stream=None):
        """projs as for Batch.prepare_apply; v buffers from new_v."""
        arr = (lora_apply_proj_t * len(projs))(*[
            lora_apply_proj_t(x.data_ptr(), x.stride(0), x.shape[1], A.c(), v.data_ptr(), v.stride(1), B.c(),
                              y.shape[1], y.data_ptr(), y.stride(0), float(s))
            for x, A, v, B, y, s in projs])
        for p in projs:
            v = p[2]
            assert v.dtype == torch.float32 and v.is_contiguous() and v.dim() == 3
            assert v.shape[0] >= self.v_slices and v.shape[1] == self.plan.n_rows
        h, n, L = stream_handle(stream), len(projs), self._launch

        def run():
            call_apply(L, arr, n, h)
        run.keep = (projs, arr)
        return run

    def apply(self, projs, stream=None):
        self.prepare_apply(projs, stream)()


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


class AdapterPool:
    """Adapters paged into one device pool on demand (S-LoRA article,
    "Unified Paging").  LoraPool (the library's pool manager) decides which
    pages hold which adapter and keeps the row-offset tables; this class
    copies the rows of newly placed adapters in on its own stream (one
    host-to-device copy of the packed rows, then lora_pool_scatter into their
    pages) together with their table entries.

    weights(a) returns, per row table t, adapter a's rows as host bf16 bits
    [rank][row_len[t]].  acquire() pins a batch's adapters and starts the
    copies; the compute stream waits for them with wait(); release_after()
    unpins the adapters once the work enqueued so far on a stream has finished
    (an adapter is only evicted after its last batch has run)."""

    def __init__(self, n_pages, page_elems, n_adapters, max_rank, row_len, weights, device="cuda"):
        self.mgr = LoraPool(n_pages, page_elems, n_adapters, max_rank, row_len)
        self.device = torch.device(device)
        self.row_len = [int(r) for r in row_len]
        self.page_elems, self.n_adapters, self.max_rank = int(page_elems), int(n_adapters), int(max_rank)
        self.weights = weights
        self.pool = torch.zeros(int(n_pages) * self.page_elems, dtype=torch.int16, device=self.device)
        self.chunks = [-(-r // self.page_elems) for r in self.row_len]
        self.tables = [torch.zeros(self.n_adapters * self.max_rank * c, dtype=torch.int64, device=self.device)
                       for c in self.chunks]
        self.stream = torch.cuda.Stream(device=self.device)
        self._done = HipEvent()      # the last upload on self.stream
        self._uploading = False
        self._pending = []           # (event, adapters): pins to drop once the event completes
        self._stage = self._meta = None
        self.loaded = 0              # adapters copied in so far
        self._t = (HipEvent(timing=True), HipEvent(timing=True))  # around the last upload's device work

    def rows(self, table):
        """lora_rows_t descriptor of row table `table` in the pool."""
        return Rows(self.pool, self.tables[table], self.n_adapters, self.max_rank, self.row_len[table],
                    self.page_elems)

    def _collect(self, block):
        while self._pending and (block or self._pending[0][0].query()):
            ev, ads = self._pending.pop(0)
            ev.synchronize()
            self.mgr.release(ads)
            block = False

    def acquire(self, adapters, ranks):
        """Pins the adapters, evicting unpinned ones if needed, and enqueues
        the copies of those not resident.  Returns the adapters copied in."""
        self._collect(False)
        st, load = self.mgr.acquire(adapters, ranks, raw=True)
        while st == LORA_ECAPACITY and self._pending:
            self._collect(True)      # wait for the oldest batch in flight and retry
            st, load = self.mgr.acquire(adapters, ranks, raw=True)
        check_status(st, "lora_pool_acquire")
        if len(load):
            rank_of = {int(a): int(r) for a, r in zip(np.asarray(adapters).reshape(-1), np.asarray(ranks).reshape(-1))}
            self._upload(load, rank_of)
        return load

    def _buffers(self, n_src, n_meta):
        if self._stage is None or self._stage[0].shape[0] < n_src:
            self._stage = (torch.empty(max(n_src, 1 << 20), dtype=torch.int16, pin_memory=True),
                           torch.empty(max(n_src, 1 << 20), dtype=torch.int16, device=self.device))
        if self._meta is None or self._meta[0].shape[0] < n_meta:
            self._meta = (torch.empty(max(n_meta, 1 << 16), dtype=torch.int64, pin_memory=True),
                          torch.empty(max(n_meta, 1 << 16), dtype=torch.int64, device=self.device))

    def _upload(self, load, rank_of):
        if self._uploading:
            self._done.synchronize()  # the staging buffers may still be in flight
        so, do, ln, n_src = self.mgr.load_list(load)
        n = so.shape[0]
        blocks = [(t, int(a)) for t in range(len(self.row_len)) for a in load]
        per = [self.max_rank * c for c in self.chunks]
        n_meta = 3 * n + sum(per[t] for t, _ in blocks)
        self._buffers(n_src, n_meta)
        hs, ds = self._stage
        hm, dm = self._meta
        h = hs.numpy().view(np.uint16)
        o = 0
        for a in load:
            for t, w in enumerate(self.weights(int(a))):
                w = np.ascontiguousarray(w, dtype=np.uint16).reshape(-1)
                assert w.shape[0] == rank_of[int(a)] * self.row_len[t], "weights do not match the rank"
                h[o:o + w.shape[0]] = w
                o += w.shape[0]
        m = hm.numpy()
        m[:n], m[n:2 * n], m[2 * n:3 * n] = so, do, ln
        o = 3 * n
        for t, a in blocks:
            tab, _ = self.mgr.row_off(t)
            m[o:o + per[t]] = tab[a * per[t]:(a + 1) * per[t]]
            o += per[t]
        self._t[0].record(self.stream)
        with torch.cuda.stream(self.stream):
            ds[:n_src].copy_(hs[:n_src], non_blocking=True)
            dm[:n_meta].copy_(hm[:n_meta], non_blocking=True)
            base = dm.data_ptr()
            lens = dm[2 * n:3 * n].to(torch.int32) if n else dm[:0].to(torch.int32)
            lora_pool_scatter(ds.data_ptr(), self.pool.data_ptr(), n, base, base + 8 * n, lens.data_ptr(),
                              self.stream.cuda_stream)
            o = 3 * n
            for t, a in blocks:
                self.tables[t][a * per[t]:(a + 1) * per[t]].copy_(dm[o:o + per[t]])
                o += per[t]
            self._lens = lens    # kept alive until the next upload
        self._t[1].record(self.stream)
        self._done.record(self.stream)
        self._uploading = True
        self.loaded += len(load)

    def mgr_rank(self, a):
        """Resident rank of adapter a (from its copy list size)."""
        so, _, ln, n_src = self.mgr.load_list([int(a)])
        return n_src // sum(self.row_len)

    def last_upload_ms(self):
        """Device time of the last upload (host-to-device copies, scatter and
        table entries on the pool's stream), once it has completed."""
        self._t[1].synchronize()
        return self._t[0].elapsed_time(self._t[1])

    def wait(self, stream=None):
        """Make `stream` wait for the copies enqueued so far."""
        if self._uploading:
            self._done.wait(stream)

    def release_after(self, adapters, stream=None):
        """Unpin the adapters once the work enqueued so far on `stream` is done."""
        ev = HipEvent()
        ev.record(stream)
        self._pending.append((ev, np.ascontiguousarray(adapters, dtype=np.int32)))

    def drain(self):
        """Wait for every batch in flight and drop their pins."""
        while self._pending:
            self._collect(True)
