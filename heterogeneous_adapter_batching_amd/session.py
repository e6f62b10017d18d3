"""Device-resident batch metadata and call marshalling.

``Batch`` runs the library's segment builder and planner on the host, then
moves row_index and both work lists to the device in one pinned host->device
copy on the caller's stream; ``Batch.shrink`` / ``Batch.expand`` /
``merge`` / ``unmerge`` turn torch tensors into the C structs and call the
library.  PyTorch only provides memory and streams here.
"""
import numpy as np
import torch

from . import (LORA_OP_EXPAND, LORA_OP_SHRINK, lora_build_segments, lora_expand, lora_merge,
               lora_plan, lora_shrink, lora_unmerge, make_launch, make_rows, lora_expand_proj_t,
               lora_merge_mat_t, lora_shrink_proj_t)


def staging_layout(n_active, n_work_shrink, n_work_expand):
    """Byte offsets of (row_index, shrink work, expand work) in the staging
    buffer, and its size in int32 elements: row_index is int32 [n_active],
    each work item 4 int32 (16 bytes)."""
    ri = 0
    ws = 4 * n_active
    we = ws + 16 * n_work_shrink
    n = max(1, n_active + 4 * (n_work_shrink + n_work_expand))
    return ri, ws, we, n


def stream_handle(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


class Rows:
    """A row table on the device: pool (bf16 bits) + row_off (int64)."""

    def __init__(self, pool, row_off, n_adapters, max_rank, row_len, chunk_len):
        assert pool.is_cuda and row_off.is_cuda and row_off.dtype == torch.int64
        self.pool, self.row_off = pool, row_off
        self.n_adapters, self.max_rank, self.row_len, self.chunk_len = n_adapters, max_rank, row_len, chunk_len

    def c(self):
        return make_rows(self.pool.data_ptr(), self.row_off.data_ptr(), self.n_adapters, self.max_rank,
                         self.row_len, self.chunk_len)


class Batch:
    """Segments + shrink/expand plans of one batch, resident on the device.

    ``refresh(row_adapter)`` rebuilds everything for a new batch of the same
    or smaller size, reusing the pinned staging buffer and device buffer."""

    def __init__(self, n_rows_max, adapter_rank, d_in, d_out, device="cuda"):
        self.adapter_rank = np.ascontiguousarray(adapter_rank, dtype=np.int32)
        self.d_in, self.d_out = int(d_in), int(d_out)
        self.device = torch.device(device)
        cap = 1 + 9 * max(1, int(n_rows_max))          # row_index + two work lists of 4 ints
        self._host = torch.empty(cap, dtype=torch.int32, pin_memory=True)
        self._dev = torch.empty(cap, dtype=torch.int32, device=self.device)
        self._copied = None          # event of the last staging copy
        self.segs = None

    def refresh(self, row_adapter, stream=None):
        segs = lora_build_segments(row_adapter, self.adapter_rank)
        ws, info_s = lora_plan(LORA_OP_SHRINK, segs, self.d_in, self.d_out)
        we, info_e = lora_plan(LORA_OP_EXPAND, segs, self.d_in, self.d_out)
        na, ns, ne = segs.n_active, ws.shape[0], we.shape[0]
        if self._copied is not None:
            self._copied.synchronize()   # the staging buffer may still be in flight
        h = self._host.numpy()
        assert na + 4 * (ns + ne) <= h.shape[0], "batch larger than n_rows_max"
        h[:na] = segs.row_index
        h[na:na + 4 * ns] = ws.reshape(-1)
        h[na + 4 * ns:na + 4 * (ns + ne)] = we.reshape(-1)
        o_ri, o_ws, o_we, n = staging_layout(na, ns, ne)
        with torch.cuda.stream(stream) if stream is not None else _null():
            self._dev[:n].copy_(self._host[:n], non_blocking=True)
            self._copied = torch.cuda.Event()
            self._copied.record()
        base = self._dev.data_ptr()
        self.segs, self.work_shrink, self.work_expand = segs, ws, we
        self.info_shrink, self.info_expand = info_s, info_e
        self.shrink_launch = make_launch(base + o_ri, base + o_ws, info_s)
        self.expand_launch = make_launch(base + o_ri, base + o_we, info_e)
        return self

    @property
    def n_active(self):
        return self.segs.n_active

    def shrink(self, projs, stream=None):
        """projs: list of (x tensor bf16 [*, ldx], Rows A, v tensor fp32 [n_active, ldv])."""
        cs = [lora_shrink_proj_t(x.data_ptr(), x.stride(0), x.shape[1], A.c(), v.data_ptr(), v.stride(0))
              for x, A, v in projs]
        lora_shrink(self.shrink_launch, cs, stream_handle(stream))

    def expand(self, projs, stream=None):
        """projs: list of (v tensor fp32, Rows B, y tensor fp32 [*, ldy], scale)."""
        cs = [lora_expand_proj_t(v.data_ptr(), v.stride(0), B.c(), y.shape[1], y.data_ptr(), y.stride(0),
                                 float(s)) for v, B, y, s in projs]
        lora_expand(self.expand_launch, cs, stream_handle(stream))


class _null:
    def __enter__(self):
        return self

    def __exit__(self, *a):
        return False


def merge_mats(mats):
    """mats: list of (W tensor bf16 [d_out, ldw], Rows A, Rows B, adapter, rank, scale)."""
    return [lora_merge_mat_t(W.data_ptr(), W.stride(0), W.shape[0], W.shape[1], A.c(), B.c(),
                             int(a), int(r), float(s)) for W, A, B, a, r, s in mats]


def merge(mats, stream=None):
    lora_merge(merge_mats(mats), stream_handle(stream))


def unmerge(mats, stream=None):
    lora_unmerge(merge_mats(mats), stream_handle(stream))
