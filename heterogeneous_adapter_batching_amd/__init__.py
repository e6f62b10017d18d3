"""Heterogeneous LoRA adapter batching on MI355X (gfx950).

Thin Python binding of ``libhetlora.so`` (declared in ``include/hetlora.h``):
the functions below carry the C entry points' names and only marshal
arguments -- numpy arrays for host inputs, raw device addresses (e.g.
``tensor.data_ptr()``) for device buffers, an integer ``hipStream_t`` for the
stream.  Every step of the path runs in the library.  There is no fallback:
importing this package fails loudly when the library is not built.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhetlora.so")

LORA_ABI_VERSION = 10
LORA_STATIC_SCRATCH_BYTES = 64 << 20
LORA_MAX_RANK = 128
LORA_MAX_PROJ = 8
LORA_MAX_RANGES = 48
LORA_MAX_MERGE = 8
LORA_MAX_SLICES = 16
LORA_INLINE_ITEMS = 64
LORA_PREPARE_INLINE = 0x100
WORK_INTS = 8  # int32 fields of lora_work_t
LORA_OK, LORA_EINVAL, LORA_EADAPTER, LORA_ERANK, LORA_ESHAPE, LORA_ECAPACITY, LORA_EHIP = 0, -1, -2, -3, -4, -5, -6
LORA_OP_SHRINK, LORA_OP_EXPAND, LORA_OP_APPLY = 0, 1, 2

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built: run `python __graft_entry__.py` (build()) first")
# The library must use the same HIP runtime as the caller's streams and
# memory.  PyTorch-ROCm ships its own libamdhip64 under the same soname as the
# system one: loaded after torch, the library binds to torch's copy; loaded
# before it, the process ends up with two runtimes and launches on torch's
# streams fail.  So torch, when installed, is loaded first.
try:
    import torch  # noqa: F401
except ImportError:
    pass
_lib = ctypes.CDLL(LIB_PATH)

_i32, _i64, _f32, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
_P = ctypes.POINTER


class lora_rows_t(ctypes.Structure):
    _fields_ = [("pool", _vp), ("row_off", _vp), ("n_adapters", _i32), ("max_rank", _i32),
                ("row_len", _i32), ("chunk_len", _i32), ("neg_from", _vp)]


class lora_work_t(ctypes.Structure):
    _fields_ = [("row0", _i32), ("nrows", _i32), ("adapter", _i32), ("rank", _i32), ("kslice", _i32),
                ("nslices", _i32), ("reserved", _i32 * 2)]


class lora_range_t(ctypes.Structure):
    _fields_ = [("variant", _i32), ("begin", _i32), ("count", _i32), ("rows_per_item", _i32)]


class lora_plan_info_t(ctypes.Structure):
    _fields_ = [("op", _i32), ("n_work", _i32), ("n_active", _i32), ("max_rank", _i32),
                ("max_adapter", _i32), ("v_slices", _i32), ("d_in", _i32), ("d_out", _i32), ("n_ranges", _i32),
                ("ranges", lora_range_t * LORA_MAX_RANGES)]

    def range_list(self):
        return [(r.variant, r.begin, r.count, r.rows_per_item) for r in self.ranges[:self.n_ranges]]


class lora_launch_t(ctypes.Structure):
    _fields_ = [("row_index", _vp), ("work", _vp), ("info", lora_plan_info_t), ("live", _vp),
                ("host_work", _vp), ("host_row_index", _vp)]


class lora_device_plan_t(ctypes.Structure):
    _fields_ = [("n_rows", _i32), ("n_adapters", _i32), ("max_rank", _i32), ("d_in", _i32), ("d_out", _i32),
                ("seg_capacity", _i32), ("work_capacity", _i32), ("reserved", _i32),
                ("off_row_index", _i64), ("off_seg_start", _i64), ("off_seg_adapter", _i64),
                ("off_seg_rank", _i64), ("off_scratch", _i64), ("off_work", _i64), ("workspace_bytes", _i64),
                ("info", lora_plan_info_t)]


class lora_device_header_t(ctypes.Structure):
    _fields_ = [("status", _i32), ("n_seg", _i32), ("n_active", _i32), ("n_work", _i32),
                ("live", _i32 * LORA_MAX_RANGES)]


class lora_batch_t(ctypes.Structure):
    _fields_ = [("n_seg", _i32), ("n_active", _i32), ("n_staged", _i64), ("launch", lora_launch_t * 3)]


class lora_shrink_proj_t(ctypes.Structure):
    _fields_ = [("x", _vp), ("ldx", _i64), ("d_in", _i32), ("A", lora_rows_t), ("v", _vp), ("ldv", _i64)]


class lora_expand_proj_t(ctypes.Structure):
    _fields_ = [("v", _vp), ("ldv", _i64), ("B", lora_rows_t), ("d_out", _i32), ("y", _vp),
                ("ldy", _i64), ("scale", _f32)]


class lora_apply_proj_t(ctypes.Structure):
    _fields_ = [("x", _vp), ("ldx", _i64), ("d_in", _i32), ("A", lora_rows_t), ("v", _vp), ("ldv", _i64),
                ("B", lora_rows_t), ("d_out", _i32), ("y", _vp), ("ldy", _i64), ("scale", _f32)]


class lora_merge_mat_t(ctypes.Structure):
    _fields_ = [("W", _vp), ("ldw", _i64), ("d_out", _i32), ("d_in", _i32), ("A", lora_rows_t),
                ("B", lora_rows_t), ("adapter", _i32), ("rank", _i32), ("scale", _f32)]


_sig = {
    "lora_abi_version": (_i32, []),
    "lora_status_string": (ctypes.c_char_p, [_i32]),
    "lora_build_segments": (_i32, [_i32, _vp, _i32, _vp, _i32, _vp, _vp, _vp, _vp, _P(_i32), _P(_i32)]),
    "lora_plan": (_i32, [_i32, _i32, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _P(lora_plan_info_t)]),
    "lora_plan_table": (_i32, [_i32, _i32, _vp, _vp, _vp, _i32, _i32, _vp, _vp, _i32, _vp, _P(lora_plan_info_t)]),
    "lora_shrink": (_i32, [_P(lora_launch_t), _i32, _P(lora_shrink_proj_t), _vp]),
    "lora_expand": (_i32, [_P(lora_launch_t), _i32, _P(lora_expand_proj_t), _vp]),
    "lora_apply": (_i32, [_P(lora_launch_t), _i32, _P(lora_apply_proj_t), _vp]),
    "lora_apply_static": (_i32, [_P(lora_launch_t), _i32, _P(lora_apply_proj_t), _vp]),
    "lora_merge": (_i32, [_i32, _P(lora_merge_mat_t), _vp]),
    "lora_unmerge": (_i32, [_i32, _P(lora_merge_mat_t), _vp]),
    "lora_rows_dense_offsets": (_i32, [_i32, _i32, _vp, _i32, _i32, _vp, _P(_i64)]),
    "lora_mixture_row_adapter": (_i32, [_i32, _vp, _i32, _i32, _vp]),
    "lora_mixture_rows": (_i32, [_i32, _i32, _vp, _i32, _i32, _vp, _i32, _vp, _vp, _vp]),
    "lora_batch_prepare": (_i32, [_i32, _vp, _i32, _vp, _i32, _i32, ctypes.c_uint32, _i32, _vp, _vp, _vp, _vp,
                                  _i64, _vp, _vp, _P(lora_batch_t)]),
    "lora_device_plan": (_i32, [_i32, _i32, _i32, _i32, _i32, _P(lora_device_plan_t)]),
    "lora_batch_build_device": (_i32, [_P(lora_device_plan_t), _vp, _vp, _vp, _vp, _P(lora_launch_t)]),
    "lora_pool_create": (_i32, [_i64, _i32, _i32, _i32, _i32, _vp, _P(_vp)]),
    "lora_pool_destroy": (_i32, [_vp]),
    "lora_pool_acquire": (_i32, [_vp, _i32, _vp, _vp, _vp, _P(_i32)]),
    "lora_pool_release": (_i32, [_vp, _i32, _vp]),
    "lora_pool_row_off": (_i32, [_vp, _i32, _P(_P(_i64)), _P(_i32)]),
    "lora_pool_stats": (_i32, [_vp, _P(_i32), _P(_i64), _P(_i32)]),
    "lora_pool_load_list": (_i32, [_vp, _i32, _vp, _i64, _vp, _vp, _vp, _P(_i64), _P(_i64)]),
    "lora_pool_scatter": (_i32, [_vp, _vp, _i64, _vp, _vp, _vp, _vp]),
}
# HIP runtime calls the binding makes itself (events), resolved through the
# library's handle so they bind to the runtime the library uses
_sig.update({
    "hipEventCreateWithFlags": (ctypes.c_int, [_P(_vp), ctypes.c_uint]),
    "hipEventRecord": (ctypes.c_int, [_vp, _vp]),
    "hipEventSynchronize": (ctypes.c_int, [_vp]),
    "hipEventQuery": (ctypes.c_int, [_vp]),
    "hipStreamWaitEvent": (ctypes.c_int, [_vp, _vp, ctypes.c_uint]),
    "hipEventElapsedTime": (ctypes.c_int, [_P(ctypes.c_float), _vp, _vp]),
    "hipEventDestroy": (ctypes.c_int, [_vp]),
})
for _name, (_res, _args) in _sig.items():
    _fn = getattr(_lib, _name)
    _fn.restype, _fn.argtypes = _res, _args


class LoraError(RuntimeError):
    def __init__(self, code, where):
        self.code = code
        super().__init__(f"{where}: {lora_status_string(code)} ({code})")


def _check(code, where):
    if code != LORA_OK:
        raise LoraError(code, where)


check_status = _check

# lora_batch_prepare(n_rows, row_adapter, n_adapters, adapter_rank, d_in, d_out, op_mask, seg_capacity,
#                    seg_start, seg_adapter, seg_rank, staging, staging_capacity, dev_staging, stream, out):
# the raw call, for a caller that binds its pointers once (session.Batch); returns the status
batch_prepare = _lib.lora_batch_prepare


def lora_batch_prepare(row_adapter, adapter_rank, d_in, d_out, op_mask, staging, dev_staging, stream=None,
                       seg_capacity=None, raw=False):
    """Segment table + plans of the ops in op_mask, written to the host int32
    array `staging` and copied to the device pointer `dev_staging` on `stream`
    (a hipStream_t handle or None).  Returns (status, lora_batch_t, (seg_start,
    seg_adapter, seg_rank)); raises LoraError unless raw=True."""
    ra = np.ascontiguousarray(row_adapter, dtype=np.int32)
    rk = np.ascontiguousarray(adapter_rank, dtype=np.int32)
    cap = max(1, min(ra.shape[0], rk.shape[0])) if seg_capacity is None else int(seg_capacity)
    segs = (np.empty(cap + 1, np.int32), np.empty(max(cap, 1), np.int32), np.empty(max(cap, 1), np.int32))
    assert staging.dtype == np.int32 and staging.flags.c_contiguous
    out = lora_batch_t()
    st = _lib.lora_batch_prepare(ra.shape[0], _ptr(ra), rk.shape[0], _ptr(rk), int(d_in), int(d_out), int(op_mask),
                                 cap, *(a.ctypes.data for a in segs), staging.ctypes.data, staging.shape[0],
                                 dev_staging, stream, ctypes.byref(out))
    if not raw:
        _check(st, "lora_batch_prepare")
    return st, out, segs


def lora_device_plan(n_rows, n_adapters, max_rank, d_in, d_out, raw=False):
    """Layout of a device-built apply plan for the given bounds: returns
    (status, lora_device_plan_t); raises LoraError unless raw=True."""
    out = lora_device_plan_t()
    st = _lib.lora_device_plan(int(n_rows), int(n_adapters), int(max_rank), int(d_in), int(d_out),
                               ctypes.byref(out))
    if not raw:
        _check(st, "lora_device_plan")
    return st, out


def lora_batch_build_device(plan, row_adapter_ptr, adapter_rank_ptr, workspace_ptr, stream=None, raw=False):
    """Enqueue the device plan builder on `stream` (device pointers in,
    nothing copied).  Returns (status, lora_launch_t); raises LoraError unless
    raw=True.  The device-side status is in the workspace header."""
    out = lora_launch_t()
    st = _lib.lora_batch_build_device(ctypes.byref(plan), row_adapter_ptr, adapter_rank_ptr, workspace_ptr, stream,
                                      ctypes.byref(out))
    if not raw:
        _check(st, "lora_batch_build_device")
    return st, out


class LoraPool:
    """Host-side pool manager (lora_pool_*): pages of a device pool assigned
    to adapters on demand.  row_len: the row length of each row table."""

    def __init__(self, n_pages, page_elems, n_adapters, max_rank, row_len):
        self.row_len = np.ascontiguousarray(row_len, dtype=np.int32)
        self.n_pages, self.page_elems = int(n_pages), int(page_elems)
        self.n_adapters, self.max_rank = int(n_adapters), int(max_rank)
        h = _vp()
        _check(_lib.lora_pool_create(self.n_pages, self.page_elems, self.n_adapters, self.max_rank,
                                     self.row_len.shape[0], self.row_len.ctypes.data, ctypes.byref(h)),
               "lora_pool_create")
        self._h = h

    def __del__(self):
        if getattr(self, "_h", None) and _lib is not None:
            _lib.lora_pool_destroy(self._h)
            self._h = None

    def acquire(self, adapters, ranks, raw=False):
        """Returns the adapters whose rows must be copied in (int32 array), or
        (status, that array) with raw=True."""
        a = np.ascontiguousarray(adapters, dtype=np.int32)
        r = np.ascontiguousarray(ranks, dtype=np.int32)
        load = np.empty(max(1, a.shape[0]), np.int32)
        nl = _i32(0)
        st = _lib.lora_pool_acquire(self._h, a.shape[0], _ptr(a), _ptr(r), load.ctypes.data, ctypes.byref(nl))
        if raw:
            return st, load[:nl.value].copy()
        _check(st, "lora_pool_acquire")
        return load[:nl.value].copy()

    def release(self, adapters, raw=False):
        a = np.ascontiguousarray(adapters, dtype=np.int32)
        st = _lib.lora_pool_release(self._h, a.shape[0], _ptr(a))
        if raw:
            return st
        _check(st, "lora_pool_release")

    def row_off(self, table):
        """(view of the host row-offset table, chunks per row); the view is
        valid until the next acquire."""
        p, ch = _P(_i64)(), _i32(0)
        _check(_lib.lora_pool_row_off(self._h, int(table), ctypes.byref(p), ctypes.byref(ch)), "lora_pool_row_off")
        n = self.n_adapters * self.max_rank * ch.value
        return np.ctypeslib.as_array(p, shape=(n,)), ch.value

    def stats(self):
        """(resident adapters, free pages, pinned adapters)."""
        r, f, p = _i32(0), _i64(0), _i32(0)
        _check(_lib.lora_pool_stats(self._h, ctypes.byref(r), ctypes.byref(f), ctypes.byref(p)), "lora_pool_stats")
        return r.value, f.value, p.value

    def load_list(self, adapters):
        """(src_off int64, dst_off int64, len int32, packed source elements)."""
        a = np.ascontiguousarray(adapters, dtype=np.int32)
        n, src = _i64(0), _i64(0)
        st = _lib.lora_pool_load_list(self._h, a.shape[0], _ptr(a), 0, None, None, None, ctypes.byref(n),
                                      ctypes.byref(src))
        if st not in (LORA_OK, LORA_ECAPACITY):
            _check(st, "lora_pool_load_list")
        so, do, ln = np.empty(n.value, np.int64), np.empty(n.value, np.int64), np.empty(n.value, np.int32)
        _check(_lib.lora_pool_load_list(self._h, a.shape[0], _ptr(a), n.value, _ptr(so), _ptr(do), _ptr(ln),
                                        ctypes.byref(n), ctypes.byref(src)), "lora_pool_load_list")
        return so, do, ln, src.value


def lora_pool_scatter(src_ptr, pool_ptr, n, src_off_ptr, dst_off_ptr, len_ptr, stream=None):
    _check(_lib.lora_pool_scatter(src_ptr, pool_ptr, int(n), src_off_ptr, dst_off_ptr, len_ptr, stream),
           "lora_pool_scatter")


def _ptr(a):
    return a.ctypes.data if a is not None and a.size else None


def lora_abi_version():
    return _lib.lora_abi_version()


def lora_status_string(code):
    return _lib.lora_status_string(int(code)).decode()


class Segments:
    """Host result of lora_build_segments."""

    def __init__(self, row_index, seg_start, seg_adapter, seg_rank):
        self.row_index, self.seg_start, self.seg_adapter, self.seg_rank = row_index, seg_start, seg_adapter, seg_rank

    @property
    def n_seg(self):
        return int(self.seg_adapter.shape[0])

    @property
    def n_active(self):
        return int(self.row_index.shape[0])


def lora_build_segments(row_adapter, adapter_rank, seg_capacity=None, raw=False, out=None):
    """Segment table of a batch (host).  Returns Segments (views into `out`,
    a tuple of int32 arrays (row_index, seg_start, seg_adapter, seg_rank), when
    given); with raw=True returns (status, n_seg, n_active) instead of raising,
    for error-path tests."""
    ra = np.ascontiguousarray(row_adapter, dtype=np.int32)
    rk = np.ascontiguousarray(adapter_rank, dtype=np.int32)
    n_rows, n_ad = ra.shape[0], rk.shape[0]
    if out is not None:
        row_index, seg_start, seg_adapter, seg_rank = out
        cap = min(seg_adapter.shape[0], seg_start.shape[0] - 1) if seg_capacity is None else int(seg_capacity)
        assert row_index.shape[0] >= n_rows and seg_rank.shape[0] >= cap
    else:
        cap = min(n_ad, n_rows) if seg_capacity is None else int(seg_capacity)
        row_index = np.empty(max(n_rows, 1), np.int32)
        seg_start = np.empty(cap + 1, np.int32)
        seg_adapter = np.empty(max(cap, 1), np.int32)
        seg_rank = np.empty(max(cap, 1), np.int32)
    n_seg, n_act = _i32(-7), _i32(-7)
    st = _lib.lora_build_segments(n_rows, _ptr(ra), n_ad, _ptr(rk), cap, row_index.ctypes.data,
                                  seg_start.ctypes.data, seg_adapter.ctypes.data, seg_rank.ctypes.data,
                                  ctypes.byref(n_seg), ctypes.byref(n_act))
    if raw:
        return st, n_seg.value, n_act.value
    _check(st, "lora_build_segments")
    ns, na = n_seg.value, n_act.value
    if out is not None:
        return Segments(row_index[:na], seg_start[:ns + 1], seg_adapter[:ns], seg_rank[:ns])
    return Segments(row_index[:na].copy(), seg_start[:ns + 1].copy(), seg_adapter[:ns].copy(),
                    seg_rank[:ns].copy())


def lora_plan(op, segs, d_in, d_out, work_capacity=None, work_out=None, info_out=None):
    """Launch plan (host).  Returns (work int32 [n_work, WORK_INTS], lora_plan_info_t);
    with work_out / info_out the results are written there (work as a view)."""
    if work_out is not None:
        work = work_out
        cap = work.shape[0] if work_capacity is None else int(work_capacity)
    else:
        cap = (LORA_MAX_SLICES + 1) * segs.n_active if work_capacity is None else int(work_capacity)
        work = np.zeros((max(cap, 1), WORK_INTS), np.int32)
    info = lora_plan_info_t() if info_out is None else info_out
    st = _lib.lora_plan(int(op), segs.n_seg, segs.seg_start.ctypes.data, _ptr(segs.seg_adapter),
                        _ptr(segs.seg_rank), int(d_in), int(d_out), cap, work.ctypes.data, ctypes.byref(info))
    _check(st, "lora_plan")
    if work_out is not None:
        return work[:info.n_work], info
    return work[:info.n_work].copy(), info


def lora_plan_table(op, segs, d_in, d_out, shrink_table, expand_table, raw=False):
    """Launch plan with the caller's tile table (the offline tile search's
    planner): shrink_table int8 [8][4][4][2] of (shape, slices), expand_table
    int8 [8][4][4].  Returns (work, info), or (status, work, info) with raw=True."""
    st_tab = np.ascontiguousarray(shrink_table, dtype=np.int8)
    ex_tab = np.ascontiguousarray(expand_table, dtype=np.int8)
    assert st_tab.shape == (8, 4, 4, 2) and ex_tab.shape == (8, 4, 4)
    cap = (LORA_MAX_SLICES + 1) * max(1, segs.n_active)
    work = np.zeros((cap, WORK_INTS), np.int32)
    info = lora_plan_info_t()
    st = _lib.lora_plan_table(int(op), segs.n_seg, segs.seg_start.ctypes.data, _ptr(segs.seg_adapter),
                              _ptr(segs.seg_rank), int(d_in), int(d_out), st_tab.ctypes.data, ex_tab.ctypes.data,
                              cap, work.ctypes.data, ctypes.byref(info))
    if raw:
        return st, work[:max(0, info.n_work)].copy(), info
    _check(st, "lora_plan_table")
    return work[:info.n_work].copy(), info


def make_rows(pool_ptr, row_off_ptr, n_adapters, max_rank, row_len, chunk_len, neg_from_ptr=None):
    return lora_rows_t(pool_ptr, row_off_ptr, int(n_adapters), int(max_rank), int(row_len), int(chunk_len),
                       neg_from_ptr)


def make_launch(row_index_ptr, work_ptr, info):
    return lora_launch_t(row_index_ptr, work_ptr, info)


def call_shrink(launch, arr, n, stream):
    """lora_shrink with a prebuilt ctypes projection array (no per-call marshalling)."""
    _check(_lib.lora_shrink(ctypes.byref(launch), n, arr, stream), "lora_shrink")


def call_expand(launch, arr, n, stream):
    _check(_lib.lora_expand(ctypes.byref(launch), n, arr, stream), "lora_expand")


def call_apply(launch, arr, n, stream):
    _check(_lib.lora_apply(ctypes.byref(launch), n, arr, stream), "lora_apply")


def call_merge(arr, n, stream, unmerge=False):
    fn = _lib.lora_unmerge if unmerge else _lib.lora_merge
    _check(fn(n, arr, stream), "lora_unmerge" if unmerge else "lora_merge")


def lora_shrink(launch, projs, stream):
    arr = (lora_shrink_proj_t * len(projs))(*projs)
    _check(_lib.lora_shrink(ctypes.byref(launch), len(projs), arr, stream), "lora_shrink")


def lora_expand(launch, projs, stream):
    arr = (lora_expand_proj_t * len(projs))(*projs)
    _check(_lib.lora_expand(ctypes.byref(launch), len(projs), arr, stream), "lora_expand")


def lora_apply(launch, projs, stream):
    arr = (lora_apply_proj_t * len(projs))(*projs)
    _check(_lib.lora_apply(ctypes.byref(launch), len(projs), arr, stream), "lora_apply")


def lora_merge(mats, stream):
    arr = (lora_merge_mat_t * len(mats))(*mats)
    _check(_lib.lora_merge(len(mats), arr, stream), "lora_merge")


def lora_unmerge(mats, stream):
    arr = (lora_merge_mat_t * len(mats))(*mats)
    _check(_lib.lora_unmerge(len(mats), arr, stream), "lora_unmerge")


def lora_rows_dense_offsets(rank, max_rank, row_len, chunk_len):
    """Dense packed row-offset table (host).  Returns (row_off int64, pool_elems)."""
    rk = np.ascontiguousarray(rank, dtype=np.int32)
    chunks = -(-int(row_len) // int(chunk_len)) if chunk_len > 0 else 1
    off = np.empty(max(1, rk.shape[0] * int(max_rank) * chunks), np.int64)
    pe = _i64(0)
    _check(_lib.lora_rows_dense_offsets(rk.shape[0], int(max_rank), _ptr(rk), int(row_len), int(chunk_len),
                                        off.ctypes.data, ctypes.byref(pe)), "lora_rows_dense_offsets")
    return off[:rk.shape[0] * int(max_rank) * chunks].copy(), pe.value


def lora_mixture_row_adapter(row_adapter, merged, base_rows=True, raw=False):
    """deLoRA mixture batch (host): rows on the merged adapter -> -1; released
    rows -> the merged adapter's composite (minus the merged adapter: the
    backbone output) when base_rows, else left released.  With raw=True
    returns (status, out) instead of raising."""
    ra = np.ascontiguousarray(row_adapter, dtype=np.int32)
    out = np.empty(max(1, ra.shape[0]), np.int32)
    st = _lib.lora_mixture_row_adapter(ra.shape[0], _ptr(ra), int(merged), int(bool(base_rows)), out.ctypes.data)
    if raw:
        return st, out[:ra.shape[0]]
    _check(st, "lora_mixture_row_adapter")
    return out[:ra.shape[0]].copy()


def lora_mixture_rows(rank, merged, chunks, row_off, max_rank, out_max_rank, raw=False):
    """deLoRA composite row table (host): returns (out_row_off int64, out_rank
    int32, out_neg_from int32).  With raw=True returns (status, ...)."""
    rk = np.ascontiguousarray(rank, dtype=np.int32)
    ro = np.ascontiguousarray(row_off, dtype=np.int64)
    n = rk.shape[0]
    out_off = np.zeros(max(1, n * int(out_max_rank) * int(chunks)), np.int64)
    out_rank = np.zeros(max(1, n), np.int32)
    out_neg = np.zeros(max(1, n), np.int32)
    st = _lib.lora_mixture_rows(n, int(max_rank), _ptr(rk), int(merged), int(chunks), _ptr(ro), int(out_max_rank),
                                out_off.ctypes.data, out_rank.ctypes.data, out_neg.ctypes.data)
    res = (out_off[:n * int(out_max_rank) * int(chunks)], out_rank[:n], out_neg[:n])
    if raw:
        return (st,) + res
    _check(st, "lora_mixture_rows")
    return res
