"""lora_apply_static (the entry point that allocates nothing: v lives in an
array the library holds per device) against lora_apply on the same batch,
through the C ABI: two calls in a row, the second on a smaller batch, each
bit-identical to lora_apply with caller-owned v (the same kernels in the same
order) and within the oracle's bound."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import heterogeneous_adapter_batching_amd as hl
import workloads
from heterogeneous_adapter_batching_amd.session import Batch, stream_handle
from workloads.device import to_device

from gpu_helpers import check_delta, rows_of

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _apply_both(W):
    """y from lora_apply (caller-owned v) and from lora_apply_static, on
    separate copies of y0; returns (batch, y_apply, y_static)."""
    dw = to_device(W)
    d_in = max(p.d_in for p in W.projections)
    d_out = max(p.d_out for p in W.projections)
    b = Batch(W.n_rows, W.adapter_rank, d_in, d_out).refresh(W.row_adapter)
    ldv = -(-int(W.adapter_rank.max()) // 4) * 4
    vs = [b.new_v(ldv, fill=float("nan")) for _ in W.projections]
    ys_static = [d.y.clone() for d in dw.projections]
    b.apply([(d.x, rows_of(dw.pool, p.A, d.A_off), v, rows_of(dw.pool, p.B, d.B_off), d.y, W.scale)
             for p, d, v in zip(W.projections, dw.projections, vs)])
    # the static entry point: v and ldv in the projections are ignored (NULL here)
    arr = (hl.lora_apply_proj_t * len(W.projections))(*[
        hl.lora_apply_proj_t(d.x.data_ptr(), d.x.stride(0), p.d_in, rows_of(dw.pool, p.A, d.A_off).c(), None, 0,
                             rows_of(dw.pool, p.B, d.B_off).c(), p.d_out, y.data_ptr(), y.stride(0), W.scale)
        for p, d, y in zip(W.projections, dw.projections, ys_static)])
    st = hl._lib.lora_apply_static(ctypes.byref(b.apply_launch), len(W.projections), arr, stream_handle())
    assert st == hl.LORA_OK, hl.lora_status_string(st)
    torch.cuda.synchronize()
    return b, [d.y.cpu().numpy() for d in dw.projections], [y.cpu().numpy() for y in ys_static]


def test_static_apply_matches_apply_twice_second_smaller():
    # 1: segments of 1 to 300 rows (fused one-row segments, split-K short
    #    segments, long MFMA segments), ranks 1..64, two projections, paged rows
    lens = [1, 1, 3, 17, 300, 9, 1, 130]
    ra = np.repeat(np.array([0, 1, 2, 3, 4, 5, -1, 6], np.int32), lens)
    W1 = workloads.gen_custom(41, ra, [8, 64, 1, 33, 16, 24, 40], 1024, 768, n_proj=2, layout="paged",
                              page_elems=256)
    # 2: the tiny workload (64 rows, rank 8, d 512): a smaller plan reuses the array
    W2 = workloads.gen_config(0)
    for name, W in (("mixed", W1), ("tiny", W2)):
        b, ya, ys = _apply_both(W)
        for pi, (a, s) in enumerate(zip(ya, ys)):
            assert np.array_equal(a, s), (name, pi)
        rep = check_delta(W, b, None, ys, check_v=False)
        _say(name, "rows", W.n_rows, "v slices", b.info_apply.v_slices, "static == apply, oracle:", rep)
