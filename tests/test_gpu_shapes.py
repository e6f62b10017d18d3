"""Every kernel shape on every kind of segment, against the oracle (GPU).

The tile table that the offline search writes may give any bucket any
candidate, so each shrink shape (split-K over 16 rows, items of 64 and of 128
rows) with 1 to 16 K slices, and each expand shape (MFMA items of 16, 64 and
128 rows, the VALU decode kernel over items of two rows), must be right on
every segment length and rank, not only where today's table uses it.  A table
that holds one choice everywhere (lora_plan_table) puts every segment of a
batch on that shape; the batch mixes one-row, short and long segments of
ranks 1 to 128 (the VALU kernel's second rank group starts at 65), the
widths are ragged 64-multiples (a last 512-column group only partly inside
d_out), and the pool is dense, paged with pages that are a multiple of 512
elements (row offsets read through the scalar cache) and paged with 192-element
pages (they are not).  y is compared with the oracle's per-row fp64 delta on
every row; v row by row; released rows bit for bit.
"""
import sys
import types

import numpy as np
import pytest
import torch

import heterogeneous_adapter_batching_amd as hl
import workloads
from heterogeneous_adapter_batching_amd.session import stream_handle
from heterogeneous_adapter_batching_amd.tile_search import read_table
from workloads.device import to_device

from gpu_helpers import check_delta, rows_of

pytestmark = pytest.mark.gpu

# 19 adapters: one-row, 2-row, 3-row, short and long segments, ranks 1..128,
# and released rows between them
_LENS = [1, 1, 1, 2, 3, 1, 2, 5, 17, 40, 70, 129, 300, 1, 2, 1, 4, 9, 200]
_RANKS = [1, 16, 17, 64, 65, 100, 128, 32, 8, 128, 33, 64, 16, 96, 127, 2, 70, 48, 128]


def _batch(seed):
    rng = np.random.default_rng(seed)
    ra = np.concatenate([np.full(n, a, np.int32) for a, n in enumerate(_LENS)])
    ra = ra[rng.permutation(ra.shape[0])]
    ra[rng.choice(ra.shape[0], size=37, replace=False)] = -1
    return ra, np.asarray(_RANKS, np.int32)


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _run(W, st_tab, ex_tab):
    """lora_shrink then lora_expand with plans from the given table."""
    dw = to_device(W)
    segs = hl.lora_build_segments(W.row_adapter, W.adapter_rank)
    d_in = max(p.d_in for p in W.projections)
    d_out = max(p.d_out for p in W.projections)
    ws, si = hl.lora_plan_table(hl.LORA_OP_SHRINK, segs, d_in, d_out, st_tab, ex_tab)
    we, ei = hl.lora_plan_table(hl.LORA_OP_EXPAND, segs, d_in, d_out, st_tab, ex_tab)
    assert si.v_slices == ei.v_slices
    ri = torch.from_numpy(np.ascontiguousarray(segs.row_index)).cuda()
    ws_d = torch.from_numpy(np.ascontiguousarray(ws)).cuda()
    we_d = torch.from_numpy(np.ascontiguousarray(we)).cuda()
    ldv = -(-int(W.adapter_rank.max()) // 4) * 4
    vs = [torch.full((si.v_slices, max(1, segs.n_active), ldv), float("nan"), dtype=torch.float32, device="cuda")
          for _ in W.projections]
    A = [rows_of(dw.pool, p.A, dp.A_off) for p, dp in zip(W.projections, dw.projections)]
    B = [rows_of(dw.pool, p.B, dp.B_off) for p, dp in zip(W.projections, dw.projections)]
    h = stream_handle()
    Ls = hl.make_launch(ri.data_ptr(), ws_d.data_ptr(), si)
    hl.lora_shrink(Ls, [hl.lora_shrink_proj_t(dp.x.data_ptr(), dp.x.stride(0), p.d_in, a.c(), v.data_ptr(), ldv)
                        for p, dp, a, v in zip(W.projections, dw.projections, A, vs)], h)
    Le = hl.make_launch(ri.data_ptr(), we_d.data_ptr(), ei)
    hl.lora_expand(Le, [hl.lora_expand_proj_t(v.data_ptr(), ldv, b.c(), p.d_out, dp.y.data_ptr(), dp.y.stride(0),
                                              W.scale)
                        for p, dp, b, v in zip(W.projections, dw.projections, B, vs)], h)
    torch.cuda.synchronize()
    batch = types.SimpleNamespace(segs=segs, work_expand=we)
    return batch, [v.cpu().numpy() for v in vs], [dp.y.cpu().numpy() for dp in dw.projections]


_LAYOUTS = [("dense", None), ("paged", 1024), ("paged", 192)]


@pytest.mark.parametrize("layout,page", _LAYOUTS, ids=["dense", "paged1024", "paged192"])
@pytest.mark.parametrize("shape", [0, 1, 2])
def test_every_shrink_shape(shape, layout, page):
    st0, ex0 = read_table()
    ra, ranks = _batch(7)
    W = workloads.gen_custom(11, ra, ranks, 1344, 1088, n_proj=2, layout=layout, page_elems=page)
    for sl in (1, 3, 16):
        st, ex = st0.copy(), ex0.copy()
        st[...] = (shape, sl)
        ex[...] = 1
        batch, vs, ys = _run(W, st, ex)
        rep = check_delta(W, batch, vs, ys)
        _say("shrink shape", shape, "slices", sl, layout, page, rep)


@pytest.mark.parametrize("layout,page", _LAYOUTS, ids=["dense", "paged1024", "paged192"])
@pytest.mark.parametrize("shape", [0, 1, 2, 4])
def test_every_expand_shape(shape, layout, page):
    st0, ex0 = read_table()
    ra, ranks = _batch(8)
    W = workloads.gen_custom(12, ra, ranks, 1088, 1600, n_proj=2, layout=layout, page_elems=page)
    st, ex = st0.copy(), ex0.copy()
    st[...] = (0, 2)
    ex[...] = shape
    batch, vs, ys = _run(W, st, ex)
    rep = check_delta(W, batch, vs, ys)
    _say("expand shape", shape, layout, page, rep)
