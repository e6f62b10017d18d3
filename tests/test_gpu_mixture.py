"""GPU parity of deLoRA mixture inference (VaLoRA blog, section 4.4.2): with
adapter m merged, rows on other adapters get y += s x A_x^T B_x - s x A_m^T B_m
through composite adapters (lora_mixture_rows, neg_from on the A side), rows
on m are untouched, and released rows get the backbone output y += -s x A_m^T
B_m (or stay untouched with base_rows=False).  Compared with the oracle's
mixture_ref; tolerances as in test_gpu_parity (contract bounds plus the
precision check), untouched rows bit-exact."""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
import heterogeneous_adapter_batching_amd as hl
from heterogeneous_adapter_batching_amd.session import Batch, Rows, mixture_tables
from workloads.device import to_device

from gpu_helpers import ABS_TOL, REL_F_EXPECT, REL_F_TOL

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _run_mixture(W, m, path, base_rows=True):
    dw = to_device(W)
    ra = hl.lora_mixture_row_adapter(W.row_adapter, m, base_rows=base_rows)
    out_max = int(max(W.adapter_rank[a] + (W.adapter_rank[m] if a != m else 0) for a in range(len(W.adapter_rank))))
    out_max = -(-out_max // 4) * 4
    projs, crank = [], None
    for p, d in zip(W.projections, dw.projections):
        ca, cb, neg, crank = mixture_tables((p.A.row_off, p.B.row_off, p.A.max_rank, p.A.chunks, p.B.chunks),
                                            W.adapter_rank, m, out_max)
        A = Rows(dw.pool, ca, p.A.n_adapters, out_max, p.A.row_len, p.A.chunk_len, neg_from=neg)
        B = Rows(dw.pool, cb, p.B.n_adapters, out_max, p.B.row_len, p.B.chunk_len)
        projs.append((d, A, B, (ca, cb, neg)))
    d_in = max(p.d_in for p in W.projections)
    d_out = max(p.d_out for p in W.projections)
    b = Batch(max(1, W.n_rows), crank, d_in, d_out).refresh(ra)
    ldv = out_max
    vs = [b.new_v(ldv, fill=float("nan")) for _ in projs]
    if path == "apply":
        b.apply([(d.x, A, v, B, d.y, W.scale) for (d, A, B, _), v in zip(projs, vs)])
    else:
        b.shrink([(d.x, A, v) for (d, A, B, _), v in zip(projs, vs)])
        b.expand([(v, B, d.y, W.scale) for (d, A, B, _), v in zip(projs, vs)])
    torch.cuda.synchronize()
    return b, [d.y.cpu().numpy() for d, _, _, _ in projs]


def _check(W, m, ys, base_rows=True):
    for p, y in zip(W.projections, ys):
        ref = oracle.mixture_ref(W.row_adapter, W.adapter_rank, m, p.x, p.y0, W.pool, p.A, p.B, W.scale,
                                 base_rows=base_rows)
        num = den = amax = 0.0
        for i in range(W.n_rows):
            a = int(W.row_adapter[i])
            if (a < 0 and not base_rows) or a == m:
                assert np.array_equal(y[i], p.y0[i]), f"row {i} (adapter {a}) must be untouched"
                continue
            d_ref = ref[i] - p.y0[i].astype(np.float64)
            d_gpu = y[i].astype(np.float64) - p.y0[i].astype(np.float64)
            num += float(np.sum((d_gpu - d_ref) ** 2))
            den += float(np.sum(d_ref ** 2))
            amax = max(amax, float(np.max(np.abs(y[i].astype(np.float64) - ref[i]))))
        relF = (num / den) ** 0.5 if den > 0 else 0.0
        assert relF <= REL_F_TOL and amax <= ABS_TOL, (p.name, relF, amax)
        assert relF <= REL_F_EXPECT, (p.name, relF)
        _say(p.name, "relF", relF, "max abs", amax)


@pytest.mark.parametrize("path,base_rows", [("apply", True), ("split", True), ("apply", False)])
def test_mixture_decode_rows(path, base_rows):
    """One-token rows on 48 adapters, adapter 5 merged (lora_apply: the fused
    kernel), two released rows (backbone output, or untouched)."""
    ra = np.array(list(range(48)) + [5, 5, -1, 7, -1], np.int32)
    W = workloads.gen_custom(31, ra, np.full(48, 16), 4096, 4096, n_proj=2)
    _say("mixture decode", path, "base rows", base_rows)
    _, ys = _run_mixture(W, 5, path, base_rows)
    _check(W, 5, ys, base_rows)


@pytest.mark.parametrize("layout", ["dense", "paged"])
def test_mixture_segments(layout):
    """Segments of 1 to 300 rows, ranks 8..64, adapter 1 merged: short-segment
    and long-segment shrink kernels, MFMA and VALU expand."""
    lens = [1, 2, 17, 130, 300, 9, 1]
    ra = np.repeat(np.array([0, 1, 2, 3, 2, 4, -1], np.int32), lens)
    W = workloads.gen_custom(32, ra, [8, 24, 64, 16, 40], 1024, 768, n_proj=2, layout=layout, page_elems=256)
    for path in ("apply", "split"):
        _say("mixture segments", layout, path)
        _, ys = _run_mixture(W, 1, path)
        _check(W, 1, ys)
