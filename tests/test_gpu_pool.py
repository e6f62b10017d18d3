"""GPU side of the unified adapter pool: the scatter kernel places rows
bit-exactly, and batches served from a pool that is too small for all
adapters (so adapters are evicted and copied in again between batches) give
the oracle's delta, bit-identical to the same batches on a dense layout."""
import sys

import numpy as np
import pytest
import torch

import heterogeneous_adapter_batching_amd as hl
import workloads
from heterogeneous_adapter_batching_amd.session import AdapterPool, Batch
from workloads.device import to_device

from gpu_helpers import check_delta, rows_of, run_delta

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def test_pool_scatter_bit_exact():
    rng = np.random.default_rng(5)
    n_pages, page = 600, 1024
    lens = rng.integers(1, page // 8 + 1, size=500) * 8
    dst_pages = rng.choice(n_pages, size=500, replace=False)
    src_off = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    dst_off = (dst_pages * page).astype(np.int64)
    src = rng.integers(0, 1 << 16, size=int(lens.sum()), dtype=np.uint16)
    ref = rng.integers(0, 1 << 16, size=n_pages * page, dtype=np.uint16)
    pool = torch.from_numpy(ref.view(np.int16).copy()).cuda()
    for so, do, ln in zip(src_off, dst_off, lens):
        ref[do:do + ln] = src[so:so + ln]
    d_src = torch.from_numpy(src.view(np.int16)).cuda()
    d_so, d_do = torch.from_numpy(src_off).cuda(), torch.from_numpy(dst_off).cuda()
    d_len = torch.from_numpy(lens.astype(np.int32)).cuda()
    hl.lora_pool_scatter(d_src.data_ptr(), pool.data_ptr(), lens.shape[0], d_so.data_ptr(), d_do.data_ptr(),
                         d_len.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert np.array_equal(pool.cpu().numpy().view(np.uint16), ref)
    assert hl._lib.lora_pool_scatter(d_src.data_ptr() + 2, pool.data_ptr(), 1, d_so.data_ptr(), d_do.data_ptr(),
                                     d_len.data_ptr(), None) == hl.LORA_EINVAL


def _adapter_rows(W, a):
    """Adapter a's rows per table (A then B of each projection) as bf16 bits."""
    out = []
    for p in W.projections:
        for desc in (p.A, p.B):
            r = int(W.adapter_rank[a])
            rows = np.empty((r, desc.row_len), np.uint16)
            for j in range(r):
                o = int(desc.row_off[(a * desc.max_rank + j) * desc.chunks])
                rows[j] = W.pool[o:o + desc.row_len]
            out.append(rows)
    return out


def test_adapter_pool_batches_with_eviction():
    rng = np.random.default_rng(11)
    n_ad, d_in, d_out = 10, 1024, 768
    ranks = rng.choice([8, 16, 32], size=n_ad).astype(np.int32)
    n_rows = 900
    W = workloads.gen_custom(11, np.zeros(n_rows, np.int32), ranks, d_in, d_out, n_proj=2, layout="dense")
    assert all(p.A.chunks == 1 and p.B.chunks == 1 for p in W.projections)
    page = 256
    row_len = [d_in, d_out, d_in, d_out]
    per_rank_row = sum(-(-r // page) for r in row_len)  # 14 pages
    n_pages = 1500                                        # about 4 rank-32 adapters
    pool = AdapterPool(n_pages, page, n_ad, int(ranks.max()), row_len, lambda a: _adapter_rows(W, a))
    stream = torch.cuda.current_stream()
    loaded, copied = [], []
    for b in range(6):
        S = rng.choice(n_ad, size=3, replace=False)
        # long segments on two adapters, single rows on the third, some rows released
        ra = np.full(n_rows, -1, np.int32)
        idx = rng.permutation(n_rows)
        ra[idx[:400]] = S[0]
        ra[idx[400:700]] = S[1]
        ra[idx[700:705]] = S[2]
        load = pool.acquire(S, ranks[S])
        loaded.append(len(load))
        copied += [int(a) for a in load]
        pool.wait(stream)
        dw = to_device(W)
        batch = Batch(n_rows, W.adapter_rank, d_in, d_out).refresh(ra)
        ldv = 32
        vs = [batch.new_v(ldv, fill=float("nan")) for _ in W.projections]
        batch.shrink([(dp.x, pool.rows(2 * i), vs[i]) for i, dp in enumerate(dw.projections)])
        batch.expand([(vs[i], pool.rows(2 * i + 1), dp.y, W.scale) for i, dp in enumerate(dw.projections)])
        pool.release_after(S, stream)
        torch.cuda.synchronize()
        ys = [dp.y.cpu().numpy() for dp in dw.projections]
        _, _, ys_dense = run_delta(W, row_adapter=ra)
        for a, d in zip(ys, ys_dense):
            assert np.array_equal(a, d), "pool and dense layouts differ"
        rows = list(idx[:8]) + list(idx[400:408]) + list(idx[700:705]) + list(idx[705:708])
        _say("batch", b, "adapters", S.tolist(), "copied in", load.tolist(),
             check_delta(W, batch, None, ys, row_adapter=ra, rows=rows, check_v=False))
    pool.drain()
    n_res, free, n_pin = pool.mgr.stats()
    _say("loads per batch", loaded, "resident", n_res, "free pages", free)
    assert n_pin == 0 and pool.loaded == sum(loaded)
    assert len(copied) > len(set(copied)), "no adapter was evicted and copied in again"
