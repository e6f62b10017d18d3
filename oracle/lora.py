"""Heterogeneous LoRA delta and merge/unmerge in fp64 (test infrastructure only).

Delta (BEE-30060 page, Punica paragraph; S-LoRA article, Batching section,
formula 2): for every row i whose adapter a = row_adapter[i] is >= 0, with
rank r = adapter_rank[a],

    v_i[j]  = sum_k x[i, k] * A_a[j, k]                 (j < r)
    y[i, n] = y0[i, n] + s * sum_j v_i[j] * B_a[j, n]

and y[i, :] = y0[i, :] for released rows (LoRazor article: released requests
get no LoRA work).

Merge (VaLoRA blog section 4.4.1; S-LoRA article, formula 1):

    W'[n, k]  = RNE_bf16( W[n, k] + s * sum_j B_a[j, n] * A_a[j, k] )
    W''[n, k] = RNE_bf16( W'[n, k] - s * sum_j B_a[j, n] * A_a[j, k] )

All arithmetic is fp64 on the exact values of the bf16 inputs; the only
rounding to bf16 is the final one of the merge and of the unmerge.

Adapter rows are read through the row-offset table (S-LoRA article, Unified
Paging: a rank-R weight occupies R hidden-size pages): chunk c of row j of
adapter a begins at pool[row_off[(a*max_rank + j)*chunks + c]] and holds
min(chunk_len, row_len - c*chunk_len) elements.
"""
import numpy as np

from .bf16 import bf16_to_f64, f64_to_bf16_rne


def gather_rows_ref(pool, row_off, max_rank, row_len, chunk_len, adapter, rank):
    """Rows 0..rank-1 of ``adapter`` as an fp64 [rank, row_len] array."""
    chunks = -(-row_len // chunk_len)
    out = np.empty((rank, row_len), dtype=np.float64)
    for j in range(rank):
        for c in range(chunks):
            lo = c * chunk_len
            n = min(chunk_len, row_len - lo)
            o = int(row_off[(adapter * max_rank + j) * chunks + c])
            out[j, lo:lo + n] = bf16_to_f64(pool[o:o + n])
    return out


def _rows(pool, desc, adapter, rank, cache):
    key = (id(desc), adapter)
    if key not in cache:
        cache[key] = gather_rows_ref(pool, desc.row_off, desc.max_rank, desc.row_len,
                                     desc.chunk_len, adapter, rank)
    return cache[key]


def apply_ref(row_adapter, adapter_rank, x_bits, y0, pool, A, B, scale, rows=None, cache=None):
    """Per-row loop: returns (y, v) where y[i] is the fp64 output row i and
    v[i] the fp64 rank-r intermediate, for each i in ``rows`` (default: all).

    ``A`` and ``B`` carry ``row_off, max_rank, row_len, chunk_len`` attributes.
    """
    cache = {} if cache is None else cache
    n_rows = len(row_adapter)
    rows = range(n_rows) if rows is None else rows
    y, v = {}, {}
    for i in rows:
        a = int(row_adapter[i])
        y_i = np.asarray(y0[i], dtype=np.float64).copy()
        if a >= 0:
            r = int(adapter_rank[a])
            Aa = _rows(pool, A, a, r, cache)          # [r, d_in]
            Ba = _rows(pool, B, a, r, cache)          # [r, d_out]
            xi = bf16_to_f64(x_bits[i])
            v_i = np.array([np.dot(xi, Aa[j]) for j in range(r)])
            delta = np.zeros_like(y_i)
            for j in range(r):
                delta += v_i[j] * Ba[j]
            y_i += scale * delta
            v[i] = v_i
        y[i] = y_i
    return y, v


def merge_dense_ref(W_bits, A64, B64, scale):
    """W [d_out, d_in] bf16 bits, A [r, d_in], B [r, d_out] fp64 ->
    bf16 bits of RNE(W + scale * B^T A)."""
    W = bf16_to_f64(W_bits)
    dW = B64.T @ A64                                   # [d_out, d_in]
    return f64_to_bf16_rne(W + scale * dW)


def merge_ref(W_bits, pool, A, B, adapter, rank, scale):
    Aa = gather_rows_ref(pool, A.row_off, A.max_rank, A.row_len, A.chunk_len, adapter, rank)
    Ba = gather_rows_ref(pool, B.row_off, B.max_rank, B.row_len, B.chunk_len, adapter, rank)
    return merge_dense_ref(W_bits, Aa, Ba, scale)


def unmerge_ref(W_bits, pool, A, B, adapter, rank, scale):
    return merge_ref(W_bits, pool, A, B, adapter, rank, -scale)
