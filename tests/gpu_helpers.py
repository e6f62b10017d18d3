"""Shared code of the GPU parity tests: run the HIP path through the C ABI and
compare with the oracle on the same seeded inputs."""
import numpy as np
import torch

import oracle
from heterogeneous_adapter_batching_amd.session import Batch, Rows, merge, unmerge
from workloads.device import bits_to_device, to_device

REL_F_TOL = 4e-3      # contract bound (relative Frobenius of the delta)
ABS_TOL = 2e-2        # contract bound (max abs error of y)
REL_F_EXPECT = 1e-4   # fp32 sums of exact bf16 products with a hi+lo split v land near 1e-6
# Bit equality with the oracle's single rounding of the exact fp64 value.  The
# kernel accumulates Delta W in fp32, and where the fp32 value straddles a
# rounding boundary the bits differ (every element stays within the error
# bound check_merge_bits also applies).  An unmerge cancels W' against
# s*Delta W, so its result is small where the merge's was large and more
# elements straddle: an fp32 accumulation of Delta W in rank order, emulated
# in numpy on the vision switch's 4096 x 4096 rank-64 matrices, gives
# 0.99995 equal for the merge and 0.99985 for the unmerge; the kernel
# measures 0.99996 and 0.99987.
MERGE_MIN_EQUAL = 0.9999
UNMERGE_MIN_EQUAL = 0.9995


def rows_of(pool, desc, off):
    return Rows(pool, off, desc.n_adapters, desc.max_rank, desc.row_len, desc.chunk_len)


def run_delta(W, row_adapter=None, dw=None, scale=None, ldv=None):
    """Shrink + expand for every projection of W; returns (batch, v list, y list) on the host."""
    dw = dw if dw is not None else to_device(W)
    ra = W.row_adapter if row_adapter is None else np.asarray(row_adapter, np.int32)
    d_in = max(p.d_in for p in W.projections)
    d_out = max(p.d_out for p in W.projections)
    batch = Batch(max(1, W.n_rows), W.adapter_rank, d_in, d_out).refresh(ra)
    ldv = ldv or -(-int(W.adapter_rank.max()) // 4) * 4
    vs = [batch.new_v(ldv, fill=float("nan")) for _ in W.projections]
    s = W.scale if scale is None else scale
    batch.shrink([(dp.x, rows_of(dw.pool, p.A, dp.A_off), v)
                  for p, dp, v in zip(W.projections, dw.projections, vs)])
    batch.expand([(v, rows_of(dw.pool, p.B, dp.B_off), dp.y, s)
                  for p, dp, v in zip(W.projections, dw.projections, vs)])
    torch.cuda.synchronize()
    return batch, [v.cpu().numpy() for v in vs], [dp.y.cpu().numpy() for dp in dw.projections]


def run_apply(W, row_adapter=None, dw=None, scale=None, ldv=None, inline=False):
    """lora_apply (fused where the plan says so) for every projection of W;
    returns (batch, y list) on the host.  inline: the batch is prepared with
    LORA_PREPARE_INLINE (a small all-fused plan rides in the launch arguments)."""
    dw = dw if dw is not None else to_device(W)
    ra = W.row_adapter if row_adapter is None else np.asarray(row_adapter, np.int32)
    d_in = max(p.d_in for p in W.projections)
    d_out = max(p.d_out for p in W.projections)
    batch = Batch(max(1, W.n_rows), W.adapter_rank, d_in, d_out, inline=inline).refresh(ra)
    ldv = ldv or -(-int(W.adapter_rank.max()) // 4) * 4
    s = W.scale if scale is None else scale
    vs = [batch.new_v(ldv, fill=float("nan")) for _ in W.projections]
    batch.apply([(dp.x, rows_of(dw.pool, p.A, dp.A_off), v, rows_of(dw.pool, p.B, dp.B_off), dp.y, s)
                 for p, dp, v in zip(W.projections, dw.projections, vs)])
    torch.cuda.synchronize()
    return batch, [dp.y.cpu().numpy() for dp in dw.projections]


def check_delta(W, batch, vs, ys, row_adapter=None, rows=None, scale=None, check_v=True):
    """Compare GPU y (and v) with the oracle on `rows` (default: all rows).

    vs[pi] is the GPU v buffer [v_slices, n_active, ldv]: a row's v is the sum
    of its first nslices slices in slice order (what the expand uses); the
    columns beyond the rank and the slices beyond nslices must be unwritten."""
    seg_slices = {}
    for w in (batch.work_expand if check_v else []):
        for p_ in range(int(w[0]), int(w[0]) + int(w[1])):
            seg_slices[p_] = int(w[5])
    ra = W.row_adapter if row_adapter is None else np.asarray(row_adapter, np.int32)
    s = W.scale if scale is None else scale
    rows = list(range(W.n_rows)) if rows is None else list(rows)
    pos = {int(r): p for p, r in enumerate(batch.segs.row_index)}
    report = []
    for pi, p in enumerate(W.projections):
        yref, vref = oracle.apply_ref(ra, W.adapter_rank, p.x, p.y0, W.pool, p.A, p.B, s, rows=rows)
        num = den = 0.0
        amax = 0.0
        for i in rows:
            y_gpu = ys[pi][i].astype(np.float64)
            if ra[i] < 0:
                assert np.array_equal(ys[pi][i], p.y0[i]), f"released row {i} touched"
                continue
            d_ref = yref[i] - p.y0[i].astype(np.float64)
            d_gpu = y_gpu - p.y0[i].astype(np.float64)
            num += float(np.sum((d_gpu - d_ref) ** 2))
            den += float(np.sum(d_ref ** 2))
            amax = max(amax, float(np.max(np.abs(y_gpu - yref[i]))))
            if check_v and vs is not None:
                r = int(W.adapter_rank[ra[i]])
                ns = seg_slices[pos[i]]
                vsl = vs[pi][:, pos[i], :]
                vg = vsl[0].copy()
                for sl in range(1, ns):
                    vg += vsl[sl]
                np.testing.assert_allclose(vg[:r], vref[i], rtol=1e-4, atol=1e-4 * (1 + np.abs(vref[i]).max()))
                assert np.all(np.isnan(vsl[:ns, r:])), "v columns beyond the rank were written"
                assert np.all(np.isnan(vsl[ns:])), "v slices beyond the row's slice count were written"
        relF = (num / den) ** 0.5 if den > 0 else 0.0
        assert np.isfinite(relF) and relF <= REL_F_TOL, (p.name, relF)
        assert amax <= ABS_TOL, (p.name, amax)
        assert relF <= REL_F_EXPECT, (p.name, relF)
        report.append((p.name, relF, amax))
    return report


def ulp_compare(got_bits, ref_bits):
    """Fraction of bf16 elements equal, and max |bit difference| of the rest."""
    g = got_bits.astype(np.int32).reshape(-1)
    r = ref_bits.astype(np.int32).reshape(-1)
    eq = g == r
    return float(eq.mean()), int(np.max(np.abs(g - r))) if not eq.all() else 0


def check_merge_bits(got_bits, W_bits, Aa, Ba, scale, min_equal=MERGE_MIN_EQUAL):
    """Merged W from the GPU against the oracle.

    The oracle rounds the exact W + s*B^T A once to bf16.  The kernel rounds
    W + s*dW once too, but accumulates dW over the rank in fp32, so an element
    may differ from the oracle's bits where that fp32 error straddles a
    rounding boundary -- rarely, and by several ulps only where W and s*dW
    nearly cancel.  Required: >= min_equal of the elements bit-identical, and
    every element within half a bf16 ulp plus an fp32 accumulation bound of
    one fp32 ulp per added term, (r + 4) * 2^-23 * |s| * (|B|^T |A|), plus the
    final fp32 rounding 2^-23 * |exact|, of the exact value."""
    ref = oracle.merge_dense_ref(W_bits, Aa, Ba, scale)
    frac, maxd = ulp_compare(got_bits, ref)
    exact = oracle.bf16_to_f64(W_bits) + scale * (Ba.T @ Aa)
    got = oracle.bf16_to_f64(got_bits)
    r = Aa.shape[0]
    mag = np.abs(Ba).T @ np.abs(Aa)
    a = np.maximum(np.abs(got), 2.0 ** -126)
    ulp = np.exp2(np.floor(np.log2(a)) - 7)
    bound = 0.5 * ulp + (r + 4) * 2.0 ** -23 * abs(scale) * mag + 2.0 ** -23 * np.abs(exact)
    worst = float(np.max(np.abs(got - exact) / bound))
    assert frac >= min_equal, (frac, maxd)
    assert worst <= 1.0, worst
    return frac, maxd, worst


def run_merge(W_bits_list, dw, descs, adapter, rank, scale, unmerge_too=False):
    """Merge adapter into each W (list of uint16 arrays) on the GPU; returns merged (and restored) bits."""
    Ws = [bits_to_device(w) for w in W_bits_list]
    mats = [(Wt, rows_of(dw.pool, A, Aoff), rows_of(dw.pool, B, Boff), adapter, rank, scale)
            for Wt, (A, Aoff, B, Boff) in zip(Ws, descs)]
    merge(mats)
    torch.cuda.synchronize()
    merged = [w.cpu().numpy().view(np.uint16).copy() for w in Ws]
    restored = None
    if unmerge_too:
        unmerge(mats)
        torch.cuda.synchronize()
        restored = [w.cpu().numpy().view(np.uint16).copy() for w in Ws]
    return merged, restored
