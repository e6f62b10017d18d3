"""Pins for the CPU oracle: it is checked against things other than itself.

* bf16 rounding: hand-derived edge cases (tests/golden/bf16_rne_cases.txt) and
  torch's float32 -> bfloat16 cast (a library routine) on random float32 values.
* segments: hand-worked cases and error cases (tests/golden/segments_worked.json)
  plus structural invariants on random batches.
* delta: a hand-worked rank-2 example with non-square shapes (catches a
  transposed operand), the rank-1 closed form (bit-exact), the all-rows-on-one-
  adapter special case against a single numpy matmul, s = 0, released rows,
  permutation of rows, and dense vs paged storage of the same values.
* merge: a hand-worked example, the single rounding on hand-derived ties, the
  exact rank-1 case, merged == unmerged inference (S-LoRA formula 1 vs 2), and
  merge followed by unmerge restoring W within the bf16 bound.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import (apply_ref, bf16_to_f64, build_segments_ref, dense_offsets_ref,
                    f64_to_bf16_rne, gather_rows_ref, merge_dense_ref, merge_ref,
                    unmerge_ref, SegmentError)
from workloads import RowsDesc, build_pool, to_bf16_bits

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _bits(vals):
    """Exact bf16 values (given as floats) -> bits, via torch's cast (exact here)."""
    return to_bf16_bits(np.asarray(vals, dtype=np.float32))


def _pool_from(mats_by_key, n_ad, max_rank, layout="dense", page=64, seed=0):
    items = [(k, m[0].shape[1], m) for k, m in mats_by_key.items()]
    return build_pool(items, n_ad, max_rank, layout, page, np.random.default_rng(seed))


# ----------------------------------------------------------------------------- bf16
def test_bf16_rne_golden_cases():
    with open(os.path.join(GOLD, "bf16_rne_cases.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            val, hexbits = line.split()[:2]
            v = float(val) if val in ("inf", "-inf", "nan") else float.fromhex(val)
            got = int(f64_to_bf16_rne(np.array([v]))[0])
            assert got == int(hexbits, 16), (line, hex(got))


def test_bf16_decode_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x0001, 0x0080, 0x7F7F, 0x7F80, 0xFF80, 0x8000], np.uint16)
    want = [1.0, -2.0, 2.0 ** -133, 2.0 ** -126, (2 - 2 ** -7) * 2.0 ** 127, math.inf, -math.inf, -0.0]
    got = bf16_to_f64(bits)
    for g, w in zip(got, want):
        assert g == w
    assert np.signbit(got[-1])
    assert np.isnan(bf16_to_f64(np.array([0x7FC1], np.uint16))[0])


def test_bf16_rne_matches_torch_cast_on_float32():
    rng = np.random.default_rng(7)
    u = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    want = to_bf16_bits(f)
    got = f64_to_bf16_rne(f.astype(np.float64))
    assert np.array_equal(got, want)
    # decode(encode(bf16 value)) is the identity on finite bf16 values
    allbits = np.arange(0, 2 ** 16, dtype=np.uint32).astype(np.uint16)
    vals = bf16_to_f64(allbits)
    fin = np.isfinite(vals)
    back = f64_to_bf16_rne(vals[fin])
    assert np.array_equal(back, allbits[fin])


# ----------------------------------------------------------------------------- segments
def _gold_segments():
    with open(os.path.join(GOLD, "segments_worked.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _gold_segments()["cases"])
def test_segments_golden(case):
    s = build_segments_ref(case["row_adapter"], case["adapter_rank"])
    for k in ("row_index", "seg_start", "seg_adapter", "seg_rank"):
        assert getattr(s, k).tolist() == case[k], k


@pytest.mark.parametrize("case", _gold_segments()["errors"])
def test_segments_golden_errors(case):
    with pytest.raises(SegmentError) as e:
        build_segments_ref(case["row_adapter"], case["adapter_rank"])
    assert e.value.kind == case["kind"]


def test_segments_invariants_random():
    rng = np.random.default_rng(11)
    for _ in range(300):
        n = int(rng.integers(0, 40))
        n_ad = int(rng.integers(1, 9))
        ranks = rng.integers(1, 129, size=n_ad)
        ra = rng.integers(-1, n_ad, size=n)
        s = build_segments_ref(ra, ranks)
        active = np.nonzero(ra >= 0)[0]
        assert sorted(s.row_index.tolist()) == active.tolist()           # a permutation of active rows
        assert s.seg_start[0] == 0 and s.seg_start[-1] == len(active)
        assert np.all(np.diff(s.seg_start) > 0)
        assert np.all(np.diff(s.seg_adapter) > 0)
        assert set(s.seg_adapter.tolist()) == set(ra[active].tolist())
        for g in range(s.n_seg):
            rows = s.row_index[s.seg_start[g]:s.seg_start[g + 1]]
            assert np.all(ra[rows] == s.seg_adapter[g])
            assert np.all(np.diff(rows) > 0)                                # stable within a segment
            assert s.seg_rank[g] == ranks[s.seg_adapter[g]]


def test_dense_offsets_golden():
    with open(os.path.join(GOLD, "delta_worked.json")) as f:
        g = json.load(f)["dense_offsets"]
    off = dense_offsets_ref(g["adapter_rank"], g["max_rank"], g["row_len"], g["chunk_len"])
    assert off.tolist() == g["expected"]


# ----------------------------------------------------------------------------- delta
def _tiny_problem(x, A_list, B_list, row_adapter, y0, layout="dense", page=64):
    n_ad = len(A_list)
    ranks = np.array([a.shape[0] for a in A_list], np.int32)
    mr = int(ranks.max())
    pool, d = _pool_from({"A": [_bits(a) for a in A_list], "B": [_bits(b) for b in B_list]},
                         n_ad, mr, layout, page)
    return dict(row_adapter=np.asarray(row_adapter, np.int32), adapter_rank=ranks,
                x_bits=_bits(x), y0=np.asarray(y0, np.float32), pool=pool, A=d["A"], B=d["B"])


def test_delta_golden_worked_example():
    with open(os.path.join(GOLD, "delta_worked.json")) as f:
        g = json.load(f)["delta"]
    p = _tiny_problem(np.array(g["x"]), [np.array(g["A"])], [np.array(g["B"])],
                      g["row_adapter"], np.array(g["y0"]))
    y, v = apply_ref(scale=g["scale"], **p)
    assert v[0].tolist() == g["v_expected"][0]
    assert y[0].tolist() == g["y_expected"][0]
    assert y[1].tolist() == g["y_expected"][1]
    assert 1 not in v


def test_delta_rank1_closed_form_bit_exact():
    x = np.arange(-3, 5, dtype=np.float64)[None, :]           # [-3..4]
    a = np.zeros((1, 8)); a[0, 2] = 1.0                         # e_2
    b = np.array([[1.0, 0.5, -2.0, 4.0]])
    p = _tiny_problem(x, [a], [b], [0], np.zeros((1, 4)))
    y, _ = apply_ref(scale=2.0, **p)
    assert y[0].tolist() == [-2.0, -1.0, 4.0, -8.0]


def test_delta_one_adapter_equals_dense_gemm():
    rng = np.random.default_rng(3)
    n, d_in, d_out, r = 24, 64, 96, 8
    X = rng.standard_normal((n, d_in))
    A = rng.standard_normal((r, d_in)) / 8
    B = rng.standard_normal((r, d_out)) / 3
    y0 = rng.standard_normal((n, d_out)).astype(np.float32)
    p = _tiny_problem(X, [A, A * 0.5], [B, B], np.zeros(n), y0)
    y, _ = apply_ref(scale=2.0, **p)
    Xe, Ae, Be = (bf16_to_f64(_bits(m)) for m in (X, A, B))
    want = y0.astype(np.float64) + 2.0 * (Xe @ Ae.T) @ Be       # textbook GEMM chain
    got = np.stack([y[i] for i in range(n)])
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_delta_scale_zero_and_released_rows_keep_y0():
    W = workloads.gen_custom(5, [0, -1, 1, 1, -1, 0], [4, 2], 64, 64)
    pr = W.projections[0]
    for scale in (0.0, 2.0):
        y, v = apply_ref(W.row_adapter, W.adapter_rank, pr.x, pr.y0, W.pool, pr.A, pr.B, scale)
        for i in range(W.n_rows):
            if scale == 0.0 or W.row_adapter[i] < 0:
                assert np.array_equal(y[i], pr.y0[i].astype(np.float64))
        assert set(v) == {0, 2, 3, 5}


def test_delta_permutation_invariance():
    W = workloads.gen_custom(6, [0, 1, 2, 0, 2, 2, 1, 0], [3, 5, 8], 64, 128)
    pr = W.projections[0]
    perm = np.random.default_rng(1).permutation(W.n_rows)
    y, _ = apply_ref(W.row_adapter, W.adapter_rank, pr.x, pr.y0, W.pool, pr.A, pr.B, 2.0)
    yp, _ = apply_ref(W.row_adapter[perm], W.adapter_rank, pr.x[perm], pr.y0[perm],
                      W.pool, pr.A, pr.B, 2.0)
    for k, i in enumerate(perm):
        assert np.array_equal(yp[k], y[i])


def test_gather_dense_vs_paged_same_values():
    ra = [0, 1, 2, 1, 0]
    Wd = workloads.gen_custom(9, ra, [3, 8, 5], 128, 192, layout="dense")
    Wp = workloads.gen_custom(9, ra, [3, 8, 5], 128, 192, layout="paged", page_elems=64)
    pd, pp = Wd.projections[0], Wp.projections[0]
    assert pp.B.chunks == 3 and pp.A.chunks == 2
    for a, r in enumerate([3, 8, 5]):
        for kind in ("A", "B"):
            dd, dp = getattr(pd, kind), getattr(pp, kind)
            gd = gather_rows_ref(Wd.pool, dd.row_off, dd.max_rank, dd.row_len, dd.chunk_len, a, r)
            gp = gather_rows_ref(Wp.pool, dp.row_off, dp.max_rank, dp.row_len, dp.chunk_len, a, r)
            assert np.array_equal(gd, gp) and np.all(np.isfinite(gd))
    yd, _ = apply_ref(Wd.row_adapter, Wd.adapter_rank, pd.x, pd.y0, Wd.pool, pd.A, pd.B, 2.0)
    yp, _ = apply_ref(Wp.row_adapter, Wp.adapter_rank, pp.x, pp.y0, Wp.pool, pp.A, pp.B, 2.0)
    for i in yd:
        assert np.array_equal(yd[i], yp[i])


def test_gather_reads_the_right_page():
    # a wrong page index would land on a NaN hole of the paged pool
    Wp = workloads.gen_custom(2, [0, 1], [2, 4], 64, 256, layout="paged", page_elems=64)
    pr = Wp.projections[0]
    assert np.isnan(bf16_to_f64(Wp.pool)).mean() > 0.4        # holes are NaN
    y, _ = apply_ref(Wp.row_adapter, Wp.adapter_rank, pr.x, pr.y0, Wp.pool, pr.A, pr.B, 2.0)
    assert all(np.all(np.isfinite(y[i])) for i in y)


# ----------------------------------------------------------------------------- merge
def test_merge_golden_worked_example():
    with open(os.path.join(GOLD, "delta_worked.json")) as f:
        g = json.load(f)
    m = g["merge"]
    out = merge_dense_ref(_bits(m["W"]), np.array(m["A"], float), np.array(m["B"], float), m["scale"])
    assert bf16_to_f64(out).tolist() == m["W_expected"]
    for c in g["merge_rounding"]:
        out = merge_dense_ref(_bits(c["W"]), np.array(c["A"], float), np.array(c["B"], float), c["scale"])
        assert [hex(int(b)) for b in out.reshape(-1)] == c["W_bits"], c["_work"]


def test_merge_rank1_exact_outer_product():
    a = np.array([[1.0, -0.5, 0.25, 2.0]])                       # [1, d_in=4]
    b = np.array([[4.0, -1.0, 0.125]])                           # [1, d_out=3]
    W0 = np.zeros((3, 4))
    out = bf16_to_f64(merge_dense_ref(_bits(W0), a, b, 2.0))
    assert np.array_equal(out, 2.0 * np.outer(b[0], a[0]))       # W'[n][k] = s b[n] a[k]


def _merge_problem(seed, d_out, d_in, r):
    rng = np.random.default_rng(seed)
    W = _bits(rng.standard_normal((d_out, d_in)) / math.sqrt(d_in))
    A = _bits(rng.standard_normal((r, d_in)) / math.sqrt(d_in))
    B = _bits(rng.standard_normal((r, d_out)) / math.sqrt(r))
    return W, A, B


@pytest.mark.parametrize("d_out,d_in,r", [(64, 192, 8), (512, 512, 8), (256, 128, 64)])
def test_merged_equals_unmerged_inference(d_out, d_in, r):
    W, A, B = _merge_problem(d_out + r, d_out, d_in, r)
    Wp = merge_dense_ref(W, bf16_to_f64(A), bf16_to_f64(B), 2.0)
    rng = np.random.default_rng(4)
    x = bf16_to_f64(_bits(rng.standard_normal((16, d_in))))
    merged = x @ bf16_to_f64(Wp).T                                 # formula 1
    unmerged = x @ bf16_to_f64(W).T + 2.0 * (x @ bf16_to_f64(A).T) @ bf16_to_f64(B)  # formula 2
    relF = np.linalg.norm(merged - unmerged) / np.linalg.norm(unmerged)
    assert relF < 4e-3
    # a transposed Delta W or a dropped scale would be far outside that bound
    wrong = x @ bf16_to_f64(W).T + (x @ bf16_to_f64(A).T) @ bf16_to_f64(B)
    assert np.linalg.norm(merged - wrong) / np.linalg.norm(unmerged) > 1e-1


@pytest.mark.parametrize("d_out,d_in,r", [(512, 512, 8), (256, 384, 64)])
def test_merge_unmerge_restores_w(d_out, d_in, r):
    W, A, B = _merge_problem(r, d_out, d_in, r)
    pool, d = _pool_from({"A": [A], "B": [B]}, 1, r)
    Wm = merge_ref(W, pool, d["A"], d["B"], 0, r, 2.0)
    Wr = unmerge_ref(Wm, pool, d["A"], d["B"], 0, r, 2.0)
    w0, w2 = bf16_to_f64(W), bf16_to_f64(Wr)
    relF = np.linalg.norm(w2 - w0) / np.linalg.norm(w0)
    assert relF <= 4e-3 and np.max(np.abs(w2 - w0)) <= 2e-2
    assert not np.array_equal(Wm, W)


def test_workload_shapes_and_determinism():
    a = workloads.gen_config(0)
    b = workloads.gen_config(0)
    assert np.array_equal(a.pool, b.pool) and np.array_equal(a.row_adapter, b.row_adapter)
    assert a.n_rows == 64 and a.projections[0].x.shape == (64, 512)
    assert len(np.unique(np.diff(np.nonzero(np.diff(np.r_[-2, a.row_adapter]))[0]))) >= 1
    s = build_segments_ref(a.row_adapter, a.adapter_rank)
    assert s.n_active == 64 and 1 <= s.n_seg <= 4


# ----------------------------------------------------------------------------- deLoRA mixture
def test_mixture_rank1_closed_form_bit_exact():
    """Adapter 0 (rank 1) merged; a row on adapter 1 gets s*(v_1 B_1 - v_0 B_0):
    x = [3, 0, 5, 0, ...], A_0 = e_0, A_1 = e_2 -> v_0 = 3, v_1 = 5."""
    x = np.zeros((3, 8)); x[:, 0] = 3.0; x[:, 2] = 5.0
    a0 = np.zeros((1, 8)); a0[0, 0] = 1.0
    a1 = np.zeros((1, 8)); a1[0, 2] = 1.0
    b0 = np.array([[1.0, 1.0, 1.0, 1.0]])
    b1 = np.array([[1.0, 0.5, -2.0, 4.0]])
    p = _tiny_problem(x, [a0, a1], [b0, b1], [1, 0, -1], np.zeros((3, 4)))
    y = oracle.mixture_ref(p["row_adapter"], p["adapter_rank"], 0, p["x_bits"], p["y0"], p["pool"],
                           p["A"], p["B"], 2.0)
    assert y[0].tolist() == [4.0, -1.0, -26.0, 34.0]     # 2*(5*b1 - 3*b0)
    assert y[1].tolist() == [0.0] * 4                     # on the merged adapter: W_merge serves it
    assert y[2].tolist() == [-6.0] * 4                    # released: backbone, -2*3*b0
    y = oracle.mixture_ref(p["row_adapter"], p["adapter_rank"], 0, p["x_bits"], p["y0"], p["pool"],
                           p["A"], p["B"], 2.0, base_rows=False)
    assert y[2].tolist() == [0.0] * 4                     # released, output not wanted: untouched


@pytest.mark.parametrize("layout", ["dense", "paged"])
def test_mixture_equals_unmerged_inference(layout):
    """VaLoRA's identity: x (W_merge - dW_m + dW_x)^T with W_merge = W + dW_m equals the
    unmerged output x W^T + s x A_x^T B_x, for rows on any adapter; rows on m get
    x W_merge^T; released rows get the backbone output x W^T (the identity with
    dW_x = 0), or keep y0 with base_rows=False.  Exact real arithmetic, so fp64
    agrees to rounding."""
    rng = np.random.default_rng(11)
    d_in, d_out, s, m = 96, 64, 2.0, 1
    ranks = [4, 8, 3]
    A = [rng.standard_normal((r, d_in)) / 8 for r in ranks]
    B = [rng.standard_normal((r, d_out)) / 3 for r in ranks]
    ra = np.array([0, 1, 2, -1, 2, 1, 0, 0], np.int32)
    x = rng.standard_normal((len(ra), d_in))
    p = _tiny_problem(x, A, B, ra, np.zeros((len(ra), d_out)), layout=layout)
    Ae, Be, xe = [bf16_to_f64(_bits(a)) for a in A], [bf16_to_f64(_bits(b)) for b in B], bf16_to_f64(p["x_bits"])
    Wb = rng.standard_normal((d_out, d_in)) / 10
    Wm = Wb + s * Be[m].T @ Ae[m]                          # merged weights (unrounded)
    y0 = xe @ Wm.T                                         # shared merged GEMM
    y = oracle.mixture_ref(ra, p["adapter_rank"], m, p["x_bits"], y0, p["pool"], p["A"], p["B"], s)
    y_pad = oracle.mixture_ref(ra, p["adapter_rank"], m, p["x_bits"], y0, p["pool"], p["A"], p["B"], s,
                               base_rows=False)
    for i, a in enumerate(ra):
        if a < 0:
            want = xe[i] @ Wb.T                                  # backbone alone
            np.testing.assert_array_equal(y_pad[i], y0[i])
        elif a == m:
            want = xe[i] @ Wm.T
        else:
            want = xe[i] @ Wb.T + s * (xe[i] @ Ae[a].T) @ Be[a]    # unmerged, adapter a
        np.testing.assert_allclose(y[i], want, rtol=1e-11, atol=1e-11)
    # adding the merged adapter instead of subtracting it would be far off
    bad = xe[0] @ Wm.T + s * (xe[0] @ Ae[0].T) @ Be[0]
    assert np.max(np.abs(bad - (xe[0] @ Wb.T + s * (xe[0] @ Ae[0].T) @ Be[0]))) > 1e-2


def test_shared_x_workload_recipe():
    """Projections that share x take one array (the group's first projection's
    draw); everything else is the same instance as without sharing."""
    W = workloads.gen_config(2, shared_qkv=True)
    W0 = workloads.gen_config(2)
    assert W.projections[0].x is W.projections[1].x is W.projections[2].x
    assert W.projections[3].x is not W.projections[0].x
    assert np.array_equal(W.projections[0].x, W0.projections[0].x)
    assert np.array_equal(W.projections[3].x, W0.projections[3].x)
    assert np.array_equal(W.row_adapter, W0.row_adapter) and np.array_equal(W.pool, W0.pool)
