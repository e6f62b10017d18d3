"""CPU tests of the C-ABI library: exports, host-side entry points, error paths.

No kernel is launched here.  The library's host functions (segment builder,
planner, dense offsets) are compared bit-exactly with the oracle's definitions;
shrink/expand/merge are called only with arguments that fail validation, which
returns before any HIP call.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import heterogeneous_adapter_batching_amd as hl
import oracle
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(lora_\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert len(names) >= 9, names
    lib = ctypes.CDLL(hl.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert hl.lora_abi_version() == hl.LORA_ABI_VERSION
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert hl.lora_status_string(code) != "unknown status"


# ---------------------------------------------------------------- segments
def _same(a, b):
    for k in ("row_index", "seg_start", "seg_adapter", "seg_rank"):
        assert np.array_equal(getattr(a, k), getattr(b, k)), k


@pytest.mark.parametrize("k", [0, 1, 2, 3, 4])
def test_build_segments_matches_oracle_on_workloads(k):
    # structure only: the big workloads' tensors are not drawn
    S = workloads.structure(k)
    for ra in S.batches.values():
        _same(hl.lora_build_segments(ra, S.adapter_rank), oracle.build_segments_ref(ra, S.adapter_rank))


def test_build_segments_matches_oracle_random():
    rng = np.random.default_rng(5)
    for t in range(1000):
        n = int(rng.integers(0, 50))
        n_ad = int(rng.integers(1, 12))
        ranks = rng.integers(1, 129, size=n_ad)
        mode = t % 4
        if mode == 0:
            ra = rng.integers(-1, n_ad, size=n)
        elif mode == 1:        # all released
            ra = np.full(n, -1)
        elif mode == 2:        # one adapter, non-adjacent repeats
            ra = np.where(rng.random(n) < 0.5, -1, int(rng.integers(0, n_ad)))
        else:                  # runs of repeated adapters
            ra = np.repeat(rng.integers(-1, n_ad, size=max(1, n // 5)), 5)[:n]
        _same(hl.lora_build_segments(ra, ranks), oracle.build_segments_ref(ra, ranks))


def test_build_segments_error_codes_and_no_writes():
    lib = hl._lib
    sentinel = -12345

    def call(ra, rk, cap):
        ra = np.asarray(ra, np.int32); rk = np.asarray(rk, np.int32)
        outs = [np.full(max(1, len(ra)), sentinel, np.int32), np.full(cap + 1, sentinel, np.int32),
                np.full(max(1, cap), sentinel, np.int32), np.full(max(1, cap), sentinel, np.int32)]
        ns, na = ctypes.c_int32(sentinel), ctypes.c_int32(sentinel)
        st = lib.lora_build_segments(len(ra), ra.ctypes.data if len(ra) else None, len(rk),
                                     rk.ctypes.data if len(rk) else None, cap,
                                     *[o.ctypes.data for o in outs], ctypes.byref(ns), ctypes.byref(na))
        return st, outs, ns.value, na.value

    st, outs, ns, na = call([0, 2], [4, 4], 2)
    assert st == hl.LORA_EADAPTER and all(np.all(o == sentinel) for o in outs) and ns == sentinel
    st, outs, *_ = call([0, -2], [4], 1)
    assert st == hl.LORA_EADAPTER
    st, outs, *_ = call([0], [0], 1)
    assert st == hl.LORA_ERANK and all(np.all(o == sentinel) for o in outs)
    st, outs, *_ = call([0], [129], 1)
    assert st == hl.LORA_ERANK
    st, outs, ns, na = call([0, 1, 2, 1], [4, 4, 4], 2)           # needs 3 segments
    assert st == hl.LORA_ECAPACITY and ns == 3 and na == 4
    assert all(np.all(o == sentinel) for o in outs)
    st, outs, ns, na = call([], [4], 0)                             # empty batch
    assert st == hl.LORA_OK and ns == 0 and na == 0 and outs[1][0] == 0
    st, outs, ns, na = call([-1, -1], [4], 0)                       # all released
    assert st == hl.LORA_OK and ns == 0 and na == 0
    assert lib.lora_build_segments(-1, None, 1, None, 0, None, None, None, None, None, None) == hl.LORA_EINVAL


# ---------------------------------------------------------------- plan
def test_plan_coverage_invariants():
    rng = np.random.default_rng(8)
    cases = [np.repeat(rng.integers(-1, 20, size=40), rng.integers(1, 400, size=40)) for _ in range(30)]
    cases += [np.arange(64), np.zeros(64, int), np.full(3000, 2), np.array([5])]
    for ra in cases:
        ranks = rng.integers(1, 129, size=int(ra.max()) + 1 if ra.max() >= 0 else 1)
        segs = hl.lora_build_segments(ra, ranks)
        for d_in, d_out in ((512, 512), (4096, 4096), (8192, 28672), (64, 192)):
            slices = []
            for op in (hl.LORA_OP_SHRINK, hl.LORA_OP_EXPAND):
                work, info = hl.lora_plan(op, segs, d_in, d_out)
                assert info.n_active == segs.n_active and info.n_work == work.shape[0]
                slices.append(oracle.check_plan_coverage(segs, work, info.range_list(),
                                                         op == hl.LORA_OP_SHRINK, info.v_slices))
                if segs.n_seg:
                    assert info.max_rank == segs.seg_rank.max()
                    assert info.max_adapter == segs.seg_adapter.max()
                assert work.shape[0] <= hl.LORA_MAX_SLICES * segs.n_active
                assert all(ns <= d_in // 64 for ns in slices[-1].values())
            assert slices[0] == slices[1], "shrink and expand agree on K slices"


def test_table_plans_follow_the_given_table():
    """lora_plan_table (the tile search's planner): with the compiled-in table
    it plans exactly as lora_plan for every op; with a table that holds one
    choice everywhere every segment gets that shape and K-slice count (capped
    at d_in/64), its plans pass the oracle's coverage checker, and its items
    stay within the shape's rows; tables with entries out of range, null
    tables and widths it cannot plan are refused."""
    from heterogeneous_adapter_batching_amd.tile_search import read_table
    st0, ex0 = read_table()
    rng = np.random.default_rng(21)
    ra = np.repeat(rng.permutation(6), [1, 2, 3, 17, 300, 70])
    ranks = np.array([8, 16, 64, 128, 32, 1], np.int32)
    segs = hl.lora_build_segments(ra, ranks)
    for op in (hl.LORA_OP_SHRINK, hl.LORA_OP_EXPAND, hl.LORA_OP_APPLY):
        for d_in, d_out in ((1024, 2048), (4096, 4096), (8192, 28672)):
            w0, i0 = hl.lora_plan(op, segs, d_in, d_out)
            w1, i1 = hl.lora_plan_table(op, segs, d_in, d_out, st0, ex0)
            assert np.array_equal(w0, w1) and i0.range_list() == i1.range_list() and i0.v_slices == i1.v_slices
    rows = {hl.LORA_OP_SHRINK: {0: 16, 1: 64, 2: 128}, hl.LORA_OP_EXPAND: {0: 16, 1: 64, 2: 128, 3: 32, 4: 2}}
    for op, shapes in rows.items():
        for shape, mt in shapes.items():
            for sl in (1, 2, 4, 8, 16):
                for d_in in (256, 4096):
                    st, ex = st0.copy(), ex0.copy()
                    st[...] = (shape if op == hl.LORA_OP_SHRINK else 0, sl)
                    ex[...] = shape if op == hl.LORA_OP_EXPAND else 0
                    if shape == 4:   # the VALU expand takes segments of at most 2 rows
                        segs2 = hl.lora_build_segments([0, 1, 1, 2], [8, 16, 64])
                    else:
                        segs2 = segs
                    work, info = hl.lora_plan_table(op, segs2, d_in, 2048, st, ex)
                    ns = oracle.check_plan_coverage(segs2, work, info.range_list(), op == hl.LORA_OP_SHRINK,
                                                    info.v_slices)
                    want = min(sl, d_in // 64)
                    assert set(ns.values()) == {want} and info.v_slices == want
                    assert all(1 <= w[1] <= mt for w in work)
                    assert all(v // 4 == shape for v, *_ in info.range_list())
    bad = []
    for i, v in ((0, -1), (0, 3), (1, 0), (1, 17)):
        st = st0.copy()
        st[7, 2, 1, i] = v
        bad.append((st, ex0))
    for v in (-1, 5):
        ex = ex0.copy()
        ex[0, 0, 0] = v
        bad.append((st0, ex))
    for st, ex in bad:
        status, _, _ = hl.lora_plan_table(hl.LORA_OP_SHRINK, segs, 1024, 2048, st, ex, raw=True)
        assert status == hl.LORA_EINVAL
    st_null = hl._lib.lora_plan_table(hl.LORA_OP_SHRINK, segs.n_seg, segs.seg_start.ctypes.data,
                                      segs.seg_adapter.ctypes.data, segs.seg_rank.ctypes.data, 1024, 2048, None,
                                      ex0.ctypes.data, 0, None, ctypes.byref(hl.lora_plan_info_t()))
    assert st_null == hl.LORA_EINVAL
    status, _, _ = hl.lora_plan_table(hl.LORA_OP_SHRINK, segs, 1000, 2048, st0, ex0, raw=True)
    assert status == hl.LORA_ESHAPE


def test_block_moves_group_the_segments_one_launch_runs():
    """The tile search's block moves treat the buckets of one op, d bucket,
    launch class and shape as one launch.  Against the planner: with one
    shape everywhere, segments whose ranks share a launch class get the same
    expand variant (a host plan runs one launch per expand range), and
    shrink variants of the same shape whose classes the launcher runs
    together (ranks up to 64) or apart (rank 128); different classes get
    different expand variants."""
    from heterogeneous_adapter_batching_amd.tile_search import RANK_REP, _launch_class, read_table
    st0, ex0 = read_table()
    for shape in (0, 1, 2):
        st, ex = st0.copy(), ex0.copy()
        st[...] = (shape, 1)
        ex[...] = shape
        ranks = np.array(RANK_REP, np.int32)            # one adapter per rank bucket
        ra = np.repeat(np.arange(4), [40, 40, 40, 40]).astype(np.int32)
        segs = hl.lora_build_segments(ra, ranks)
        for op in (hl.LORA_OP_SHRINK, hl.LORA_OP_EXPAND):
            work, info = hl.lora_plan_table(op, segs, 1024, 1024, st, ex)
            var_of_rank = {}
            for v, b, c, _ in info.range_list():
                for w in work[b:b + c]:
                    var_of_rank.setdefault(int(w[3]), set()).add(v)
            assert all(len(vs) == 1 for vs in var_of_rank.values())
            var = {r: next(iter(var_of_rank[RANK_REP[r]])) for r in range(4)}
            name = "shrink" if op == hl.LORA_OP_SHRINK else "expand"
            for r1 in range(4):
                for r2 in range(4):
                    same = _launch_class(name, r1) == _launch_class(name, r2)
                    v1, v2 = var[r1], var[r2]
                    assert v1 // 4 == v2 // 4 == shape
                    if op == hl.LORA_OP_EXPAND:
                        assert (v1 == v2) == same
                    else:   # the launcher runs shrink classes 0-2 of a shape together, class 3 alone
                        assert ((v1 % 4 < 3) == (v2 % 4 < 3)) == same


def test_tile_table_source_round_trips(tmp_path):
    """The tile search reads the compiled-in table's source and writes it back
    unchanged but for its note line."""
    from heterogeneous_adapter_batching_amd import tile_search
    st0, ex0 = tile_search.read_table()
    out = tmp_path / "t.inc"
    tile_search.write_table(st0, ex0, str(out), "note")
    st1, ex1 = tile_search.read_table(str(out))
    assert np.array_equal(st0, st1) and np.array_equal(ex0, ex1)
    keep = [ln for ln in open(tile_search.TABLE).read().splitlines() if not ln.startswith("// Written by")]
    assert [ln for ln in out.read_text().splitlines() if ln != "// note"] == keep


def test_plan_errors():
    segs = hl.lora_build_segments([0, 0, 1], [8, 16])
    with pytest.raises(hl.LoraError) as e:
        hl.lora_plan(hl.LORA_OP_SHRINK, segs, 100, 512)
    assert e.value.code == hl.LORA_ESHAPE
    with pytest.raises(hl.LoraError) as e:
        hl.lora_plan(7, segs, 512, 512)
    assert e.value.code == hl.LORA_EINVAL
    with pytest.raises(hl.LoraError) as e:
        hl.lora_plan(hl.LORA_OP_SHRINK, segs, 512, 512, work_capacity=1)
    assert e.value.code == hl.LORA_ECAPACITY
    empty = hl.lora_build_segments([-1, -1], [8])
    work, info = hl.lora_plan(hl.LORA_OP_EXPAND, empty, 512, 512)
    assert info.n_work == 0 and info.n_ranges == 0


# ---------------------------------------------------------------- dense offsets
def test_dense_offsets_match_oracle():
    import json
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "delta_worked.json")))["dense_offsets"]
    off, pe = hl.lora_rows_dense_offsets(g["adapter_rank"], g["max_rank"], g["row_len"], g["chunk_len"])
    assert off.tolist() == g["expected"] and pe == 6 * 104
    rng = np.random.default_rng(2)
    for _ in range(50):
        n_ad = int(rng.integers(1, 9)); mr = int(rng.integers(1, 129))
        rk = rng.integers(1, mr + 1, size=n_ad)
        rl = int(rng.integers(1, 5000)); cl = 64 * int(rng.integers(1, 40))
        off, _ = hl.lora_rows_dense_offsets(rk, mr, rl, cl)
        assert np.array_equal(off, oracle.dense_offsets_ref(rk, mr, rl, cl))
    with pytest.raises(hl.LoraError) as e:
        hl.lora_rows_dense_offsets([4], 4, 512, 100)
    assert e.value.code == hl.LORA_ESHAPE
    with pytest.raises(hl.LoraError) as e:
        hl.lora_rows_dense_offsets([5], 4, 512, 64)
    assert e.value.code == hl.LORA_ERANK


# ---------------------------------------------------------------- launch validation (no launch)
def _launch(op, n_work=1, max_rank=16, max_adapter=0):
    info = hl.lora_plan_info_t()
    info.op, info.n_work, info.n_active, info.max_rank, info.max_adapter = op, n_work, n_work, max_rank, max_adapter
    info.v_slices = 1
    info.d_in = info.d_out = 512
    info.n_ranges = 1
    info.ranges[0].variant, info.ranges[0].begin, info.ranges[0].count, info.ranges[0].rows_per_item = 0, 0, n_work, 16
    return hl.lora_launch_t(0x1000, 0x2000, info)


def _rows(row_len=512, chunk_len=512, max_rank=16, n_ad=4, pool=0x10000):
    return hl.lora_rows_t(pool, 0x20000, n_ad, max_rank, row_len, chunk_len)


def test_shrink_expand_merge_validation_errors():
    lib = hl._lib
    L = _launch(hl.LORA_OP_SHRINK)

    def shrink(**kw):
        p = dict(x=0x30000, ldx=512, d_in=512, A=_rows(), v=0x40000, ldv=16)
        p.update(kw)
        arr = (hl.lora_shrink_proj_t * 1)(hl.lora_shrink_proj_t(**p))
        return lib.lora_shrink(ctypes.byref(L), 1, arr, None)

    assert shrink(x=None) == hl.LORA_EINVAL
    assert shrink(x=0x30008) == hl.LORA_EINVAL                 # misaligned
    assert shrink(d_in=500, ldx=512, A=_rows(row_len=500)) == hl.LORA_ESHAPE
    assert shrink(ldx=256) == hl.LORA_EINVAL                   # ld < d
    assert shrink(ldv=8) == hl.LORA_EINVAL                     # ldv < max rank
    assert shrink(A=_rows(max_rank=8)) == hl.LORA_ERANK
    assert shrink(A=_rows(n_ad=0)) == hl.LORA_EADAPTER
    assert shrink(A=_rows(chunk_len=100)) == hl.LORA_ESHAPE
    assert shrink(A=_rows(row_len=1024)) == hl.LORA_ESHAPE
    Lbad = _launch(hl.LORA_OP_EXPAND)
    arr = (hl.lora_shrink_proj_t * 1)(hl.lora_shrink_proj_t(0x30000, 512, 512, _rows(), 0x40000, 16))
    assert lib.lora_shrink(ctypes.byref(Lbad), 1, arr, None) == hl.LORA_EINVAL   # wrong op
    assert lib.lora_shrink(ctypes.byref(L), 0, arr, None) == hl.LORA_EINVAL
    assert lib.lora_shrink(ctypes.byref(L), 9, arr, None) == hl.LORA_EINVAL

    LE = _launch(hl.LORA_OP_EXPAND)

    def expand(**kw):
        p = dict(v=0x40000, ldv=16, B=_rows(), d_out=512, y=0x50000, ldy=512, scale=2.0)
        p.update(kw)
        arr = (hl.lora_expand_proj_t * 1)(hl.lora_expand_proj_t(**p))
        return lib.lora_expand(ctypes.byref(LE), 1, arr, None)

    assert expand(y=None) == hl.LORA_EINVAL
    assert expand(y=0x50004) == hl.LORA_EINVAL
    assert expand(ldy=510) == hl.LORA_EINVAL
    assert expand(d_out=96, ldy=96, B=_rows(row_len=96)) == hl.LORA_ESHAPE
    assert expand(B=_rows(max_rank=4)) == hl.LORA_ERANK

    def merge(**kw):
        p = dict(W=0x60000, ldw=512, d_out=512, d_in=512, A=_rows(), B=_rows(), adapter=0, rank=16, scale=2.0)
        p.update(kw)
        arr = (hl.lora_merge_mat_t * 1)(hl.lora_merge_mat_t(**p))
        return lib.lora_merge(1, arr, None), lib.lora_unmerge(1, arr, None)

    assert merge(W=None) == (hl.LORA_EINVAL,) * 2
    assert merge(rank=0) == (hl.LORA_ERANK,) * 2
    assert merge(rank=32) == (hl.LORA_ERANK,) * 2              # beyond the tables' max_rank
    assert merge(adapter=4) == (hl.LORA_EADAPTER,) * 2
    assert merge(adapter=-1) == (hl.LORA_EADAPTER,) * 2
    assert merge(d_in=100) == (hl.LORA_ESHAPE,) * 2
    assert merge(ldw=256) == (hl.LORA_EINVAL,) * 2
    assert lib.lora_merge(0, None, None) == hl.LORA_EINVAL
    assert lib.lora_merge(9, None, None) == hl.LORA_EINVAL


def test_launch_rejects_variants_no_kernel_runs():
    """Expand variants of rank class 3 exist only for the VALU decode shape's
    numbering; no MFMA expand kernel runs them (its rank classes stop at 128
    ranks in class 2), and the decode shape has class 0 only.  A hand-made
    launch that names one is refused before anything is launched, for the
    expand and for the expand part of an apply plan."""
    lib = hl._lib
    n_rc = 4
    e_shapes, bgmv = 5, 4
    expand0, fused = 3 * n_rc, 3 * n_rc + 5 * n_rc
    earr = (hl.lora_expand_proj_t * 1)(hl.lora_expand_proj_t(0x40000, 16, _rows(), 512, 0x50000, 512, 2.0))
    aarr = (hl.lora_apply_proj_t * 1)(hl.lora_apply_proj_t(0x30000, 512, 512, _rows(), 0x40000, 16, _rows(),
                                                           512, 0x50000, 512, 2.0))
    bad = [s * n_rc + 3 for s in range(e_shapes)] + [bgmv * n_rc + c for c in (1, 2)] + [-1, e_shapes * n_rc]
    for ev in bad:
        LE = _launch(hl.LORA_OP_EXPAND)
        LE.info.ranges[0].variant = ev
        assert lib.lora_expand(ctypes.byref(LE), 1, earr, None) == hl.LORA_EINVAL, ev
        LA = _launch(hl.LORA_OP_APPLY)
        LA.info.ranges[0].variant = expand0 + ev
        if expand0 + ev not in (fused,) and not 0 <= expand0 + ev < expand0:
            assert lib.lora_apply(ctypes.byref(LA), 1, aarr, None) == hl.LORA_EINVAL, ev
    LA = _launch(hl.LORA_OP_APPLY)
    LA.info.ranges[0].variant = fused + 1
    assert lib.lora_apply(ctypes.byref(LA), 1, aarr, None) == hl.LORA_EINVAL
    LS = _launch(hl.LORA_OP_SHRINK)
    LS.info.ranges[0].variant = 3 * n_rc
    sarr = (hl.lora_shrink_proj_t * 1)(hl.lora_shrink_proj_t(0x30000, 512, 512, _rows(), 0x40000, 16))
    assert lib.lora_shrink(ctypes.byref(LS), 1, sarr, None) == hl.LORA_EINVAL


def test_launch_rejects_projections_wider_than_the_plan():
    """A plan is cut for the d_in / d_out it was made with (its K slices, and
    whether a segment is fused): a wider projection is refused, as is a
    fused range at a width the fused kernel does not cover, and a plan
    summary with no widths."""
    lib = hl._lib
    LS = _launch(hl.LORA_OP_SHRINK)
    arr = (hl.lora_shrink_proj_t * 1)(hl.lora_shrink_proj_t(0x30000, 1024, 1024, _rows(1024, 1024), 0x40000, 16))
    assert lib.lora_shrink(ctypes.byref(LS), 1, arr, None) == hl.LORA_ESHAPE
    LE = _launch(hl.LORA_OP_EXPAND)
    arr = (hl.lora_expand_proj_t * 1)(hl.lora_expand_proj_t(0x40000, 16, _rows(1024, 1024), 1024, 0x50000, 1024, 2.0))
    assert lib.lora_expand(ctypes.byref(LE), 1, arr, None) == hl.LORA_ESHAPE
    LE.info.d_out = 0
    assert lib.lora_expand(ctypes.byref(LE), 1, arr, None) == hl.LORA_ESHAPE
    fused = 3 * 4 + 5 * 4
    for d_in, d_out in ((8192, 4096), (4096, 28672)):
        LA = _launch(hl.LORA_OP_APPLY)
        LA.info.ranges[0].variant = fused
        LA.info.d_in, LA.info.d_out = d_in, d_out
        arr = (hl.lora_apply_proj_t * 1)(hl.lora_apply_proj_t(0x30000, d_in, d_in, _rows(d_in, d_in), 0x40000, 16,
                                                             _rows(d_out, d_out), d_out, 0x50000, d_out, 2.0))
        assert lib.lora_apply(ctypes.byref(LA), 1, arr, None) == hl.LORA_ESHAPE, (d_in, d_out)


def test_plan_records_its_widths():
    segs = hl.lora_build_segments([0, 0, 1], [8, 16])
    for op in (hl.LORA_OP_SHRINK, hl.LORA_OP_EXPAND, hl.LORA_OP_APPLY):
        _, info = hl.lora_plan(op, segs, 1024, 28672)
        assert (info.d_in, info.d_out) == (1024, 28672)
    _, dp = hl.lora_device_plan(64, 8, 16, 2048, 512)
    assert (dp.info.d_in, dp.info.d_out) == (2048, 512)


def test_pool_rejects_pages_past_the_scatter_piece():
    with pytest.raises(hl.LoraError) as e:
        hl.LoraPool(4, 65536 + 64, 2, 16, [512])
    assert e.value.code == hl.LORA_ESHAPE
    hl.LoraPool(4, 65536, 2, 16, [512])


def test_static_apply_refuses_plans_past_its_array():
    """lora_apply_static checks that every projection's v region fits the
    library's array before it touches the device (so this runs without a
    GPU): 8 projections x 16 slices x 65,536 rows x 128 ranks do not fit."""
    lib = hl._lib
    L = _launch(hl.LORA_OP_APPLY)
    L.info.n_active, L.info.v_slices, L.info.max_rank = 65536, 16, 128
    arr = (hl.lora_apply_proj_t * 8)(*[hl.lora_apply_proj_t(0x30000, 512, 512, _rows(), None, 0, _rows(), 512,
                                                            0x50000, 512, 2.0) for _ in range(8)])
    assert lib.lora_apply_static(ctypes.byref(L), 8, arr, None) == hl.LORA_ECAPACITY
    # one projection of 16 x 8192 x 128 floats (64 MiB) still fits; two do not
    L.info.n_active, L.info.v_slices, L.info.max_rank = 8192, 16, 128
    assert lib.lora_apply_static(ctypes.byref(L), 2, arr, None) == hl.LORA_ECAPACITY
    assert lib.lora_apply_static(None, 1, arr, None) == hl.LORA_EINVAL
    assert lib.lora_apply_static(ctypes.byref(L), 0, arr, None) == hl.LORA_EINVAL


def test_empty_batch_launches_nothing():
    # n_work == 0 returns OK before any HIP call (works without a GPU)
    lib = hl._lib
    L = _launch(hl.LORA_OP_SHRINK, n_work=0)
    L.info.n_ranges = 0
    arr = (hl.lora_shrink_proj_t * 1)(hl.lora_shrink_proj_t(0x30000, 512, 512, _rows(), 0x40000, 16))
    assert lib.lora_shrink(ctypes.byref(L), 1, arr, None) == hl.LORA_OK


def test_batch_prepare_errors_and_size():
    """lora_batch_prepare validates before it copies, and on a staging buffer
    that is too small reports the exact size: row_index plus every requested
    plan (no copy is enqueued on these paths, so no GPU is needed)."""
    ra = np.repeat([0, 1, 2, -1], [5, 70, 300, 3])
    rank = [8, 16, 64]
    segs = hl.lora_build_segments(ra, rank)
    n_work = {op: hl.lora_plan(op, segs, 4096, 4096)[0].shape[0]
              for op in (hl.LORA_OP_SHRINK, hl.LORA_OP_EXPAND, hl.LORA_OP_APPLY)}
    fake_dev = 0x10000  # never dereferenced: every call below returns before the copy
    for mask, ops in ((1, [0]), (2, [1]), (4, [2]), (7, [0, 1, 2]), (5, [0, 2])):
        need = segs.n_active + hl.WORK_INTS * sum(n_work[o] for o in ops)
        for cap in (0, segs.n_active, need - 1):
            st, out, _ = hl.lora_batch_prepare(ra, rank, 4096, 4096, mask, np.zeros(cap, np.int32), fake_dev,
                                               raw=True)
            assert st == hl.LORA_ECAPACITY
            assert out.n_staged == (ra.shape[0] if cap < ra.shape[0] else need)
    big = np.zeros(100000, np.int32)
    st, out, _ = hl.lora_batch_prepare(ra, rank, 4096, 4096, 7, big, fake_dev, seg_capacity=2, raw=True)
    assert st == hl.LORA_ECAPACITY and out.n_seg == 3 and out.n_staged == 0
    for mask in (0, 8, 15):
        assert hl.lora_batch_prepare(ra, rank, 4096, 4096, mask, big, fake_dev, raw=True)[0] == hl.LORA_EINVAL
    assert hl.lora_batch_prepare(ra, rank, 4096, 4096, 7, big, None, raw=True)[0] == hl.LORA_EINVAL
    assert hl.lora_batch_prepare(ra, rank, 4096, 4000, 7, big, fake_dev, raw=True)[0] == hl.LORA_ESHAPE
    assert hl.lora_batch_prepare([0, 5], rank, 4096, 4096, 7, big, fake_dev, raw=True)[0] == hl.LORA_EADAPTER


def test_apply_plan_partitions_segments():
    """An apply plan fuses exactly the segments of one row, or of len * rank
    <= 1024, with d_in, d_out <= 4096 (one item per row); every other segment
    is covered by its shrink items (each row x K slice once) and its expand
    items (each row once); fused items cover one row."""
    N_SHRINK = 3 * 4            # shrink variants
    FUSED = N_SHRINK + 5 * 4    # the fused variant follows the expand variants
    rng = np.random.default_rng(12)
    cases = [np.arange(64), np.zeros(64, int), np.repeat(rng.integers(-1, 30, size=40), rng.integers(1, 5, size=40)),
             np.repeat(rng.integers(0, 8, size=20), rng.integers(1, 300, size=20)), np.array([3])]
    for ra in cases:
        ranks = rng.integers(1, 129, size=int(ra.max()) + 1)
        segs = hl.lora_build_segments(ra, ranks)
        for d_in, d_out in ((512, 512), (4096, 4096), (4096, 8192), (8192, 4096), (64, 4096)):
            work, info = hl.lora_plan(hl.LORA_OP_APPLY, segs, d_in, d_out)
            _, info_s = hl.lora_plan(hl.LORA_OP_SHRINK, segs, d_in, d_out)
            assert info.op == hl.LORA_OP_APPLY and info.n_work == work.shape[0]
            assert work.shape[0] <= (hl.LORA_MAX_SLICES + 1) * segs.n_active
            cov_s = np.zeros((segs.n_active, hl.LORA_MAX_SLICES), int)
            cov_e = np.zeros(segs.n_active, int)
            fused_rows = set()
            prev_v = -1
            for v, begin, count, mt in info.range_list():
                assert v > prev_v
                prev_v = v
                for w in work[begin:begin + count]:
                    row0, nrows, ad, rk, ks, ns = (int(t) for t in w[:6])
                    assert 1 <= nrows <= mt
                    if v < N_SHRINK:
                        cov_s[row0:row0 + nrows, ks] += 1
                    else:
                        cov_e[row0:row0 + nrows] += 1
                        if v == FUSED:
                            assert nrows == 1 and ns == 1
                            fused_rows.add(row0)
            assert np.all(cov_e == 1)
            assert info.v_slices <= max(1, info_s.v_slices)
            for s in range(segs.n_seg):
                lo, hi = int(segs.seg_start[s]), int(segs.seg_start[s + 1])
                rk = int(segs.seg_rank[s])
                fused = (hi - lo == 1 or (hi - lo) * rk <= 1024) and d_in <= 4096 and d_out <= 4096
                assert all((q in fused_rows) == fused for q in range(lo, hi))
                if fused:
                    assert np.all(cov_s[lo:hi] == 0)
                else:
                    ns = int(work[[i for i in range(work.shape[0]) if work[i, 0] == lo][0], 5])
                    assert np.all(cov_s[lo:hi, :ns] == 1) and np.all(cov_s[lo:hi, ns:] == 0)


def test_one_hip_runtime_in_process():
    """Importing the binding first must not bring a second HIP runtime into the
    process: torch ships its own libamdhip64 under the system one's soname, so
    the binding loads torch before the library (fresh interpreter, no GPU needed)."""
    import subprocess
    import sys
    code = ("import heterogeneous_adapter_batching_amd, torch\n"
            "paths = set()\n"
            "for line in open('/proc/self/maps'):\n"
            "    f = line.split()[-1]\n"
            "    if 'libamdhip64' in f: paths.add(__import__('os').path.realpath(f))\n"
            "print(len(paths), sorted(paths))\n")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300,
                         cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert out.returncode == 0, out.stderr
    n = int(out.stdout.split()[0])
    assert n == 1, out.stdout


def test_mixture_row_adapter():
    ra = np.array([0, 2, -1, 2, 1, 0, 2], np.int32)
    out = hl.lora_mixture_row_adapter(ra, 2)               # released row -> minus the merged adapter
    assert out.tolist() == [0, -1, 2, -1, 1, 0, -1]
    out = hl.lora_mixture_row_adapter(ra, 2, base_rows=False)   # released row stays untouched
    assert out.tolist() == [0, -1, -1, -1, 1, 0, -1]
    st, _ = hl.lora_mixture_row_adapter(ra, -1, raw=True)
    assert st == hl.LORA_EINVAL


@pytest.mark.parametrize("chunks", [1, 3])
def test_mixture_rows_composite_table(chunks):
    """Composite adapter a != m: rows j < r_a are a's, rows r_a + i are m's row i;
    m keeps its own rows, all negated; neg_from = r_a (m: 0)."""
    rng = np.random.default_rng(chunks)
    rank = np.array([3, 8, 5, 1], np.int32)
    max_rank, m, out_max = 8, 2, 16
    row_off = rng.integers(0, 1 << 40, size=len(rank) * max_rank * chunks).astype(np.int64) * 8
    off, crank, neg = hl.lora_mixture_rows(rank, m, chunks, row_off, max_rank, out_max)
    R = lambda t, a, j, c, mr: t[(a * mr + j) * chunks + c]
    for a in range(len(rank)):
        r = rank[m] if a == m else rank[a] + rank[m]
        assert crank[a] == r and neg[a] == (0 if a == m else rank[a])
        for j in range(out_max):
            for c in range(chunks):
                if j >= r:
                    want = 0
                elif a == m or j < rank[a]:
                    want = R(row_off, a, j, c, max_rank)
                else:
                    want = R(row_off, m, j - rank[a], c, max_rank)
                assert R(off, a, j, c, out_max) == want, (a, j, c)


def test_mixture_rows_errors():
    rank = np.array([64, 70, 8], np.int32)
    row_off = np.zeros(3 * 80, np.int64)
    st, *_ = hl.lora_mixture_rows(rank, 1, 1, row_off, 80, 128, raw=True)
    assert st == hl.LORA_ERANK                       # 64 + 70 > 128
    st, *_ = hl.lora_mixture_rows(rank, 3, 1, row_off, 80, 128, raw=True)
    assert st == hl.LORA_EINVAL                      # merged adapter out of range
    st, *_ = hl.lora_mixture_rows(rank, 2, 1, row_off, 80, 64, raw=True)
    assert st == hl.LORA_ERANK                       # 70 + 8 > out_max_rank
    st, off, crank, neg = hl.lora_mixture_rows(rank, 2, 1, row_off, 80, 128, raw=True)
    assert st == hl.LORA_OK and crank.tolist() == [72, 78, 8] and neg.tolist() == [64, 70, 0]


def test_batch_prepare_inline_copies_nothing():
    """With LORA_PREPARE_INLINE and the apply op alone, a small all-fused plan
    (64 one-token rows, rank 16, d 4096) is left in the staging buffer: no
    copy is enqueued (so this runs without a GPU), the launch's device arrays
    are NULL and its host pointers point into staging."""
    import ctypes
    staging = np.zeros(4096, np.int32)
    ra = np.arange(64, dtype=np.int32)
    st, out, segs = hl.lora_batch_prepare(ra, np.full(64, 16), 4096, 4096,
                                          (1 << hl.LORA_OP_APPLY) | hl.LORA_PREPARE_INLINE, staging, 0x1000)
    assert st == hl.LORA_OK
    L = out.launch[hl.LORA_OP_APPLY]
    assert not L.row_index and not L.work
    assert L.host_row_index == staging.ctypes.data
    assert L.host_work == staging.ctypes.data + 4 * 64
    assert L.info.n_work == 64 and L.info.range_list() == [(3 * 4 + 5 * 4, 0, 64, 1)]
    assert out.n_staged == 64 + hl.WORK_INTS * 64
    assert np.array_equal(staging[:64], np.arange(64))
    assert out.launch[hl.LORA_OP_SHRINK].info.op == -1 and out.launch[hl.LORA_OP_EXPAND].info.op == -1
    # lora_apply refuses, before any HIP call, a launch with neither device
    # arrays nor a complete inline plan
    lib = hl._lib
    arr = (hl.lora_apply_proj_t * 1)(hl.lora_apply_proj_t(0x30000, 4096, 4096, _rows(4096, 4096, 16, 64),
                                                         0x40000, 16, _rows(4096, 4096, 16, 64), 4096, 0x50000,
                                                         4096, 1.0))

    def apply_with(edit):
        L2 = hl.lora_launch_t.from_buffer_copy(L)
        edit(L2)
        return lib.lora_apply(ctypes.byref(L2), 1, arr, None)

    def no_host_work(L2):
        L2.host_work = None

    def no_host_rows(L2):
        L2.host_row_index = None

    def too_many(L2):  # 65 items: past what the launch arguments hold
        L2.info.n_work = L2.info.ranges[0].count = hl.LORA_INLINE_ITEMS + 1

    def not_fused(L2):
        L2.info.ranges[0].variant = 0

    for edit in (no_host_work, no_host_rows, too_many, not_fused):
        assert apply_with(edit) == hl.LORA_EINVAL, edit.__name__
    # a flag bit the call does not know
    st, *_ = hl.lora_batch_prepare(ra, np.full(64, 16), 4096, 4096, (1 << hl.LORA_OP_APPLY) | 0x200, staging,
                                   0x1000, raw=True)
    assert st == hl.LORA_EINVAL
