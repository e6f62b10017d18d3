"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Tolerances: relative Frobenius error of the delta <= 4e-3 and max abs error of
y <= 2e-2 (the contract), plus a precision check relF <= 1e-4 (the kernels add
exact bf16 products in fp32 with v split into two bf16 terms, so ~1e-6 is
expected; a single-bf16 v would show up near 1e-3).  Metadata and the
structural invariants (released rows, permutation, dense vs paged storage,
s = 0, repeat runs) are bit-exact.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads import Projection, RowsDesc, Workload, build_pool, to_bf16_bits
from workloads.device import to_device

from gpu_helpers import UNMERGE_MIN_EQUAL, check_delta, check_merge_bits, run_apply, run_delta, run_merge, ulp_compare, rows_of

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _explicit_workload(x, A_list, B_list, row_adapter, y0, scale=2.0, layout="dense", page=64):
    ranks = np.array([a.shape[0] for a in A_list], np.int32)
    mr = int(ranks.max())
    bits = lambda m: to_bf16_bits(np.asarray(m, np.float32))
    pool, d = build_pool([("A", x.shape[1], [bits(a) for a in A_list]),
                          ("B", y0.shape[1], [bits(b) for b in B_list])],
                         len(A_list), mr, layout, page, np.random.default_rng(0))
    proj = Projection("p", x.shape[1], y0.shape[1], bits(x), np.asarray(y0, np.float32), d["A"], d["B"])
    ra = np.asarray(row_adapter, np.int32)
    return Workload("explicit", 0, len(ra), ra, ranks, pool, [proj], scale, {"main": ra})


# ------------------------------------------------------------------ workloads 0 and 1
def test_tiny_sgmv_parity():
    W = workloads.gen_config(0)
    _say("tiny: rows", W.n_rows, "segments", oracle.build_segments_ref(W.row_adapter, W.adapter_rank).n_seg)
    batch, vs, ys = run_delta(W)
    ref = oracle.build_segments_ref(W.row_adapter, W.adapter_rank)
    assert np.array_equal(batch.segs.row_index, ref.row_index)
    _say(check_delta(W, batch, vs, ys))


@pytest.mark.parametrize("which", ["hetero", "homo"])
def test_decode_bgmv_parity(which):
    W = workloads.gen_config(1)
    ra = W.batches[which]
    _say("decode", which)
    batch, vs, ys = run_delta(W, ra)
    _say(check_delta(W, batch, vs, ys, row_adapter=ra))


def test_tiny_merge_parity_and_restore():
    W = workloads.gen_config(0)
    dw = to_device(W)
    p = W.projections[0]
    Wb = W.merge.weight(0, 0)
    r = int(W.adapter_rank[W.merge.adapter])
    merged, restored = run_merge([Wb], dw, [(p.A, dw.projections[0].A_off, p.B, dw.projections[0].B_off)],
                                 W.merge.adapter, r, W.scale, unmerge_too=True)
    Aa = oracle.gather_rows_ref(W.pool, p.A.row_off, p.A.max_rank, p.A.row_len, p.A.chunk_len, 0, r)
    Ba = oracle.gather_rows_ref(W.pool, p.B.row_off, p.B.max_rank, p.B.row_len, p.B.chunk_len, 0, r)
    _say("tiny merge (equal fraction, max ulp, worst/bound):", check_merge_bits(merged[0], Wb, Aa, Ba, W.scale))
    # restore after unmerge, against the oracle's own unmerge of the GPU result and against W
    _say("tiny unmerge (equal fraction, max ulp, worst/bound):",
         check_merge_bits(restored[0], merged[0], Aa, Ba, -W.scale, min_equal=UNMERGE_MIN_EQUAL))
    w0, w2 = oracle.bf16_to_f64(Wb), oracle.bf16_to_f64(restored[0])
    relF = np.linalg.norm(w2 - w0) / np.linalg.norm(w0)
    assert relF <= 4e-3 and np.max(np.abs(w2 - w0)) <= 2e-2
    # merged == unmerged inference (S-LoRA formula 1 vs formula 2)
    x = oracle.bf16_to_f64(p.x)
    f1 = x @ oracle.bf16_to_f64(merged[0]).T
    f2 = x @ w0.T + W.scale * (x @ Aa.T) @ Ba
    assert np.linalg.norm(f1 - f2) / np.linalg.norm(f2) <= 4e-3


# ------------------------------------------------------------------ exact cases and invariants
def test_rank1_closed_form_bit_exact():
    d = 64
    x = np.zeros((3, d)); x[0, :8] = np.arange(-3, 5); x[1, :8] = np.arange(5, -3, -1); x[2, 2] = 7
    a = np.zeros((1, d)); a[0, 2] = 1.0
    b = np.zeros((1, d)); b[0, :4] = [1.0, 0.5, -2.0, 4.0]; b[0, 63] = 0.25
    W = _explicit_workload(x, [a], [b], [0, 0, -1], np.zeros((3, d)))
    _, _, ys = run_delta(W)
    want = np.zeros((3, d), np.float32)
    for i in range(2):
        want[i] = 2.0 * x[i, 2] * b[0]
    assert np.array_equal(ys[0], want)
    assert ys[0][0, :4].tolist() == [-2.0, -1.0, 4.0, -8.0]


def test_scale_zero_keeps_y():
    W = workloads.gen_custom(21, np.repeat([0, 1, 2, -1], [5, 40, 130, 3]), [7, 33, 64], 256, 320)
    _, _, ys = run_delta(W, scale=0.0)
    assert np.array_equal(ys[0], W.projections[0].y0)


def test_permutation_bit_identical():
    ra = np.repeat([0, 1, 2, 3, 1], [1, 20, 70, 300, 9])
    W = workloads.gen_custom(22, ra, [16, 64, 8, 32], 512, 576, n_proj=2)
    _, _, ys = run_delta(W)
    perm = np.random.default_rng(3).permutation(W.n_rows)
    Wp = Workload(W.name, W.seed, W.n_rows, W.row_adapter[perm], W.adapter_rank, W.pool,
                  [Projection(p.name, p.d_in, p.d_out, p.x[perm], p.y0[perm], p.A, p.B) for p in W.projections],
                  W.scale)
    _, _, ysp = run_delta(Wp)
    for y, yp in zip(ys, ysp):
        assert np.array_equal(yp, y[perm])


def test_released_rows_untouched_and_active_rows_unchanged():
    rng = np.random.default_rng(4)
    ra = np.repeat(rng.integers(0, 6, size=12), rng.integers(1, 60, size=12))
    W = workloads.gen_custom(23, ra, [4, 16, 24, 40, 64, 128], 384, 448)
    keep = rng.random(W.n_rows) < 0.6
    ra_rel = np.where(keep, ra, -1)
    batch, vs, ys = run_delta(W, ra_rel)
    p = W.projections[0]
    assert np.array_equal(ys[0][~keep], p.y0[~keep])
    # the same batch with the released rows deleted gives bit-identical active rows
    idx = np.nonzero(keep)[0]
    Wd = Workload(W.name, W.seed, len(idx), ra[idx], W.adapter_rank, W.pool,
                  [Projection(p.name, p.d_in, p.d_out, p.x[idx], p.y0[idx], p.A, p.B)], W.scale)
    _, _, ysd = run_delta(Wd)
    assert np.array_equal(ysd[0], ys[0][idx])
    check_delta(W, batch, vs, ys, row_adapter=ra_rel)


@pytest.mark.parametrize("page", [64, 192])
def test_dense_vs_paged_bit_identical(page):
    ra = np.repeat([2, 0, 1, 2], [3, 100, 17, 260])
    Wd = workloads.gen_custom(24, ra, [12, 48, 100], 640, 896, layout="dense")
    Wp = workloads.gen_custom(24, ra, [12, 48, 100], 640, 896, layout="paged", page_elems=page)
    assert Wp.projections[0].B.chunks > 1
    _, vd, yd = run_delta(Wd)
    batch, vp, yp = run_delta(Wp)
    assert np.array_equal(yd[0], yp[0])
    assert np.array_equal(np.nan_to_num(vd[0], nan=7.0), np.nan_to_num(vp[0], nan=7.0))
    check_delta(Wp, batch, vp, yp)


@pytest.mark.parametrize("path", ["split", "apply", "apply_shared_x"])
def test_repeat_runs_bit_identical(path):
    """10 runs from the same inputs give the same bits (a race on LDS or a
    reduction whose order depends on timing would show up here): one-row,
    short and long segments, several K slices, three projections."""
    from gpu_helpers import run_apply
    from workloads.device import reset_outputs
    ra = np.repeat([0, 1, 2, 3], [1, 33, 513, 700])
    shared = [(0, 1, 2)] if path == "apply_shared_x" else ()
    W = workloads.gen_custom(25, ra, [16, 96, 64, 40], 4096, 1024, n_proj=3, shared_x=shared)
    dw = to_device(W)
    run = (lambda: run_delta(W, dw=dw)[2]) if path == "split" else (lambda: run_apply(W, dw=dw)[1])
    y1 = run()
    for _ in range(9):
        reset_outputs(W, dw)
        for a, b in zip(y1, run()):
            assert np.array_equal(a, b)


def test_repeat_merge_bit_identical():
    """10 merges of a 4096 x 4096 W (many tiles, rank 16) give the same bits."""
    W = workloads.gen_config(1)
    dw = to_device(W)
    p, d = W.projections[0], dw.projections[0]
    w = W.merge.weight(0, 0)
    r = int(W.adapter_rank[W.merge.adapter])
    descs = [(p.A, d.A_off, p.B, d.B_off)]
    first, _ = run_merge([w], dw, descs, W.merge.adapter, r, W.scale)
    for _ in range(9):
        again, _ = run_merge([w], dw, descs, W.merge.adapter, r, W.scale)
        assert np.array_equal(first[0], again[0])


def test_empty_batch_no_work():
    W = workloads.gen_custom(26, [-1, -1, -1], [8], 128, 128)
    batch, vs, ys = run_delta(W)
    assert batch.n_active == 0 and batch.info_shrink.n_work == 0
    assert np.array_equal(ys[0], W.projections[0].y0)


@pytest.mark.parametrize("seed", range(100, 110))
def test_random_shapes_parity(seed):
    """Every kernel variant: segment lengths 1..700, ranks 1..128, d 64..2048 with ragged 64-multiples."""
    rng = np.random.default_rng(seed)
    n_ad = int(rng.integers(1, 10))
    ranks = rng.integers(1, 129, size=n_ad)
    ranks[0] = int(rng.choice([1, 8, 16, 17, 32, 33, 64, 65, 127, 128]))
    lens = rng.choice([1, 2, 3, 5, 9, 16, 17, 31, 64, 65, 127, 128, 129, 300, 700], size=int(rng.integers(1, 9)))
    ra = np.repeat(rng.integers(-1, n_ad, size=len(lens)), lens)
    d_in = 64 * int(rng.integers(1, 33))
    d_out = 64 * int(rng.integers(1, 33))
    layout = "paged" if seed % 3 == 0 else "dense"
    W = workloads.gen_custom(seed, ra, ranks, d_in, d_out, n_proj=1 + seed % 3, layout=layout,
                             page_elems=64 * int(rng.integers(1, 5)))
    _say("random", seed, "rows", W.n_rows, "ranks", ranks.tolist(), "d", d_in, d_out, layout)
    batch, vs, ys = run_delta(W)
    _say(check_delta(W, batch, vs, ys))


@pytest.mark.parametrize("seed", range(200, 216))
def test_random_wide_shapes_parity(seed):
    """The tile table's large-d buckets: d_in up to 16384 and d_out up to
    28672 with every length and rank bucket, through the shrink + expand
    path and lora_apply, dense and paged; every row of a batch up to 300
    rows, else a seeded sample of 300 (released rows among them checked
    untouched)."""
    rng = np.random.default_rng(seed)
    n_ad = int(rng.integers(1, 12))
    ranks = rng.integers(1, 129, size=n_ad)
    lens = rng.choice([1, 2, 3, 4, 5, 8, 9, 16, 17, 32, 33, 64, 65, 200, 256, 257, 600], size=int(rng.integers(1, 10)))
    ra = np.repeat(rng.integers(-1, n_ad, size=len(lens)), lens)
    d_in = int(rng.choice([1024, 2048, 4096, 6144, 8192, 12288, 16384]))
    d_out = int(rng.choice([1024, 4096, 8192, 12288, 16384, 28672]))
    layout = "paged" if seed % 2 else "dense"
    W = workloads.gen_custom(seed, ra, ranks, d_in, d_out, n_proj=1 + seed % 2, layout=layout,
                             page_elems=64 * int(rng.choice([16, 64, 128])))
    rows = None if W.n_rows <= 300 else sorted(rng.choice(W.n_rows, 300, replace=False).tolist())
    _say("wide", seed, "rows", W.n_rows, "ranks", ranks.tolist(), "d", d_in, d_out, layout)
    batch, vs, ys = run_delta(W)
    _say(check_delta(W, batch, vs, ys, rows=rows))
    batch, ys = run_apply(W)
    _say(check_delta(W, batch, None, ys, rows=rows, check_v=False))


@pytest.mark.parametrize("d_out,d_in,r", [(64, 192, 1), (576, 320, 17), (1024, 512, 64), (256, 704, 128)])
def test_merge_shapes_parity(d_out, d_in, r):
    rng = np.random.default_rng(d_out + d_in + r)
    n_ad = 3
    ranks = np.array([r, max(1, r // 2), 5])
    W = workloads.gen_custom(int(d_out + r), [0], ranks, d_in, d_out, layout="paged" if r % 2 else "dense",
                             page_elems=128)
    dw = to_device(W)
    p = W.projections[0]
    Wb = to_bf16_bits(rng.standard_normal((d_out, d_in)).astype(np.float32) / np.sqrt(d_in))
    a = int(rng.integers(0, n_ad)) if r > 1 else 0
    ra_ = int(ranks[a])
    merged, restored = run_merge([Wb], dw, [(p.A, dw.projections[0].A_off, p.B, dw.projections[0].B_off)],
                                 a, ra_, 2.0, unmerge_too=True)
    Aa = oracle.gather_rows_ref(W.pool, p.A.row_off, p.A.max_rank, p.A.row_len, p.A.chunk_len, a, ra_)
    Ba = oracle.gather_rows_ref(W.pool, p.B.row_off, p.B.max_rank, p.B.row_len, p.B.chunk_len, a, ra_)
    _say("merge", d_out, d_in, r, check_merge_bits(merged[0], Wb, Aa, Ba, 2.0))
    _say("unmerge", d_out, d_in, r, check_merge_bits(restored[0], merged[0], Aa, Ba, -2.0, min_equal=UNMERGE_MIN_EQUAL))
    w0, w2 = oracle.bf16_to_f64(Wb), oracle.bf16_to_f64(restored[0])
    assert np.linalg.norm(w2 - w0) / np.linalg.norm(w0) <= 4e-3


def test_merge_mixed_launch():
    """One launch merges matrices of different shapes and ranks: the launch
    compiles for its largest rank (128, four 32-rank groups), each matrix stops
    at its own rank, and the tiles past d_in (waves with no columns still load
    their share of the B strip) and past d_out are partial."""
    from heterogeneous_adapter_batching_amd.session import merge, unmerge
    from workloads.device import bits_to_device
    rng = np.random.default_rng(77)
    specs = [(192, 704, 128, "dense"), (576, 320, 40, "paged"), (1024, 1536, 5, "dense"), (64, 192, 97, "paged")]
    mats, refs, keep = [], [], []
    for i, (d_out, d_in, r, layout) in enumerate(specs):
        W = workloads.gen_custom(300 + i, [0], np.array([r], np.int32), d_in, d_out, layout=layout, page_elems=128)
        dw = to_device(W)
        p, dp = W.projections[0], dw.projections[0]
        Wb = to_bf16_bits(rng.standard_normal((d_out, d_in)).astype(np.float32) / np.sqrt(d_in))
        Wt = bits_to_device(Wb)
        mats.append((Wt, rows_of(dw.pool, p.A, dp.A_off), rows_of(dw.pool, p.B, dp.B_off), 0, r, 1.5))
        Aa = oracle.gather_rows_ref(W.pool, p.A.row_off, p.A.max_rank, p.A.row_len, p.A.chunk_len, 0, r)
        Ba = oracle.gather_rows_ref(W.pool, p.B.row_off, p.B.max_rank, p.B.row_len, p.B.chunk_len, 0, r)
        refs.append((Wb, Aa, Ba))
        keep.append(dw)
    merge(mats)
    torch.cuda.synchronize()
    merged = [m[0].cpu().numpy().view(np.uint16).copy() for m in mats]
    for (d_out, d_in, r, _), got, (Wb, Aa, Ba) in zip(specs, merged, refs):
        _say("mixed merge", d_out, d_in, r, check_merge_bits(got, Wb, Aa, Ba, 1.5))
    unmerge(mats)
    torch.cuda.synchronize()
    for m, got, (Wb, Aa, Ba) in zip(mats, merged, refs):
        back = m[0].cpu().numpy().view(np.uint16)
        _say("mixed unmerge", check_merge_bits(back, got, Aa, Ba, -1.5, min_equal=UNMERGE_MIN_EQUAL))


# ------------------------------------------------------------------ lora_apply (fused decode rows)
def _apply_check(W, ra=None):
    from gpu_helpers import run_apply
    batch, ys = run_apply(W, ra)
    n_fused = sum(c for v, b, c, m in batch.info_apply.range_list() if v == 32)
    rep = check_delta(W, batch, None, ys, row_adapter=ra, check_v=False)
    _say("apply: fused items", n_fused, rep)
    return n_fused


@pytest.mark.parametrize("which", ["hetero", "homo"])
def test_apply_decode_parity(which):
    W = workloads.gen_config(1)
    n_fused = _apply_check(W, W.batches[which])
    # hetero: 64 one-row segments; homo: one 64-row rank-16 segment, fused row by row (64 * 16 <= 1024)
    assert n_fused == 64


def test_apply_tiny_and_mixed_lengths():
    _apply_check(workloads.gen_config(0))
    # one-row segments of several ranks (1..128: several rank groups of 16) next to longer ones
    ra = np.repeat([0, 1, 2, 3, 4, 5, 6], [1, 1, 1, 1, 40, 1, 300])
    W = workloads.gen_custom(31, ra, [1, 16, 17, 33, 64, 128, 8], 4096, 3072, n_proj=2)
    assert _apply_check(W) == 5    # 5 one-row segments (the projections share each item)


@pytest.mark.parametrize("page", [64, 448])
def test_apply_paged_and_small_d(page):
    ra = np.repeat([2, 0, 1, 3], [1, 1, 77, 1])
    W = workloads.gen_custom(32, ra, [24, 5, 64, 96], 448, 1984, layout="paged", page_elems=page)
    _apply_check(W)


def test_apply_matches_shrink_expand_when_nothing_fuses():
    # d_out beyond the fused limit: apply runs the shrink and expand kernels, bit-identical to them
    ra = np.repeat([0, 1, 2], [1, 5, 130])
    W = workloads.gen_custom(33, ra, [16, 32, 64], 1024, 4160)
    from gpu_helpers import run_apply
    batch, ya = run_apply(W)
    assert all(v != 32 for v, b, c, m in batch.info_apply.range_list())
    _, _, yd = run_delta(W)
    assert np.array_equal(ya[0], yd[0])


@pytest.mark.parametrize("case", ["hetero", "homo", "tiny", "not_inline"])
def test_apply_inline_plan_bit_identical(case):
    """A plan carried in the launch arguments gives the same bits as the
    copied one; a plan too large or not all fused falls back to the copy."""
    from gpu_helpers import run_apply
    if case in ("hetero", "homo"):
        W = workloads.gen_config(1)
        ra = W.batches[case]
    elif case == "tiny":
        W, ra = workloads.gen_config(0), None
    else:  # a long rank-64 segment: shrink + expand ranges, copied
        ra = np.repeat([0, 1, 2], [1, 3, 200])
        W = workloads.gen_custom(34, ra, [16, 8, 64], 4096, 4096, n_proj=2)
    b0, y0 = run_apply(W, ra)
    b1, y1 = run_apply(W, ra, inline=True)
    L = b1.apply_launch
    assert bool(L.work) == (case == "not_inline") and bool(L.row_index) == (case == "not_inline")
    for a, b in zip(y0, y1):
        assert np.array_equal(a, b)
    rep = check_delta(W, b0, None, y1, row_adapter=ra, check_v=False)
    _say("inline", case, rep)


# ------------------------------------------------------------------ batch preparation
def test_batch_prepare_layout_and_upload():
    """lora_batch_prepare writes row_index and the requested plans back to back
    into the staging buffer (bit-identical to lora_build_segments + lora_plan),
    points each launch into the device buffer, and the device copy equals the
    staging buffer; a Batch refreshed over a sequence of batches keeps serving
    the current one."""
    import heterogeneous_adapter_batching_amd as hl
    from heterogeneous_adapter_batching_amd.session import Batch
    rng = np.random.default_rng(31)
    rank = rng.choice([8, 16, 32, 64], size=20).astype(np.int32)
    ra = np.repeat(rng.integers(-1, 20, size=40), rng.integers(1, 90, size=40)).astype(np.int32)
    segs = hl.lora_build_segments(ra, rank)
    plans = {op: hl.lora_plan(op, segs, 4096, 2048) for op in (hl.LORA_OP_SHRINK, hl.LORA_OP_EXPAND, hl.LORA_OP_APPLY)}
    need = segs.n_active + hl.WORK_INTS * sum(p[0].shape[0] for p in plans.values())
    host = torch.zeros(need + 64, dtype=torch.int32).pin_memory()
    dev = torch.full((need + 64,), -7, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    st, out, (s0, s1, s2) = hl.lora_batch_prepare(ra, rank, 4096, 2048, 7, host.numpy(), dev.data_ptr(),
                                                  stream.cuda_stream)
    torch.cuda.synchronize()
    assert out.n_seg == segs.n_seg and out.n_active == segs.n_active and out.n_staged == need
    assert np.array_equal(s0[:segs.n_seg + 1], segs.seg_start) and np.array_equal(s1[:segs.n_seg], segs.seg_adapter)
    assert np.array_equal(s2[:segs.n_seg], segs.seg_rank)
    h = host.numpy()
    assert np.array_equal(h[:segs.n_active], segs.row_index)
    off = segs.n_active
    for op in (hl.LORA_OP_SHRINK, hl.LORA_OP_EXPAND, hl.LORA_OP_APPLY):
        work, info = plans[op]
        L = out.launch[op]
        assert L.row_index == dev.data_ptr() and L.work == dev.data_ptr() + 4 * off
        assert L.info.op == op and L.info.n_work == work.shape[0] and L.info.range_list() == info.range_list()
        assert np.array_equal(h[off:off + hl.WORK_INTS * work.shape[0]].reshape(-1, hl.WORK_INTS), work)
        off += hl.WORK_INTS * work.shape[0]
    d = dev.cpu().numpy()
    assert np.array_equal(d[:need], h[:need]) and (d[need:] == -7).all()
    # only the apply plan: the other launches are marked unusable
    st, out, _ = hl.lora_batch_prepare(ra, rank, 4096, 2048, 4, host.numpy(), dev.data_ptr(), stream.cuda_stream)
    torch.cuda.synchronize()
    assert out.launch[0].info.op == -1 and out.launch[1].info.op == -1 and out.launch[2].info.op == 2
    assert out.launch[2].work == dev.data_ptr() + 4 * segs.n_active
    # Batch: a small staging buffer grows, and each refresh describes its own batch
    b = Batch(8, rank, 4096, 2048)
    for k in range(4):
        rak = ra[rng.permutation(ra.shape[0])][: 50 + 400 * k]
        b.refresh(rak)
        ref = hl.lora_build_segments(rak, rank)
        assert np.array_equal(b.segs.row_index, ref.row_index) and b.n_active == ref.n_active
        we, ie = hl.lora_plan(hl.LORA_OP_EXPAND, ref, 4096, 2048)
        assert np.array_equal(b.work_expand, we) and b.info_expand.range_list() == ie.range_list()
        torch.cuda.synchronize()
        got = b._dev.cpu().numpy()
        assert np.array_equal(got[:ref.n_active], ref.row_index)


# ------------------------------------------------------------------ projections that share x
def _shared_x_workload(layout, seed=41):
    """q/k/v (projections 0-2) read one x, o its own.  Long segments (the
    grouped long-segment shrink), one of rank above 64 (its own kernel, not
    grouped), one short segment, rows scattered over the batch."""
    rng = np.random.default_rng(seed)
    ranks = np.array([8, 16, 32, 64, 100, 40], np.int32)
    lens = [300, 520, 270, 700, 290, 3]
    ra = np.repeat(rng.permutation(6), lens).astype(np.int32)
    ra = ra[rng.permutation(ra.shape[0])]
    return workloads.gen_custom(seed, ra, ranks, 4096, 1024, n_proj=4, layout=layout, page_elems=512,
                                shared_x=[(0, 1, 2)])


@pytest.mark.parametrize("layout", ["dense", "paged"])
def test_shared_x_parity(layout):
    W = _shared_x_workload(layout)
    assert W.projections[0].x is W.projections[2].x
    _say("shared x", layout, "rows", W.n_rows)
    batch, vs, ys = run_delta(W)
    _say(check_delta(W, batch, vs, ys))


def test_shared_x_apply_and_storage():
    """lora_apply over the same batch (its shrink ranges group q/k/v too)
    matches the oracle, and dense and paged storage give bit-identical y."""
    from gpu_helpers import run_apply
    Wd, Wp = _shared_x_workload("dense"), _shared_x_workload("paged")
    ys_d = run_delta(Wd)[2]
    ys_p = run_delta(Wp)[2]
    for a, b in zip(ys_d, ys_p):
        assert np.array_equal(a, b)
    batch, ys = run_apply(Wd)
    _say("shared x apply", check_delta(Wd, batch, None, ys, check_v=False))


def test_shared_x_against_separate_copies():
    """The same values with a private copy of x per projection (no grouping):
    the group's first projection sums in the same order (bit-identical y);
    the others start their K steps elsewhere, so they agree to fp32 rounding."""
    from workloads import Projection as Proj
    W = _shared_x_workload("dense")
    _, _, ys_g = run_delta(W)
    W.projections = [Proj(p.name, p.d_in, p.d_out, p.x.copy(), p.y0, p.A, p.B) for p in W.projections]
    _, _, ys_s = run_delta(W)
    assert np.array_equal(ys_g[0], ys_s[0]) and np.array_equal(ys_g[3], ys_s[3])
    for pi in (1, 2):
        d_g = ys_g[pi].astype(np.float64) - W.projections[pi].y0
        d_s = ys_s[pi].astype(np.float64) - W.projections[pi].y0
        rel = np.linalg.norm(d_g - d_s) / np.linalg.norm(d_s)
        _say("shared vs separate x, projection", pi, rel)
        assert rel <= 1e-5


# ------------------------------------------------------------------ vision task heads
def test_task_heads_in_one_launch():
    """Per-adapter vision task heads (VaLoRA 4.2.2: a linear layer that is part
    of the adapter replaces the LM head for tasks with a small label set) are
    a shrink whose A rows are the head's class rows: logits = x . H_a^T, with
    heads of different widths in one launch and the LM-head rows (-1) left
    alone."""
    rng = np.random.default_rng(23)
    classes = np.array([10, 37, 100, 3, 128], np.int32)
    lens = [300, 2, 270, 1, 40]
    ra = np.concatenate([np.repeat(np.arange(5), lens), np.full(25, -1)]).astype(np.int32)
    ra = ra[rng.permutation(ra.shape[0])]
    d = 2048
    W = workloads.gen_custom(23, ra, classes, d, 64, n_proj=1, layout="paged", page_elems=512)
    batch, vs, ys = run_delta(W)   # the expand half is ordinary LoRA work on the same rows
    p = W.projections[0]
    _, vref = oracle.apply_ref(W.row_adapter, W.adapter_rank, p.x, p.y0, W.pool, p.A, p.B, W.scale)
    pos = {int(r): i for i, r in enumerate(batch.segs.row_index)}
    seg_slices = {}
    for w in batch.work_expand:
        for q in range(int(w[0]), int(w[0]) + int(w[1])):
            seg_slices[q] = int(w[5])
    worst = 0.0
    for i in range(W.n_rows):
        a = int(W.row_adapter[i])
        if a < 0:
            assert i not in pos
            continue
        c = int(classes[a])
        logits = vs[0][:seg_slices[pos[i]], pos[i], :].sum(axis=0)
        ref = vref[i]
        assert logits.shape[0] >= c and np.all(np.isnan(vs[0][:, pos[i], c:])), "columns past the head's width written"
        err = np.abs(logits[:c] - ref) / (1e-3 + np.abs(ref).max())
        worst = max(worst, float(err.max()))
    _say("task heads: worst relative logit error", worst)
    assert worst <= 1e-4
