"""Device-built batches on the GPU (lora_batch_build_device).

The builder's segment table must equal lora_build_segments' and, range by
range, its work items must equal the items lora_plan(LORA_OP_APPLY) gives
the same variant for the same batch, bit for bit.  lora_apply through the
device-built launch must then give y bit-identical to the host-built launch
(and so stay within the oracle's bound).  Invalid inputs leave an error
status and an empty plan."""
import numpy as np
import pytest
import torch

import heterogeneous_adapter_batching_amd as hl
import oracle
import workloads
from heterogeneous_adapter_batching_amd.session import DeviceBatch
from workloads.device import to_device

from gpu_helpers import check_delta, rows_of, run_apply
from test_device_plan import FUSED, launch_group

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _host_plan(ra, ranks, d_in, d_out):
    segs = hl.lora_build_segments(ra, ranks)
    work, info = hl.lora_plan(hl.LORA_OP_APPLY, segs, d_in, d_out)
    return segs, {v: work[b:b + c] for v, b, c, m in info.range_list()}, info


def _padded(ra, n_rows):
    out = np.full(n_rows, -1, np.int32)
    out[:len(ra)] = ra
    return out


def check_against_oracle(ra, ranks, segs, items, v_slices):
    """The device-built segment table against the oracle's, bit for bit, and
    the device-built work lists against the oracle's coverage invariants: the
    shrink items and the fused rows cover every (active row, K slice) pair of
    its segment once, the expand items and the fused rows every active row
    once, each with its segment's adapter and rank."""
    ref = oracle.build_segments_ref(ra, ranks)
    for k in ("row_index", "seg_start", "seg_adapter", "seg_rank"):
        assert np.array_equal(getattr(segs, k), np.asarray(getattr(ref, k))), k
    for side in ("shrink", "expand"):
        keys = [g for g in sorted(items) if g == FUSED or (g < 12) == (side == "shrink")]
        work = [items[g] for g in keys]
        begin, ranges = 0, []
        for g, w in zip(keys, work):
            ranges.append((g, begin, w.shape[0], 128))
            begin += w.shape[0]
        work = np.concatenate(work) if work else np.zeros((0, hl.WORK_INTS), np.int32)
        oracle.check_plan_coverage(ref, work, ranges, side == "shrink", v_slices)


def build_and_compare(ra, ranks, d_in, d_out, n_rows=None, max_rank=None, db=None):
    """Build on the device and compare with the host planner and the oracle;
    returns the DeviceBatch."""
    ranks = np.asarray(ranks, np.int32)
    ra = _padded(np.asarray(ra, np.int32), n_rows or len(ra))
    db = db or DeviceBatch(len(ra), len(ranks), max_rank or int(ranks.max()), d_in, d_out)
    db.build(torch.from_numpy(ra).cuda(), torch.from_numpy(ranks).cuda())
    h, segs, items = db.read()
    hs, host_items, info = _host_plan(ra, ranks, d_in, d_out)
    assert h.status == hl.LORA_OK
    assert (h.n_seg, h.n_active, h.n_work) == (hs.n_seg, hs.n_active, info.n_work)
    for k in ("row_index", "seg_start", "seg_adapter", "seg_rank"):
        assert np.array_equal(getattr(segs, k), getattr(hs, k)), k
    # each range (launch group) holds the host plan's items of its variants,
    # variant after variant
    assert {launch_group(v) for v in host_items} <= set(items)
    for g, got in items.items():
        parts = [host_items[v] for v in sorted(host_items) if launch_group(v) == g]
        exp = np.concatenate(parts) if parts else np.zeros((0, hl.WORK_INTS), np.int32)
        assert np.array_equal(got, exp), g
    check_against_oracle(ra, ranks, segs, items, db.plan.info.v_slices)
    return db


@pytest.mark.parametrize("k", [0, 1, 2, 3, 4])
def test_builder_matches_host_on_workloads(k):
    S = workloads.structure(k)
    d_in = max(d for _, d, _ in S.projs)
    d_out = max(d for _, _, d in S.projs)
    for name, ra in S.batches.items():
        _say("workload", k, name, "rows", len(ra))
        build_and_compare(ra, S.adapter_rank, d_in, d_out)


@pytest.mark.parametrize("seed", range(8))
def test_builder_matches_host_random(seed):
    rng = np.random.default_rng(1000 + seed)
    n_rows = int(rng.integers(1, 5000))
    n_ad = int(rng.integers(1, 600))
    max_rank = int(rng.choice([8, 16, 64, 128]))
    ranks = rng.integers(1, max_rank + 1, n_ad).astype(np.int32)
    p = 1.0 / np.arange(1, n_ad + 1) ** rng.uniform(0.0, 2.0)
    ra = rng.choice(n_ad, n_rows, p=p / p.sum()).astype(np.int32)
    ra[rng.random(n_rows) < 0.2] = -1
    d_in = int(rng.choice([64, 512, 4096, 8192]))
    d_out = int(rng.choice([128, 4096, 28672]))
    _say("seed", seed, "rows", n_rows, "adapters", n_ad, "max_rank", max_rank, "d", d_in, d_out)
    build_and_compare(ra, ranks, d_in, d_out, max_rank=max_rank)


def test_builder_edges():
    ranks = np.full(4096, 16, np.int32)
    # every row released
    build_and_compare(np.full(64, -1), ranks[:8], 4096, 4096)
    # one row, the largest adapter id
    build_and_compare([4095], ranks, 4096, 4096)
    # the largest bounds: 65536 rows over all 4096 adapters, ranks 1..128
    rng = np.random.default_rng(5)
    r = rng.integers(1, 129, 4096).astype(np.int32)
    build_and_compare(rng.integers(-1, 4096, 65536), r, 8192, 8192)
    # one adapter holds every row (16 waves' blocks all on one id)
    build_and_compare(np.full(65536, 7), r, 4096, 4096)


def test_rebuild_smaller_batch_ignores_stale_items():
    """A large batch, then a small one in the same workspace: the second
    plan's counts exclude the first one's items, which stay in memory."""
    ranks = np.array([16, 64, 32, 128, 8], np.int32)
    big = np.repeat([0, 1, 2, 3, 4], [700, 300, 129, 65, 1])
    db = build_and_compare(big, ranks, 4096, 4096, n_rows=2048)
    small = np.repeat([3, 1], [2, 40])
    build_and_compare(small, ranks, 4096, 4096, n_rows=2048, db=db)


def test_invalid_inputs_give_status_and_empty_plan():
    ranks = np.full(8, 16, np.int32)
    db = DeviceBatch(64, 8, 16, 4096, 4096)
    ra = np.zeros(64, np.int32)
    ra[10] = 8  # id == n_adapters
    db.build(torch.from_numpy(ra).cuda(), torch.from_numpy(ranks).cuda())
    h = db.header()
    assert h.status == hl.LORA_EADAPTER and h.n_work == 0 and list(h.live[:db.plan.info.n_ranges]) == [0]
    ra[10] = -2
    db.build(torch.from_numpy(ra).cuda(), torch.from_numpy(ranks).cuda())
    assert db.header().status == hl.LORA_EADAPTER
    ra[10] = 3
    bad = ranks.copy()
    bad[5] = 17  # above the plan's max_rank
    db.build(torch.from_numpy(ra).cuda(), torch.from_numpy(bad).cuda())
    h = db.header()
    assert h.status == hl.LORA_ERANK and h.n_work == 0
    # a valid batch afterwards builds normally
    build_and_compare(ra, ranks, 4096, 4096, max_rank=16, db=db)


def run_apply_device(W, row_adapter=None, n_rows=None):
    """lora_apply through a device-built launch for every projection of W;
    returns (DeviceBatch, y list) on the host."""
    dw = to_device(W)
    ra = _padded(W.row_adapter if row_adapter is None else np.asarray(row_adapter, np.int32), n_rows or W.n_rows)
    d_in = max(p.d_in for p in W.projections)
    d_out = max(p.d_out for p in W.projections)
    db = DeviceBatch(len(ra), len(W.adapter_rank), int(W.adapter_rank.max()), d_in, d_out)
    db.build(torch.from_numpy(ra).cuda(), torch.from_numpy(np.asarray(W.adapter_rank, np.int32)).cuda())
    ldv = -(-int(W.adapter_rank.max()) // 4) * 4
    vs = [db.new_v(ldv, fill=float("nan")) for _ in W.projections]
    db.apply([(dp.x, rows_of(dw.pool, p.A, dp.A_off), v, rows_of(dw.pool, p.B, dp.B_off), dp.y, W.scale)
              for p, dp, v in zip(W.projections, dw.projections, vs)])
    torch.cuda.synchronize()
    assert db.header().status == hl.LORA_OK
    return db, [dp.y.cpu().numpy() for dp in dw.projections]


def _same_as_host(W, ra=None):
    """Host-built and device-built lora_apply give the same y, bit for bit;
    returns the host Batch and the device y."""
    hb, yh = run_apply(W, ra)
    _, yd = run_apply_device(W, ra)
    for a, b in zip(yh, yd):
        assert np.array_equal(a, b)
    return hb, yd


@pytest.mark.parametrize("which", ["hetero", "homo"])
def test_apply_device_decode_bit_identical(which):
    W = workloads.gen_config(1)
    hb, yd = _same_as_host(W, W.batches[which])
    rep = check_delta(W, hb, None, yd, row_adapter=W.batches[which], check_v=False)
    _say(which, rep)


def test_apply_device_mixed_lengths_and_paged():
    # fused one-row segments, short and long shrink + expand segments
    ra = np.repeat([0, 1, 2, 3, 4, 5, 6], [1, 1, 1, 1, 40, 1, 300])
    _same_as_host(workloads.gen_custom(31, ra, [1, 16, 17, 33, 64, 128, 8], 4096, 3072, n_proj=2))
    # paged rows, nothing fused (d_out above the fused limit), released rows
    ra = np.repeat([2, -1, 0, 1, 3, -1], [1, 5, 1, 77, 130, 3])
    _same_as_host(workloads.gen_custom(32, ra, [24, 5, 64, 96], 448, 4160, layout="paged", page_elems=192))


def test_apply_device_prefill_bit_identical():
    W = workloads.gen_config(2)
    _same_as_host(W)


def test_apply_device_padded_rows_untouched():
    """Capacity above the batch: padding rows are released and their y stays."""
    W = workloads.gen_config(0)
    _, yh = run_apply(W)
    _, yd = run_apply_device(W, n_rows=256)
    assert np.array_equal(yh[0], yd[0])


def test_apply_device_more_items_than_resident_workgroups():
    """Each grid-stride kernel walks several items per workgroup: 3000 rows on
    800 adapters (segments of ~4 rows).  At d 1024 every segment is fused
    (3000 fused rows); with d_in 8192 none is, so the shrink and expand
    launch groups the tile table picks for such segments take them, each
    with more items than a CU-filling grid has workgroups."""
    rng = np.random.default_rng(77)
    ra = rng.integers(0, 800, 3000).astype(np.int32)
    ranks = rng.choice([4, 8, 16], 800).astype(np.int32)
    W = workloads.gen_custom(35, ra, ranks, 1024, 1024, n_proj=2)
    hb, _ = _same_as_host(W)
    assert sum(c for v, b, c, m in hb.info_apply.range_list() if v == 32) == 3000
    W = workloads.gen_custom(36, ra, ranks, 8192, 1024, n_proj=2)
    hb, _ = _same_as_host(W)
    variants = {v: c for v, b, c, m in hb.info_apply.range_list()}
    assert 32 not in variants
    assert sum(c for v, c in variants.items() if v < 12) > 1000      # shrink items
    assert sum(c for v, c in variants.items() if 12 <= v < 32) > 1000  # expand items


def test_apply_device_shared_x_bit_identical():
    """q, k and v read one x: the device-built launch runs the grouped
    long-segment shrink (tasks = item x group, counted from the live count)."""
    ra = np.repeat([0, 1, 2, 3], [300, 1, 150, 520])
    W = workloads.gen_custom(41, ra, [16, 64, 32, 8], 4096, 4096, n_proj=4, shared_x=[(0, 1, 2)])
    _same_as_host(W)
    W = workloads.gen_custom(42, ra, [16, 64, 32, 8], 1024, 8192, n_proj=3, layout="paged", page_elems=1024,
                             shared_x=[(0, 1, 2)])
    _same_as_host(W)
