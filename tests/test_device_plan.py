"""Device-built plans, host side (CPU only): the layout lora_device_plan fixes
from bounds must hold the host planner's plan of every batch within those
bounds, launch group by launch group.  The GPU tests check that the builder
fills it with exactly those items."""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import heterogeneous_adapter_batching_amd as hl

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

LEN_EDGES = [1, 2, 4, 5, 8, 9, 16, 17, 32, 33, 64, 65, 256, 257]
FUSED = 3 * 4 + 5 * 4   # apply variants: 3 shrink shapes x 4 rank classes, 5 expand shapes x 4, then fused


def launch_group(v):
    """The launch group of an apply variant in a device-built plan, keyed by
    its smallest variant: the shrink of ranks up to 64 shares one launch per
    shape (split-K, 64-row and 128-row items), the MFMA expand (shapes 0-3)
    one launch per rank class; ranks above 64 of the shrink, the BGMV expand
    and the fused rows are launches of their own."""
    if v < 12:
        shape, cls = divmod(v, 4)
        return shape * 4 if cls < 3 else v
    if v < FUSED:
        shape, cls = divmod(v - 12, 4)
        return v if shape == 4 else 12 + cls
    return v


RANK_EDGES = [1, 8, 16, 17, 32, 33, 64, 65, 128]


def host_plan(row_adapter, ranks, d_in, d_out):
    segs = hl.lora_build_segments(row_adapter, ranks)
    work, info = hl.lora_plan(hl.LORA_OP_APPLY, segs, d_in, d_out)
    return segs, work, info


def check_fits(row_adapter, ranks, bounds, d_in, d_out):
    """The host apply plan's items of every launch group fit the device
    layout's range of that group."""
    n_rows, n_adapters, max_rank = bounds
    _, plan = hl.lora_device_plan(n_rows, n_adapters, max_rank, d_in, d_out)
    dev = {g: (b, c, m) for g, b, c, m in plan.info.range_list()}
    _, _, info = host_plan(row_adapter, ranks, d_in, d_out)
    need = {}
    for v, _, count, rows_per in info.range_list():
        g = launch_group(v)
        assert g in dev, (v, g, sorted(dev))
        assert rows_per <= dev[g][2]
        need[g] = need.get(g, 0) + count
    for g, n in need.items():
        assert n <= dev[g][1], (g, n, dev[g][1])
    assert info.v_slices <= plan.info.v_slices
    return plan, info


def batch_from_lengths(lengths, n_rows, n_adapters, rng, released=0):
    """Rows of segments with the given lengths (one adapter each, distinct),
    shuffled, the rest released."""
    ids = rng.permutation(n_adapters)[:len(lengths)]
    ra = np.full(n_rows, -1, np.int32)
    pos = 0
    for a, ln in zip(ids, lengths):
        ra[pos:pos + ln] = a
        pos += ln
    return ra[rng.permutation(n_rows)]


@pytest.mark.parametrize("d", [(512, 512), (4096, 4096), (8192, 8192), (8192, 28672), (4096, 1024)])
def test_layout_holds_adversarial_batches(d):
    d_in, d_out = d
    rng = np.random.default_rng(7)
    for n_rows in (1, 3, 64, 300, 2048):
        for max_rank in (16, 64, 128):
            n_adapters = 512
            ranks_pool = [r for r in RANK_EDGES if r <= max_rank]
            cases = []
            # one segment of each edge length, all ranks at max
            for ln in LEN_EDGES + [n_rows]:
                if ln <= n_rows:
                    cases.append(([ln], max_rank))
            # as many segments as fit, of one edge length each
            for ln in LEN_EDGES:
                k = min(n_rows // ln, n_adapters)
                if k:
                    cases.append(([ln] * k, None))
            for lengths, r in cases:
                ranks = rng.choice(ranks_pool, n_adapters).astype(np.int32)
                if r is not None:
                    ranks[:] = r
                ra = batch_from_lengths(lengths, n_rows, n_adapters, rng)
                check_fits(ra, ranks, (n_rows, n_adapters, max_rank), d_in, d_out)


def test_layout_holds_random_batches():
    rng = np.random.default_rng(11)
    for _ in range(300):
        n_rows = int(rng.integers(1, 3000))
        n_adapters = int(rng.integers(1, 300))
        max_rank = int(rng.choice([4, 16, 32, 48, 64, 100, 128]))
        d_in = int(rng.choice([64, 512, 4096, 8192, 16384]))
        d_out = int(rng.choice([64, 1024, 4096, 8192, 28672]))
        ranks = rng.integers(1, max_rank + 1, n_adapters).astype(np.int32)
        # a Zipf-like adapter choice gives a few long segments and many short
        p = 1.0 / np.arange(1, n_adapters + 1) ** rng.uniform(0.0, 2.0)
        ra = rng.choice(n_adapters, n_rows, p=p / p.sum()).astype(np.int32)
        ra[rng.random(n_rows) < rng.uniform(0, 0.5)] = -1
        check_fits(ra, ranks, (n_rows, n_adapters, max_rank), d_in, d_out)


def test_decode_layout_is_one_fused_range():
    """64 one-token rows, rank <= 16, d 4096: every segment is fused whatever
    the adapters, so the device layout is the fused range alone, 64 items."""
    _, plan = hl.lora_device_plan(64, 1024, 16, 4096, 4096)
    assert plan.info.range_list() == [(FUSED, 0, 64, 1)]
    assert plan.info.v_slices == 1 and plan.info.n_active == 64 and plan.info.max_adapter == 1023


def test_launch_groups():
    """Each range is keyed by its group's smallest variant, groups are
    disjoint, and the prefill-sized layout holds exactly the launch groups
    that some segment within its bounds reaches (from the host planner, one
    segment of each length-bucket edge and rank edge at a time)."""
    for v in range(FUSED + 1):
        g = launch_group(v)
        assert g <= v and launch_group(g) == g
    _, plan = hl.lora_device_plan(9436, 16, 64, 4096, 4096)
    keys = [g for g, *_ in plan.info.range_list()]
    assert keys == sorted(set(keys)) and all(launch_group(g) == g for g in keys)
    reach = set()
    for n in LEN_EDGES + [9436]:
        for r in [e for e in RANK_EDGES if e <= 64]:
            _, _, info = host_plan(np.zeros(n, np.int32), [r], 4096, 4096)
            reach |= {launch_group(v) for v, *_ in info.range_list()}
    assert keys == sorted(reach)
    assert FUSED in keys and len(keys) <= 10


def test_layout_offsets_and_sizes():
    for bounds in [(1, 1, 1, 64, 64), (64, 64, 16, 4096, 4096), (8448, 128, 64, 8192, 28672),
                   (65536, 4096, 128, 4096, 4096)]:
        _, p = hl.lora_device_plan(*bounds)
        n_rows, n_adapters = bounds[0], bounds[1]
        assert p.seg_capacity == min(n_rows, n_adapters)
        offs = [p.off_row_index, p.off_seg_start, p.off_seg_adapter, p.off_seg_rank, p.off_scratch, p.off_work,
                p.workspace_bytes]
        assert all(o % 256 == 0 for o in offs)
        assert offs[0] >= ctypes.sizeof(hl.lora_device_header_t)
        sizes = [4 * n_rows, 4 * (p.seg_capacity + 1), 4 * p.seg_capacity, 4 * p.seg_capacity, 4 * n_rows,
                 32 * p.work_capacity]
        for a, b, sz in zip(offs, offs[1:], sizes):
            assert b - a >= sz
        rl = p.info.range_list()
        assert [v for v, *_ in rl] == sorted(v for v, *_ in rl)  # shrink, expand, fused order
        begin = 0
        for v, b, c, m in rl:
            assert b == begin and c > 0
            begin += c
        assert begin == p.work_capacity == p.info.n_work


def test_device_plan_errors():
    ok = (64, 16, 16, 4096, 4096)
    assert hl.lora_device_plan(*ok, raw=True)[0] == hl.LORA_OK
    for bad, code in [((0, 16, 16, 4096, 4096), hl.LORA_EINVAL), ((65537, 16, 16, 4096, 4096), hl.LORA_EINVAL),
                      ((64, 0, 16, 4096, 4096), hl.LORA_EINVAL), ((64, 4097, 16, 4096, 4096), hl.LORA_EINVAL),
                      ((64, 16, 0, 4096, 4096), hl.LORA_ERANK), ((64, 16, 129, 4096, 4096), hl.LORA_ERANK),
                      ((64, 16, 16, 4000, 4096), hl.LORA_ESHAPE), ((64, 16, 16, 4096, 0), hl.LORA_ESHAPE)]:
        assert hl.lora_device_plan(*bad, raw=True)[0] == code, bad


def test_build_device_rejects_a_plan_it_did_not_lay_out():
    """The builder trusts the capacities only after recomputing them; the
    host checks run before anything touches the device."""
    _, plan = hl.lora_device_plan(64, 16, 16, 4096, 4096)
    plan.info.ranges[0].count += 1
    st, _ = hl.lora_batch_build_device(plan, 256, 256, 256, None, raw=True)
    assert st == hl.LORA_EINVAL
    _, plan = hl.lora_device_plan(64, 16, 16, 4096, 4096)
    st, _ = hl.lora_batch_build_device(plan, 256, 256, 256 + 16, None, raw=True)  # misaligned workspace
    assert st == hl.LORA_EINVAL
    st, _ = hl.lora_batch_build_device(plan, None, 256, 256, None, raw=True)
    assert st == hl.LORA_EINVAL


STRUCTS = ["lora_rows_t", "lora_work_t", "lora_range_t", "lora_plan_info_t", "lora_launch_t", "lora_batch_t",
           "lora_shrink_proj_t", "lora_expand_proj_t", "lora_apply_proj_t", "lora_merge_mat_t",
           "lora_device_plan_t", "lora_device_header_t"]


def test_struct_layouts_match_header(tmp_path):
    """sizeof and every field offset of the binding's ctypes structs equal
    the C compiler's, from include/hetlora.h."""
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "hetlora.h"', 'int main(void) {']
    for name in STRUCTS:
        cls = getattr(hl, name)
        lines.append(f'  printf("{name} %zu\\n", sizeof({name}));')
        for fname, _ in cls._fields_:
            lines.append(f'  printf("{name}.{fname} %zu\\n", offsetof({name}, {fname}));')
    lines += ['  return 0;', '}']
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(REPO, "include"), str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    got = dict(line.split() for line in out if line)
    for name in STRUCTS:
        cls = getattr(hl, name)
        assert int(got[name]) == ctypes.sizeof(cls), name
        for fname, _ in cls._fields_:
            assert int(got[f"{name}.{fname}"]) == getattr(cls, fname).offset, (name, fname)


def test_launch_group_rules_match_the_library(tmp_path):
    """The C rules (lv_launch_group, lv_group_member in variants.h) against
    the statement above: every variant's group and every group's members."""
    src = tmp_path / "groups.c"
    src.write_text('''#include <stdio.h>
#include "hetlora.h"
#include "variants.h"
int main(void) {
    for (int v = 0; v < LV_APPLY_VARIANTS; ++v) printf("g %d %d\\n", v, lv_launch_group(v));
    for (int key = 0; key < LV_APPLY_VARIANTS; ++key)
        for (int i = 0; i < 8 && lv_group_member(key, i) >= 0; ++i) printf("m %d %d\\n", key, lv_group_member(key, i));
    return 0;
}
''')
    exe = tmp_path / "groups"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(REPO, "include"), "-I",
                    os.path.join(REPO, "heterogeneous_adapter_batching_amd", "csrc"), str(src), "-o", str(exe)],
                   check=True)
    lines = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    groups = {int(v): int(g) for k, v, g in (l.split() for l in lines if l.startswith("g"))}
    assert groups == {v: launch_group(v) for v in range(FUSED + 1)}
    members = {}
    for k, key, v in (l.split() for l in lines if l.startswith("m")):
        members.setdefault(int(key), []).append(int(v))
    for key in set(groups.values()):
        assert members[key] == sorted(v for v in groups if groups[v] == key), key
