"""Offline tile search: the tile table's choices measured on the GPU.

VaLoRA blog, section 4.3.2 (profile-based optimal tiling search): the input
shapes an operator will see are profiled offline over the candidate tilings,
the space pruned by the on-chip memory limit and by 64/128 multiples, and the
best tiling of each shape is kept in a table that the operator looks up at run
time.  Here the table is ``csrc/tile_table.inc`` (keyed by segment-length
bucket, rank bucket and d bucket; see ``csrc/variants.h``), compiled into the
library, and this script writes it.

Candidates per bucket:

* shrink: the three shapes (4 waves splitting K over 16 rows; items of 64;
  items of 128 rows) x K slices 1, 2, 4, 8, 16, pruned to slices <= d_in/64
  (a slice is at least one 64-wide K block) -- every shape fits the 160 KiB
  LDS at every rank, so the LDS limit prunes nothing further;
* expand: the MFMA kernel with items of 16, 64 or 128 rows, and the VALU
  kernel for segments of at most 2 rows.

Every candidate is timed through ``lora_plan_table`` (the planner with a
caller's table) and the library as built, in two phases:

1. Workload shapes.  The batches the library is measured on -- one-token
   decode over 64 adapters (heterogeneous and one-adapter), the 16-request
   prefill, one vision layer, the 70B-class mixed batch and its one-adapter
   twin (same rows, the token-weighted mean rank) -- are built with
   their exact row maps, ranks and projection widths (random bf16 values drawn
   on the GPU: only shapes matter for time).  Each table bucket that one of
   their segments falls in is searched by coordinate descent from the current
   table: the bucket's candidates are tried in turn with the rest of the table
   fixed, each judged by the summed time of lora_apply, lora_shrink and
   lora_expand (over all projections, one call each, warm, median of
   ``--reps``) on the batches that touch the bucket.  Each pass first tries
   block moves: the buckets that share one launch (same op, d bucket, launch
   class and shape) set to one candidate at once, which a move of one
   bucket cannot reach when moving it alone would split that launch.  Judging a choice inside
   the whole batch, not alone, sees what a choice costs its neighbours: two
   buckets on different kernel shapes are separate launches, and each launch
   has its own tail.
2. Other buckets.  A bucket no batch above reaches is timed alone: a batch of
   segments of one length, rank and width inside it (8192 rows, 256 segments
   at most, one projection), cold (a 512 MB read evicts the Infinity Cache
   before each call), the op the bucket serves only.

In the workload phase a candidate replaces the current choice only when it is
faster by more than ``--min-gain`` (1%; block moves ``--min-gain-block``,
0.5%) and stays so when both are timed again; in the isolated phase, whose single-projection timings are noisier, when
it is faster by more than ``--min-gain-alone`` (3%).  Re-running on an
unchanged device then changes little by noise.  The descent repeats (at most
``--passes`` times) until a pass changes nothing.

Usage (from the repository root, on one MI355X, with the library built):

    python -m heterogeneous_adapter_batching_amd.tile_search \\
        [--reps 9] [--out heterogeneous_adapter_batching_amd/csrc/tile_table.inc] \\
        [--summary profiles/tile_search.md]

then rebuild the library (the table is compiled in).
"""
import argparse
import ctypes
import datetime
import os
import re
import sys
import time

import numpy as np
import torch

from . import (LORA_OP_APPLY, LORA_OP_EXPAND, LORA_OP_SHRINK, _lib, check_status, lora_apply_proj_t,
               lora_build_segments, lora_expand_proj_t, lora_launch_t, lora_plan_table, lora_rows_dense_offsets,
               lora_shrink_proj_t, make_rows)
from .session import HipEvent

HERE = os.path.dirname(os.path.abspath(__file__))
TABLE = os.path.join(HERE, "csrc", "tile_table.inc")

# a representative of each bucket (see lv_len_bucket, lv_rank_bucket, lv_d_bucket)
LEN_REP = [1, 3, 6, 12, 24, 48, 160, 1024]
RANK_REP = [16, 32, 64, 128]
D_IN_REP = [1024, 4096, 8192, 16384]      # shrink: d_in decides the bucket
D_OUT_REP = [1024, 4096, 8192, 28672]     # expand: d_out decides the bucket
LEN_NAMES = ["len 1     ", "len 2-4   ", "len 5-8   ", "len 9-16  ", "len 17-32 ", "len 33-64 ", "65-256    ",
             "257+      "]
ROWS_TARGET = 8192       # rows per timed batch of the isolated phase
MAX_SEGMENTS = 256
SHRINK_CAND = [(s, k) for s in (0, 1, 2) for k in (1, 2, 4, 8, 16)]
EXPAND_CAND = [0, 3, 1, 2, 4]   # items of 16, 32, 64, 128 rows; the VALU decode kernel
FUSED_MAX_D, FUSED_MAX_ROWRANK = 4096, 1024   # lv_fused: such segments never read the table in an apply plan
OPS = (LORA_OP_APPLY, LORA_OP_SHRINK, LORA_OP_EXPAND)
OP_NAMES = {LORA_OP_SHRINK: "shrink", LORA_OP_EXPAND: "expand", LORA_OP_APPLY: "apply"}


def len_bucket(n):
    return 0 if n <= 1 else 1 if n <= 4 else 2 if n <= 8 else 3 if n <= 16 else 4 if n <= 32 else 5 if n <= 64 \
        else 6 if n <= 256 else 7


def rank_bucket(r):
    return 0 if r <= 16 else 1 if r <= 32 else 2 if r <= 64 else 3


def d_bucket(d):
    return 0 if d <= 1024 else 1 if d <= 4096 else 2 if d <= 8192 else 3


def read_table(path=TABLE):
    """(shrink int8 [8][4][4][2] of (shape, slices), expand int8 [8][4][4]) from the table source."""
    src = open(path).read()
    s_part = src[src.index("kShrinkCfg"):src.index("kExpandShape")]
    e_part = src[src.index("kExpandShape"):]
    pairs = [(int(a), int(b)) for a, b in re.findall(r"S\((\d+),\s*(\d+)\)", s_part)]
    assert len(pairs) == 8 * 4 * 4, len(pairs)
    body = e_part[e_part.index("{"):]
    vals = [int(v) for v in re.findall(r"-?\d+", re.sub(r"/\*.*?\*/", "", body))]
    assert len(vals) == 8 * 4 * 4, len(vals)
    return np.array(pairs, np.int8).reshape(8, 4, 4, 2), np.array(vals, np.int8).reshape(8, 4, 4)


def write_table(shrink, expand, path, note):
    lines = ["// Tile-config table: per op, the kernel shape chosen for a segment by",
             "// (segment-length bucket, rank bucket, d bucket); for the shrink also the",
             "// number of K slices the reduction over d_in is split into (each slice is its",
             "// own workgroup, the expand adds the slices up).",
             "//   length buckets: 1, 2-4, 5-8, 9-16, 17-32, 33-64, 65-256, 257+",
             "//   rank buckets:   <=16, <=32, <=64, <=128",
             "//   d buckets (d_in for the shrink, d_out for the expand): <=1024, <=4096, <=8192, larger",
             "// Shrink shapes: 0 = 4 waves split K over 16 rows, 1 = 4 x 16 rows, 2 = 4 x 32 rows.",
             "// Expand shapes: 0/1/2/3 = MFMA work items of 16/64/128/32 rows, 4 = VALU",
             "// decode items of at most 2 rows.",
             "// " + note,
             "struct ShrinkCfg {",
             "    int8_t shape;",
             "    int8_t slices;",
             "};",
             "#define S(shape, slices) {shape, slices}",
             "#define ROWS_D(a, b, c, d) {a, b, c, d}",
             "static LV_TABLE_SPACE const ShrinkCfg kShrinkCfg[LV_LEN_BUCKETS][LV_RANK_BUCKETS][LV_D_BUCKETS] = {"]
    for l in range(8):
        rows = []
        for r in range(4):
            rows.append("ROWS_D(" + ", ".join("S(%d, %d)" % tuple(int(v) for v in shrink[l, r, d])
                                              for d in range(4)) + ")")
        lines.append("    /* %s*/ {%s, %s," % (LEN_NAMES[l], rows[0], rows[1]))
        lines.append("                     %s, %s}," % (rows[2], rows[3]))
    lines += ["};", "#undef S",
              "static LV_TABLE_SPACE const int8_t kExpandShape[LV_LEN_BUCKETS][LV_RANK_BUCKETS][LV_D_BUCKETS] = {"]
    for l in range(8):
        lines.append("    /* %s*/ {%s}," % (LEN_NAMES[l], ", ".join(
            "{" + ", ".join(str(int(expand[l, r, d])) for d in range(4)) + "}" for r in range(4))))
    lines += ["};", "#undef ROWS_D", ""]
    open(path, "w").write("\n".join(lines))


def _median_us(call, stream, reps, flush=None):
    ts = []
    for k in range(reps + 1):
        if flush is not None:
            flush.max()  # a read evicts the Infinity Cache without leaving dirty lines behind
        e0, e1 = HipEvent(timing=True), HipEvent(timing=True)
        e0.record(stream)
        call()
        e1.record(stream)
        e1.synchronize()
        if k > 0:
            ts.append(e0.elapsed_time(e1) * 1e3)
    return float(np.median(ts))


class Case:
    """One batch on the device: its row map and ranks, every projection's x,
    A and B (dense row tables), v and y; times lora_apply / lora_shrink /
    lora_expand over all projections under a given table."""

    def __init__(self, label, row_adapter, ranks, projs, seed, cold=False):
        self.label = label
        self.ra = np.ascontiguousarray(row_adapter, np.int32)
        self.ranks = np.ascontiguousarray(ranks, np.int32)
        self.segs = lora_build_segments(self.ra, self.ranks)
        self.n_rows = self.ra.shape[0]
        self.d_in = max(di for _, di, _ in projs)
        self.d_out = max(do for _, _, do in projs)
        self.max_rank = int(self.ranks.max())
        self.ldv = -(-self.max_rank // 4) * 4
        self.stream = torch.cuda.current_stream()
        g = torch.Generator(device="cuda").manual_seed(seed)
        n_act = max(1, self.segs.n_active)
        self.row_index = torch.from_numpy(np.ascontiguousarray(self.segs.row_index)).cuda()
        self._keep = [self.row_index]
        self.sp, self.ep, self.ap = [], [], []
        for _, d_in, d_out in projs:
            def rows(row_len):
                off, n = lora_rows_dense_offsets(self.ranks, self.max_rank, row_len, row_len)
                pool = (torch.randn(int(n), generator=g, device="cuda") * 0.05).to(torch.bfloat16)
                off_d = torch.from_numpy(off).cuda()
                self._keep += [pool, off_d]
                return make_rows(pool.data_ptr(), off_d.data_ptr(), self.ranks.shape[0], self.max_rank, row_len,
                                 row_len)
            A, B = rows(d_in), rows(d_out)
            x = torch.randn(self.n_rows, d_in, generator=g, device="cuda").to(torch.bfloat16)
            y = torch.zeros(self.n_rows, d_out, dtype=torch.float32, device="cuda")
            v = torch.zeros(16, n_act, self.ldv, dtype=torch.float32, device="cuda")   # any slice count
            self._keep += [x, y, v]
            self.sp.append(lora_shrink_proj_t(x.data_ptr(), d_in, d_in, A, v.data_ptr(), self.ldv))
            self.ep.append(lora_expand_proj_t(v.data_ptr(), self.ldv, B, d_out, y.data_ptr(), d_out, 1.0))
            self.ap.append(lora_apply_proj_t(x.data_ptr(), d_in, d_in, A, v.data_ptr(), self.ldv, B, d_out,
                                             y.data_ptr(), d_out, 1.0))
        n = len(projs)
        self.arr = {LORA_OP_SHRINK: (lora_shrink_proj_t * n)(*self.sp),
                    LORA_OP_EXPAND: (lora_expand_proj_t * n)(*self.ep),
                    LORA_OP_APPLY: (lora_apply_proj_t * n)(*self.ap)}
        self.fn = {LORA_OP_SHRINK: _lib.lora_shrink, LORA_OP_EXPAND: _lib.lora_expand, LORA_OP_APPLY: _lib.lora_apply}
        self.flush = torch.ones(128 << 20, dtype=torch.int32, device="cuda") if cold else None
        self.n_proj = n

    def buckets(self):
        """Table entries this batch's plans read: ('shrink', l, r, d_in bucket)
        and ('expand', l, r, d_out bucket)."""
        out = set()
        for a, b, rk in zip(self.segs.seg_start[:-1], self.segs.seg_start[1:], self.segs.seg_rank):
            ln, rk = int(b - a), int(rk)
            out.add(("shrink", len_bucket(ln), rank_bucket(rk), d_bucket(self.d_in)))
            out.add(("expand", len_bucket(ln), rank_bucket(rk), d_bucket(self.d_out)))
        return out

    def time(self, op, st_tab, ex_tab, reps):
        st, work, info = lora_plan_table(op, self.segs, self.d_in, self.d_out, st_tab, ex_tab, raw=True)
        check_status(st, "lora_plan_table")
        work_d = torch.from_numpy(np.ascontiguousarray(work)).cuda()
        L = lora_launch_t()
        L.row_index, L.work, L.info = self.row_index.data_ptr(), work_d.data_ptr(), info
        fn, arr, h = self.fn[op], self.arr[op], self.stream.cuda_stream

        def call():
            check_status(fn(ctypes.byref(L), self.n_proj, arr, h), OP_NAMES[op])
        return _median_us(call, self.stream, reps, self.flush)

    def total(self, st_tab, ex_tab, reps, ops=OPS):
        return {op: self.time(op, st_tab, ex_tab, reps) for op in ops}


def workload_cases():
    """The batches the library is measured on, from the seeded workload
    generators' structures (no tensors drawn on the host)."""
    import workloads
    cases = []
    S = workloads.structure(1)
    for key in ("hetero", "homo"):
        cases.append(("decode " + key, S.batches[key], S.adapter_rank, S.projs))
    for k, name in ((2, "prefill"), (3, "vision layer"), (4, "70B mix")):
        S = workloads.structure(k)
        cases.append((name, S.row_adapter, S.adapter_rank, S.projs))
    S = workloads.structure_twin(4)   # the 70B mix on one adapter of its mean rank
    cases.append(("70B twin", S.row_adapter, S.adapter_rank, S.projs))
    return cases


def search_workloads(cases, st_tab, ex_tab, reps, min_gain, log, report, pass_no):
    """One pass of coordinate descent over the buckets the cases touch."""
    touch = {}
    for c in cases:
        for bk in c.buckets():
            touch.setdefault(bk, []).append(c)
    order = sorted(touch, key=lambda b: (b[0] != "shrink", -b[1], b[2], b[3]))

    def cost(cs, st, ex):
        return sum(sum(c.total(st, ex, reps).values()) for c in cs)
    for bk in order:
        op, l, r, d = bk
        cs = touch[bk]
        cur = tuple(int(v) for v in st_tab[l, r, d]) if op == "shrink" else int(ex_tab[l, r, d])
        cands = SHRINK_CAND if op == "shrink" else EXPAND_CAND
        res = {}
        for cand in cands:
            st, ex = st_tab.copy(), ex_tab.copy()
            if op == "shrink":
                if cand[1] > D_IN_REP[d] // 64:
                    continue
                st[l, r, d] = cand
            else:
                if cand == 4 and l > 1:
                    continue
                ex[l, r, d] = cand
            res[cand] = (cost(cs, st, ex), st, ex)
        best = min(res, key=lambda k: res[k][0])
        t_cur = res[cur][0] if cur in res else float("inf")
        chosen = cur
        if best != cur and res[best][0] < (1 - min_gain) * t_cur:
            # confirm: both again, interleaved
            t2c = cost(cs, *res[cur][1:]) if cur in res else float("inf")
            t2b = cost(cs, *res[best][1:])
            if t2b < (1 - min_gain) * t2c:
                chosen = best
        if op == "shrink":
            st_tab[l, r, d] = chosen
        else:
            ex_tab[l, r, d] = chosen
        report.append((op, l, r, d, "pass %d: %s" % (pass_no, "+".join(c.label for c in cs)), cur, t_cur, chosen,
                       res[chosen][0]))
        log("pass %d: workloads %s bucket (%s, %s, %s) on %s: current %s %.1f us, chosen %s %.1f us (best %s %.1f)"
            % (pass_no, op, LEN_NAMES[l].strip(), RANK_REP[r], d, "+".join(c.label for c in cs), cur, t_cur, chosen,
               res[chosen][0], best, res[best][0]))
    return set(touch)


def _launch_class(op, r):
    """Rank buckets whose segments one launch runs together: the expand's
    rank classes (ranks <= 32 share the one-K-step kernel), the shrink's
    ranks <= 64 (one launch per shape) against rank 128."""
    if op == "expand":
        return 0 if r <= 1 else r - 1
    return 0 if r <= 2 else 1


def search_blocks(cases, st_tab, ex_tab, reps, min_gain, log, report, pass_no):
    """Block moves: the buckets the batches touch that now share one launch
    (same op, d bucket, launch class and shape) set to one candidate
    together.  One bucket at a time, the descent cannot move segments that
    share a launch to another shape without splitting that launch first,
    which costs more than the move gains; together they move as one launch.
    The groups are disjoint, so each is formed from the table as the pass
    found it."""
    touch = {}
    for c in cases:
        for bk in c.buckets():
            touch.setdefault(bk, []).append(c)
    groups = {}
    for op, l, r, d in touch:
        shape = int(st_tab[l, r, d][0]) if op == "shrink" else int(ex_tab[l, r, d])
        groups.setdefault((op, d, _launch_class(op, r), shape), []).append((op, l, r, d))

    def cost(cs, st, ex):
        return sum(sum(c.total(st, ex, reps).values()) for c in cs)
    for key in sorted(groups):
        bks = sorted(groups[key])
        if len(bks) < 2:
            continue
        op, d = key[0], key[1]
        cs = sorted({id(c): c for bk in bks for c in touch[bk]}.values(), key=lambda c: c.label)
        res = {"current": (cost(cs, st_tab, ex_tab), st_tab.copy(), ex_tab.copy())}
        for cand in (SHRINK_CAND if op == "shrink" else EXPAND_CAND):
            st, ex = st_tab.copy(), ex_tab.copy()
            if op == "shrink":
                if cand[1] > D_IN_REP[d] // 64:
                    continue
                for _, l, r, _ in bks:
                    st[l, r, d] = cand
            else:
                if cand == 4 and any(l > 1 for _, l, _, _ in bks):
                    continue
                for _, l, r, _ in bks:
                    ex[l, r, d] = cand
            if np.array_equal(st, st_tab) and np.array_equal(ex, ex_tab):
                continue
            res[cand] = (cost(cs, st, ex), st, ex)
        best = min(res, key=lambda k: res[k][0])
        t_cur = res["current"][0]
        chosen = "current"
        if best != "current" and res[best][0] < (1 - min_gain) * t_cur:
            t2c = cost(cs, *res["current"][1:])
            t2b = cost(cs, *res[best][1:])
            if t2b < (1 - min_gain) * t2c:
                chosen = best
        where = "block, pass %d: %s" % (pass_no, "+".join(c.label for c in cs))
        for _, l, r, _ in bks:
            cur = tuple(int(v) for v in st_tab[l, r, d]) if op == "shrink" else int(ex_tab[l, r, d])
            new = cur if chosen == "current" else chosen
            report.append((op, l, r, d, where, cur, t_cur, new, res[chosen][0]))
        if chosen != "current":
            st_tab[...] = res[chosen][1]
            ex_tab[...] = res[chosen][2]
        log("block %d: %s d %d class %d shape %d (%s) on %s: current %.1f us, chosen %s %.1f us (best %s %.1f)"
            % (pass_no, op, d, key[2], key[3], ", ".join("%s/%d" % (LEN_NAMES[l].strip(), RANK_REP[r]) for _, l, r, _ in bks),
               "+".join(c.label for c in cs), t_cur, chosen, res[chosen][0], best, res[best][0]))


def search_isolated(st_tab, ex_tab, skip, reps, min_gain, log, report):
    for l in range(8):
        for r in range(4):
            for d in range(4):
                L, R = LEN_REP[l], RANK_REP[r]
                n_seg = max(1, min(MAX_SEGMENTS, ROWS_TARGET // L))
                ra = np.repeat(np.arange(n_seg, dtype=np.int32), L)
                ranks = np.full(n_seg, R, np.int32)
                if ("shrink", l, r, d) not in skip:
                    c = Case("alone", ra, ranks, [("p", D_IN_REP[d], 1024)], seed=1000 + 16 * l + 4 * r + d,
                             cold=True)
                    res = {}
                    for cand in SHRINK_CAND:
                        if cand[1] > D_IN_REP[d] // 64:
                            continue
                        st = st_tab.copy()
                        st[l, r, d] = cand
                        res[cand] = c.time(LORA_OP_SHRINK, st, ex_tab, reps)
                    _pick(res, "shrink", l, r, d, tuple(int(v) for v in st_tab[l, r, d]), st_tab, min_gain, c.n_rows,
                          log, report)
                    del c
                if ("expand", l, r, d) not in skip:
                    c = Case("alone", ra, ranks, [("p", 1024, D_OUT_REP[d])], seed=2000 + 16 * l + 4 * r + d,
                             cold=True)
                    res = {}
                    for cand in EXPAND_CAND:
                        if cand == 4 and l > 1:
                            continue
                        st, ex = st_tab.copy(), ex_tab.copy()
                        st[l, r, 0] = (0, 1)   # one K slice: the expand alone
                        ex[l, r, d] = cand
                        res[cand] = c.time(LORA_OP_EXPAND, st, ex, reps)
                    _pick(res, "expand", l, r, d, int(ex_tab[l, r, d]), ex_tab, min_gain, c.n_rows, log, report)
                    del c
                torch.cuda.empty_cache()


def _pick(res, op, l, r, d, cur, tab, min_gain, rows, log, report):
    best = min(res, key=res.get)
    chosen = best if (cur not in res or res[best] < (1 - min_gain) * res[cur]) else cur
    tab[l, r, d] = chosen
    report.append((op, l, r, d, "alone, %d rows" % rows, cur, res.get(cur, float("nan")), chosen, res[chosen]))
    log("alone %s len %d rank %d d %d: current %s %.1f us, chosen %s %.1f us"
        % (op, LEN_REP[l], RANK_REP[r], (D_IN_REP if op == "shrink" else D_OUT_REP)[d], cur,
           res.get(cur, float("nan")), chosen, res[chosen]))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--reps", type=int, default=9)
    ap.add_argument("--min-gain", type=float, default=0.01)
    ap.add_argument("--min-gain-alone", type=float, default=0.03)
    ap.add_argument("--min-gain-block", type=float, default=0.005,
                    help="block moves are judged on sums over whole batches, steadier than one bucket's")
    ap.add_argument("--passes", type=int, default=3, help="coordinate-descent passes at most (stops when one "
                    "changes nothing)")
    ap.add_argument("--out", default=TABLE)
    ap.add_argument("--summary", default=None)
    ap.add_argument("--skip-isolated", action="store_true", help="search the workload buckets only")
    args = ap.parse_args()
    assert torch.cuda.is_available(), "the tile search times kernels on the GPU"
    t0 = time.time()

    def log(msg):
        print("[%4.0f s] %s" % (time.time() - t0, msg), flush=True)
    st0, ex0 = read_table()
    st_tab, ex_tab = st0.copy(), ex0.copy()
    cases = [Case(lbl, ra, rk, projs, seed=3000 + i) for i, (lbl, ra, rk, projs) in enumerate(workload_cases())]
    before = {c.label: c.total(st0, ex0, args.reps) for c in cases}
    log("workload batches built; before: " + "; ".join(
        "%s %s" % (k, ", ".join("%s %.1f" % (OP_NAMES[o], t) for o, t in v.items())) for k, v in before.items()))
    report = []
    for k in range(args.passes):
        before_pass = (st_tab.copy(), ex_tab.copy())
        search_blocks(cases, st_tab, ex_tab, args.reps, args.min_gain_block, log, report, k + 1)
        touched = search_workloads(cases, st_tab, ex_tab, args.reps, args.min_gain, log, report, k + 1)
        if np.array_equal(before_pass[0], st_tab) and np.array_equal(before_pass[1], ex_tab):
            break
    after = {c.label: c.total(st_tab, ex_tab, args.reps) for c in cases}
    again = {c.label: c.total(st0, ex0, args.reps) for c in cases}
    log("after: " + "; ".join(
        "%s %s" % (k, ", ".join("%s %.1f" % (OP_NAMES[o], t) for o, t in v.items())) for k, v in after.items()))
    del cases
    torch.cuda.empty_cache()
    if not args.skip_isolated:
        search_isolated(st_tab, ex_tab, touched, args.reps, args.min_gain_alone, log, report)
    dev = torch.cuda.get_device_properties(0).name
    note = ("Written by heterogeneous_adapter_batching_amd/tile_search.py on %s (%s): buckets the measured "
            "batches reach are chosen inside those batches, the others alone." % (dev, datetime.date.today()))
    write_table(st_tab, ex_tab, args.out, note)
    log("wrote " + args.out)
    if args.summary:
        _summary(args, dev, before, after, again, report)
        log("wrote " + args.summary)


def _summary(args, dev, before, after, again, report):
    with open(args.summary, "w") as f:
        f.write("# Tile search: the tile table's buckets, timed\n\n")
        f.write("Command (from the repository root, on one MI355X, library built with the table before the "
                "search):\n\n")
        f.write("    python -m heterogeneous_adapter_batching_amd.tile_search %s\n\n" % " ".join(sys.argv[1:]))
        f.write("Device: %s.  Median of %d calls per timing; a choice changes only when faster by more than "
                "%.0f%% twice (buckets timed in the batches; %.1f%% for block moves) or %.0f%% (buckets timed "
                "alone).\n\n" % (dev, args.reps, 100 * args.min_gain, 100 * args.min_gain_block,
                                   100 * args.min_gain_alone))
        f.write("## Measured batches, whole (us per call over all projections, warm)\n\n")
        f.write("| batch | op | table before | table after | table before, timed again at the end |\n"
                "|---|---|---|---|---|\n")
        for k in before:
            for o in OPS:
                f.write("| %s | %s | %.1f | %.1f | %.1f |\n" % (k, OP_NAMES[o], before[k][o], after[k][o], again[k][o]))
        f.write("\n## Buckets\n\n`where`: the descent pass and the batches a bucket was judged on (sum of apply + shrink + "
                "expand over them; `block`: the bucket moved together with the others of its launch, the times are the "
                "block's), or `alone` (the op alone on a batch of that bucket's segments, cold).  Shrink entries are "
                "(shape, K slices); expand entries the shape.\n\n")
        f.write("| op | length | rank | d | where | current | us | chosen | us |\n|---|---|---|---|---|---|---|---|---|\n")
        for op, l, r, d, where, cur, t_cur, chosen, t_ch in report:
            f.write("| %s | %s | %d | %d | %s | %s | %.1f | %s | %.1f |\n"
                    % (op, LEN_NAMES[l].strip(), RANK_REP[r], (D_IN_REP if op == "shrink" else D_OUT_REP)[d], where,
                       cur, t_cur, chosen, t_ch))


if __name__ == "__main__":
    sys.exit(main())
