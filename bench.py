#!/usr/bin/env python3
"""Benchmark of the heterogeneous LoRA hot path on one MI355X.

The benchmark line (default, `--workload mix70b`): the 70B-shaped paged mix,
the largest configuration.  One step = one pass of the whole path over one
batch of 8,448 rows (256 decode rows, 128 of them released; 8 prefill
segments of 1024 rows) on q/o (8192 -> 8192) and up (8192 -> 28672), with
128 adapters of ranks 16/32/64 held in a pool of 8192-element pages under a
random page table: the host builds the segment table and the apply plan and
copies them to the device (lora_batch_prepare), then lora_apply runs the
shrink and expand over the active rows.  Steps alternate between two device
copies of the inputs (same values, other addresses), so every step streams
from HBM.  `value` is the step's algorithmic bytes (x rows, each distinct
adapter's A and B rows once, v written and read, y read and written in fp32)
over the wall-clock time per step.  lora_apply is issued in pieces split at
its launch boundaries (all shrink ranges, then each expand range, then the
fused range: the launches lora_apply makes, in its order), so that the
timed steps can hold one pair of HIP events around the dominant launch:
`roofline` describes it.  The same line carries the vision workload's mode
switch (merge, then unmerge, of its rank-64 adapter into 32 layers x q/k/v/o
W[4096x4096], each phase cold) as `merge_us_per_layer`, the ratio against
the homogeneous twin, a per-piece table, and `cpu_baseline`: the CPU oracle
timed on a bounded sample of the same work and checked against the GPU's
results.  All events are recorded without the system-scope fence: a default
event writes back and invalidates the GPU caches when it completes, which
idles the GPU between the kernels it separates.

`--workload decode`: the decode configuration, a Llama-7B-shaped layer of 64
one-token rows at d 4096 (q/k/v/o, rank 16).  One step: the fully
heterogeneous batch (64 adapters) and the homogeneous batch (1 adapter)
through lora_apply, then merge and unmerge of adapter 0 into the layer's four
W[4096x4096]; steps rotate over 8 layer copies (cold Infinity Cache).  With
--path split it calls lora_shrink and lora_expand instead; with --metadata
device both batches are built on the GPU (lora_batch_build_device).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
       python bench.py --workload decode [--layers L] [--path apply|split] [--metadata host|inline|device]
       python bench.py --workload tiny|prefill|vision|mixture|swap|heads
                       (the other workloads; swap: adapter pool; heads: per-adapter vision task heads)
       python bench.py --workload prefill|vision --shared-x           (the same with q/k/v reading one x)
       python bench.py --workload prefill|vision|mix70b --twin        (shrink/expand tables and the twin ratio)
       python bench.py --workload prefill|vision|mix70b --metadata device  (apply: host- vs device-built plan)
       python bench.py --copy-calibration                             (counter calibration under rocprofv3)
       python bench.py --flush-study                                  (kernel times after a write or a read cache flush, and in a step)
       python bench.py --traffic-record PMC_DIR --traffic-grid N      (write the dominant launch's traffic record)
       python bench.py --rmw-ceiling                                  (in-place streaming rate of this HBM)
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
METRIC = "hetero-LoRA shrink+expand µs, GB/s & TFLOP/s vs roofline; merge µs/layer"


class ColdCache:
    """Evicts the 256 MB Infinity Cache before a cold timing by reading a
    512 MB buffer (one reduction over it).  A write-based flush (a fill)
    would leave the cache full of dirty lines, and the kernel timed next
    would pay their write-back on its own reads: the prefill shrink takes
    ~116 us after a 1 GiB fill against ~67 us after a 1 GiB read
    (`--flush-study`)."""

    def __init__(self, device="cuda"):
        import torch
        self.buf = torch.ones(128 << 20, dtype=torch.int32, device=device)

    def __call__(self):
        self.sink = self.buf.max()


def flush_study():
    """The prefill workload's lora_shrink (9,436 rows, q/k/v/o at d 4096:
    326 MB of algorithmic bytes) timed after three cache states: after a
    1 GiB fill (the Infinity Cache left full of dirty lines), after a 1 GiB
    read (evicted, clean), and right after the batch's own lora_expand (y
    just written: the state a step leaves behind); and the decode layer's
    heterogeneous lora_apply (the fused kernel) after the first two; and
    every launch of the 70B mix's lora_apply, alone after a 1 GiB read and
    inside a step that follows a whole step."""
    import torch
    import workloads
    from heterogeneous_adapter_batching_amd.session import Batch, HipEvent, Rows
    from workloads.device import to_device
    W = workloads.gen_config(2)
    dw = to_device(W)
    d_in = max(p.d_in for p in W.projections)
    d_out = max(p.d_out for p in W.projections)
    b = Batch(W.n_rows, W.adapter_rank, d_in, d_out).refresh(W.row_adapter)
    ldv = -(-int(W.adapter_rank.max()) // 4) * 4
    A = [Rows(dw.pool, d.A_off, p.A.n_adapters, p.A.max_rank, p.A.row_len, p.A.chunk_len)
         for p, d in zip(W.projections, dw.projections)]
    B = [Rows(dw.pool, d.B_off, p.B.n_adapters, p.B.max_rank, p.B.row_len, p.B.chunk_len)
         for p, d in zip(W.projections, dw.projections)]
    v = [b.new_v(ldv) for _ in W.projections]
    do_s = b.prepare_shrink([(d.x, A[i], v[i]) for i, d in enumerate(dw.projections)])
    do_e = b.prepare_expand([(v[i], B[i], d.y, W.scale) for i, d in enumerate(dw.projections)])
    nbytes = delta_cost(W, W.row_adapter)["shrink_bytes"]
    big = torch.ones(256 << 20, dtype=torch.int32, device="cuda")
    out = {}
    for name in ("after a 1 GiB fill", "after a 1 GiB read", "after its own expand"):
        ts = []
        for rep in range(12):
            if name == "after a 1 GiB fill":
                big.fill_(rep)
            elif name == "after a 1 GiB read":
                big.max()
            else:
                do_e()
            e0, e1 = HipEvent(timing=True), HipEvent(timing=True)
            e0.record()
            do_s()
            e1.record()
            e1.synchronize()
            if rep >= 2:
                ts.append(e0.elapsed_time(e1) * 1e3)
        us = float(np.median(ts))
        out[name] = {"us_median": round(us, 2), "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    # the decode layer's heterogeneous batch: one fused lora_apply (77.6 MB)
    Wd = workloads.gen_config(1)
    dd = to_device(Wd)
    ra = Wd.batches["hetero"]
    bd = Batch(Wd.n_rows, Wd.adapter_rank, 4096, 4096, inline=True).refresh(ra)
    ldvd = -(-int(Wd.adapter_rank.max()) // 4) * 4
    do_a = bd.prepare_apply([(d.x, Rows(dd.pool, d.A_off, p.A.n_adapters, p.A.max_rank, p.A.row_len, p.A.chunk_len),
                              bd.new_v(ldvd), Rows(dd.pool, d.B_off, p.B.n_adapters, p.B.max_rank, p.B.row_len,
                                                    p.B.chunk_len), d.y, Wd.scale)
                             for p, d in zip(Wd.projections, dd.projections)])
    nd = delta_cost(Wd, ra)
    nd = nd["shrink_bytes"] + nd["expand_bytes"]
    dec = {}
    for name in ("after a 1 GiB fill", "after a 1 GiB read"):
        ts = []
        for rep in range(12):
            if name == "after a 1 GiB fill":
                big.fill_(rep)
            else:
                big.max()
            e0, e1 = HipEvent(timing=True), HipEvent(timing=True)
            e0.record()
            do_a()
            e1.record()
            e1.synchronize()
            if rep >= 2:
                ts.append(e0.elapsed_time(e1) * 1e3)
        us = float(np.median(ts))
        dec[name] = {"us_median": round(us, 2), "hbm_frac": round(nd / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    del dd, bd, do_a, dw, b, do_s, do_e
    # the 70B mix's lora_apply split at its launch boundaries: each piece
    # alone after a 1 GiB read, and the same pieces in a step that follows a
    # whole step (the state the bench line's steps run in)
    Wm = workloads.gen_config(4)
    dm = to_device(Wm)
    bm = Batch(Wm.n_rows, Wm.adapter_rank, max(p.d_in for p in Wm.projections),
               max(p.d_out for p in Wm.projections), inline=True).refresh(Wm.row_adapter)
    ldvm = -(-int(Wm.adapter_rank.max()) // 4) * 4
    pm = apply_pieces(bm, [(d.x, Rows(dm.pool, d.A_off, p.A.n_adapters, p.A.max_rank, p.A.row_len, p.A.chunk_len),
                            bm.new_v(ldvm), Rows(dm.pool, d.B_off, p.B.n_adapters, p.B.max_rank, p.B.row_len,
                                                  p.B.chunk_len), d.y, Wm.scale)
                           for p, d in zip(Wm.projections, dm.projections)])
    clean = {i: [] for i in range(len(pm))}
    stepped = {i: [] for i in range(len(pm))}
    for rep in range(12):
        for i, (_, _, fn, _) in enumerate(pm):
            big.max()
            e0, e1 = HipEvent(timing=True), HipEvent(timing=True)
            e0.record(); fn(); e1.record()
            e1.synchronize()
            if rep >= 2:
                clean[i].append(e0.elapsed_time(e1) * 1e3)
        ev = [HipEvent(timing=True) for _ in range(len(pm) + 1)]
        for _, _, fn, _ in pm:
            fn()
        for i, (_, _, fn, _) in enumerate(pm):
            ev[i].record(); fn()
        ev[len(pm)].record()
        ev[-1].synchronize()
        if rep >= 2:
            for i in range(len(pm)):
                stepped[i].append(ev[i].elapsed_time(ev[i + 1]) * 1e3)
    mix = {}
    for i, (name, _, _, items) in enumerate(pm):
        parts = ("shrink",) if name == "shrink" else ("expand",)
        nb, _ = piece_cost(Wm, items, parts)
        c_us, s_us = float(np.median(clean[i])), float(np.median(stepped[i]))
        mix["%s (%d items)" % (name, items.shape[0])] = {
            "alg_MB": round(nb / 1e6, 1),
            "after a 1 GiB read": {"us_median": round(c_us, 2), "hbm_frac": round(nb / c_us / 1e3 / HBM_PEAK_GBS, 4)},
            "in a step after a step": {"us_median": round(s_us, 2), "hbm_frac": round(nb / s_us / 1e3 / HBM_PEAK_GBS, 4)}}
    print(json.dumps({"study": "a kernel's time after three cache states",
                      "prefill lora_shrink (326 MB)": out,
                      "decode heterogeneous lora_apply, fused (%.1f MB)" % (nd / 1e6): dec,
                      "70B mix lora_apply, launch by launch": mix}), flush=True)


KERNELS_SRC = os.path.join(ROOT, "heterogeneous_adapter_batching_amd", "csrc", "kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "merge_kernel_traffic.json")
SECTION = "// " + "-" * 66 + " "


def merge_source_digest():
    """sha256 of the merge kernel's device code (its section of kernels.hip)."""
    src = open(KERNELS_SRC).read()
    a = src.index(SECTION + "merge\n")
    b = src.index(SECTION + "host side\n")
    return hashlib.sha256(src[a:b].encode()).hexdigest()


def merge_traffic():
    """HBM bytes per merge launch from the committed rocprofv3 counters:
    FETCH_SIZE and WRITE_SIZE (KiB per dispatch, one pass each) of the merge
    kernel, each scaled by copy_bytes / (the same counter's KiB for one plain
    copy of copy_bytes).  None when the record is missing or was taken on a
    different version of the merge kernel's source."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("merge_source_sha256") != merge_source_digest():
        return None
    c = rec["copy"]
    f_fetch = c["bytes"] / (c["fetch_kib"] * 1024.0)
    f_write = c["bytes"] / (c["write_kib"] * 1024.0)
    return round(rec["merge"]["fetch_kib"] * 1024.0 * f_fetch + rec["merge"]["write_kib"] * 1024.0 * f_write)


def copy_calibration():
    """One plain device-to-device copy of 1 GiB (after a warm-up copy), for
    calibrating the FETCH_SIZE / WRITE_SIZE counters under rocprofv3 --pmc."""
    import torch
    n = 1 << 30
    src = torch.full((n,), 1, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n}), flush=True)


def rmw_ceiling(reps=24):
    """The rate at which this device streams an in-place read-modify-write,
    with a plain library kernel (torch's elementwise add), launches back to
    back: (1) of the merge's size (4 x W[4096x4096] bf16 = 128 MiB read and
    written), rotating over 4 such buffers so that the reads find nothing in
    the Infinity Cache; its writes (128 MiB) still fit in that cache, and part
    of their write-back falls to the next launch.  (2) sustained: fp32
    buffers of 2.95 GB (the 70B step's y rows twice over), rotating over 2,
    where every launch pays for its own writes except the last ~256 MB."""
    import torch
    from heterogeneous_adapter_batching_amd.session import HipEvent
    out = {}
    for name, n, dtype, nbuf, k_reps in (("merge-sized", 4 * 4096 * 4096, torch.bfloat16, 4, reps),
                                         ("sustained", 16384 * 45056, torch.float32, 2, 8)):
        bufs = [torch.zeros(n, dtype=dtype, device="cuda") for _ in range(nbuf)]
        for k in range(2 * nbuf):
            bufs[k % nbuf].add_(1.0)
        torch.cuda.synchronize()
        ev = [HipEvent(timing=True) for _ in range(k_reps + 1)]
        for k in range(k_reps):
            ev[k].record()
            bufs[k % nbuf].add_(1.0)
        ev[k_reps].record()
        torch.cuda.synchronize()
        us = float(np.median([ev[k].elapsed_time(ev[k + 1]) * 1e3 for k in range(k_reps)]))
        nbytes = 2 * n * bufs[0].element_size()
        out[name] = {"rmw_bytes": nbytes, "us_median": round(us, 2), "GB_s": round(nbytes / (us * 1e-6) / 1e9, 1),
                     "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        del bufs
    print(json.dumps(out), flush=True)


def delta_cost(W, row_adapter):
    """Algorithmic bytes/flops of shrink and expand for every projection of W."""
    ra = np.asarray(row_adapter)
    act = ra[ra >= 0]
    distinct = np.unique(act)
    r_act = W.adapter_rank[act].astype(np.int64)
    r_dis = W.adapter_rank[distinct].astype(np.int64)
    cost = {"shrink_bytes": 0, "expand_bytes": 0, "flops": 0}
    seen_x = set()  # projections that share one x read it once
    for p in W.projections:
        x_bytes = 0 if id(p.x) in seen_x else act.size * p.d_in * 2
        seen_x.add(id(p.x))
        cost["shrink_bytes"] += x_bytes + int(r_dis.sum()) * p.d_in * 2 + int(r_act.sum()) * 4
        cost["expand_bytes"] += int(r_act.sum()) * 4 + int(r_dis.sum()) * p.d_out * 2 + act.size * p.d_out * 8
        cost["flops"] += int(2 * r_act.sum() * (p.d_in + p.d_out))
    return cost


def merge_cost(d_out, d_in, r, n):
    return {"bytes": n * (4 * d_out * d_in + r * (d_in + d_out) * 2), "flops": n * 2 * r * d_out * d_in}


def cpu_baseline(W, batches, merge_ws, gpu=None, min_seconds=10.0, max_seconds=30.0):
    """The oracle as it stands, on a bounded sample of the same workload: work
    units (the oracle delta for all rows and projections of one batch, or the
    oracle merge + unmerge of one of the layer's W) are run in turn until at
    least `min_seconds` have passed and every unit has run once; the rate is
    the units' algorithmic bytes over the elapsed time.  `gpu` holds the GPU
    results of the same units (y per batch and projection from y0, merged W
    bits), which each unit's first oracle result is compared with (the
    comparison's own time is left out of the rate): the returned `parity`
    reports the delta's relative Frobenius and max abs error against the
    4e-3 / 2e-2 bounds, and for the merge the fraction of bits identical to
    the oracle's and the worst error against the exact W + s*B^T A over its
    bound (half a bf16 ulp plus the fp32 accumulation allowance; <= 1 is
    within)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    p0 = W.projections[0]
    r = int(W.adapter_rank[W.merge.adapter])

    parity = {"delta_relF_max": 0.0, "delta_abs_max": 0.0, "merge_equal_fraction_min": 1.0,
              "merge_worst_over_bound": 0.0, "checked": []}
    check_s = [0.0]

    def delta_unit(name, ra):
        def run():
            for pi, p in enumerate(W.projections):
                yrows, _ = oracle.apply_ref(ra, W.adapter_rank, p.x, p.y0, W.pool, p.A, p.B, W.scale)
                if gpu is not None and (name, pi) not in parity["checked"]:
                    t_check = time.perf_counter()
                    yref = np.stack([yrows[i] for i in range(len(ra))])
                    yg = gpu["delta"][name][pi].astype(np.float64)
                    d_ref, d_gpu = yref - p.y0, yg - p.y0
                    relf = float(np.linalg.norm(d_gpu - d_ref) / max(np.linalg.norm(d_ref), 1e-300))
                    parity["delta_relF_max"] = max(parity["delta_relF_max"], relf)
                    parity["delta_abs_max"] = max(parity["delta_abs_max"], float(np.max(np.abs(yg - yref))))
                    parity["checked"].append((name, pi))
                    check_s[0] += time.perf_counter() - t_check
            c = delta_cost(W, ra)
            return c["shrink_bytes"] + c["expand_bytes"], "delta"
        return run

    def merge_unit(i):
        def run():
            p = W.projections[W.merge.projs[i]]
            wm = oracle.merge_ref(merge_ws[i], W.pool, p.A, p.B, W.merge.adapter, r, W.scale)
            if gpu is not None and ("merge", i) not in parity["checked"] and i < len(gpu["merge"]):
                t_check = time.perf_counter()
                a, b = np.asarray(wm, np.uint16), gpu["merge"][i]
                parity["merge_equal_fraction_min"] = min(parity["merge_equal_fraction_min"], float(np.mean(a == b)))
                Aa = oracle.gather_rows_ref(W.pool, p.A.row_off, p.A.max_rank, p.A.row_len, p.A.chunk_len,
                                            W.merge.adapter, r)
                Ba = oracle.gather_rows_ref(W.pool, p.B.row_off, p.B.max_rank, p.B.row_len, p.B.chunk_len,
                                            W.merge.adapter, r)
                exact = oracle.bf16_to_f64(merge_ws[i]) + W.scale * (Ba.T @ Aa)
                got = oracle.bf16_to_f64(b)
                ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(got), 2.0 ** -126))) - 7)
                bound = (0.5 * ulp + (r + 4) * 2.0 ** -23 * abs(W.scale) * (np.abs(Ba).T @ np.abs(Aa)) +
                         2.0 ** -23 * np.abs(exact))
                parity["merge_worst_over_bound"] = max(parity["merge_worst_over_bound"],
                                                       float(np.max(np.abs(got - exact) / bound)))
                parity["checked"].append(("merge", i))
                check_s[0] += time.perf_counter() - t_check
            oracle.unmerge_ref(wm, W.pool, p.A, p.B, W.merge.adapter, r, W.scale)
            return 2 * merge_cost(p.d_out, p.d_in, r, 1)["bytes"], "merge"
        return run

    units = [delta_unit(n, ra) for n, ra in batches.items()] + [merge_unit(i) for i in range(len(merge_ws))]
    t0 = time.perf_counter()
    nbytes, done, k = 0, {"delta": 0, "merge": 0}, 0
    while True:
        b, kind = units[k % len(units)]()
        nbytes += b
        done[kind] += 1
        k += 1
        dt = time.perf_counter() - t0 - check_s[0]
        if (k >= len(units) and dt >= min_seconds) or dt >= max_seconds:
            break
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": int(cores), "kind": "oracle",
            "sample": "%d oracle delta passes (all 64 rows x q/k/v/o of the hetero or homo batch) and %d oracle "
                      "merge+unmerge passes of one W[4096x4096], run in turn for %.1f s"
                      % (done["delta"], done["merge"], dt),
            "seconds": round(dt, 3), "cpu_model": _cpu_model(),
            "parity": None if gpu is None else dict(
                parity, checked=len(parity["checked"]),
                within_bounds=bool(parity["delta_relF_max"] <= 4e-3 and parity["delta_abs_max"] <= 2e-2 and
                                   parity["merge_worst_over_bound"] <= 1.0))}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--layers", type=int, default=8, help="layer copies the steps rotate over")
    ap.add_argument("--workload", default="mix70b", choices=["decode", "tiny", "prefill", "vision", "mix70b",
                                                             "mixture", "swap", "heads"],
                    help="mix70b (default) is the benchmark line (with the vision mode switch); decode is the "
                         "decode layer's line; the others time shrink+expand of that workload for the kernel "
                         "tables")
    ap.add_argument("--path", default="apply", choices=["apply", "split"],
                    help="apply (default): lora_apply, one-row segments fused; split: lora_shrink then lora_expand")
    ap.add_argument("--metadata", default="inline", choices=["host", "inline", "device"],
                    help="decode: inline (default) prepares each batch with lora_batch_prepare on the host and "
                         "passes the small all-fused plan in the kernel's launch arguments (no copy; with "
                         "--path split, whose plans are not all fused, the plans are copied as with host); host "
                         "copies the prepared metadata to the device instead; device builds it on the GPU (lora_batch_build_device) "
                         "from device-resident row maps")
    ap.add_argument("--twin", action="store_true",
                    help="with --workload prefill|vision|mix70b: also time the homogeneous twin (the same rows on one "
                         "adapter of the token-weighted mean rank) and report the heterogeneous / homogeneous ratio")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--shared-x", action="store_true",
                    help="with --workload prefill|vision: q, k and v take one x (the layer input), o its own")
    ap.add_argument("--flush-study", action="store_true",
                    help="time the prefill shrink after a write-based and a read-based cache flush and after its "
                         "own expand, then exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one 1 GiB device copy (counter calibration under rocprofv3 --pmc) and exit")
    ap.add_argument("--rmw-ceiling", action="store_true",
                    help="time a plain in-place read-modify-write stream of the merge's size (cold) and exit")
    ap.add_argument("--traffic-record", default=None, metavar="PMC_DIR",
                    help="(no GPU) write the dominant launch's traffic record from the --pmc runs under PMC_DIR")
    ap.add_argument("--traffic-kernel", default="expand_kernel<1>")
    ap.add_argument("--traffic-grid", type=int, default=0, help="workgroups of the recorded launch")
    args = ap.parse_args()
    if args.traffic_record:
        return traffic_record(args)
    if args.flush_study:
        return flush_study()
    if args.copy_calibration:
        return copy_calibration()
    if args.rmw_ceiling:
        return rmw_ceiling()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this path is single-GPU by design (no sharding, no collectives); "
              "run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.workload == "mixture":
        return mixture_workload(args)
    if args.workload == "swap":
        return swap_workload(args)
    if args.workload == "heads":
        return heads_workload(args)
    if args.workload == "mix70b" and not (args.twin or args.metadata == "device"):
        return headline(args)
    if args.workload != "decode":
        return other_workload(args)
    return decode_workload(args)


def decode_workload(args):
    """The decode configuration's line (see the module docstring's last
    paragraph)."""
    import torch
    import workloads
    from heterogeneous_adapter_batching_amd.session import Batch, DeviceBatch, HipEvent, Rows, prepare_merge
    from workloads.device import bits_to_device, to_device

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    layers = []
    for l in range(max(1, args.layers)):
        Wl = workloads.gen_config(1, seed=1 + 1000 * l)   # layer 0 = the seeded decode instance
        dwl = to_device(Wl)
        rows = lambda desc, off: Rows(dwl.pool, off, desc.n_adapters, desc.max_rank, desc.row_len, desc.chunk_len)
        A = [rows(p.A, d.A_off) for p, d in zip(Wl.projections, dwl.projections)]
        B = [rows(p.B, d.B_off) for p, d in zip(Wl.projections, dwl.projections)]
        mh = [Wl.merge.weight(0, i) for i in Wl.merge.projs]
        Wt = [bits_to_device(w) for w in mh]
        layers.append(dict(W=Wl, dw=dwl, A=A, B=B, Wt=Wt, merge_host=mh))
    W = layers[0]["W"]
    het, homo = W.batches["hetero"], W.batches["homo"]
    r_m = int(W.adapter_rank[W.merge.adapter])
    ldv = 16
    stream = torch.cuda.current_stream()
    on_device = args.metadata == "device"
    if on_device:
        assert args.path == "apply", "device-built plans are apply plans"
        rk_d = torch.from_numpy(np.asarray(W.adapter_rank, np.int32)).to(dev)
        het_d = torch.from_numpy(np.asarray(het, np.int32)).to(dev)
        homo_d = torch.from_numpy(np.asarray(homo, np.int32)).to(dev)
        max_rank = int(W.adapter_rank.max())
        bh = DeviceBatch(64, len(W.adapter_rank), max_rank, 4096, 4096).build(het_d, rk_d)
        bo = DeviceBatch(64, len(W.adapter_rank), max_rank, 4096, 4096).build(homo_d, rk_d)
    else:
        # inline plans are apply plans: the split path copies its plans
        inline = args.metadata == "inline" and args.path == "apply"
        bh = Batch(64, W.adapter_rank, 4096, 4096, inline=inline).refresh(het)
        bo = Batch(64, W.adapter_rank, 4096, 4096, inline=inline).refresh(homo)
        # both decode plans are all fused and small: they must travel inline
        assert not inline or not (bh.apply_launch.work or bo.apply_launch.work), "plan did not go inline"
    vs = {id(b): [b.new_v(ldv) for _ in W.projections] for b in (bh, bo)}
    split = args.path == "split"
    for L in layers:
        L["calls"] = []
        for b in (bh, bo):
            v = vs[id(b)]
            pr = L["dw"].projections
            if split:
                L["calls"].append((b.prepare_shrink([(d.x, L["A"][i], v[i]) for i, d in enumerate(pr)]),
                                   b.prepare_expand([(v[i], L["B"][i], d.y, W.scale) for i, d in enumerate(pr)])))
            else:
                L["calls"].append((b.prepare_apply([(d.x, L["A"][i], v[i], L["B"][i], d.y, W.scale)
                                                    for i, d in enumerate(pr)]),))
        mats = [(L["Wt"][i], L["A"][i], L["B"][i], W.merge.adapter, r_m, W.scale) for i in range(len(L["Wt"]))]
        L["merge"], L["unmerge"] = prepare_merge(mats), prepare_merge(mats, unmerge=True)
    merge_host = layers[0]["merge_host"]
    n_mats = len(layers[0]["Wt"])

    # merge and unmerge run back to back between one pair of events (the same
    # kernel twice: the per-launch figure is half the pair, and an event pair
    # per launch would add its dispatch gap to each)
    if split:
        groups = ["hetero_shrink", "hetero_expand", "homo_shrink", "homo_expand", "merge_unmerge"]
    else:
        groups = ["hetero_apply", "homo_apply", "merge_unmerge"]
    if on_device:
        groups = ["metadata"] + groups
        build_h, build_o = bh.prepare_build(het_d, rk_d, stream), bo.prepare_build(homo_d, rk_d, stream)

    # One step, two ways.  Timed steps record one event pair, around the
    # merge and unmerge (the roofline kernel): nothing else is added to the
    # timed region.  Profiled steps (after the timed ones, untimed) record an
    # event between every group: group g runs between events g and g + 1.
    # Host metadata: both batches are prepared (host plan + metadata upload)
    # before the first group; device metadata: both builder kernels are the
    # first group.
    def step(ev, k, every_group):
        L = layers[k % len(layers)]
        g = 0
        if on_device:
            if every_group:
                ev[0].record(stream)
            build_h()
            build_o()
            g = 1
        else:
            bh.refresh(het, stream)
            bo.refresh(homo, stream)
        if every_group:
            ev[g].record(stream)
        for fns in L["calls"]:
            for fn in fns:
                fn()
                g += 1
                if every_group:
                    ev[g].record(stream)
        if not every_group:
            ev[0].record(stream)
        L["merge"]()
        L["unmerge"]()
        ev[g + 1 if every_group else 1].record(stream)

    def new_events(n):
        return [HipEvent(timing=True) for _ in range(n)]

    # the GPU results the CPU baseline leg checks against the oracle: layer 0's
    # batches from y0 and its merged W (both restored afterwards)
    gpu_results = None
    if not args.no_cpu_baseline:
        L0 = layers[0]
        gpu_results = {"delta": {}, "merge": []}
        for name, fns in zip(("hetero", "homo"), L0["calls"]):
            for p, d in zip(W.projections, L0["dw"].projections):
                d.y.copy_(torch.from_numpy(p.y0))
            for fn in fns:
                fn()
            torch.cuda.synchronize()
            gpu_results["delta"][name] = [d.y.cpu().numpy() for d in L0["dw"].projections]
        for p, d in zip(W.projections, L0["dw"].projections):
            d.y.copy_(torch.from_numpy(p.y0))
        L0["merge"]()
        torch.cuda.synchronize()
        gpu_results["merge"] = [w.cpu().numpy().view(np.uint16).copy() for w in L0["Wt"]]
        for w, h in zip(L0["Wt"], L0["merge_host"]):
            w.copy_(torch.from_numpy(np.ascontiguousarray(h).view(np.int16)))
        torch.cuda.synchronize()

    for k in range(args.warmup):
        step(new_events(2), k, False)
    torch.cuda.synchronize()
    evs = [new_events(2) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k], args.warmup + k, False)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    merge_pair_us = [ev[0].elapsed_time(ev[1]) * 1e3 for ev in evs]

    pevs = [new_events(len(groups) + 1) for _ in range(args.steps)]
    for k in range(args.steps):
        step(pevs[k], args.warmup + args.steps + k, True)
    torch.cuda.synchronize()

    # the two batches' calls alone, back to back over the layer copies (no
    # mode switch between them, as in a run of decode steps): each call then
    # follows the other batch's, not an unmerge's 128 MB of fresh W writes
    loop_us = None
    if not on_device:
        n_calls = len(layers[0]["calls"][0]) + len(layers[0]["calls"][1])
        lev = [new_events(n_calls + 1) for _ in range(args.steps + args.warmup)]
        for k, ev in enumerate(lev):
            L = layers[k % len(layers)]
            bh.refresh(het, stream)
            bo.refresh(homo, stream)
            g = 0
            ev[0].record(stream)
            for fns in L["calls"]:
                for fn in fns:
                    fn()
                    g += 1
                    ev[g].record(stream)
        torch.cuda.synchronize()
        loop_us = [[ev[i].elapsed_time(ev[i + 1]) * 1e3 for ev in lev[args.warmup:]] for i in range(n_calls)]

    # launch floor: one near-empty kernel (a 1-element fill) between the same
    # kind of events, on the same stream
    tiny = torch.zeros(1, dtype=torch.int32, device=dev)
    floor = []
    for k in range(40):
        a, z = HipEvent(timing=True), HipEvent(timing=True)
        a.record(stream); tiny.fill_(k); z.record(stream)
        z.synchronize()
        if k >= 10:
            floor.append(a.elapsed_time(z) * 1e3)

    us = {g: [] for g in groups}
    for ev in pevs:
        for gi, g in enumerate(groups):
            us[g].append(ev[gi].elapsed_time(ev[gi + 1]) * 1e3)
    med = {g: float(np.median(us[g])) for g in groups}
    # the roofline kernel from the timed steps themselves
    us["merge_unmerge"] = merge_pair_us
    med["merge_unmerge"] = float(np.median(merge_pair_us))

    ch, co = delta_cost(W, het), delta_cost(W, homo)
    mc = merge_cost(4096, 4096, r_m, n_mats)
    alg = {"hetero_shrink": (ch["shrink_bytes"], ch["flops"] * 0.5),
           "hetero_expand": (ch["expand_bytes"], ch["flops"] * 0.5),
           "homo_shrink": (co["shrink_bytes"], co["flops"] * 0.5),
           "homo_expand": (co["expand_bytes"], co["flops"] * 0.5),
           "hetero_apply": (ch["shrink_bytes"] + ch["expand_bytes"], ch["flops"]),
           "homo_apply": (co["shrink_bytes"] + co["expand_bytes"], co["flops"]),
           "merge_unmerge": (2 * mc["bytes"], 2 * mc["flops"]),
           "metadata": (0, 0)}
    alg = {g: alg[g] for g in groups}
    step_bytes = sum(b for b, _ in alg.values())
    kernels = {}
    for g in groups:
        b, f = alg[g]
        if g == "metadata":  # the builder kernels: no HBM traffic to speak of
            kernels[g] = {"us_median": round(med[g], 3), "us_p10": round(float(np.percentile(us[g], 10)), 3),
                          "us_p90": round(float(np.percentile(us[g], 90)), 3), "launches": 2}
            continue
        gbs = b / (med[g] * 1e-6) / 1e9
        kernels[g] = {"us_median": round(med[g], 3), "us_p10": round(float(np.percentile(us[g], 10)), 3),
                      "us_p90": round(float(np.percentile(us[g], 90)), 3), "alg_bytes": int(b),
                      "GB_s": round(gbs, 1), "TFLOP_s": round(f / (med[g] * 1e-6) / 1e12, 3),
                      "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    # dominant kernel: largest share of GPU time; merge and unmerge are the same kernel
    mavg = med["merge_unmerge"] / 2
    dom = max((g for g in groups if g != "metadata"), key=lambda g: med[g])
    traffic = None
    if dom == "merge_unmerge":
        d_us, d_bytes, name = mavg, mc["bytes"], "merge_kernel (merge/unmerge, 4 x W[4096x4096], rank 16)"
        traffic = merge_traffic()
    else:
        d_us, d_bytes, name = med[dom], alg[dom][0], dom
    achieved = d_bytes / (d_us * 1e-6) / 1e9
    out = {
        "metric": METRIC,
        "value": round(step_bytes / (dt / args.steps) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(dt / args.steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "decode BGMV, Llama-7B-shaped layer: 64 one-token rows, d 4096, q/k/v/o, "
                               "rank 16; hetero (64 adapters) + homo (1 adapter) batches via lora_%s, then merge+unmerge "
                               "of one adapter into the layer's 4 W[4096x4096]; steps rotate over %d layer copies"
                               % ("apply" if not split else "shrink/lora_expand", len(layers)),
                   "rows": 64, "d": 4096, "rank": 16, "adapters": 64, "projections": 4,
                   "layer_copies": len(layers)},
        "roofline": {"bound": "hbm", "kernel": name, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "us_per_launch": round(d_us, 3), "alg_bytes_per_launch": int(d_bytes)},
        "kernels": kernels,
        "hetero_over_homo": round(sum(med[g] for g in groups if g.startswith("hetero")) /
                                  sum(med[g] for g in groups if g.startswith("homo")), 3),
        "path": args.path,
        "metadata": "host" if (args.metadata == "inline" and split) else args.metadata,
        "merge_us_per_layer": round(mavg, 3),
        "launch_floor_us": round(float(np.median(floor)), 3),
        "step_alg_bytes": int(step_bytes),
    }
    if loop_us is not None:
        # the same groups as the step's (minus the mode switch), timed in the
        # loop of calls alone
        lg = [g for g in groups if g not in ("merge_unmerge", "metadata")]
        out["calls_back_to_back"] = {}
        for g, t in zip(lg, loop_us):
            b, _ = alg[g]
            m = float(np.median(t))
            out["calls_back_to_back"][g] = {"us_median": round(m, 3), "hbm_frac": round(b / (m * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(W, {"hetero": het, "homo": homo}, merge_host, gpu_results)
    print(json.dumps(out), flush=True)


# ---------------------------------------------------------------------------
# The benchmark line: the 70B-shaped paged mix, plus the vision mode switch
# ---------------------------------------------------------------------------
APPLY_EXPAND0, APPLY_FUSED = 3 * 4, 3 * 4 + 5 * 4   # apply-plan variant numbering (shrink, expand, fused)
EXPAND_SHAPES = {0: 16, 1: 64, 2: 128, 3: 32, 4: 2}
MIX70B_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "mix70b_dominant_traffic.json")


def kernel_section_digest(name):
    """sha256 of one section of kernels.hip (the kernel's device code)."""
    src = open(KERNELS_SRC).read()
    a = src.index(SECTION + name + "\n")
    b = src.index(SECTION, a + len(SECTION))
    return hashlib.sha256(src[a:b].encode()).hexdigest()


PLAN_SOURCES = [os.path.join(ROOT, "heterogeneous_adapter_batching_amd", "csrc", f)
                for f in ("tile_table.inc", "plan_rules.h", "variants.h")]


def plan_digest():
    """sha256 of the sources that decide which items a launch holds (the tile
    table and the plan rules): a launch's counters describe that launch only
    while they are unchanged."""
    h = hashlib.sha256()
    for f in PLAN_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def recorded_traffic(path, kernel):
    """HBM bytes per launch of `kernel` from committed rocprofv3 counters
    (FETCH_SIZE and WRITE_SIZE in KiB per dispatch, one pass each, each
    scaled by a plain copy's bytes over the same counter's reading); None when
    there is no record for this kernel, or its source section, the tile table
    or the plan rules have changed since."""
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("kernel") != kernel or rec.get("source_sha256") != kernel_section_digest(rec.get("section", "")):
        return None
    if rec.get("plan_sha256") != plan_digest():
        return None
    c = rec["copy"]
    return round(rec["fetch_kib"] * c["bytes"] / c["fetch_kib"] + rec["write_kib"] * c["bytes"] / c["write_kib"])


def _pmc_groups(path):
    """rocprofv3 --pmc counter CSV -> {(kernel, grid workgroups): [value per dispatch]}."""
    import csv
    import re
    g = {}
    for r in csv.DictReader(open(path)):
        name = re.sub(r"\(anonymous namespace\)::", "", r["Kernel_Name"])
        name = re.sub(r"\([A-Za-z]*Args\)$", "", re.sub(r"^void ", "", name))
        wg = int(r.get("Workgroup_Size", r.get("Workgroup_Size_X", 256)) or 256)
        grid = int(r.get("Grid_Size", r.get("Grid_Size_X", 0)) or 0) // max(wg, 1)
        g.setdefault((name, grid), []).append(float(r["Counter_Value"]))
    return g


def traffic_record(args):
    """Write the committed traffic record of the 70B-mix step's dominant launch
    from four rocprofv3 --pmc runs under args.traffic_record: bench_FETCH_SIZE,
    bench_WRITE_SIZE (this script's default line) and copy_FETCH_SIZE,
    copy_WRITE_SIZE (--copy-calibration), each holding run_counter_collection.csv.
    The launch is the one of kernel args.traffic_kernel over args.traffic_grid
    workgroups (the grid the kernel trace shows for it)."""
    d = args.traffic_record

    def mean(op, counter, key):
        g = _pmc_groups(os.path.join(d, "%s_%s" % (op, counter), "run_counter_collection.csv"))
        v = g[key] if key is not None else max(g.values(), key=np.mean)   # the copy: the largest dispatches
        return float(np.mean(v)), len(v)
    key = (args.traffic_kernel, args.traffic_grid)
    f, n = mean("bench", "FETCH_SIZE", key)
    w, _ = mean("bench", "WRITE_SIZE", key)
    cf, _ = mean("copy", "FETCH_SIZE", None)
    cw, _ = mean("copy", "WRITE_SIZE", None)
    section = args.traffic_kernel.split("_kernel")[0]
    rec = {"what": "rocprofv3 --pmc counters (KiB per dispatch, mean over dispatches), one counter per run: the "
                   "dominant launch of the 70B-mix benchmark step (%s over %d workgroups) and one plain 1 GiB "
                   "device copy for calibration" % key,
           "kernel": args.traffic_kernel, "section": section,
           "source_sha256": kernel_section_digest(section), "plan_sha256": plan_digest(),
           "grid_workgroups": args.traffic_grid, "fetch_kib": round(f, 1), "write_kib": round(w, 1),
           "dispatches": n,
           "copy": {"bytes": 1 << 30, "fetch_kib": round(cf, 1), "write_kib": round(cw, 1),
                    "kernel": "the largest dispatch group of the calibration run (the 1 GiB copy)"},
           "commands": ["rocprofv3 --pmc %s --output-format csv -d %s/bench_%s -o run -- python3 bench.py "
                        "--no-cpu-baseline --steps 4 --warmup 2" % (c, d, c) for c in ("FETCH_SIZE", "WRITE_SIZE")]
                       + ["rocprofv3 --pmc %s --output-format csv -d %s/copy_%s -o run -- python3 bench.py "
                          "--copy-calibration" % (c, d, c) for c in ("FETCH_SIZE", "WRITE_SIZE")]
                       + ["python bench.py --traffic-record %s --traffic-kernel '%s' --traffic-grid %d"
                          % (d, args.traffic_kernel, args.traffic_grid)]}
    with open(MIX70B_TRAFFIC_FILE, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec, indent=1))


def piece_name(variant):
    if variant < APPLY_EXPAND0:
        return "shrink"
    if variant < APPLY_FUSED:
        ev = variant - APPLY_EXPAND0
        shape, cls = divmod(ev, 4)
        if shape == 4:
            return "bgmv_expand_kernel"
        return "expand_kernel<%d> (items of <= %d rows)" % ((1, 2, 4)[cls], EXPAND_SHAPES[shape])
    return "fused_kernel"


def piece_cost(W, work, parts):
    """Algorithmic bytes and flops of a set of apply-plan items over every
    projection of W.  parts: which halves the items compute ("shrink",
    "expand" or both for fused items): x rows (bf16) read and v written by
    the shrink; v read, y read and written (fp32) by the expand; each
    distinct adapter's A rows (shrink) and B rows (expand) once."""
    nb = fl = 0
    rows_r = []          # (row, rank) of every row the items cover, once
    seen, adapters = set(), set()
    for w in work:
        row0, nrows, a, r = int(w[0]), int(w[1]), int(w[2]), int(w[3])
        adapters.add((a, r))
        for q in range(row0, row0 + nrows):
            if q not in seen:
                seen.add(q)
                rows_r.append(r)
    rows_r = np.asarray(rows_r, np.int64)
    n = rows_r.size
    for p in W.projections:
        if "shrink" in parts:
            nb += n * p.d_in * 2 + sum(r * p.d_in * 2 for _, r in adapters) + int(rows_r.sum()) * 4
            fl += 2 * int(rows_r.sum()) * p.d_in
        if "expand" in parts:
            nb += int(rows_r.sum()) * 4 + sum(r * p.d_out * 2 for _, r in adapters) + n * p.d_out * 8
            fl += 2 * int(rows_r.sum()) * p.d_out
    return nb, fl


def apply_pieces(batch, projs):
    """lora_apply of the batch's current apply plan issued in pieces, each a
    lora_apply call on a copy of the launch that keeps some of its ranges:
    all shrink ranges (one call: the launcher groups them exactly as
    lora_apply does), then every expand range alone, then the fused range.
    lora_apply itself makes the same launches in the same order (one launch
    per expand range), so the pieces are the call split at its launch
    boundaries, which lets events sit between them.  The pieces keep the
    ranges of the plan current when they are made (the same batch is
    refreshed with the same rows every step) and read its buffers at each
    call.  Returns [(name, range indices, fn, items)]."""
    import ctypes
    from heterogeneous_adapter_batching_amd import lora_apply_proj_t, lora_launch_t, call_apply
    from heterogeneous_adapter_batching_amd.session import stream_handle
    L = batch.apply_launch
    info = L.info
    ranges = info.range_list()
    groups = []
    sh = [i for i, (v, _, c, _) in enumerate(ranges) if v < APPLY_EXPAND0 and c > 0]
    if sh:
        groups.append(("shrink", sh))
    for i, (v, _, c, _) in enumerate(ranges):
        if APPLY_EXPAND0 <= v < APPLY_FUSED and c > 0:
            groups.append((piece_name(v), [i]))
    for i, (v, _, c, _) in enumerate(ranges):
        if v == APPLY_FUSED and c > 0:
            groups.append(("fused_kernel", [i]))
    arr = (lora_apply_proj_t * len(projs))(*[
        lora_apply_proj_t(x.data_ptr(), x.stride(0), x.shape[1], A.c(), v.data_ptr(), v.stride(1), B.c(),
                          y.shape[1], y.data_ptr(), y.stride(0), float(s))
        for x, A, v, B, y, s in projs])
    h = stream_handle()
    work = batch.work_apply.copy()
    out = []
    for name, idx in groups:
        sub = lora_launch_t.from_buffer_copy(L)
        sub.info.n_ranges = len(idx)
        for j, i in enumerate(idx):
            sub.info.ranges[j] = L.info.ranges[i]
        items = np.concatenate([work[ranges[i][1]:ranges[i][1] + ranges[i][2]] for i in idx])

        def fn(sub=sub):
            # the plan's buffers of the batch's latest refresh (they move when
            # a refresh grows them)
            sub.row_index, sub.work, sub.live = L.row_index, L.work, L.live
            sub.host_work, sub.host_row_index = L.host_work, L.host_row_index
            call_apply(sub, arr, len(projs), h)
        fn.keep = (sub, arr, projs)
        out.append((name, idx, fn, items))
    return out


def cpu_baseline_mix(W, gpu_y, V, vision_merge, min_seconds=10.0, max_seconds=30.0):
    """The oracle as it stands, timed on a bounded sample of the benchmark's
    work on the host cores, and checked against the GPU's results of the same
    work.  Units, run in turn until `min_seconds` have passed and every unit
    ran once: (1) the oracle delta of a 1-in-16 sample of the 70B mix's rows
    (every 16th row, released ones included: they cost a copy) for one
    projection, cycling over q, o and up; (2) the oracle merge + unmerge of
    one vision W[4096x4096] with the rank-64 adapter.  The rate is the units'
    algorithmic bytes (the same definitions as the GPU figures) over the
    elapsed time; the comparisons' own time is left out."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    ra = np.asarray(W.row_adapter)
    sample = np.arange(0, W.n_rows, 16)
    act = sample[ra[sample] >= 0]
    distinct = np.unique(ra[act])
    r_act = W.adapter_rank[ra[act]].astype(np.int64)
    parity = {"delta_relF_max": 0.0, "delta_abs_max": 0.0, "rows_checked": 0, "released_untouched": True,
              "merge_equal_fraction": None, "merge_worst_over_bound": None}
    check_s = [0.0]

    def delta_unit(pi):
        def run():
            p = W.projections[pi]
            yrows, _ = oracle.apply_ref(ra, W.adapter_rank, p.x, p.y0, W.pool, p.A, p.B, W.scale, rows=sample)
            if ("delta", pi) not in done_checks:
                t0 = time.perf_counter()
                yg = gpu_y[pi]
                num = den = 0.0
                for i in sample:
                    if ra[i] < 0:
                        parity["released_untouched"] &= bool(np.array_equal(yg[i], p.y0[i]))
                        continue
                    dr = yrows[i] - p.y0[i]
                    dg = yg[i].astype(np.float64) - p.y0[i]
                    num += float(np.sum((dg - dr) ** 2))
                    den += float(np.sum(dr ** 2))
                    parity["delta_abs_max"] = max(parity["delta_abs_max"], float(np.max(np.abs(dg - dr))))
                    parity["rows_checked"] += 1
                parity["delta_relF_max"] = max(parity["delta_relF_max"], (num / den) ** 0.5)
                done_checks.add(("delta", pi))
                check_s[0] += time.perf_counter() - t0
            nb = act.size * p.d_in * 2 + act.size * p.d_out * 8 + int(r_act.sum()) * 8 + \
                int(W.adapter_rank[distinct].sum()) * (p.d_in + p.d_out) * 2
            return nb, "delta"
        return run

    def merge_unit():
        spec = V.merge
        p = V.projections[spec.projs[0]]
        r = int(V.adapter_rank[spec.adapter])
        w0, got = vision_merge

        def run():
            wm = oracle.merge_ref(w0, V.pool, p.A, p.B, spec.adapter, r, V.scale)
            if "merge" not in done_checks:
                t0 = time.perf_counter()
                parity["merge_equal_fraction"] = float(np.mean(np.asarray(wm, np.uint16) == got))
                Aa = oracle.gather_rows_ref(V.pool, p.A.row_off, p.A.max_rank, p.A.row_len, p.A.chunk_len,
                                            spec.adapter, r)
                Ba = oracle.gather_rows_ref(V.pool, p.B.row_off, p.B.max_rank, p.B.row_len, p.B.chunk_len,
                                            spec.adapter, r)
                exact = oracle.bf16_to_f64(w0) + V.scale * (Ba.T @ Aa)
                g = oracle.bf16_to_f64(got)
                ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(g), 2.0 ** -126))) - 7)
                bound = (0.5 * ulp + (r + 4) * 2.0 ** -23 * abs(V.scale) * (np.abs(Ba).T @ np.abs(Aa)) +
                         2.0 ** -23 * np.abs(exact))
                parity["merge_worst_over_bound"] = float(np.max(np.abs(g - exact) / bound))
                done_checks.add("merge")
                check_s[0] += time.perf_counter() - t0
            oracle.unmerge_ref(wm, V.pool, p.A, p.B, spec.adapter, r, V.scale)
            return 2 * merge_cost(p.d_out, p.d_in, r, 1)["bytes"], "merge"
        return run

    done_checks = set()
    units = [delta_unit(pi) for pi in range(len(W.projections))] + [merge_unit()]
    t0 = time.perf_counter()
    nbytes, done, k = 0, {"delta": 0, "merge": 0}, 0
    while True:
        b, kind = units[k % len(units)]()
        nbytes += b
        done[kind] += 1
        k += 1
        dt = time.perf_counter() - t0 - check_s[0]
        if (k >= len(units) and dt >= min_seconds) or dt >= max_seconds:
            break
    parity["within_bounds"] = bool(parity["delta_relF_max"] <= 4e-3 and parity["delta_abs_max"] <= 2e-2 and
                                   parity["released_untouched"] and parity["merge_worst_over_bound"] <= 1.0)
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": int(cores), "kind": "oracle",
            "sample": "%d oracle delta passes over every 16th row of the 70B mix (%d rows, %d active) for one "
                      "projection each (q, o, up in turn) and %d oracle merge+unmerge passes of one vision "
                      "W[4096x4096] with the rank-64 adapter, run in turn for %.1f s"
                      % (done["delta"], sample.size, act.size, done["merge"], dt),
            "seconds": round(dt, 3), "cpu_model": _cpu_model(), "parity": parity}


def headline(args):
    """The benchmark line.  Workload: the 70B-shaped paged mix (d 8192; q and
    o 8192 -> 8192, up 8192 -> 28672; 256 decode rows of which 128 are
    released, plus 8 prefill segments of 1024 rows; 128 adapters of ranks
    16/32/64 in a paged pool of 8192-element pages).  One step = one pass of
    the whole path over that batch: the host builds the segment table and the
    apply plan and copies them to the device (lora_batch_prepare), then
    lora_apply runs the shrink and expand of every projection over the
    active rows, gathering adapter rows through the page table.  Steps
    alternate between two device copies of the inputs (same values, other
    addresses), so no step finds the previous one's data in the Infinity
    Cache.  Inputs are resident in HBM before the timed region.

    Beside it, in the same line: the vision workload's mode switch (merge of
    its rank-64 adapter into 32 layers x q/k/v/o W[4096x4096], then unmerge),
    as merge and unmerge µs per layer, each phase cold (it streams 4.3 GB of
    W); and the heterogeneous / homogeneous time ratio against the mix's
    homogeneous twin (the same rows on one adapter of the token-weighted
    mean rank), both cold (a 512 MB read before each timed call evicts the
    Infinity Cache: ColdCache)."""
    import torch
    import workloads
    from heterogeneous_adapter_batching_amd.session import Batch, HipEvent, Rows, prepare_merge
    from workloads.device import bits_to_device, to_device

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    t_setup = time.perf_counter()
    W = workloads.gen_config(4)
    d_in = max(p.d_in for p in W.projections)
    d_out = max(p.d_out for p in W.projections)
    ldv = -(-int(W.adapter_rank.max()) // 4) * 4
    dw0 = to_device(W)
    b = Batch(W.n_rows, W.adapter_rank, d_in, d_out, inline=True).refresh(W.row_adapter)
    copies = []
    for c in range(2):
        if c == 0:
            pool, xs, ys = dw0.pool, [d.x for d in dw0.projections], [d.y for d in dw0.projections]
            offs = [(d.A_off, d.B_off) for d in dw0.projections]
        else:
            pool = dw0.pool.clone()
            xs = [d.x.clone() for d in dw0.projections]
            ys = [d.y.clone() for d in dw0.projections]
            offs = [(d.A_off.clone(), d.B_off.clone()) for d in dw0.projections]
        projs = []
        for p, x, y, (ao, bo) in zip(W.projections, xs, ys, offs):
            A = Rows(pool, ao, p.A.n_adapters, p.A.max_rank, p.A.row_len, p.A.chunk_len)
            B = Rows(pool, bo, p.B.n_adapters, p.B.max_rank, p.B.row_len, p.B.chunk_len)
            projs.append((x, A, b.new_v(ldv), B, y, W.scale))
        copies.append(dict(pool=pool, projs=projs, run=b.prepare_apply(projs), pieces=apply_pieces(b, projs)))
    names = [n for n, _, _, _ in copies[0]["pieces"]]

    # GPU results the CPU baseline checks (copy 0, one lora_apply from y0)
    gpu_y = None
    if not args.no_cpu_baseline:
        copies[0]["run"]()
        torch.cuda.synchronize()
        gpu_y = [d.y.cpu().numpy() for d in dw0.projections]
        for p, d in zip(W.projections, dw0.projections):
            d.y.copy_(torch.from_numpy(p.y0))
        torch.cuda.synchronize()

    def step(k, ev=None, dom=None):
        """One step on copy k mod 2: host preparation, then the pieces; with
        `ev` an event before every piece and one after the last (all pieces),
        or around piece `dom` only."""
        C = copies[k % 2]
        b.refresh(W.row_adapter, stream)
        for i, (_, _, fn, _) in enumerate(C["pieces"]):
            if ev is not None and (dom is None or i == dom):
                ev[0 if dom is not None else i].record(stream)
            fn()
            if ev is not None and dom == i:
                ev[1].record(stream)
        if ev is not None and dom is None:
            ev[len(C["pieces"])].record(stream)

    new_events = lambda n: [HipEvent(timing=True) for _ in range(n)]
    # warm-up steps, with an event between every piece: they name the dominant piece
    wev = [new_events(len(names) + 1) for _ in range(max(1, args.warmup))]
    for k in range(max(1, args.warmup)):
        step(k, wev[k])
    torch.cuda.synchronize()
    wmed = [float(np.median([e[i].elapsed_time(e[i + 1]) for e in wev])) for i in range(len(names))]
    dom = int(np.argmax(wmed))

    # timed steps: one event pair, around the dominant piece
    evs = [new_events(2) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(k, evs[k], dom)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    dom_us = [e[0].elapsed_time(e[1]) * 1e3 for e in evs]

    # per-piece table: as many steps again, an event between every piece
    pev = [new_events(len(names) + 1) for _ in range(args.steps)]
    for k in range(args.steps):
        step(k, pev[k])
    torch.cuda.synchronize()
    piece_us = [[e[i].elapsed_time(e[i + 1]) * 1e3 for e in pev] for i in range(len(names))]
    # the whole lora_apply as one call, between one event pair (same steps)
    aev = [new_events(2) for _ in range(args.steps)]
    for k in range(args.steps):
        C = copies[k % 2]
        b.refresh(W.row_adapter, stream)
        aev[k][0].record(stream)
        C["run"]()
        aev[k][1].record(stream)
    torch.cuda.synchronize()
    apply_us = float(np.median([e[0].elapsed_time(e[1]) * 1e3 for e in aev]))

    cost = delta_cost(W, W.row_adapter)
    step_bytes = cost["shrink_bytes"] + cost["expand_bytes"]
    pieces = {}
    for i, (name, idx, _, items) in enumerate(copies[0]["pieces"]):
        parts = ("shrink",) if name == "shrink" else ("shrink", "expand") if name == "fused_kernel" else ("expand",)
        nb, fl = piece_cost(W, items, parts)
        us = float(np.median(piece_us[i]))
        key = name if name not in pieces else "%s #%d" % (name, i)
        pieces[key] = {"us_median": round(us, 2), "us_p10": round(float(np.percentile(piece_us[i], 10)), 2),
                       "us_p90": round(float(np.percentile(piece_us[i], 90)), 2), "items": int(items.shape[0]),
                       "alg_bytes": int(nb), "GB_s": round(nb / us / 1e3, 1),
                       "hbm_frac": round(nb / us / 1e3 / HBM_PEAK_GBS, 4), "TFLOP_s": round(fl / us / 1e6, 2)}
    dname, _, _, ditems = copies[0]["pieces"][dom]
    dparts = ("shrink",) if dname == "shrink" else ("shrink", "expand") if dname == "fused_kernel" else ("expand",)
    d_bytes, d_flops = piece_cost(W, ditems, dparts)
    d_us = float(np.median(dom_us))
    achieved = d_bytes / (d_us * 1e-6) / 1e9
    kernel_label = dname.split(" ")[0]
    traffic = recorded_traffic(MIX70B_TRAFFIC_FILE, kernel_label)

    # homogeneous twin, cold: lora_apply between an event pair after a cache flush
    flush = ColdCache(dev)
    Wt = workloads.gen_twin(4)
    dwt = to_device(Wt)
    bt = Batch(Wt.n_rows, Wt.adapter_rank, d_in, d_out, inline=True).refresh(Wt.row_adapter)
    ldvt = -(-int(Wt.adapter_rank.max()) // 4) * 4
    twin_runs = []
    for c in range(2):
        # two device copies of the twin's inputs (same values, own addresses),
        # as the heterogeneous step has
        pool_t = dwt.pool if c == 0 else dwt.pool.clone()
        twin_runs.append(bt.prepare_apply(
            [(d.x if c == 0 else d.x.clone(),
              Rows(pool_t, d.A_off, p.A.n_adapters, p.A.max_rank, p.A.row_len, p.A.chunk_len),
              bt.new_v(ldvt), Rows(pool_t, d.B_off, p.B.n_adapters, p.B.max_rank, p.B.row_len, p.B.chunk_len),
              d.y if c == 0 else d.y.clone(), Wt.scale)
             for p, d in zip(Wt.projections, dwt.projections)]))
    run_t = twin_runs[0]
    cold = {"hetero": [], "homo": []}
    for it in range(args.warmup + args.steps):
        for name, fn in (("hetero", copies[0]["run"]), ("homo", run_t)):
            flush()
            e = new_events(2)
            e[0].record(stream); fn(); e[1].record(stream)
            torch.cuda.synchronize()
            if it >= args.warmup:
                cold[name].append(e[0].elapsed_time(e[1]) * 1e3)
    # the same pair in the step's steady state: calls back to back over the
    # two input copies, so every call pays the Infinity Cache write-back that
    # the call before it left (a flush before each call instead pays the
    # timed call's own last dirty lines outside the timed region)
    steady = {}
    for name, runs in (("hetero", [C["run"] for C in copies]), ("homo", twin_runs)):
        sev = [new_events(2) for _ in range(args.warmup + args.steps)]
        for k, e in enumerate(sev):
            (b if name == "hetero" else bt).refresh(W.row_adapter if name == "hetero" else Wt.row_adapter, stream)
            e[0].record(stream); runs[k % 2](); e[1].record(stream)
        torch.cuda.synchronize()
        steady[name] = float(np.median([e[0].elapsed_time(e[1]) * 1e3 for e in sev[args.warmup:]]))
    ct = delta_cost(Wt, Wt.row_adapter)
    twin = {"rank": int(Wt.adapter_rank[0]), "hetero_us": round(float(np.median(cold["hetero"])), 2),
            "homo_us": round(float(np.median(cold["homo"])), 2),
            "hetero_over_homo_time": round(float(np.median(cold["hetero"]) / np.median(cold["homo"])), 3),
            "steady_hetero_us": round(steady["hetero"], 2), "steady_homo_us": round(steady["homo"], 2),
            "steady_hetero_over_homo_time": round(steady["hetero"] / steady["homo"], 3),
            "hetero_over_homo_bytes": round(step_bytes / (ct["shrink_bytes"] + ct["expand_bytes"]), 3)}
    del dwt, bt, run_t, twin_runs

    # the vision mode switch: merge adapter 0 (rank 64) into 32 layers x
    # q/k/v/o W[4096x4096], then unmerge; each layer's matrices are copies of
    # the seeded layer-0 draws (same values, own addresses: 4.3 GB streamed
    # per phase, far past the Infinity Cache)
    V = workloads.gen_config(3, n_layers=32)
    dv = to_device(V)
    spec = V.merge
    rv = int(V.adapter_rank[spec.adapter])
    Av = [Rows(dv.pool, d.A_off, p.A.n_adapters, p.A.max_rank, p.A.row_len, p.A.chunk_len)
          for p, d in zip(V.projections, dv.projections)]
    Bv = [Rows(dv.pool, d.B_off, p.B.n_adapters, p.B.max_rank, p.B.row_len, p.B.chunk_len)
          for p, d in zip(V.projections, dv.projections)]
    w_host = [spec.weight(0, pi) for pi in spec.projs]
    w_dev0 = [bits_to_device(w) for w in w_host]
    mats = [[w_dev0[i] if l == 0 else w_dev0[i].clone() for i in range(len(spec.projs))] for l in range(spec.n_layers)]
    calls = [(prepare_merge([(mats[l][i], Av[pi], Bv[pi], spec.adapter, rv, V.scale)
                             for i, pi in enumerate(spec.projs)]),
              prepare_merge([(mats[l][i], Av[pi], Bv[pi], spec.adapter, rv, V.scale)
                             for i, pi in enumerate(spec.projs)], unmerge=True)) for l in range(spec.n_layers)]
    calls[0][0]()
    torch.cuda.synchronize()
    vision_merged = mats[0][0].cpu().numpy().view(np.uint16).copy()
    calls[0][1]()
    torch.cuda.synchronize()
    sw = []
    for rep in range(4):
        e = new_events(3)
        e[0].record(stream)
        for m, _ in calls:
            m()
        e[1].record(stream)
        for _, u in calls:
            u()
        e[2].record(stream)
        torch.cuda.synchronize()
        if rep > 0:
            sw.append((e[0].elapsed_time(e[1]) * 1e3, e[1].elapsed_time(e[2]) * 1e3))
    mb = merge_cost(4096, 4096, rv, len(spec.projs) * spec.n_layers)
    mus, uus = float(np.median([t[0] for t in sw])), float(np.median([t[1] for t in sw]))
    switch = {"layers": spec.n_layers, "matrices": len(spec.projs) * spec.n_layers, "rank": rv,
              "merge_us_per_layer": round(mus / spec.n_layers, 2), "unmerge_us_per_layer": round(uus / spec.n_layers, 2),
              "switch_ms": round((mus + uus) / 1e3, 3), "alg_bytes_per_phase": int(mb["bytes"]),
              "merge_hbm_frac": round(mb["bytes"] / mus / 1e3 / HBM_PEAK_GBS, 4),
              "unmerge_hbm_frac": round(mb["bytes"] / uus / 1e3 / HBM_PEAK_GBS, 4),
              "merge_TFLOP_s": round(mb["flops"] / mus / 1e6, 2)}
    del mats, calls, w_dev0

    # launch floor: one near-empty kernel between the same kind of events
    tiny = torch.zeros(1, dtype=torch.int32, device=dev)
    floor = []
    for k in range(40):
        a_, z_ = HipEvent(timing=True), HipEvent(timing=True)
        a_.record(stream); tiny.fill_(k); z_.record(stream)
        z_.synchronize()
        if k >= 10:
            floor.append(a_.elapsed_time(z_) * 1e3)

    ms = dt / args.steps * 1e3
    out = {
        "metric": METRIC,
        "value": round(step_bytes / (dt / args.steps) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "70B-shaped paged mix: 256 decode rows (128 released) + 8 prefill segments of 1024 "
                               "rows; q/o 8192->8192 and up 8192->28672; 128 adapters of ranks 16/32/64 in a pool of "
                               "8192-element pages under a random page table; step = host segment table + apply "
                               "plan + upload, then lora_apply (shrink + expand, all projections); plus the vision "
                               "mode switch (merge/unmerge of a rank-64 adapter into 32 x 4 W[4096x4096])",
                   "rows": int(W.n_rows), "active_rows": int((W.row_adapter >= 0).sum()),
                   "segments": int(b.segs.n_seg), "d": 8192, "d_up": 28672, "adapters": int(W.n_adapters),
                   "projections": len(W.projections), "input_copies": 2},
        "step_alg_bytes": int(step_bytes), "step_flops": int(cost["flops"]),
        "TFLOP_s": round(cost["flops"] / (ms * 1e-3) / 1e12, 2),
        "hbm_frac": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "kernel": "%s, %s" % (dname, "lora_apply's launch over %d items x %d "
                                                           "projections" % (ditems.shape[0], len(W.projections))),
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "us_per_launch": round(d_us, 3), "alg_bytes_per_launch": int(d_bytes)},
        "pieces": pieces,
        "lora_apply_one_call_us": round(apply_us, 2),
        "twin": twin,
        "switch": switch,
        "merge_us_per_layer": switch["merge_us_per_layer"],
        "launch_floor_us": round(float(np.median(floor)), 3),
        "setup_s": round(time.perf_counter() - t_setup, 1),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_mix(W, gpu_y, V, (w_host[0], vision_merged))
    print(json.dumps(out), flush=True)


def other_workload(args):
    """Kernel timing of the tiny, prefill, vision or 70B workload: shrink and
    expand over all projections per step (HIP events on the launch stream,
    median over the timed steps), plus for the vision workload the mode switch
    (merge then unmerge of adapter 0 into 32 layers x 4 W[4096x4096])."""
    import torch
    import workloads
    from heterogeneous_adapter_batching_amd.session import Batch, HipEvent, Rows, prepare_merge
    from workloads.device import bits_to_device, to_device

    k = {"tiny": 0, "prefill": 2, "vision": 3, "mix70b": 4}[args.workload]
    kw = {"n_layers": 32} if k == 3 else {}
    if getattr(args, "shared_x", False):
        assert k in (2, 3), "--shared-x applies to the prefill and vision workloads (q/k/v share x)"
        kw["shared_qkv"] = True
    flush = ColdCache("cuda")   # Infinity Cache flush between steps

    def setup(W):
        dw = to_device(W)
        rows = lambda desc, off: Rows(dw.pool, off, desc.n_adapters, desc.max_rank, desc.row_len, desc.chunk_len)
        A = [rows(p.A, d.A_off) for p, d in zip(W.projections, dw.projections)]
        B = [rows(p.B, d.B_off) for p, d in zip(W.projections, dw.projections)]
        d_in = max(p.d_in for p in W.projections)
        d_out = max(p.d_out for p in W.projections)
        b = Batch(W.n_rows, W.adapter_rank, d_in, d_out).refresh(W.row_adapter)
        ldv = -(-int(W.adapter_rank.max()) // 4) * 4
        return dw, A, B, d_in, d_out, b, ldv

    def time_split(W, dw, A, B, b, ldv, cold=True):
        """Shrink and expand µs over the timed steps: cold (a cache-flushing
        read before each step: ColdCache) or warm (the same launches back to back)."""
        v = [b.new_v(ldv) for _ in W.projections]
        do_s = b.prepare_shrink([(d.x, A[i], v[i]) for i, d in enumerate(dw.projections)])
        do_e = b.prepare_expand([(v[i], B[i], d.y, W.scale) for i, d in enumerate(dw.projections)])
        res = {"shrink": [], "expand": []}
        for it in range(args.warmup + args.steps):
            if cold:
                flush()
            e = [HipEvent(timing=True) for _ in range(3)]
            e[0].record(); do_s(); e[1].record(); do_e(); e[2].record()
            torch.cuda.synchronize()
            if it >= args.warmup:
                res["shrink"].append(e[0].elapsed_time(e[1]) * 1e3)
                res["expand"].append(e[1].elapsed_time(e[2]) * 1e3)
        return res

    W = workloads.gen_config(k, **kw)
    dw, A, B, d_in, d_out, b, ldv = setup(W)
    res = time_split(W, dw, A, B, b, ldv)
    warm = time_split(W, dw, A, B, b, ldv, cold=False)
    c = delta_cost(W, W.row_adapter)
    out = {"workload": args.workload + ("+shared-x" if getattr(args, "shared_x", False) else ""),
           "rows": W.n_rows, "active": int((W.row_adapter >= 0).sum()),
           "segments": b.segs.n_seg, "layout": W.layout, "kernels": {}}
    for g, nb, fl in (("shrink", c["shrink_bytes"], c["flops"] * 0.5), ("expand", c["expand_bytes"], c["flops"] * 0.5)):
        us = float(np.median(res[g]))
        out["kernels"][g] = {"us_median": round(us, 2), "alg_bytes": int(nb), "GB_s": round(nb / us / 1e3, 1),
                             "hbm_frac": round(nb / us / 1e3 / HBM_PEAK_GBS, 4),
                             "TFLOP_s": round(fl / us / 1e6, 2),
                             "us_p10": round(float(np.percentile(res[g], 10)), 2),
                             "us_p90": round(float(np.percentile(res[g], 90)), 2),
                             "warm_us_median": round(float(np.median(warm[g])), 2)}
    tot = sum(np.median(res[g]) for g in res)
    nb = c["shrink_bytes"] + c["expand_bytes"]
    out["shrink_expand_us"] = round(float(tot), 2)
    out["shrink_expand_hbm_frac"] = round(nb / tot / 1e3 / HBM_PEAK_GBS, 4)
    if getattr(args, "twin", False):
        assert k in (2, 3, 4), "--twin applies to the prefill, vision and 70B workloads"
        Wt = workloads.gen_twin(k)
        dwt, At, Bt, _, _, bt, ldvt = setup(Wt)
        rt = time_split(Wt, dwt, At, Bt, bt, ldvt)
        wt = time_split(Wt, dwt, At, Bt, bt, ldvt, cold=False)
        ct = delta_cost(Wt, Wt.row_adapter)
        tt = sum(np.median(rt[g]) for g in rt)
        # back to back, each step pays the write-back the step before it left
        # in the Infinity Cache (the flushed timing leaves its own to the flush)
        warm_h = sum(np.median(warm[g]) for g in warm)
        warm_t = sum(np.median(wt[g]) for g in wt)
        nbt = ct["shrink_bytes"] + ct["expand_bytes"]
        out["twin"] = {"rank": int(Wt.adapter_rank[0]), "shrink_us": round(float(np.median(rt["shrink"])), 2),
                       "expand_us": round(float(np.median(rt["expand"])), 2), "shrink_expand_us": round(float(tt), 2),
                       "alg_bytes": int(nbt), "hbm_frac": round(nbt / tt / 1e3 / HBM_PEAK_GBS, 4),
                       "hetero_over_homo_time": round(float(tot / tt), 3),
                       "warm_shrink_expand_us": round(float(warm_t), 2),
                       "warm_hetero_shrink_expand_us": round(float(warm_h), 2),
                       "warm_hetero_over_homo_time": round(float(warm_h / warm_t), 3),
                       "hetero_over_homo_bytes": round(nb / nbt, 3)}
        del dwt, bt
    if args.metadata == "device":
        # lora_apply with the host-built plan, against the builder kernel plus
        # lora_apply with the device-built plan (every range launched at its
        # capacity), each from a flushed cache
        from heterogeneous_adapter_batching_amd.session import DeviceBatch
        va = [b.new_v(ldv) for _ in W.projections]
        do_a = b.prepare_apply([(d.x, A[i], va[i], B[i], d.y, W.scale) for i, d in enumerate(dw.projections)])
        db = DeviceBatch(W.n_rows, len(W.adapter_rank), int(W.adapter_rank.max()), d_in, d_out)
        ra_d = torch.from_numpy(np.asarray(W.row_adapter, np.int32)).cuda()
        rk_d = torch.from_numpy(np.asarray(W.adapter_rank, np.int32)).cuda()
        db.build(ra_d, rk_d)
        vd = [db.new_v(ldv) for _ in W.projections]
        do_d = db.prepare_apply([(d.x, A[i], vd[i], B[i], d.y, W.scale) for i, d in enumerate(dw.projections)])
        r2 = {"apply_host_plan": [], "build": [], "apply_device_plan": []}
        for it in range(args.warmup + args.steps):
            e = [HipEvent(timing=True) for _ in range(5)]
            flush()
            e[0].record(); do_a(); e[1].record()
            flush()
            e[2].record(); db.build(ra_d, rk_d); e[3].record(); do_d(); e[4].record()
            torch.cuda.synchronize()
            if it >= args.warmup:
                r2["apply_host_plan"].append(e[0].elapsed_time(e[1]) * 1e3)
                r2["build"].append(e[2].elapsed_time(e[3]) * 1e3)
                r2["apply_device_plan"].append(e[3].elapsed_time(e[4]) * 1e3)
        assert db.header().status == 0
        out["device_metadata"] = {g: round(float(np.median(r2[g])), 2) for g in r2}
        out["device_metadata"]["ranges"] = db.plan.info.n_ranges
        out["device_metadata"]["work_capacity"] = db.plan.work_capacity
    if k == 3:
        spec = W.merge
        r = int(W.adapter_rank[spec.adapter])
        # each layer's matrices are copies of the seeded layer-0 draws (same
        # values, own addresses: every phase streams all of them from HBM)
        w0 = {pi: bits_to_device(spec.weight(0, pi)) for pi in spec.projs}
        mats = {}
        for l in range(spec.n_layers):
            for pi in spec.projs:
                mats[(l, pi)] = w0[pi] if l == 0 else w0[pi].clone()
        calls = [(prepare_merge([(mats[(l, pi)], A[pi], B[pi], spec.adapter, r, W.scale) for pi in spec.projs]),
                  prepare_merge([(mats[(l, pi)], A[pi], B[pi], spec.adapter, r, W.scale) for pi in spec.projs],
                                unmerge=True)) for l in range(spec.n_layers)]
        ts = []
        for rep in range(3):
            torch.cuda.synchronize()
            e = [HipEvent(timing=True) for _ in range(3)]
            e[0].record()
            for m, _ in calls:
                m()
            e[1].record()
            for _, u in calls:
                u()
            e[2].record()
            torch.cuda.synchronize()
            ts.append((e[0].elapsed_time(e[1]) * 1e3, e[1].elapsed_time(e[2]) * 1e3))
        mb = merge_cost(4096, 4096, r, 4 * spec.n_layers)["bytes"]
        mus, uus = float(np.median([t[0] for t in ts])), float(np.median([t[1] for t in ts]))
        out["switch"] = {"merge_us": round(mus, 1), "unmerge_us": round(uus, 1),
                         "merge_us_per_layer": round(mus / spec.n_layers, 2), "alg_bytes_per_phase": int(mb),
                         "merge_hbm_frac": round(mb / mus / 1e3 / HBM_PEAK_GBS, 4),
                         "unmerge_hbm_frac": round(mb / uus / 1e3 / HBM_PEAK_GBS, 4)}
    print(json.dumps(out), flush=True)


def mixture_workload(args):
    """deLoRA mixture inference (VaLoRA blog, section 4.4.2) on the decode
    layer: adapter 0 merged, the other 63 one-token rows get
    +s x A_x^T B_x - s x A_0^T B_0 through composite adapters in one
    lora_apply (the fused kernel), timed next to the plain heterogeneous
    lora_apply of the same rows (no adapter merged); HIP events, medians,
    a 512 MB read between steps (ColdCache) to evict the Infinity Cache."""
    import torch
    import workloads
    from heterogeneous_adapter_batching_amd import lora_mixture_row_adapter
    from heterogeneous_adapter_batching_amd.session import Batch, HipEvent, Rows, mixture_tables
    from workloads.device import to_device

    W = workloads.gen_config(1)
    dw = to_device(W)
    m = W.merge.adapter
    ra = W.batches["hetero"]
    ra_mix = lora_mixture_row_adapter(ra, m)
    r_max = int(W.adapter_rank.max())
    out_max = 2 * r_max
    mix, plain, crank = [], [], None
    for p, d in zip(W.projections, dw.projections):
        ca, cb, neg, crank = mixture_tables((p.A.row_off, p.B.row_off, p.A.max_rank, p.A.chunks, p.B.chunks),
                                            W.adapter_rank, m, out_max)
        mix.append((d, Rows(dw.pool, ca, p.A.n_adapters, out_max, p.A.row_len, p.A.chunk_len, neg_from=neg),
                    Rows(dw.pool, cb, p.B.n_adapters, out_max, p.B.row_len, p.B.chunk_len), (ca, cb, neg)))
        plain.append((d, Rows(dw.pool, d.A_off, p.A.n_adapters, p.A.max_rank, p.A.row_len, p.A.chunk_len),
                      Rows(dw.pool, d.B_off, p.B.n_adapters, p.B.max_rank, p.B.row_len, p.B.chunk_len)))
    bm = Batch(W.n_rows, crank, 4096, 4096).refresh(ra_mix)
    bp = Batch(W.n_rows, W.adapter_rank, 4096, 4096).refresh(np.where(ra == m, -1, ra).astype(np.int32))
    vm = [bm.new_v(out_max) for _ in mix]
    vp = [bp.new_v(r_max) for _ in plain]
    run_mix = bm.prepare_apply([(d.x, A, v, B, d.y, W.scale) for (d, A, B, _), v in zip(mix, vm)])
    run_plain = bp.prepare_apply([(d.x, A, v, B, d.y, W.scale) for (d, A, B), v in zip(plain, vp)])
    flush = ColdCache("cuda")
    res = {"mixture_apply": [], "unmerged_apply": []}
    for it in range(args.warmup + args.steps):
        for name, fn in (("mixture_apply", run_mix), ("unmerged_apply", run_plain)):
            flush()
            e = [HipEvent(timing=True) for _ in range(2)]
            e[0].record(); fn(); e[1].record()
            torch.cuda.synchronize()
            if it >= args.warmup:
                res[name].append(e[0].elapsed_time(e[1]) * 1e3)
    act = ra_mix >= 0
    n, d_in, d_out, r = int(act.sum()), 4096, 4096, int(W.adapter_rank[1])
    rm = int(W.adapter_rank[m])
    n_proj = len(W.projections)
    # algorithmic bytes: x, y read+write, each distinct adapter's A and B once, the merged adapter's once, v
    plain_b = n_proj * (n * d_in * 2 + n * d_out * 8 + n * r * (d_in + d_out) * 2 + n * r * 8)
    mix_b = plain_b + n_proj * (rm * (d_in + d_out) * 2 + n * rm * 8)
    out = {"workload": "mixture", "rows": n, "merged_adapter": int(m), "kernels": {}}
    for name, nb in (("mixture_apply", mix_b), ("unmerged_apply", plain_b)):
        us = float(np.median(res[name]))
        out["kernels"][name] = {"us_median": round(us, 2), "alg_bytes": int(nb), "GB_s": round(nb / us / 1e3, 1),
                                "hbm_frac": round(nb / us / 1e3 / HBM_PEAK_GBS, 4)}
    out["mixture_over_unmerged"] = round(out["kernels"]["mixture_apply"]["us_median"] /
                                         out["kernels"]["unmerged_apply"]["us_median"], 3)
    print(json.dumps(out), flush=True)


def swap_workload(args):
    """Unified adapter pool (S-LoRA's unified paging): the vision workload's
    32 rank-64 adapters (q/k/v/o: 8 row tables of 4096) paged on demand into
    a pool that holds 16 of them.  Reports (1) copy-in of 16 adapters (packed
    rows host -> device, then the scatter into their pages) on the pool's
    stream, (2) the scatter kernel alone, against HBM, and (3) the vision
    shrink + expand on the compute stream alone and with a copy-in of 16
    other adapters running beside it on the pool's stream."""
    import torch
    import workloads
    from heterogeneous_adapter_batching_amd.session import AdapterPool, Batch, HipEvent, Rows
    from heterogeneous_adapter_batching_amd import lora_pool_scatter
    from workloads.device import to_device

    W = workloads.gen_config(3, n_layers=1)
    dw = to_device(W)
    n_ad, r = W.n_adapters, int(W.adapter_rank.max())
    tables = [d for p in W.projections for d in (p.A, p.B)]

    def rows_of_adapter(a):
        out = []
        for d in tables:
            blk = np.empty((int(W.adapter_rank[a]), d.row_len), np.uint16)
            for j in range(blk.shape[0]):
                o = int(d.row_off[(a * d.max_rank + j) * d.chunks])
                blk[j] = W.pool[o:o + d.row_len]
            out.append(blk)
        return out
    host_rows = {a: rows_of_adapter(a) for a in range(n_ad)}
    page = 4096
    per_adapter = r * sum(d.row_len for d in tables) * 2          # bytes
    pool = AdapterPool(16 * r * len(tables), page, n_ad, r, [d.row_len for d in tables], host_rows.__getitem__)
    res = {"copy_in_16": [], "scatter_16": [], "compute_alone": [], "compute_with_copy_in": []}
    # the vision batch on the compute stream, from the dense layout
    rows = lambda desc, off: Rows(dw.pool, off, desc.n_adapters, desc.max_rank, desc.row_len, desc.chunk_len)
    A = [rows(p.A, d.A_off) for p, d in zip(W.projections, dw.projections)]
    B = [rows(p.B, d.B_off) for p, d in zip(W.projections, dw.projections)]
    b = Batch(W.n_rows, W.adapter_rank, 4096, 4096).refresh(W.row_adapter)
    v = [b.new_v(r) for _ in W.projections]
    do_s = b.prepare_shrink([(d.x, A[i], v[i]) for i, d in enumerate(dw.projections)])
    do_e = b.prepare_expand([(v[i], B[i], d.y, W.scale) for i, d in enumerate(dw.projections)])
    compute = torch.cuda.current_stream()
    flush = ColdCache("cuda")
    sets = [np.arange(0, 16), np.arange(16, 32)]
    cur = 1  # the set resident last (none yet): each acquire below loads the other one
    for it in range(args.warmup + args.steps):
        for _ in range(2):
            cur = 1 - cur
            S = sets[cur]
            flush()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            load = pool.acquire(S, W.adapter_rank[S])
            t1 = time.perf_counter()
            assert len(load) == 16
            pool.release_after(S, pool.stream)
            pool.drain()
            if it >= args.warmup:
                res["copy_in_16"].append(pool.last_upload_ms() * 1e3)
                res.setdefault("host_pack_16", []).append((t1 - t0) * 1e3)  # ms: manager + packing + enqueue
            # the scatter alone, from the packed rows now on the device
            so, do, ln, n_src = pool.mgr.load_list(S)
            d_so, d_do = torch.from_numpy(so).cuda(), torch.from_numpy(do).cuda()
            d_ln = torch.from_numpy(ln).cuda()
            torch.cuda.synchronize()
            e = [HipEvent(timing=True) for _ in range(2)]
            e[0].record(compute)
            lora_pool_scatter(pool._stage[1].data_ptr(), pool.pool.data_ptr(), so.shape[0], d_so.data_ptr(),
                              d_do.data_ptr(), d_ln.data_ptr(), compute.cuda_stream)
            e[1].record(compute)
            torch.cuda.synchronize()
            if it >= args.warmup:
                res["scatter_16"].append(e[0].elapsed_time(e[1]) * 1e3)
        # compute alone, then with the copy-in of the set not resident
        for name in ("compute_alone", "compute_with_copy_in"):
            flush()
            torch.cuda.synchronize()
            if name == "compute_with_copy_in":
                # the copy-in is enqueued (host packing done) before the compute starts
                cur = 1 - cur
                S = sets[cur]
                assert len(pool.acquire(S, W.adapter_rank[S])) == 16
            e = [HipEvent(timing=True) for _ in range(2)]
            e[0].record(compute)
            do_s()
            do_e()
            e[1].record(compute)
            torch.cuda.synchronize()
            if name == "compute_with_copy_in":
                pool.release_after(S, pool.stream)
                pool.drain()
            if it >= args.warmup:
                res[name].append(e[0].elapsed_time(e[1]) * 1e3)
    med = {k: float(np.median(v_)) for k, v_ in res.items()}
    nbytes = 16 * per_adapter
    out = {"workload": "swap", "adapters": n_ad, "rank": r, "pool_adapters": 16,
           "adapter_bytes": per_adapter, "kernels": {
               "copy_in_16": {"us_median": round(med["copy_in_16"], 1), "bytes": nbytes,
                              "GB_s": round(nbytes / med["copy_in_16"] / 1e3, 1),
                              "what": "device time on the pool stream: host->device copy of the packed rows, "
                                      "scatter into pages, table entries",
                              "host_acquire_ms": round(med["host_pack_16"], 2)},
               "scatter_16": {"us_median": round(med["scatter_16"], 2), "alg_bytes": 2 * nbytes,
                              "GB_s": round(2 * nbytes / med["scatter_16"] / 1e3, 1),
                              "hbm_frac": round(2 * nbytes / med["scatter_16"] / 1e3 / HBM_PEAK_GBS, 4)},
               "vision_shrink_expand": {"alone_us": round(med["compute_alone"], 1),
                                        "with_copy_in_us": round(med["compute_with_copy_in"], 1),
                                        "what": "one layer's shrink + expand on the compute stream, alone and "
                                                "while the pool stream copies 16 adapters in"}}}
    print(json.dumps(out), flush=True)


def heads_workload(args):
    """Vision task heads (VaLoRA 4.2.2): each of the vision workload's 32
    adapters carries a head with U{2..128} classes (one linear layer over
    d 4096), all heads in one launch: logits = x . H_a^T for every row, the
    shrink kernels with the head's class rows as the A table.  Input: the
    vision workload's rows and adapter choice; heads drawn like A."""
    import torch
    import workloads
    from heterogeneous_adapter_batching_amd.session import Batch, HipEvent, Rows
    from workloads.device import to_device

    V = workloads.gen_config(3, n_layers=1)
    classes = np.random.default_rng([3, 7]).integers(2, 129, size=V.n_adapters).astype(np.int32)
    W = workloads.gen_custom(3, V.row_adapter, classes, 4096, 64, n_proj=1, layout="dense")
    dw = to_device(W)
    p, d = W.projections[0], dw.projections[0]
    H = Rows(dw.pool, d.A_off, p.A.n_adapters, p.A.max_rank, p.A.row_len, p.A.chunk_len)
    b = Batch(W.n_rows, W.adapter_rank, 4096, 64).refresh(W.row_adapter)
    v = [b.new_v(128)]
    run = b.prepare_shrink([(d.x, H, v[0])])
    flush = ColdCache("cuda")
    ts = []
    for it in range(args.warmup + args.steps):
        flush()
        e = [HipEvent(timing=True) for _ in range(2)]
        e[0].record()
        run()
        e[1].record()
        torch.cuda.synchronize()
        if it >= args.warmup:
            ts.append(e[0].elapsed_time(e[1]) * 1e3)
    act = W.row_adapter[W.row_adapter >= 0]
    c_act = classes[act].astype(np.int64)
    distinct = np.unique(act)
    nbytes = int(act.size * 4096 * 2 + classes[distinct].sum() * 4096 * 2 + c_act.sum() * 4 * b.v_slices)
    flops = int(2 * 4096 * c_act.sum())
    us = float(np.median(ts))
    out = {"workload": "heads", "rows": int(act.size), "heads": int(V.n_adapters),
           "classes_min_max": [int(classes.min()), int(classes.max())],
           "kernels": {"heads_shrink": {"us_median": round(us, 2), "alg_bytes": nbytes,
                                        "GB_s": round(nbytes / us / 1e3, 1),
                                        "hbm_frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4),
                                        "TFLOP_s": round(flops / us / 1e6, 2)}}}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
