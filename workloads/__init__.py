"""Seeded synthetic inputs for heterogeneous LoRA batching.

This module only *draws inputs*: it holds none of the method's arithmetic
(no shrink, expand, merge, segment grouping or rounding of results).  Both the
CPU oracle (``oracle/``) and the HIP path consume exactly the arrays produced
here, so the two sides are compared on identical inputs.

Shapes follow the model-shaped stand-ins of the five workloads:

* ``tiny``     -- 64 rows, d 512, 4 adapters of rank 8, 8 request segments,
                  plus a merge of adapter 0 into one W[512x512].
* ``decode``   -- Llama-7B-shaped layer, 64 one-token rows, d 4096, q/k/v/o,
                  rank 16; a fully heterogeneous batch (row i -> adapter i) and
                  a homogeneous batch (every row -> adapter 0).
* ``prefill``  -- 16 requests with lognormal prompt lengths (median 512,
                  sigma 0.6, clipped to [32, 2048]), 16 adapters of ranks drawn
                  from {8,16,32,64}, truncated Zipf(1.1) adapter choice.
* ``vision``   -- Qwen-VL-7B-like mix: 24 requests of U{256..1024} visual
                  tokens + 32 text tokens, 32 adapters of rank 64, Zipf(1.1);
                  plus a mode switch over 32 layers x q/k/v/o W[4096x4096].
* ``mix70b``   -- 70B-shaped mix: d 8192, q/o (8192->8192) and MLP up
                  (8192->28672); 256 decode rows (half released) plus 8 prefill
                  segments of 1024 rows; 128 adapters of ranks {16,32,64}; all
                  adapter rows live in a paged pool of 8192-element pages placed
                  by a random page table.

Value distributions: x ~ N(0,1), A ~ N(0,1/d_in), B ~ N(0,1/r), W ~ N(0,1/d_in)
drawn in fp32 and rounded to bf16 (round-to-nearest-even, by torch's CPU cast);
y0 ~ N(0,1) kept in fp32; scale s = 2.0.

Adapter weights follow the d-vector layout of unified paging (S-LoRA,
"Unified Paging": a rank-R weight occupies R vectors of the hidden size):
A of adapter a is r_a rows of d_in elements, B is r_a rows of d_out elements,
so the delta is y += s * (x @ A^T) @ B and the merge is W += s * B^T @ A with
W stored [d_out][d_in].  Rows are addressed through a row-offset table with the
library's descriptor semantics: chunk c of row j of adapter a starts at
``pool[row_off[(a*max_rank + j)*chunks + c]]`` and covers ``chunk_len``
elements (the last chunk only up to ``row_len``).

Random numbers: every tensor is drawn in fixed row blocks, each block from its
own ``numpy.random.default_rng([seed, tag..., block])`` stream, so the values do
not depend on the number of threads used to draw them.  The batch structure
(lengths, adapter choice, ranks, released rows, page permutation) comes from
``default_rng([seed, 0])``.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Callable, Dict, List, NamedTuple, Optional

import numpy as np

__all__ = [
    "RowsDesc", "Projection", "MergeSpec", "Workload", "GENERATORS", "gen_config",
    "to_bf16_bits", "normal_f32", "build_pool", "NAN_BF16",
]

NAN_BF16 = np.uint16(0x7FC0)  # quiet NaN: fills holes so stray reads show up
_BLOCK_ELEMS = 1 << 21  # elements per independently seeded draw block
_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))

# Tags keep every tensor on its own random stream.
_TAG_X, _TAG_A, _TAG_B, _TAG_Y0, _TAG_W = 1, 2, 3, 4, 5


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (uint16), round-to-nearest-even (torch CPU cast)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def normal_f32(seed: int, key: tuple, shape: tuple, std: float = 1.0) -> np.ndarray:
    """N(0, std^2) fp32 array drawn in row blocks, one keyed stream per block."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    out = np.empty(n, dtype=np.float32)
    nblk = max(1, (n + _BLOCK_ELEMS - 1) // _BLOCK_ELEMS)

    def fill(b):
        lo, hi = b * _BLOCK_ELEMS, min(n, (b + 1) * _BLOCK_ELEMS)
        rng = np.random.default_rng([seed, *key, b])
        rng.standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])
        if std != 1.0:
            out[lo:hi] *= np.float32(std)

    if nblk == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(fill, range(nblk)))
    return out.reshape(shape)


def bf16_normal(seed, key, shape, std=1.0):
    return to_bf16_bits(normal_f32(seed, key, shape, std))


@dataclass
class RowsDesc:
    """Adapter rows of one matrix kind (A or B of one projection) inside a pool.

    Mirrors the library's row descriptor: ``row_off`` int64, indexed
    ``(a*max_rank + j)*chunks + c``; offsets are in bf16 elements from the pool
    base and multiples of 8 (16-byte aligned)."""
    row_off: np.ndarray
    n_adapters: int
    max_rank: int
    row_len: int
    chunk_len: int

    @property
    def chunks(self) -> int:
        return (self.row_len + self.chunk_len - 1) // self.chunk_len


@dataclass
class Projection:
    name: str
    d_in: int
    d_out: int
    x: np.ndarray        # uint16 bf16 bits [n_rows, d_in]
    y0: np.ndarray       # float32 [n_rows, d_out]
    A: RowsDesc          # r_a rows of d_in per adapter
    B: RowsDesc          # r_a rows of d_out per adapter


@dataclass
class MergeSpec:
    """Mode switch: merge adapter ``adapter`` into ``n_layers x len(projs)`` W.

    Matrix (layer, p) is W[d_out, d_in] of projection ``projs[p]`` (an index
    into ``Workload.projections``); the adapter rows are that projection's
    ``adapter`` rows in the pool (the same rows for every layer: one layer's
    adapters are drawn).  ``weight(layer, p)`` draws W lazily as bf16 bits."""
    adapter: int
    n_layers: int
    projs: List[int]
    weight: Callable[[int, int], np.ndarray]


@dataclass
class Workload:
    name: str
    seed: int
    n_rows: int
    row_adapter: np.ndarray          # int32 [n_rows], -1 = released
    adapter_rank: np.ndarray         # int32 [n_adapters]
    pool: np.ndarray                 # uint16 bf16 bits, all adapter rows
    projections: List[Projection]
    scale: float = 2.0
    batches: Dict[str, np.ndarray] = field(default_factory=dict)
    merge: Optional[MergeSpec] = None
    layout: str = "dense"

    @property
    def n_adapters(self) -> int:
        return int(self.adapter_rank.shape[0])


# ----------------------------------------------------------------------------
# pool placement (input layout only)
# ----------------------------------------------------------------------------
def build_pool(items, n_adapters, max_rank, layout, page_elems, rng):
    """Place adapter rows in one pool.

    ``items`` is a list of (key, row_len, rows) where ``rows[a]`` is a uint16
    array [r_a, row_len].  Returns (pool, {key: RowsDesc}).

    dense: every row is one chunk, rows packed back to back in item order.
    paged: every row is split into pages of ``page_elems`` elements; all pages
    are scattered by a random permutation over twice as many page slots; unused
    slots and the tail of a partly used page hold NaN.  A trailing NaN page
    backs the offsets of rank slots j >= r_a, which the kernels never read.
    """
    descs = {}
    if layout == "dense":
        total = sum(int(sum(r.shape[0] for r in rows)) * rl for _, rl, rows in items)
        nan_base = total
        pool = np.empty(total + max(rl for _, rl, _ in items), dtype=np.uint16)
        pool[nan_base:] = NAN_BF16
        cur = 0
        for key, rl, rows in items:
            off = np.full(n_adapters * max_rank, nan_base, dtype=np.int64)
            for a, m in enumerate(rows):
                for j in range(m.shape[0]):
                    pool[cur:cur + rl] = m[j]
                    off[a * max_rank + j] = cur
                    cur += rl
            descs[key] = RowsDesc(off, n_adapters, max_rank, rl, rl)
        return pool, descs
    if layout != "paged":
        raise ValueError(layout)
    P = page_elems
    need = sum(int(sum(r.shape[0] for r in rows)) * ((rl + P - 1) // P) for _, rl, rows in items)
    n_slots = 2 * need
    perm = rng.permutation(n_slots)
    pool = np.full((n_slots + 1) * P, NAN_BF16, dtype=np.uint16)
    nan_base = n_slots * P
    nxt = 0
    for key, rl, rows in items:
        ch = (rl + P - 1) // P
        off = np.full(n_adapters * max_rank * ch, nan_base, dtype=np.int64)
        for a, m in enumerate(rows):
            for j in range(m.shape[0]):
                for c in range(ch):
                    slot = int(perm[nxt]); nxt += 1
                    lo, hi = c * P, min(rl, (c + 1) * P)
                    pool[slot * P: slot * P + (hi - lo)] = m[j, lo:hi]
                    off[(a * max_rank + j) * ch + c] = slot * P
        descs[key] = RowsDesc(off, n_adapters, max_rank, rl, P)
    return pool, descs


def _zipf_choice(rng, n_ids, size, s=1.1):
    p = (np.arange(1, n_ids + 1, dtype=np.float64)) ** (-s)
    p /= p.sum()
    return rng.choice(n_ids, size=size, p=p)


class Structure(NamedTuple):
    """A workload's batch structure: no tensors drawn."""
    name: str
    row_adapter: np.ndarray
    adapter_rank: np.ndarray
    projs: list          # (name, d_in, d_out)
    batches: dict
    layout: str
    page_elems: int


_structure_only = False


def structure(k: int, seed: Optional[int] = None, **kw) -> Structure:
    """Row map(s), ranks and projection shapes of workload k, from the same
    draws as gen_config(k, seed) but without drawing its tensors."""
    return _structure_of(gen_config, k, seed, **kw)


def structure_twin(k: int, seed: Optional[int] = None) -> Structure:
    """Row map, rank and projection shapes of gen_twin(k, seed), no tensors drawn."""
    return _structure_of(gen_twin, k, seed)


def _structure_of(gen, *a, **kw):
    global _structure_only
    prev, _structure_only = _structure_only, True
    try:
        return gen(*a, **kw)
    finally:
        _structure_only = prev


def _make(name, seed, row_adapter, ranks, projs, layout, page_elems, rng,
          batches=None, merge=None, scale=2.0, shared_x=()):
    """shared_x: groups of projection indices that take the same x (one
    array, drawn for the group's first projection), as q, k and v do in a
    transformer layer."""
    row_adapter = np.asarray(row_adapter, dtype=np.int32)
    ranks = np.asarray(ranks, dtype=np.int32)
    if _structure_only:
        return Structure(name, row_adapter, ranks, [(pn, di, do) for pn, di, do in projs],
                         batches or {"main": row_adapter}, layout, page_elems)
    n_rows, n_ad = row_adapter.shape[0], ranks.shape[0]
    max_rank = int(ranks.max())
    x_of = {}
    for grp in shared_x:
        for pi in grp[1:]:
            assert projs[pi][1] == projs[grp[0]][1], "projections that share x share d_in"
            x_of[pi] = grp[0]
    items, tensors = [], []
    for pi, (pname, d_in, d_out) in enumerate(projs):
        x = tensors[x_of[pi]][3] if pi in x_of else bf16_normal(seed, (_TAG_X, pi), (n_rows, d_in))
        A = [bf16_normal(seed, (_TAG_A, pi, a), (int(ranks[a]), d_in), 1.0 / math.sqrt(d_in))
             for a in range(n_ad)]
        B = [bf16_normal(seed, (_TAG_B, pi, a), (int(ranks[a]), d_out), 1.0 / math.sqrt(int(ranks[a])))
             for a in range(n_ad)]
        y0 = normal_f32(seed, (_TAG_Y0, pi), (n_rows, d_out))
        items += [((pi, "A"), d_in, A), ((pi, "B"), d_out, B)]
        tensors.append((pname, d_in, d_out, x, y0))
    pool, descs = build_pool(items, n_ad, max_rank, layout, page_elems, rng)
    projections = [Projection(pn, di, do, x, y0, descs[(pi, "A")], descs[(pi, "B")])
                   for pi, (pn, di, do, x, y0) in enumerate(tensors)]
    return Workload(name, seed, n_rows, row_adapter, ranks, pool, projections, scale,
                    batches or {"main": row_adapter}, merge, layout)


def _merge_spec(seed, adapter, n_layers, projs):
    """projs: list of (index, d_in, d_out)."""
    dims = {i: (di, do) for i, di, do in projs}

    def weight(layer, p):
        d_in, d_out = dims[p]
        return bf16_normal(seed, (_TAG_W, layer, p), (d_out, d_in), 1.0 / math.sqrt(d_in))
    return MergeSpec(adapter, n_layers, [i for i, _, _ in projs], weight)


# ----------------------------------------------------------------------------
# the five workloads
# ----------------------------------------------------------------------------
def gen_tiny(seed=0, layout="dense", n_segments=8):
    """64 rows, d 512, 4 adapters of rank 8; segment lengths a uniform
    composition of 64 (n_segments-1 distinct cut points in 1..63), adapter per
    segment U{0..3}; merge of adapter 0 into one W[512x512]."""
    rng = np.random.default_rng([seed, 0])
    n, k = 64, n_segments
    cuts = np.sort(rng.choice(np.arange(1, n), size=k - 1, replace=False)) if k > 1 else np.array([], int)
    bounds = np.concatenate([[0], cuts, [n]])
    seg_ad = rng.integers(0, 4, size=k)
    row_adapter = np.repeat(seg_ad, np.diff(bounds))
    ranks = np.full(4, 8)
    merge = _merge_spec(seed, 0, 1, [(0, 512, 512)])
    return _make("tiny", seed, row_adapter, ranks, [("proj", 512, 512)], layout, 512, rng, merge=merge)


def gen_decode(seed=1, layout="dense"):
    """64 one-token rows, d 4096, q/k/v/o, 64 adapters of rank 16.
    Batches: 'hetero' (row i -> adapter i) and 'homo' (all rows -> adapter 0).
    Merge spec: adapter 0 into the layer's four W[4096x4096]."""
    rng = np.random.default_rng([seed, 0])
    het = np.arange(64, dtype=np.int32)
    homo = np.zeros(64, dtype=np.int32)
    projs = [(p, 4096, 4096) for p in ("q", "k", "v", "o")]
    merge = _merge_spec(seed, 0, 1, [(i, 4096, 4096) for i in range(4)])
    return _make("decode", seed, het, np.full(64, 16), projs, layout, 4096, rng,
                 batches={"hetero": het, "homo": homo}, merge=merge)


def gen_prefill(seed=2, layout="dense", shared_qkv=False):
    """16 requests, lognormal lengths, 16 adapters with ranks U{8,16,32,64},
    Zipf(1.1) adapter choice, q/k/v/o at d 4096.  shared_qkv: q, k and v
    take one x (the layer input), o its own."""
    rng = np.random.default_rng([seed, 0])
    z = rng.standard_normal(16)
    lens = np.clip(np.rint(np.exp(math.log(512.0) + 0.6 * z)), 32, 2048).astype(np.int64)
    ranks = rng.choice(np.array([8, 16, 32, 64]), size=16)
    req_ad = _zipf_choice(rng, 16, 16)
    row_adapter = np.repeat(req_ad, lens)
    projs = [(p, 4096, 4096) for p in ("q", "k", "v", "o")]
    return _make("prefill", seed, row_adapter, ranks, projs, layout, 4096, rng,
                 shared_x=[(0, 1, 2)] if shared_qkv else ())


def gen_vision(seed=3, layout="dense", n_layers=32, shared_qkv=False):
    """24 requests of U{256..1024} visual + 32 text tokens, 32 adapters of rank
    64, Zipf(1.1); q/k/v/o at d 4096; mode switch of adapter 0 over
    n_layers x 4 W[4096x4096].  shared_qkv: q, k and v take one x."""
    rng = np.random.default_rng([seed, 0])
    lens = rng.integers(256, 1025, size=24) + 32
    req_ad = _zipf_choice(rng, 32, 24)
    row_adapter = np.repeat(req_ad, lens)
    projs = [(p, 4096, 4096) for p in ("q", "k", "v", "o")]
    merge = _merge_spec(seed, 0, n_layers, [(i, 4096, 4096) for i in range(4)])
    return _make("vision", seed, row_adapter, np.full(32, 64), projs, layout, 4096, rng, merge=merge,
                 shared_x=[(0, 1, 2)] if shared_qkv else ())


def gen_mix70b(seed=4, layout="paged"):
    """d 8192, q/o (8192->8192) and up (8192->28672); 256 decode rows with
    adapter U{0..127}, a random 128 of them released (-1); 8 prefill segments
    of 1024 rows with adapter U{0..127}; 128 adapters of ranks U{16,32,64};
    adapter rows in a pool of 8192-element pages under a random page table."""
    rng = np.random.default_rng([seed, 0])
    ranks = rng.choice(np.array([16, 32, 64]), size=128)
    dec = rng.integers(0, 128, size=256)
    released = rng.choice(256, size=128, replace=False)
    dec[released] = -1
    pre = np.repeat(rng.integers(0, 128, size=8), 1024)
    row_adapter = np.concatenate([dec, pre])
    projs = [("q", 8192, 8192), ("o", 8192, 8192), ("up", 8192, 28672)]
    return _make("mix70b", seed, row_adapter, ranks, projs, layout, 8192, rng)


GENERATORS = {0: gen_tiny, 1: gen_decode, 2: gen_prefill, 3: gen_vision, 4: gen_mix70b}


def gen_config(k: int, seed: Optional[int] = None, **kw) -> Workload:
    """Workload k (0 tiny, 1 decode, 2 prefill, 3 vision, 4 70B mix); the seeded instance uses seed = k."""
    return GENERATORS[k](k if seed is None else seed, **kw)


def gen_twin(k: int, seed: Optional[int] = None) -> Workload:
    """Homogeneous twin of workload k: the same rows and projections, every
    active row on one adapter whose rank is the token-weighted mean rank of
    the heterogeneous batch (flop-matched), released rows still released."""
    S = structure(k, seed)
    ra = S.row_adapter
    active = ra >= 0
    r = int(round(float(S.adapter_rank[ra[active]].mean())))
    twin = np.where(active, 0, -1).astype(np.int32)
    sd = k if seed is None else seed
    rng = np.random.default_rng([sd, 1])
    return _make(S.name + "-twin", sd, twin, np.array([r], np.int32), S.projs, S.layout, S.page_elems, rng)


def gen_custom(seed, row_adapter, ranks, d_in, d_out, n_proj=1, layout="dense",
               page_elems=None, scale=2.0, shared_x=()):
    """Small ad-hoc workload for tests: given row->adapter map and ranks."""
    rng = np.random.default_rng([seed, 0])
    projs = [(f"p{i}", d_in, d_out) for i in range(n_proj)]
    return _make("custom", seed, row_adapter, ranks, projs, layout,
                 page_elems or max(d_in, d_out), rng, scale=scale, shared_x=shared_x)
