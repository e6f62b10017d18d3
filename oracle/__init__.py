"""CPU oracle for heterogeneous LoRA batching -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct fp64 reference of what the hot path computes.
Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  It shares no code with the HIP path (no kernels,
headers, helpers or tables) and imports nothing from it; the two meet only on
the seeded inputs drawn by ``workloads``.

What it follows (page titles as printed; sections named on the page):

* BEE-30060 "Multi-LoRA serving and adapter management", Punica paragraph:
  every request adds its own delta y_i += x_i * A_i * B_i while the base GEMM is
  shared; SGMV groups requests by adapter identity.  Same page, background
  paragraph: the update is Delta W = B * A with r*(d_in + d_out) parameters.
* S-LoRA article, "Batching" section: formula 1 (merge the adapter into W) vs
  formula 2 (compute x*A*B on the fly, batched with no padding); "Unified
  Paging" section: a rank-R adapter weight occupies R pages of hidden-size
  vectors.
* VaLoRA blog (EuroSys'25), section 4.4.1 "Swift Inference Mode Switch":
  Delta W = B x A computed at run time and added to / subtracted from W once.
* LoRazor news article, "mechanism" section: LoRA work is launched over the
  rows whose adapter is still held; released rows get no LoRA work.
* VaLoRA blog, section 4.4.2 "Mixture Inference Mode" (deLoRA): with adapter
  m merged, a request on adapter x uses W_merge - Delta W_m + Delta W_x
  (``mixture``).

Readings where the pages are silent (kept identical in the HIP path's docs):
A is stored [r][d_in] and B [r][d_out] (both as r hidden-size vectors), W as
[d_out][d_in]; shrink v = x A^T, expand y += s v B, merge W += s B^T A.
Inputs are bf16, v and y fp32, W bf16 rounded once (round-to-nearest-even)
per merge or unmerge.

Parity status: every function here is pinned by ``tests/test_oracle.py``
(closed forms, hand-worked fixtures in ``tests/golden/``, library special
cases, invariants); none is "parity unpinned".
"""
from .bf16 import bf16_to_f64, f64_to_bf16_rne
from .segments import build_segments_ref, SegmentsRef, dense_offsets_ref, SegmentError
from .lora import gather_rows_ref, apply_ref, merge_ref, unmerge_ref, merge_dense_ref
from .plan_check import check_plan_coverage
from .mixture import mixture_ref

__all__ = [
    "bf16_to_f64", "f64_to_bf16_rne", "build_segments_ref", "SegmentsRef",
    "dense_offsets_ref", "SegmentError", "gather_rows_ref", "apply_ref",
    "merge_ref", "unmerge_ref", "merge_dense_ref", "check_plan_coverage", "mixture_ref",
]
