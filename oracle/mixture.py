"""deLoRA mixture inference in fp64 (test infrastructure only).

VaLoRA blog (EuroSys'25), section 4.4.2 "Mixture Inference Mode": while
adapter m is merged into the base weights (W_merge = W_base + Delta W_m), a
request on another adapter x is served with the weights
W_merge - Delta W_deLoRA_m + Delta W_x, where Delta W_deLoRA_m equals
Delta W_m: the merged adapter is subtracted and the wanted one added, with no
change to the weights in memory.

A request with no adapter runs on the backbone alone: the LoRazor article's
mechanism section releases a request's adapter early and serves the request
on the backbone from then on.  With W_merge resident, the backbone weights
are W_merge - Delta W_m: the formula above with Delta W_x = 0.

On the delta path the merged GEMM y0 = x * W_merge^T is shared by all rows, so
row i with adapter a = row_adapter[i] gets

    y[i] = y0[i] + s * (x_i A_a^T) B_a - s * (x_i A_m^T) B_m     (a >= 0, a != m)
    y[i] = y0[i]                                                  (a == m: served by W_merge)
    y[i] = y0[i] - s * (x_i A_m^T) B_m                            (a == -1: released, backbone)

``base_rows=False`` leaves released rows at y0 instead (rows whose output is
not wanted, such as padding).

fp64 arithmetic on the exact values of the bf16 inputs, as in ``lora``.
"""
import numpy as np

from .bf16 import bf16_to_f64
from .lora import gather_rows_ref


def mixture_ref(row_adapter, adapter_rank, merged, x_bits, y0, pool, A, B, scale, rows=None, base_rows=True):
    """Returns {i: fp64 y row} for each i in ``rows`` (default: all rows)."""
    rows = range(len(row_adapter)) if rows is None else rows

    def both(a):
        r = int(adapter_rank[a])
        return (gather_rows_ref(pool, A.row_off, A.max_rank, A.row_len, A.chunk_len, a, r),
                gather_rows_ref(pool, B.row_off, B.max_rank, B.row_len, B.chunk_len, a, r))

    Am, Bm = both(int(merged))
    out = {}
    for i in rows:
        a = int(row_adapter[i])
        y = np.asarray(y0[i], dtype=np.float64).copy()
        if a >= 0 and a != int(merged):
            Aa, Ba = both(a)
            xi = bf16_to_f64(x_bits[i])
            add = (Aa @ xi) @ Ba          # s-free delta of the wanted adapter
            sub = (Am @ xi) @ Bm          # and of the merged one
            y += scale * add - scale * sub
        elif a == -1 and base_rows:
            xi = bf16_to_f64(x_bits[i])
            y -= scale * ((Am @ xi) @ Bm)  # back to the backbone: minus the merged adapter
        out[i] = y
    return out
