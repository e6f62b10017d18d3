"""Copy a workload's inputs to the GPU (plain tensor copies, no arithmetic).

bf16 data travels as int16 bit patterns; kernels read them as bf16.
"""
from dataclasses import dataclass
from typing import List

import numpy as np
import torch


@dataclass
class DeviceProjection:
    x: torch.Tensor        # int16 bits [n_rows, d_in]
    y: torch.Tensor        # float32 [n_rows, d_out], initialised to y0
    A_off: torch.Tensor    # int64
    B_off: torch.Tensor    # int64


@dataclass
class DeviceWorkload:
    pool: torch.Tensor     # int16 bits
    projections: List[DeviceProjection]


def bits_to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)


def to_device(W, device="cuda") -> DeviceWorkload:
    """Projections that share one host x array share one device x."""
    pool = bits_to_device(W.pool, device)
    projs, xs = [], {}
    for p in W.projections:
        if id(p.x) not in xs:
            xs[id(p.x)] = bits_to_device(p.x, device)
        projs.append(DeviceProjection(
            x=xs[id(p.x)],
            y=torch.from_numpy(p.y0).to(device),
            A_off=torch.from_numpy(p.A.row_off).to(device),
            B_off=torch.from_numpy(p.B.row_off).to(device)))
    return DeviceWorkload(pool, projs)


def reset_outputs(W, dw: DeviceWorkload):
    for p, d in zip(W.projections, dw.projections):
        d.y.copy_(torch.from_numpy(p.y0))
