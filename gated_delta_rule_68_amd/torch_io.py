"""Move seeded host inputs (``synth.Inputs``) into device tensors and allocate the
outputs of one call. PyTorch only provides device memory and streams here."""
from __future__ import annotations

import numpy as np
import torch

from .synth import Inputs

ACTS = ("q", "k", "v", "g", "beta", "z", "gate_x", "beta_x")


def _act_tensor(inp: Inputs, name: str, device) -> torch.Tensor:
    if inp.cfg.dtype == "bf16":
        bits = inp.bits[name]
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(getattr(inp, name), np.float32)).to(device)


def to_device(inp: Inputs, device="cuda") -> dict:
    d = {n: _act_tensor(inp, n, device) for n in ACTS}
    for n in ("conv_w", "norm_w", "ring", "state", "A_log", "dt_bias"):
        d[n] = torch.from_numpy(np.ascontiguousarray(getattr(inp, n), np.float32)).to(device)
    return d


def tiled_device_inputs(cfg, period: int = 1024, device="cuda") -> dict:
    """Device inputs of a long workload: the seeded generator draws the first `period`
    tokens of every sequence and they are repeated up to cfg.T (values keep the
    workload's distributions; tokens [0, period) are exactly the generator's)."""
    from .synth import make_inputs

    small = to_device(make_inputs(cfg, T=min(period, cfg.T)), device)
    reps = (cfg.T + period - 1) // period
    out = {}
    for n, t in small.items():
        if n in ACTS:
            out[n] = t.repeat(1, reps, *([1] * (t.dim() - 2)))[:, :cfg.T].contiguous()
        else:
            out[n] = t
    return out


def act_dtype(cfg) -> torch.dtype:
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def alloc_outputs(cfg, T: int, device="cuda", o_core: bool = True) -> dict:
    shape = (cfg.B, T, cfg.qkv)
    return {"out": torch.empty(shape, dtype=act_dtype(cfg), device=device),
            "o_core": torch.empty(shape, dtype=torch.float32, device=device) if o_core else None}


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)
