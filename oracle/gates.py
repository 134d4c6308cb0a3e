"""Gate and beta activations in fp64, written from their definitions.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle``): the fused-activation entry
points of the library are checked against the mixer oracle fed with these.

- memra-engine kda.rs, stage 4 (gates) and its per-channel forget-gate kernel: the
  KDA log gate of channel c = h*D + i is lb * sigmoid(exp(A_log[h]) * (f + dt_bias[c]))
  and beta is sigmoid of its own pre-activation.
- aprender-serve gdn_ops.rs, the per-head gates: the GDN log gate of head h is
  a[h] * softplus(alpha + dt_bias[h]) (a < 0), beta = sigmoid(beta_raw); here the same
  form serves KDA too (per channel), optionally bounded below.
"""
from __future__ import annotations

import numpy as np


def _head_of(width: int, D: int, gdn: bool) -> np.ndarray:
    """Head of every gate column: the column itself for GDN ([..., H]), c // D for KDA."""
    cols = np.arange(width)
    return cols if gdn else cols // D


def gate_sigmoid(x, A_log, dt_bias, lb, D, gdn=False):
    """g = lb * sigmoid(exp(A_log[h]) * (x + dt_bias[c])) over the last axis of x."""
    x = np.asarray(x, np.float64)
    h = _head_of(x.shape[-1], D, gdn)
    t = np.exp(np.asarray(A_log, np.float64)[h]) * (x + np.asarray(dt_bias, np.float64))
    return lb / (1.0 + np.exp(-t))


def gate_softplus(x, a, dt_bias, lb, D, gdn=False):
    """g = max(lb, a[h] * softplus(x + dt_bias[c])); softplus(t) = ln(1 + e^t)."""
    x = np.asarray(x, np.float64)
    h = _head_of(x.shape[-1], D, gdn)
    sp = np.logaddexp(0.0, x + np.asarray(dt_bias, np.float64))
    return np.maximum(lb, np.asarray(a, np.float64)[h] * sp)


def beta_sigmoid(b):
    return 1.0 / (1.0 + np.exp(-np.asarray(b, np.float64)))
