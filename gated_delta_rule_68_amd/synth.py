"""Seeded synthetic inputs for the KDA / GDN mixer.

This module only draws numbers; it holds none of the mixer's arithmetic. Both the
HIP path (through the tests and the benchmark) and the fp64 oracle receive the
arrays it returns, so the two sides always see identical values.

Recipe (one independent numpy PCG64 stream per (tensor, sequence)):

* every tensor ``name`` of sequence ``b`` draws from ``default_rng([seed, id(name), b])``;
  per-layer tensors (conv weight, A_log, dt_bias, norm weight) use ``b = 0``.
  Token rows are drawn in token order, so the first ``T'`` tokens of a run with
  ``T > T'`` are exactly the inputs of a run with ``T'`` tokens (prefix property);
* values are drawn in fp64, cast to fp32, and for bf16 configurations the
  activations (q, k, v, g, beta, z) are then rounded to bf16 (round to nearest
  even). State, conv ring, conv weight and norm weight always stay fp32;
* q, k, v raw ~ N(0, 1); conv weight ~ N(0, 0.5) (0.5 is the standard deviation);
  with grouped heads (Hk < H, GDN) q and k have Hk heads and the conv weight and
  ring have 2*Hk*D + H*D rows (planes q, k, v);
  beta = sigmoid(N(0, 1)) per (token, head);
  log gate g = max(-5, -exp(A_log[h]) * softplus(x + dt_bias)), x ~ N(0, 1),
  A_log ~ U(0, ln 16) per head, dt_bias ~ N(0, 0.1) per channel (KDA) or per head
  (GDN); in the "alternating" regime x ~ N(+2, 1) on even heads and N(-2, 1) on
  odd heads; output gate z ~ N(0, 1); norm weight ~ N(1, 0.1) per head_dim entry;
* conv ring and recurrent state are zero for prefill configurations; for the
  decode configuration the ring is N(0, 1) (it holds raw inputs) and the state
  is N(0, 0.02).
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

_TENSOR_IDS = {
    "q": 1, "k": 2, "v": 3, "conv_w": 4, "beta_x": 5, "A_log": 6, "dt_bias": 7,
    "gate_x": 8, "z": 9, "norm_w": 10, "ring": 11, "state": 12,
}


@dataclass(frozen=True)
class Config:
    """One workload: shapes, dtype and value regime."""

    name: str
    B: int
    T: int
    H: int
    D: int
    K: int = 4
    dtype: str = "bf16"          # activations: "fp32" or "bf16"
    gdn: bool = False            # scalar gate per (token, head) and SiLU output gate
    gate_regime: str = "normal"  # "normal" or "alternating" (+2 / -2 shift by head parity)
    random_init: bool = False    # random state and ring (decode) instead of zeros (prefill)
    chunk: int = 64
    Hk: int = 0                  # query / key heads (GDN grouped heads); 0 means H

    @property
    def qkv(self) -> int:
        """Width of the value-head rows (v, z, out): H * D."""
        return self.H * self.D

    @property
    def hk(self) -> int:
        return self.Hk or self.H

    @property
    def kw(self) -> int:
        """Width of the query / key rows: Hk * D."""
        return self.hk * self.D

    @property
    def conv_rows(self) -> int:
        """Conv-weight and ring rows: planes q, k (Hk * D each), v (H * D)."""
        return 2 * self.kw + self.qkv

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


# The five workloads: tiny KDA parity case, the batched decode step, single-sequence
# prefill, the scalar-gate GDN prefill, and the long batched prefill with gates pushed
# to both ends of [-5, 0] on alternate heads.
CONFIGS = {
    "tiny_kda": Config("tiny_kda", B=1, T=64, H=2, D=16, dtype="fp32"),
    "kda_decode": Config("kda_decode", B=64, T=1, H=64, D=128, random_init=True),
    "kda_prefill": Config("kda_prefill", B=1, T=4626, H=64, D=128),
    "gdn_prefill": Config("gdn_prefill", B=4, T=8192, H=32, D=128, gdn=True),
    "kda_long": Config("kda_long", B=8, T=16384, H=64, D=128, gate_regime="alternating"),
}


def _rng(seed: int, name: str, b: int = 0) -> np.random.Generator:
    return np.random.default_rng([seed, _TENSOR_IDS[name], b])


def bf16_bits(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even. Inputs are finite."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    return ((u + (((u >> 16) & 1) + 0x7FFF)) >> 16).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x)


@dataclass
class Inputs:
    """Host arrays for one call. Activations are fp32 arrays holding exactly the values
    the kernel sees (already bf16-rounded for bf16 configs); ``bits`` holds the bf16
    bit patterns of the activations for bf16 configs."""

    cfg: Config
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    z: np.ndarray
    conv_w: np.ndarray
    norm_w: np.ndarray
    ring: np.ndarray
    state: np.ndarray
    bits: dict
    # The draws the gate and beta come from (the pre-activations as the kernel sees
    # them, like the activations above, and the per-head / per-channel parameters):
    # g = max(-5, -exp(A_log[h]) * softplus(gate_x + dt_bias)), beta = sigmoid(beta_x).
    gate_x: np.ndarray = None
    beta_x: np.ndarray = None
    A_log: np.ndarray = None
    dt_bias: np.ndarray = None

    def f64(self, name: str) -> np.ndarray:
        return getattr(self, name).astype(np.float64)


def _per_seq(seed, name, B, shape_one, loc=0.0, scale=1.0) -> np.ndarray:
    out = np.empty((B,) + shape_one, dtype=np.float32)
    for b in range(B):
        out[b] = (loc + scale * _rng(seed, name, b).standard_normal(shape_one)).astype(np.float32)
    return out


def make_inputs(cfg: Config, seed: int = 0, T: int | None = None) -> Inputs:
    """Draw the inputs of ``cfg`` (optionally only the first ``T`` tokens)."""
    T = cfg.T if T is None else T
    B, H, D, K, qkv = cfg.B, cfg.H, cfg.D, cfg.K, cfg.qkv
    q = _per_seq(seed, "q", B, (T, cfg.kw))
    k = _per_seq(seed, "k", B, (T, cfg.kw))
    v = _per_seq(seed, "v", B, (T, qkv))
    conv_w = (0.5 * _rng(seed, "conv_w").standard_normal((cfg.conv_rows, K))).astype(np.float32)
    beta_x = _per_seq(seed, "beta_x", B, (T, H)).astype(np.float64)
    beta = (1.0 / (1.0 + np.exp(-beta_x))).astype(np.float32)
    A_log = _rng(seed, "A_log").uniform(0.0, np.log(16.0), H)
    gw = H if cfg.gdn else qkv
    dt_bias = 0.1 * _rng(seed, "dt_bias").standard_normal(gw)
    gx = _per_seq(seed, "gate_x", B, (T, gw)).astype(np.float64)
    head_of = np.arange(gw) if cfg.gdn else np.arange(gw) // D
    if cfg.gate_regime == "alternating":
        gx = gx + np.where(head_of % 2 == 0, 2.0, -2.0)
    g = np.maximum(-5.0, -np.exp(A_log[head_of]) * _softplus(gx + dt_bias)).astype(np.float32)
    z = _per_seq(seed, "z", B, (T, qkv))
    norm_w = (1.0 + 0.1 * _rng(seed, "norm_w").standard_normal(D)).astype(np.float32)
    if cfg.random_init:
        ring = _per_seq(seed, "ring", B, (cfg.conv_rows, K - 1))
        state = _per_seq(seed, "state", B, (H, D, D), scale=0.02)
    else:
        ring = np.zeros((B, cfg.conv_rows, K - 1), np.float32)
        state = np.zeros((B, H, D, D), np.float32)
    gate_x, beta_x32 = gx.astype(np.float32), beta_x.astype(np.float32)
    bits = {}
    if cfg.dtype == "bf16":
        acts = {"q": q, "k": k, "v": v, "g": g, "beta": beta, "z": z, "gate_x": gate_x, "beta_x": beta_x32}
        bits = {n: bf16_bits(a) for n, a in acts.items()}
        q, k, v, g, beta, z, gate_x, beta_x32 = (bf16_to_f32(bits[n]) for n in acts)
    elif cfg.dtype != "fp32":
        raise ValueError(f"unknown dtype {cfg.dtype}")
    return Inputs(cfg, q, k, v, g, beta, z, conv_w, norm_w, ring, state, bits, gate_x, beta_x32,
                  A_log.astype(np.float32), dt_bias.astype(np.float32))
