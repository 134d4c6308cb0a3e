"""Helpers for the GPU tests: run the library through its C ABI on seeded inputs,
run the oracle on the same inputs (optionally on a sample of heads / sequences),
and compare."""
from __future__ import annotations

import math

import numpy as np
import torch

import gated_delta_rule_68_amd as kda
import oracle
from gated_delta_rule_68_amd.synth import Config, Inputs, make_inputs
from gated_delta_rule_68_amd.torch_io import alloc_outputs, to_device, to_f64

DEV = "cuda"
RMS_EPS = 1e-5
TOL = {"fp32": 1e-3, "bf16": 2e-2}


def scale_of(cfg: Config) -> float:
    return 1.0 / math.sqrt(cfg.D)


def run_gpu(cfg: Config, dev: dict, mode=kda.KDA_MODE_SEQUENTIAL, decode=False,
            inplace=False, t0=0, T=None, ring=None, state=None, o_core=True):
    """One prefill (or decode) over tokens [t0, t0+T) of the device inputs.
    ring / state default to fresh copies of the config's initial values.
    Returns dict(out, o_core, ring, state) as device tensors."""
    T = cfg.T if T is None else T
    sl = slice(t0, t0 + T)
    # fresh copies: a contiguous row slice at B == 1 would be a view at an offset that
    # need not meet the entry points' 16-byte alignment
    acts = {n: dev[n][:, sl].clone(memory_format=torch.contiguous_format)
            for n in ("q", "k", "v", "g", "beta", "z")}
    ring = dev["ring"].clone() if ring is None else ring
    s_in = dev["state"].clone() if state is None else state
    s_out = s_in if inplace else torch.empty_like(s_in)
    outs = alloc_outputs(cfg, T, DEV, o_core=o_core)
    args = (acts["q"], acts["k"], acts["v"], acts["g"], acts["beta"], dev["conv_w"], ring,
            s_in, s_out, acts["z"], dev["norm_w"], outs["out"], outs["o_core"])
    if decode:
        fn = kda.gdn_decode if cfg.gdn else kda.kda_decode
        fn(*args, scale=scale_of(cfg), rms_eps=RMS_EPS)
    else:
        fn = kda.gdn_prefill if cfg.gdn else kda.kda_prefill
        q = acts["q"]
        code = kda.KDA_DTYPE_BF16 if q.dtype == torch.bfloat16 else kda.KDA_DTYPE_F32
        nbytes = kda.workspace_bytes(cfg.B, T, cfg.H, cfg.D, code, mode, gdn=cfg.gdn)
        if nbytes == (1 << 64) - 1:  # arguments the prefill refuses: the call reports it
            nbytes = 0
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=DEV) if nbytes else None
        fn(*args, scale=scale_of(cfg), rms_eps=RMS_EPS, mode=mode, workspace=ws)
    return {"out": outs["out"], "o_core": outs["o_core"], "ring": ring, "state": s_out}


def head_slice(inp: Inputs, heads, batches=None):
    """The inputs of a sub-problem made of the given heads (and sequences): heads are
    independent inside the mixer, so the oracle can run on a sample of them."""
    cfg = inp.cfg
    D, qkv = cfg.D, cfg.qkv
    bsel = np.arange(cfg.B) if batches is None else np.asarray(batches)
    ch = np.concatenate([np.arange(h * D, (h + 1) * D) for h in heads])
    rows = np.concatenate([p * qkv + ch for p in range(3)])
    f = lambda a: a.astype(np.float64)  # noqa: E731
    d = {
        "q": f(inp.q[bsel][:, :, ch]), "k": f(inp.k[bsel][:, :, ch]), "v": f(inp.v[bsel][:, :, ch]),
        "g": f(inp.g[bsel][:, :, heads] if cfg.gdn else inp.g[bsel][:, :, ch]),
        "beta": f(inp.beta[bsel][:, :, heads]), "z": f(inp.z[bsel][:, :, ch]),
        "conv_w": f(inp.conv_w[rows]), "ring": f(inp.ring[bsel][:, rows]),
        "state": f(inp.state[bsel][:, heads]), "norm_w": f(inp.norm_w),
    }
    return d, ch, rows, bsel


def oracle_run(inp: Inputs, heads=None, batches=None, T=None, threads=8):
    """Oracle over (a sample of) the problem. Returns (result dict, channel index,
    ring-row index, batch index) so GPU outputs can be sliced the same way."""
    cfg = inp.cfg
    heads = list(range(cfg.H)) if heads is None else list(heads)
    d, ch, rows, bsel = head_slice(inp, heads, batches)
    if T is not None:
        for n in ("q", "k", "v", "g", "beta", "z"):
            d[n] = np.ascontiguousarray(d[n][:, :T])
    r = oracle.mixer(**d, scale=scale_of(cfg), rms_eps=RMS_EPS, gdn=cfg.gdn, threads=threads)
    return r, ch, rows, bsel, heads


def compare_to_oracle(cfg, got: dict, ref, ch, rows, bsel, heads, T=None, tol=None):
    """rel L-inf per tensor on the sampled heads / sequences. Returns the errors."""
    tol = TOL[cfg.dtype] if tol is None else tol
    T = got["out"].shape[1] if T is None else T
    errs = {}
    out = to_f64(got["out"])[bsel][:, :T][:, :, ch]
    errs["out"] = oracle.rel_linf(out, ref["out"])
    if got.get("o_core") is not None:
        errs["o_core"] = oracle.rel_linf(to_f64(got["o_core"])[bsel][:, :T][:, :, ch], ref["o_core"])
    errs["state"] = oracle.rel_linf(to_f64(got["state"])[bsel][:, heads], ref["state"])
    errs["ring"] = oracle.rel_linf(to_f64(got["ring"])[bsel][:, rows], ref["ring"])
    for k, e in errs.items():
        assert e <= tol, f"{cfg.name}: {k} rel L-inf {e:.3e} > {tol:.1e} (all: {errs})"
    assert errs["ring"] == 0.0, f"ring must be an exact copy of raw inputs: {errs}"
    return errs


def assert_bitwise(a: dict, b: dict, keys=("out", "o_core", "ring", "state")):
    for k in keys:
        if a.get(k) is None or b.get(k) is None:
            continue
        x, y = a[k], b[k]
        assert x.shape == y.shape, (k, x.shape, y.shape)
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32),
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32)), \
            f"{k} differs bitwise (max abs diff {(x.float() - y.float()).abs().max().item()})"


def inputs_for(cfg: Config, T=None):
    inp = make_inputs(cfg, T=T)
    return inp, to_device(inp, DEV)
