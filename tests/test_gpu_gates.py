"""Fused gate activation on the GPU: the *_gated entry points take the gate and beta
pre-activations and activate them inside every arm. Checked against the fp64 oracle
fed with the oracle's own activations (oracle/gates.py) of the same pre-activations,
and, on the sequential arms, bitwise across arms (fused, split, chained decodes)."""
import math

import numpy as np
import pytest
import torch

import gated_delta_rule_68_amd as kda
import oracle
from gated_delta_rule_68_amd.synth import CONFIGS
from gated_delta_rule_68_amd.torch_io import alloc_outputs, to_f64
from oracle import gates
from tests.gpu_util import DEV, RMS_EPS, TOL, assert_bitwise, head_slice, inputs_for, scale_of

pytestmark = pytest.mark.gpu
SEQ, CHK = kda.KDA_MODE_SEQUENTIAL, kda.KDA_MODE_CHUNKED
LB = -5.0


def _print(*a):
    print(*a, flush=True)


def gate_params(inp, dev, form):
    """(gate_a, gate_bias) device tensors and the oracle's fp64 log gate and beta."""
    cfg = inp.cfg
    if form == kda.KDA_GATE_SIGMOID:
        ga = dev["A_log"]
        g = gates.gate_sigmoid(inp.gate_x, inp.A_log, inp.dt_bias, LB, cfg.D, cfg.gdn)
    else:
        a = -np.exp(inp.A_log.astype(np.float64))
        ga = torch.from_numpy(a.astype(np.float32)).to(DEV)
        g = gates.gate_softplus(inp.gate_x, a.astype(np.float32), inp.dt_bias, LB, cfg.D, cfg.gdn)
    return ga, dev["dt_bias"], g, gates.beta_sigmoid(inp.beta_x)


def run_gated(cfg, dev, ga, gb, form, mode=SEQ, decode=False, t0=0, T=None, ring=None, state=None, lb=LB):
    T = cfg.T if T is None else T
    sl = slice(t0, t0 + T)
    acts = {n: dev[n][:, sl].clone(memory_format=torch.contiguous_format)
            for n in ("q", "k", "v", "gate_x", "beta_x", "z")}  # aligned copies, not views
    ring = dev["ring"].clone() if ring is None else ring
    s_in = dev["state"].clone() if state is None else state
    s_out = s_in if state is not None else torch.empty_like(s_in)
    outs = alloc_outputs(cfg, T, DEV, o_core=True)
    args = (acts["q"], acts["k"], acts["v"], acts["gate_x"], acts["beta_x"], ga, gb, dev["conv_w"], ring,
            s_in, s_out, acts["z"], dev["norm_w"], outs["out"], outs["o_core"])
    kw = dict(gate_form=form, gate_lb=lb, scale=scale_of(cfg), rms_eps=RMS_EPS)
    if decode:
        (kda.gdn_decode_gated if cfg.gdn else kda.kda_decode_gated)(*args, **kw)
    else:
        code = kda.KDA_DTYPE_BF16 if cfg.dtype == "bf16" else kda.KDA_DTYPE_F32
        nb = kda.workspace_bytes(cfg.B, T, cfg.H, cfg.D, code, mode, gdn=cfg.gdn)
        ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=DEV) if nb else None
        (kda.gdn_prefill_gated if cfg.gdn else kda.kda_prefill_gated)(*args, **kw, mode=mode, workspace=ws)
    return {"out": outs["out"], "o_core": outs["o_core"], "ring": ring, "state": s_out}


def oracle_gated(inp, g, beta, heads, batches=None, threads=16):
    cfg = inp.cfg
    d, ch, rows, bsel = head_slice(inp, heads, batches)
    d["g"] = np.ascontiguousarray(g[bsel][:, :, heads] if cfg.gdn else g[bsel][:, :, ch])
    d["beta"] = np.ascontiguousarray(beta[bsel][:, :, heads])
    r = oracle.mixer(**d, scale=scale_of(cfg), rms_eps=RMS_EPS, gdn=cfg.gdn, threads=threads)
    return r, ch, rows, bsel


def compare(cfg, got, ref, ch, rows, bsel, heads, tol):
    errs = {"out": oracle.rel_linf(to_f64(got["out"])[bsel][:, :, ch], ref["out"]),
            "o_core": oracle.rel_linf(to_f64(got["o_core"])[bsel][:, :, ch], ref["o_core"]),
            "state": oracle.rel_linf(to_f64(got["state"])[bsel][:, heads], ref["state"]),
            "ring": oracle.rel_linf(to_f64(got["ring"])[bsel][:, rows], ref["ring"])}
    _print("errs", errs)
    for k, e in errs.items():
        assert e <= tol, f"{k}: {e:.3e} > {tol}"
    assert errs["ring"] == 0.0


FORMS = [kda.KDA_GATE_SIGMOID, kda.KDA_GATE_SOFTPLUS]


@pytest.mark.parametrize("form", FORMS, ids=["sigmoid", "softplus"])
@pytest.mark.parametrize("gdn", [False, True])
@pytest.mark.parametrize("mode,T", [(SEQ, 37), (CHK, 37), (CHK, 200)], ids=["seq37", "chunk37", "chunk200"])
def test_gated_prefill_vs_oracle(form, gdn, mode, T):
    cfg = CONFIGS["kda_decode"].with_(B=2, H=3, T=T, gdn=gdn)
    inp, dev = inputs_for(cfg)
    ga, gb, g, beta = gate_params(inp, dev, form)
    got = run_gated(cfg, dev, ga, gb, form, mode=mode)
    torch.cuda.synchronize()
    ref, ch, rows, bsel = oracle_gated(inp, g, beta, heads=[0, 1, 2])
    compare(cfg, got, ref, ch, rows, bsel, [0, 1, 2], TOL["bf16"])


@pytest.mark.parametrize("gdn", [False, True])
def test_gated_unbounded_gates_auto_vs_oracle(gdn):
    """Softplus gates with no lower bound (gate_lb = -inf) and pre-activations shifted
    up by 3, so that most log gates lie between about -50 and -3, far below the chunked
    arm's -5. AUTO at bf16, D = 128, T = 200 (which would take the chunked arm for given
    gates) runs them on the fused sequential arm and matches the oracle."""
    cfg = CONFIGS["kda_decode"].with_(B=2, H=3, T=200, gdn=gdn)
    inp, dev = inputs_for(cfg)
    assert kda.ARM_NAMES[kda.prefill_arm(cfg.B, cfg.T, cfg.H, cfg.D, kda.KDA_DTYPE_BF16,
                                         kda.KDA_MODE_AUTO, gdn=gdn)] in ("chunked", "segmented")
    shifted = (inp.gate_x.astype(np.float32) + 3.0)
    dev = dict(dev)
    dev["gate_x"] = torch.from_numpy(shifted).to(DEV, dev["gate_x"].dtype)
    gx = to_f64(dev["gate_x"].cpu())  # the values the kernels read (bf16-rounded)
    a = -np.exp(inp.A_log.astype(np.float64))
    ga = torch.from_numpy(a.astype(np.float32)).to(DEV)
    g = gates.gate_softplus(gx, a.astype(np.float32), inp.dt_bias, -np.inf, cfg.D, cfg.gdn)
    assert float(np.mean(g < -5.0)) > 0.5, "most gates should lie below -5"
    beta = gates.beta_sigmoid(inp.beta_x)
    got = run_gated(cfg, dev, ga, dev["dt_bias"], kda.KDA_GATE_SOFTPLUS, mode=kda.KDA_MODE_AUTO, lb=-np.inf)
    torch.cuda.synchronize()
    ref, ch, rows, bsel = oracle_gated(inp, g, beta, heads=[0, 1, 2])
    compare(cfg, got, ref, ch, rows, bsel, [0, 1, 2], TOL["bf16"])


@pytest.mark.parametrize("form", FORMS, ids=["sigmoid", "softplus"])
@pytest.mark.parametrize("gdn", [False, True])
@pytest.mark.parametrize("B", [2, 4], ids=["two_splits", "full_width"])
def test_gated_chunked_wide_vs_oracle(form, gdn, B):
    """H = 64 heads at B = 2 (each head split over two column blocks) and B = 4 (one
    workgroup per head): the other chunked launch widths, on sampled heads."""
    cfg = CONFIGS["kda_decode"].with_(B=B, H=64, T=130, gdn=gdn)
    inp, dev = inputs_for(cfg)
    ncol = 2 if B == 2 else 1
    assert kda.ARM_NAMES[kda.prefill_arm(cfg.B, cfg.T, cfg.H, cfg.D, kda.KDA_DTYPE_BF16, CHK, gdn=gdn)] == "chunked"
    _print("case", cfg, "column splits", ncol)
    ga, gb, g, beta = gate_params(inp, dev, form)
    got = run_gated(cfg, dev, ga, gb, form, mode=CHK)
    torch.cuda.synchronize()
    heads, batches = [0, 37, 63], [0, B - 1]
    ref, ch, rows, bsel = oracle_gated(inp, g, beta, heads=heads, batches=batches)
    compare(cfg, got, ref, ch, rows, bsel, heads, TOL["bf16"])


@pytest.mark.parametrize("form", FORMS, ids=["sigmoid", "softplus"])
@pytest.mark.parametrize("gdn", [False, True])
def test_gated_fp32_sequential_vs_oracle(form, gdn):
    cfg = CONFIGS["tiny_kda"].with_(gdn=gdn, T=40, random_init=True)
    inp, dev = inputs_for(cfg)
    ga, gb, g, beta = gate_params(inp, dev, form)
    got = run_gated(cfg, dev, ga, gb, form, mode=SEQ)
    torch.cuda.synchronize()
    ref, ch, rows, bsel = oracle_gated(inp, g, beta, heads=list(range(cfg.H)))
    compare(cfg, got, ref, ch, rows, bsel, list(range(cfg.H)), TOL["fp32"])


@pytest.mark.parametrize("gdn", [False, True])
def test_gated_sequential_arms_bitwise(gdn):
    """Fused prefill == split prefill == chained gated decodes, bit for bit."""
    form = kda.KDA_GATE_SOFTPLUS
    cfg = CONFIGS["kda_decode"].with_(B=1, H=2, T=40, D=16, dtype="fp32", gdn=gdn)
    inp, dev = inputs_for(cfg)
    ga, gb, _, _ = gate_params(inp, dev, form)
    assert kda.prefill_arm(cfg.B, cfg.T, cfg.H, cfg.D, 0, SEQ) == 2  # split
    split = run_gated(cfg, dev, ga, gb, form, mode=SEQ)
    ring, state = dev["ring"].clone(), dev["state"].clone()
    outs = []
    for t in range(cfg.T):
        outs.append(run_gated(cfg, dev, ga, gb, form, decode=True, t0=t, T=1, ring=ring, state=state)["out"])
    torch.cuda.synchronize()
    assert_bitwise(split, {"out": torch.cat(outs, 1), "ring": ring, "state": state}, keys=("out", "ring", "state"))
    # fused arm (T <= 16) against the first 16 decodes
    fused = run_gated(cfg, dev, ga, gb, form, mode=SEQ, T=16)
    torch.cuda.synchronize()
    assert_bitwise({"out": fused["out"]}, {"out": torch.cat(outs[:16], 1)}, keys=("out",))


def test_softplus_form_reproduces_the_given_gates():
    """The softplus form with a = -exp(A_log), lb = -5 is the generator's own gate, so the
    gated call agrees with the plain call on the generator's g (bf16-rounded there) to
    bf16 accuracy, on the chunked arm at full prefill width."""
    cfg = CONFIGS["kda_decode"].with_(B=1, H=64, T=300)
    inp, dev = inputs_for(cfg)
    ga, gb, _, _ = gate_params(inp, dev, kda.KDA_GATE_SOFTPLUS)
    got = run_gated(cfg, dev, ga, gb, kda.KDA_GATE_SOFTPLUS, mode=CHK)
    from tests.gpu_util import run_gpu
    ref = run_gpu(cfg, dev, mode=CHK)
    torch.cuda.synchronize()
    for k in ("out", "state"):
        e = oracle.rel_linf(to_f64(got[k]), to_f64(ref[k]))
        _print(k, e)
        assert e <= TOL["bf16"]


def _rollback_gated(cfg, dev, ga, gb, form, ring_snap, state_snap, ring, state, keep):
    code = kda.KDA_DTYPE_BF16 if cfg.dtype == "bf16" else kda.KDA_DTYPE_F32
    nb = kda.rollback_workspace_bytes(cfg.B, keep, cfg.H, cfg.D, code, gdn=cfg.gdn)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV) if nb else None
    fn = kda.gdn_rollback_gated if cfg.gdn else kda.kda_rollback_gated
    fn(dev["q"], dev["k"], dev["v"], dev["gate_x"], dev["beta_x"], ga, gb, dev["conv_w"], ring_snap,
       state_snap, ring, state, keep, gate_form=form, gate_lb=LB, workspace=ws)


@pytest.mark.parametrize("form", FORMS, ids=["sigmoid", "softplus"])
@pytest.mark.parametrize("gdn", [False, True])
def test_gated_verify_then_rollback_is_bitwise_the_gated_decode_chain(form, gdn):
    """A round verified with the gated sequential prefill, rolled back with the gated
    rollback to keep rows, equals keep chained gated decodes bit for bit."""
    cfg = CONFIGS["kda_decode"].with_(B=2, H=3, T=8, gdn=gdn)
    inp, dev = inputs_for(cfg)
    ga, gb, _, _ = gate_params(inp, dev, form)
    ring, state = dev["ring"].clone(), dev["state"].clone()
    steps = []
    for t in range(cfg.T):
        run_gated(cfg, dev, ga, gb, form, decode=True, t0=t, T=1, ring=ring, state=state)
        steps.append({"ring": ring.clone(), "state": state.clone()})
    verify = run_gated(cfg, dev, ga, gb, form, mode=SEQ)
    torch.cuda.synchronize()
    assert_bitwise(verify, steps[-1], keys=("ring", "state"))
    for keep in (1, 3, cfg.T):
        ring = torch.full_like(dev["ring"], float("nan"))
        state = torch.full_like(dev["state"], float("nan"))
        _rollback_gated(cfg, dev, ga, gb, form, dev["ring"], dev["state"], ring, state, keep)
        torch.cuda.synchronize()
        assert_bitwise({"ring": ring, "state": state}, steps[keep - 1], keys=("ring", "state"))
        _print("keep", keep, "bitwise ok")


def test_gated_rollback_split_arm_matches_gated_prefill():
    """keep > 16 rows with few (b, h) pairs: the split arm (with a workspace) equals a
    gated sequential prefill over the same first keep rows."""
    cfg = CONFIGS["kda_decode"].with_(B=1, H=2, T=40, D=16, dtype="fp32")
    inp, dev = inputs_for(cfg)
    form, keep = kda.KDA_GATE_SIGMOID, 30
    ga, gb, _, _ = gate_params(inp, dev, form)
    assert kda.prefill_arm(cfg.B, keep, cfg.H, cfg.D, kda.KDA_DTYPE_F32, SEQ) == 2
    ref = run_gated(cfg, dev, ga, gb, form, mode=SEQ, T=keep)
    ring, state = torch.empty_like(dev["ring"]), torch.empty_like(dev["state"])
    _rollback_gated(cfg, dev, ga, gb, form, dev["ring"], dev["state"], ring, state, keep)
    torch.cuda.synchronize()
    assert_bitwise({"ring": ring, "state": state}, ref, keys=("ring", "state"))
