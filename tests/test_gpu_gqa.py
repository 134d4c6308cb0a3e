"""GDN with grouped query / key heads on the GPU (gdn_prefill_gqa, gdn_decode_gqa,
gdn_rollback_gqa): parity with the grouped-head oracle (oracle/gqa.py) on every arm,
bitwise agreement of the sequential arms with chained decodes, Hk = H equal to the
plain entry points bit for bit, and the decode workload at full size on sampled
heads."""
import numpy as np
import pytest
import torch

import gated_delta_rule_68_amd as kda
import oracle
from gated_delta_rule_68_amd.synth import CONFIGS
from gated_delta_rule_68_amd.torch_io import alloc_outputs, to_f64
from oracle import gqa
from tests.gpu_util import DEV, RMS_EPS, TOL, assert_bitwise, inputs_for, run_gpu, scale_of

pytestmark = pytest.mark.gpu
SEQ, CHK, SEG = kda.KDA_MODE_SEQUENTIAL, kda.KDA_MODE_CHUNKED, kda.KDA_MODE_SEGMENTED


def _print(*a):
    print(*a, flush=True)


def run_gqa(cfg, dev, mode=SEQ, decode=False, t0=0, T=None, ring=None, state=None, gate=None):
    """One grouped-head call over rows [t0, t0+T); ring / state updated in place when
    given. gate = (form, gate_a, gate_bias, lb) feeds the pre-activations instead."""
    T = cfg.T if T is None else T
    sl = slice(t0, t0 + T)
    gname, bname = ("gate_x", "beta_x") if gate else ("g", "beta")
    acts = {n: dev[n][:, sl].clone(memory_format=torch.contiguous_format)
            for n in ("q", "k", "v", gname, bname, "z")}
    ring = dev["ring"].clone() if ring is None else ring
    s_in = dev["state"].clone() if state is None else state
    s_out = s_in if state is not None else torch.empty_like(s_in)
    outs = alloc_outputs(cfg, T, DEV, o_core=True)
    kw = {}
    if gate:
        kw = dict(gate_form=gate[0], gate_a=gate[1], gate_bias=gate[2], gate_lb=gate[3])
    args = (acts["q"], acts["k"], acts["v"], acts[gname], acts[bname], dev["conv_w"], ring, s_in, s_out,
            acts["z"], dev["norm_w"], outs["out"], outs["o_core"])
    if decode:
        kda.gdn_decode_gqa(*args, scale=scale_of(cfg), rms_eps=RMS_EPS, **kw)
    else:
        code = kda.KDA_DTYPE_BF16 if cfg.dtype == "bf16" else kda.KDA_DTYPE_F32
        nb = kda.gqa_workspace_bytes(cfg.B, T, cfg.H, cfg.hk, cfg.D, code, mode)
        ws = torch.empty(nb, dtype=torch.uint8, device=DEV) if nb else None
        kda.gdn_prefill_gqa(*args, scale=scale_of(cfg), rms_eps=RMS_EPS, mode=mode, workspace=ws, **kw)
    return {"out": outs["out"], "o_core": outs["o_core"], "ring": ring, "state": s_out}


def oracle_heads(inp, heads, batches, g=None, beta=None, T=None):
    """The oracle over value heads `heads` of sequences `batches` (first T rows):
    returns (result, value channels, grouped ring rows, batch index)."""
    cfg = inp.cfg
    T = cfg.T if T is None else T
    bsel = np.asarray(batches)
    f = lambda x: np.asarray(x, np.float64)[bsel][:, :T]  # noqa: E731
    d, rows = gqa.value_head_problem(
        f(inp.q), f(inp.k), f(inp.v), f(inp.g if g is None else g), f(inp.beta if beta is None else beta),
        inp.conv_w.astype(np.float64), inp.ring.astype(np.float64)[bsel], inp.state.astype(np.float64)[bsel],
        f(inp.z), heads)
    r = oracle.mixer(**d, norm_w=inp.norm_w.astype(np.float64), scale=scale_of(cfg), rms_eps=RMS_EPS,
                     gdn=True, threads=16)
    vc = (np.asarray(heads)[:, None] * cfg.D + np.arange(cfg.D)).ravel()
    return r, vc, rows, bsel


def compare(got, ref, vc, rows, bsel, heads, tol, T=None):
    sl = slice(0, T)
    errs = {"out": oracle.rel_linf(to_f64(got["out"])[bsel][:, sl][:, :, vc], ref["out"]),
            "o_core": oracle.rel_linf(to_f64(got["o_core"])[bsel][:, sl][:, :, vc], ref["o_core"]),
            "state": oracle.rel_linf(to_f64(got["state"])[bsel][:, heads], ref["state"]),
            "ring": oracle.rel_linf(to_f64(got["ring"])[bsel][:, rows], ref["ring"])}
    _print("errs", errs)
    for k, e in errs.items():
        assert e <= tol, f"{k}: {e:.3e} > {tol}"
    assert errs["ring"] == 0.0


# (value heads, key heads): two and four value heads per key head
GROUPS = [(8, 4), (8, 2)]


@pytest.mark.parametrize("H,Hk", GROUPS, ids=["g2", "g4"])
@pytest.mark.parametrize("mode,T,B", [(SEQ, 9, 2), (SEQ, 70, 1), (CHK, 150, 2), (SEG, 300, 2)],
                         ids=["fused", "split", "chunked", "segmented"])
def test_gqa_prefill_vs_oracle(H, Hk, mode, T, B):
    """Every arm against the grouped-head oracle. The segmented case runs several
    segments: its last segment writes the ring in the kernel, the q / k rows of a key head
    by one of its value heads (the ring is compared exactly)."""
    cfg = CONFIGS["gdn_prefill"].with_(B=B, T=T, H=H, Hk=Hk, random_init=True)
    inp, dev = inputs_for(cfg)
    arm = kda.prefill_arm(cfg.B, cfg.T, cfg.H, cfg.D, kda.KDA_DTYPE_BF16, mode, gdn=True)
    _print("case", cfg, "arm", kda.ARM_NAMES[arm])
    got = run_gqa(cfg, dev, mode=mode)
    torch.cuda.synchronize()
    heads = list(range(H))
    ref, vc, rows, bsel = oracle_heads(inp, heads, list(range(B)))
    compare(got, ref, vc, rows, bsel, heads, TOL["bf16"])


@pytest.mark.parametrize("H,Hk", GROUPS, ids=["g2", "g4"])
def test_gqa_fp32_sequential_vs_oracle(H, Hk):
    cfg = CONFIGS["gdn_prefill"].with_(B=2, T=40, H=H, Hk=Hk, D=16, dtype="fp32", random_init=True)
    inp, dev = inputs_for(cfg)
    got = run_gqa(cfg, dev, mode=SEQ)
    torch.cuda.synchronize()
    r = gqa.mixer_gqa(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.conv_w, inp.ring, inp.state, inp.z,
                      inp.norm_w, scale_of(cfg), RMS_EPS)
    errs = {n: oracle.rel_linf(to_f64(got[n]), r[n]) for n in ("out", "o_core", "state", "ring")}
    _print("errs", errs)
    assert max(errs.values()) <= TOL["fp32"] and errs["ring"] == 0.0


@pytest.mark.parametrize("T", [9, 40], ids=["fused", "split"])
def test_gqa_sequential_arms_equal_chained_decodes(T):
    cfg = CONFIGS["gdn_prefill"].with_(B=1, T=T, H=8, Hk=2, D=16, dtype="fp32", random_init=True)
    inp, dev = inputs_for(cfg)
    pre = run_gqa(cfg, dev, mode=SEQ)
    ring, state = dev["ring"].clone(), dev["state"].clone()
    outs = [run_gqa(cfg, dev, decode=True, t0=t, T=1, ring=ring, state=state)["out"] for t in range(T)]
    torch.cuda.synchronize()
    assert_bitwise(pre, {"out": torch.cat(outs, 1), "ring": ring, "state": state}, keys=("out", "ring", "state"))


@pytest.mark.parametrize("mode,T", [(SEQ, 9), (SEQ, 40), (CHK, 130)], ids=["fused", "split", "chunked"])
def test_equal_heads_match_the_plain_entry_bitwise(mode, T):
    cfg = CONFIGS["gdn_prefill"].with_(B=2, T=T, H=4, random_init=True)
    inp, dev = inputs_for(cfg)
    a = run_gqa(cfg, dev, mode=mode)
    b = run_gpu(cfg, dev, mode=mode)
    torch.cuda.synchronize()
    assert_bitwise(a, b)


def test_gqa_gated_softplus_vs_oracle():
    from oracle import gates
    cfg = CONFIGS["gdn_prefill"].with_(B=2, T=150, H=8, Hk=2, random_init=True)
    inp, dev = inputs_for(cfg)
    a = -np.exp(inp.A_log.astype(np.float64))
    ga = torch.from_numpy(a.astype(np.float32)).to(DEV)
    g = gates.gate_softplus(inp.gate_x, a.astype(np.float32), inp.dt_bias, -5.0, cfg.D, gdn=True)
    beta = gates.beta_sigmoid(inp.beta_x)
    for mode in (SEQ, CHK):
        got = run_gqa(cfg, dev, mode=mode, gate=(kda.KDA_GATE_SOFTPLUS, ga, dev["dt_bias"], -5.0))
        torch.cuda.synchronize()
        heads = list(range(cfg.H))
        ref, vc, rows, bsel = oracle_heads(inp, heads, [0, 1], g=g, beta=beta)
        compare(got, ref, vc, rows, bsel, heads, TOL["bf16"])


def test_gqa_rollback_is_bitwise_the_decode_chain():
    cfg = CONFIGS["gdn_prefill"].with_(B=2, T=8, H=8, Hk=2, random_init=True)
    inp, dev = inputs_for(cfg)
    ring, state = dev["ring"].clone(), dev["state"].clone()
    steps = []
    for t in range(cfg.T):
        run_gqa(cfg, dev, decode=True, t0=t, T=1, ring=ring, state=state)
        steps.append({"ring": ring.clone(), "state": state.clone()})
    for keep in (1, 5, cfg.T):
        ring = torch.full_like(dev["ring"], float("nan"))
        state = torch.full_like(dev["state"], float("nan"))
        nb = kda.gqa_workspace_bytes(cfg.B, keep, cfg.H, cfg.hk, cfg.D, kda.KDA_DTYPE_BF16, SEQ)
        ws = torch.empty(nb, dtype=torch.uint8, device=DEV) if nb else None
        kda.gdn_rollback_gqa(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], dev["conv_w"], dev["ring"],
                             dev["state"], ring, state, keep, workspace=ws)
        torch.cuda.synchronize()
        assert_bitwise({"ring": ring, "state": state}, steps[keep - 1], keys=("ring", "state"))


def test_gqa_decode_full_size_sampled():
    """Batched decode B=64 with 32 value heads over 16 key heads (D=128, bf16, state in
    place) against the oracle on sampled heads and sequences."""
    cfg = CONFIGS["kda_decode"].with_(gdn=True, H=32, Hk=16)
    inp, dev = inputs_for(cfg)
    got = run_gqa(cfg, dev, decode=True, T=1)
    torch.cuda.synchronize()
    heads = [0, 15, 16, 31]
    ref, vc, rows, bsel = oracle_heads(inp, heads, [0, 37, 63])
    compare(got, ref, vc, rows, bsel, heads, TOL["bf16"])


@pytest.mark.parametrize("T", [1, 3, 9])
def test_gqa_wide_conv_short_rows_vs_oracle(T):
    """K = 8 with T < K - 1 rows: the separate q / k ring roll keeps old ring slots."""
    cfg = CONFIGS["gdn_prefill"].with_(B=2, T=T, H=8, Hk=2, K=8, D=16, dtype="fp32", random_init=True)
    inp, dev = inputs_for(cfg)
    got = run_gqa(cfg, dev, mode=SEQ)
    torch.cuda.synchronize()
    r = gqa.mixer_gqa(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.conv_w, inp.ring, inp.state, inp.z,
                      inp.norm_w, scale_of(cfg), RMS_EPS)
    errs = {n: oracle.rel_linf(to_f64(got[n]), r[n]) for n in ("out", "state", "ring")}
    _print("errs", errs)
    assert max(errs.values()) <= TOL["fp32"] and errs["ring"] == 0.0


def test_gqa_rollback_split_arm_matches_prefill():
    """keep = 30 rows with 8 value heads over 2 key heads (B = 1): the split arm
    replays from the workspace; it equals a grouped sequential prefill of those rows."""
    cfg = CONFIGS["gdn_prefill"].with_(B=1, T=40, H=8, Hk=2, D=16, dtype="fp32", random_init=True)
    inp, dev = inputs_for(cfg)
    keep = 30
    assert kda.prefill_arm(cfg.B, keep, cfg.H, cfg.D, kda.KDA_DTYPE_F32, SEQ, gdn=True) == 2
    ref = run_gqa(cfg, dev, mode=SEQ, T=keep)
    ring, state = torch.empty_like(dev["ring"]), torch.empty_like(dev["state"])
    nb = kda.gqa_workspace_bytes(cfg.B, keep, cfg.H, cfg.hk, cfg.D, kda.KDA_DTYPE_F32, SEQ)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    kda.gdn_rollback_gqa(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], dev["conv_w"], dev["ring"],
                         dev["state"], ring, state, keep, workspace=ws)
    torch.cuda.synchronize()
    assert_bitwise({"ring": ring, "state": state}, ref, keys=("ring", "state"))
