"""Packed variable-length prefill on the GPU (kda_prefill_varlen, gdn_prefill_varlen):
every sequence of a packed call equals a call on that sequence alone (bit for bit on
the sequential arms, which share their per-step arithmetic), an empty sequence passes
its ring and state through, a packing of equal lengths equals the batched call bit for
bit on the chunked arm, and the chunked arm matches the oracle per sequence (also with
grouped heads and fused gates)."""
import numpy as np
import pytest
import torch

import gated_delta_rule_68_amd as kda
import oracle
from gated_delta_rule_68_amd.synth import CONFIGS
from gated_delta_rule_68_amd.torch_io import act_dtype, to_f64
from oracle import gates, gqa
from tests.gpu_util import DEV, RMS_EPS, TOL, assert_bitwise, inputs_for, run_gpu, scale_of

pytestmark = pytest.mark.gpu
SEQ, CHK = kda.KDA_MODE_SEQUENTIAL, kda.KDA_MODE_CHUNKED
ACT_NAMES = ("q", "k", "v", "g", "beta", "z", "gate_x", "beta_x")


def _print(*a):
    print(*a, flush=True)


def pack(dev, lens):
    """Rows 0..len-1 of every sequence of the batched device inputs, back to back."""
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    p = {n: torch.cat([dev[n][b, :L] for b, L in enumerate(lens)], 0).contiguous() for n in ACT_NAMES}
    return p, torch.from_numpy(cu).to(DEV), int(cu[-1])


def run_varlen(cfg, dev, lens, mode, gate=None):
    p, cu, T_total = pack(dev, lens)
    N = len(lens)
    ring, s_out = dev["ring"].clone(), torch.empty_like(dev["state"])
    out = torch.empty(T_total, cfg.qkv, dtype=act_dtype(cfg), device=DEV)
    o_core = torch.empty(T_total, cfg.qkv, dtype=torch.float32, device=DEV)
    code = kda.KDA_DTYPE_BF16 if cfg.dtype == "bf16" else kda.KDA_DTYPE_F32
    nb = kda.varlen_workspace_bytes(N, T_total, cfg.H, cfg.D, code, mode, gdn=cfg.gdn, Hk=cfg.hk)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV) if nb else None
    gname, bname = ("gate_x", "beta_x") if gate else ("g", "beta")
    kw = dict(gate_form=gate[0], gate_a=gate[1], gate_bias=gate[2], gate_lb=gate[3]) if gate else {}
    kda.prefill_varlen(p["q"], p["k"], p["v"], p[gname], p[bname], dev["conv_w"], ring, dev["state"], s_out,
                       p["z"], dev["norm_w"], out, cu, o_core, gdn=cfg.gdn, scale=scale_of(cfg), rms_eps=RMS_EPS,
                       mode=mode, workspace=ws, **kw)
    return {"out": out, "o_core": o_core, "ring": ring, "state": s_out}, cu.cpu().numpy()


def one_sequence(cfg, dev, b, L):
    """The device inputs of sequence b alone, first L rows (B = 1)."""
    d = {n: dev[n][b:b + 1, :L].contiguous() for n in ACT_NAMES}
    for n in ("conv_w", "norm_w", "A_log", "dt_bias"):
        d[n] = dev[n]
    d["ring"], d["state"] = dev["ring"][b:b + 1].contiguous(), dev["state"][b:b + 1].contiguous()
    return cfg.with_(B=1, T=L), d


LENS = [5, 0, 1, 40, 17, 3]


@pytest.mark.parametrize("gdn", [False, True])
@pytest.mark.parametrize("dtype,D", [("fp32", 16), ("bf16", 128)])
def test_sequential_varlen_equals_each_sequence_alone(gdn, dtype, D):
    cfg = CONFIGS["kda_decode"].with_(B=len(LENS), T=max(LENS), H=3, D=D, dtype=dtype, gdn=gdn)
    inp, dev = inputs_for(cfg)
    got, cu = run_varlen(cfg, dev, LENS, SEQ)
    torch.cuda.synchronize()
    for b, L in enumerate(LENS):
        if L == 0:  # ring and state pass through
            assert_bitwise({"ring": got["ring"][b], "state": got["state"][b]},
                           {"ring": dev["ring"][b], "state": dev["state"][b]}, keys=("ring", "state"))
            continue
        c1, d1 = one_sequence(cfg, dev, b, L)
        ref = run_gpu(c1, d1, mode=SEQ)
        torch.cuda.synchronize()
        rows = slice(int(cu[b]), int(cu[b + 1]))
        assert_bitwise({"out": got["out"][rows], "o_core": got["o_core"][rows], "ring": got["ring"][b],
                        "state": got["state"][b]},
                       {"out": ref["out"][0], "o_core": ref["o_core"][0], "ring": ref["ring"][0],
                        "state": ref["state"][0]})
    _print("bitwise ok", LENS)


@pytest.mark.parametrize("gdn", [False, True])
def test_chunked_equal_lengths_equal_the_batched_call(gdn):
    cfg = CONFIGS["kda_decode"].with_(B=3, T=150, H=4, gdn=gdn)
    inp, dev = inputs_for(cfg)
    got, _ = run_varlen(cfg, dev, [150] * 3, CHK)
    ref = run_gpu(cfg, dev, mode=CHK)
    torch.cuda.synchronize()
    assert_bitwise({"out": got["out"].view(3, 150, -1), "o_core": got["o_core"].view(3, 150, -1),
                    "ring": got["ring"], "state": got["state"]}, ref)


def _oracle_seq(inp, b, L, g=None, beta=None):
    cfg = inp.cfg
    f = lambda x: np.asarray(x, np.float64)[b:b + 1, :L]  # noqa: E731
    args = dict(q=f(inp.q), k=f(inp.k), v=f(inp.v), g=f(inp.g if g is None else g),
                beta=f(inp.beta if beta is None else beta), conv_w=inp.conv_w.astype(np.float64),
                ring=inp.ring[b:b + 1].astype(np.float64), state=inp.state[b:b + 1].astype(np.float64),
                z=f(inp.z), norm_w=inp.norm_w.astype(np.float64), scale=scale_of(cfg), rms_eps=RMS_EPS)
    if cfg.gdn and cfg.hk != cfg.H:
        return gqa.mixer_gqa(**args)
    return oracle.mixer(**args, gdn=cfg.gdn)


def _compare_seqs(inp, got, cu, lens, tol, g=None, beta=None):
    for b, L in enumerate(lens):
        if L == 0:
            continue
        ref = _oracle_seq(inp, b, L, g, beta)
        rows = slice(int(cu[b]), int(cu[b + 1]))
        errs = {"out": oracle.rel_linf(to_f64(got["out"][rows]), ref["out"][0]),
                "o_core": oracle.rel_linf(to_f64(got["o_core"][rows]), ref["o_core"][0]),
                "state": oracle.rel_linf(to_f64(got["state"][b]), ref["state"][0]),
                "ring": oracle.rel_linf(to_f64(got["ring"][b]), ref["ring"][0])}
        _print("seq", b, "len", L, errs)
        assert max(errs.values()) <= tol and errs["ring"] == 0.0, (b, L, errs)


CHUNK_LENS = [130, 0, 1, 64, 65, 300, 17]


@pytest.mark.parametrize("gdn", [False, True])
def test_chunked_varlen_vs_oracle(gdn):
    cfg = CONFIGS["kda_decode"].with_(B=len(CHUNK_LENS), T=max(CHUNK_LENS), H=3, gdn=gdn)
    inp, dev = inputs_for(cfg)
    got, cu = run_varlen(cfg, dev, CHUNK_LENS, CHK)
    torch.cuda.synchronize()
    _compare_seqs(inp, got, cu, CHUNK_LENS, TOL["bf16"])


@pytest.mark.parametrize("mode", [SEQ, CHK], ids=["fused", "chunked"])
def test_gdn_varlen_grouped_heads_and_gates_vs_oracle(mode):
    lens = [70, 0, 129, 9]
    cfg = CONFIGS["kda_decode"].with_(B=len(lens), T=max(lens), H=8, Hk=2, gdn=True)
    inp, dev = inputs_for(cfg)
    a = -np.exp(inp.A_log.astype(np.float64))
    ga = torch.from_numpy(a.astype(np.float32)).to(DEV)
    got, cu = run_varlen(cfg, dev, lens, mode, gate=(kda.KDA_GATE_SOFTPLUS, ga, dev["dt_bias"], -5.0))
    torch.cuda.synchronize()
    g = gates.gate_softplus(inp.gate_x, a.astype(np.float32), inp.dt_bias, -5.0, cfg.D, gdn=True)
    _compare_seqs(inp, got, cu, lens, TOL["bf16"], g=g, beta=gates.beta_sigmoid(inp.beta_x))


def test_chunked_varlen_long_mixed_lengths_sampled():
    """A serving-like mix at H=64 (column splits: N*H < 256) with long and short
    sequences; the oracle checks three of them."""
    lens = [2000, 37, 1, 700, 0, 129]
    cfg = CONFIGS["kda_decode"].with_(B=len(lens), T=max(lens), H=64)
    inp, dev = inputs_for(cfg)
    got, cu = run_varlen(cfg, dev, lens, CHK)
    torch.cuda.synchronize()
    for b in (1, 3, 5):
        L = lens[b]
        heads = [0, 33, 63]
        ch = np.concatenate([np.arange(h * cfg.D, (h + 1) * cfg.D) for h in heads])
        rows_r = np.concatenate([p * cfg.qkv + ch for p in range(3)])
        f = lambda x: np.asarray(x, np.float64)[b:b + 1, :L][:, :, ch]  # noqa: E731
        ref = oracle.mixer(q=f(inp.q), k=f(inp.k), v=f(inp.v), g=f(inp.g),
                           beta=np.asarray(inp.beta, np.float64)[b:b + 1, :L][:, :, heads],
                           conv_w=inp.conv_w[rows_r].astype(np.float64),
                           ring=inp.ring[b:b + 1][:, rows_r].astype(np.float64),
                           state=inp.state[b:b + 1][:, heads].astype(np.float64), z=f(inp.z),
                           norm_w=inp.norm_w.astype(np.float64), scale=scale_of(cfg), rms_eps=RMS_EPS,
                           threads=16)
        rows = slice(int(cu[b]), int(cu[b + 1]))
        errs = {"out": oracle.rel_linf(to_f64(got["out"][rows])[:, ch], ref["out"][0]),
                "state": oracle.rel_linf(to_f64(got["state"][b])[heads], ref["state"][0]),
                "ring": oracle.rel_linf(to_f64(got["ring"][b])[rows_r], ref["ring"][0])}
        _print("seq", b, "len", L, errs)
        assert max(errs.values()) <= TOL["bf16"] and errs["ring"] == 0.0


@pytest.mark.parametrize("mode", [SEQ, CHK], ids=["fused", "chunked"])
def test_varlen_wide_conv_short_sequences_vs_oracle(mode):
    """K = 8: sequences shorter than K - 1 rows roll rings that keep old slots."""
    lens = [1, 3, 0, 6, 8, 70]
    cfg = CONFIGS["kda_decode"].with_(B=len(lens), T=max(lens), H=3, K=8)
    inp, dev = inputs_for(cfg)
    got, cu = run_varlen(cfg, dev, lens, mode)
    torch.cuda.synchronize()
    _compare_seqs(inp, got, cu, lens, TOL["bf16"])
