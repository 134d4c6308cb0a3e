"""GPU parity of the segmented chunked prefill (KDA_MODE_SEGMENTED): each sequence is
cut into segments that run in parallel, and the segments are joined by the affine state
scan. The segmented run is checked against the fp64 oracle. Segments of one chunk give
several scan steps and a ragged last segment. The segmented arm is also checked against
the sequential arm at the single-sequence prefill workload, which AUTO sends to it."""
import numpy as np
import pytest
import torch

import gated_delta_rule_68_amd as kda
import oracle
from gated_delta_rule_68_amd.synth import CONFIGS
from gated_delta_rule_68_amd.torch_io import to_f64
from oracle import gates
from tests.gpu_util import DEV, compare_to_oracle, inputs_for, oracle_run, run_gpu
from tests.test_gpu_gates import compare as compare_gated
from tests.test_gpu_gates import gate_params, oracle_gated, run_gated
from tests.test_gpu_gqa import compare as compare_gqa
from tests.test_gpu_gqa import oracle_heads, run_gqa

pytestmark = pytest.mark.gpu
SEG, SEQ, CHK = kda.KDA_MODE_SEGMENTED, kda.KDA_MODE_SEQUENTIAL, kda.KDA_MODE_CHUNKED
TOL = 2e-2  # bf16-operand arm


def _print(*a):
    print(*a, flush=True)


def _check(cfg, heads=None, tol=TOL, **run_kw):
    inp, dev = inputs_for(cfg)
    got = run_gpu(cfg, dev, mode=SEG, **run_kw)
    torch.cuda.synchronize()
    ref, ch, rows, bsel, hh = oracle_run(inp, heads=heads, threads=16)
    errs = compare_to_oracle(cfg, got, ref, ch, rows, bsel, hh, tol=tol)
    _print("errs", errs)
    return got, dev


# At B*H = 2 the explicit mode takes one-chunk segments where they shorten the
# critical path: T = 50 and 100 run as one segment, 300 as five (three scan steps, a
# 44-row last segment), 700 as eleven.
@pytest.mark.parametrize("T", [50, 100, 300, 700])
@pytest.mark.parametrize("gdn", [False, True])
def test_one_chunk_segments_vs_oracle(T, gdn):
    cfg = CONFIGS["kda_decode"].with_(B=1, H=2, T=T, gdn=gdn)
    _print("case", cfg)
    _check(cfg)


@pytest.mark.parametrize("gdn", [False, True])
def test_many_pairs_vs_oracle(gdn):
    """B*H = 80: four segments; the 320 middle runs of pass 1 take two rounds beside the
    segment-0 runs. Sampled heads."""
    cfg = CONFIGS["kda_decode"].with_(B=2, H=40, T=300, gdn=gdn)
    _check(cfg, heads=[0, 17, 39])


def test_wide_conv_and_alternating_gates_vs_oracle():
    """K = 6 (history of five rows read from the rows before each segment) and gates
    pushed to both ends of [-5, 0] on alternate heads."""
    cfg = CONFIGS["kda_long"].with_(B=1, T=330, H=4, K=6, random_init=True)
    _check(cfg)


def test_gdn_widest_conv_vs_oracle():
    """GDN with K = 8: the widest conv history, read from the seven rows before each
    segment."""
    cfg = CONFIGS["gdn_prefill"].with_(B=1, T=330, H=3, K=8, random_init=True)
    _check(cfg)


def test_in_place_state_vs_oracle():
    cfg = CONFIGS["kda_decode"].with_(B=1, H=3, T=260)
    _check(cfg, inplace=True)


@pytest.mark.parametrize("gdn", [False, True])
def test_gated_vs_oracle(gdn):
    cfg = CONFIGS["kda_decode"].with_(B=1, H=3, T=300, gdn=gdn)
    inp, dev = inputs_for(cfg)
    form = kda.KDA_GATE_SIGMOID
    ga, gb, g, beta = gate_params(inp, dev, form)
    got = run_gated(cfg, dev, ga, gb, form, mode=SEG)
    torch.cuda.synchronize()
    ref, ch, rows, bsel = oracle_gated(inp, g, beta, heads=[0, 1, 2])
    compare_gated(cfg, got, ref, ch, rows, bsel, [0, 1, 2], TOL)


def test_grouped_heads_vs_oracle():
    cfg = CONFIGS["gdn_prefill"].with_(B=2, T=300, H=8, Hk=4, random_init=True)
    inp, dev = inputs_for(cfg)
    got = run_gqa(cfg, dev, mode=SEG)
    torch.cuda.synchronize()
    heads = list(range(cfg.H))
    ref, vc, rows, bsel = oracle_heads(inp, heads, [0, 1])
    compare_gqa(got, ref, vc, rows, bsel, heads, TOL)


def _slow_gates(inp, dev, a=-0.002):
    """Softplus gates with multiplier a: e^g stays within 1% of 1, so a segment's
    transition M is far from zero and the entry states carry the whole history.
    (Under the workloads' gates M underflows to zero within a few hundred rows.)"""
    cfg = inp.cfg
    av = np.full(cfg.H, a, np.float32)
    g = gates.gate_softplus(inp.gate_x, av, inp.dt_bias, -5.0, cfg.D, cfg.gdn)
    return torch.from_numpy(av).to(DEV), dev["dt_bias"], g, gates.beta_sigmoid(inp.beta_x)


@pytest.mark.parametrize("T", [300, 700])
@pytest.mark.parametrize("gdn", [False, True])
def test_slow_decay_history_across_segments_vs_oracle(T, gdn):
    """Slow gates and a random entry state: the outputs of later segments depend on
    the whole history through the scan (forgetting it moves them by about 50%)."""
    cfg = CONFIGS["kda_decode"].with_(B=1, H=2, T=T, gdn=gdn)
    inp, dev = inputs_for(cfg)
    ga, gb, g, beta = _slow_gates(inp, dev)
    form = kda.KDA_GATE_SOFTPLUS
    got = run_gated(cfg, dev, ga, gb, form, mode=SEG)
    torch.cuda.synchronize()
    ref, ch, rows, bsel = oracle_gated(inp, g, beta, heads=[0, 1])
    compare_gated(cfg, got, ref, ch, rows, bsel, [0, 1], TOL)


def test_slow_decay_prefill_workload_vs_oracle():
    """The single-sequence workload's shape and AUTO plan (five segments) with slow
    gates: sampled heads against the oracle."""
    cfg = CONFIGS["kda_prefill"].with_(random_init=True)
    assert kda.prefill_arm(cfg.B, cfg.T, cfg.H, cfg.D, kda.KDA_DTYPE_BF16, kda.KDA_MODE_AUTO) == 4
    inp, dev = inputs_for(cfg)
    ga, gb, g, beta = _slow_gates(inp, dev)
    got = run_gated(cfg, dev, ga, gb, kda.KDA_GATE_SOFTPLUS, mode=kda.KDA_MODE_AUTO)
    torch.cuda.synchronize()
    heads = [0, 33, 63]
    ref, ch, rows, bsel = oracle_gated(inp, g, beta, heads=heads)
    compare_gated(cfg, got, ref, ch, rows, bsel, heads, TOL)


def test_prefill_workload_auto_is_segmented():
    """Single-sequence prefill T = 4626, H = 64: AUTO takes five segments. Sampled heads
    against the oracle, everything against the sequential arm and the unsegmented
    chunked arm."""
    cfg = CONFIGS["kda_prefill"]
    assert kda.prefill_arm(cfg.B, cfg.T, cfg.H, cfg.D, kda.KDA_DTYPE_BF16, kda.KDA_MODE_AUTO) == 4
    inp, dev = inputs_for(cfg)
    got = run_gpu(cfg, dev, mode=kda.KDA_MODE_AUTO)
    torch.cuda.synchronize()
    ref, ch, rows, bsel, hh = oracle_run(inp, heads=[0, 33, 63])
    _print("oracle errs", compare_to_oracle(cfg, got, ref, ch, rows, bsel, hh, tol=TOL))
    for mode in (SEQ, CHK):
        other = run_gpu(cfg, dev, mode=mode)
        errs = {k: oracle.rel_linf(to_f64(got[k]), to_f64(other[k])) for k in ("out", "o_core", "state", "ring")}
        _print("vs mode", mode, errs)
        assert max(errs.values()) <= TOL and errs["ring"] == 0.0


def test_gdn_workload_auto_is_segmented():
    """GDN prefill B = 4, T = 8192, H = 32 (128 pairs): AUTO takes three segments
    (3456, 2368 and 2368 rows). Sampled heads against the oracle, everything against
    the sequential arm."""
    cfg = CONFIGS["gdn_prefill"]
    assert kda.prefill_arm(cfg.B, cfg.T, cfg.H, cfg.D, kda.KDA_DTYPE_BF16, kda.KDA_MODE_AUTO, gdn=True) == 4
    inp, dev = inputs_for(cfg)
    got = run_gpu(cfg, dev, mode=kda.KDA_MODE_AUTO)
    torch.cuda.synchronize()
    ref, ch, rows, bsel, hh = oracle_run(inp, heads=[7], batches=[1, 2])
    _print("oracle errs", compare_to_oracle(cfg, got, ref, ch, rows, bsel, hh, tol=TOL))
    seq = run_gpu(cfg, dev, mode=SEQ)
    errs = {k: oracle.rel_linf(to_f64(got[k]), to_f64(seq[k])) for k in ("out", "o_core", "state", "ring")}
    _print("vs sequential", errs)
    assert max(errs.values()) <= TOL and errs["ring"] == 0.0


def test_segmented_gdn_few_pairs_auto():
    """GDN, one sequence of 2048 rows, 16 heads: AUTO takes four segments (320 rows,
    then 576); checked against the sequential arm."""
    cfg = CONFIGS["gdn_prefill"].with_(B=1, T=2048, H=16)
    assert kda.prefill_arm(cfg.B, cfg.T, cfg.H, cfg.D, kda.KDA_DTYPE_BF16, kda.KDA_MODE_AUTO, gdn=True) == 4
    inp, dev = inputs_for(cfg)
    got = run_gpu(cfg, dev, mode=kda.KDA_MODE_AUTO)
    ref = run_gpu(cfg, dev, mode=SEQ)
    torch.cuda.synchronize()
    errs = {k: oracle.rel_linf(to_f64(got[k]), to_f64(ref[k])) for k in ("out", "o_core", "state", "ring")}
    _print("vs sequential", errs)
    assert max(errs.values()) <= TOL and errs["ring"] == 0.0


@pytest.mark.parametrize("H,nseg", [(32, 9), (8, 10)])
def test_auto_plans_with_few_heads_slow_gates(H, nseg):
    """A single sequence of 4626 rows with 32 and with 8 heads: AUTO's timed plan takes
    nine segments (576 rows, then 512) and ten (a first segment of 64 rows, then 512).
    Slow gates, so every segment's entry state carries the history through its
    transition M; every head against the sequential arm under the same gates."""
    from tests.test_abi_host import _segments_from_workspace
    cfg = CONFIGS["kda_prefill"].with_(H=H, random_init=True)
    assert kda.prefill_arm(cfg.B, cfg.T, cfg.H, cfg.D, kda.KDA_DTYPE_BF16, kda.KDA_MODE_AUTO) == 4
    assert _segments_from_workspace(cfg.B, cfg.T, cfg.H, kda.KDA_MODE_AUTO) == nseg
    inp, dev = inputs_for(cfg)
    ga, gb, _, _ = _slow_gates(inp, dev)
    got = run_gated(cfg, dev, ga, gb, kda.KDA_GATE_SOFTPLUS, mode=kda.KDA_MODE_AUTO)
    ref = run_gated(cfg, dev, ga, gb, kda.KDA_GATE_SOFTPLUS, mode=SEQ)
    torch.cuda.synchronize()
    errs = {k: oracle.rel_linf(to_f64(got[k]), to_f64(ref[k])) for k in ("out", "o_core", "state", "ring")}
    _print("vs sequential", errs)
    assert max(errs.values()) <= TOL and errs["ring"] == 0.0


def test_without_o_core_same_outputs():
    """o_core = NULL: the same out, ring and state bit for bit as with it."""
    cfg = CONFIGS["kda_decode"].with_(B=1, H=2, T=300)
    inp, dev = inputs_for(cfg)
    a = run_gpu(cfg, dev, mode=SEG)
    b = run_gpu(cfg, dev, mode=SEG, o_core=False)
    torch.cuda.synchronize()
    assert b["o_core"] is None
    for k in ("out", "state", "ring"):
        assert torch.equal(a[k], b[k]), k


def test_repeated_calls_reuse_the_workspace():
    """The workspace's constant blocks are rebuilt by every call: a second call on a
    workspace full of the first call's values gives the same result bit for bit."""
    cfg = CONFIGS["kda_decode"].with_(B=1, H=2, T=300)
    inp, dev = inputs_for(cfg)
    a = run_gpu(cfg, dev, mode=SEG)
    b = run_gpu(cfg, dev, mode=SEG)
    torch.cuda.synchronize()
    for k in ("out", "o_core", "state", "ring"):
        assert torch.equal(a[k], b[k]), k
