"""GPU parity of the chunked prefill arm (D = 128, bf16 MFMA operands) against the fp64
oracle and against the sequential arm on identical inputs. Conv kernels of up to 4 taps
run the 32-row chunk kernel (kda_c32.hip), wider ones the 64-row kernel with its column
splits (kda_chunk.hip)."""
import numpy as np
import pytest
import torch

import gated_delta_rule_68_amd as kda
import oracle
from gated_delta_rule_68_amd.synth import CONFIGS, make_inputs
from gated_delta_rule_68_amd.torch_io import tiled_device_inputs, to_f64
from tests.gpu_util import (DEV, compare_to_oracle, inputs_for, oracle_run, run_gpu)

pytestmark = pytest.mark.gpu
SEQ, CHK = kda.KDA_MODE_SEQUENTIAL, kda.KDA_MODE_CHUNKED
TOL = 2e-2  # bf16-operand arm


def _print(*a):
    print(*a, flush=True)


def _rel(a, b):
    return oracle.rel_linf(to_f64(a), to_f64(b))


def _vs_sequential(cfg, dev, got, keys=("out", "o_core", "state", "ring"), tol=TOL):
    ref = run_gpu(cfg, dev, mode=SEQ)
    errs = {k: _rel(got[k], ref[k]) for k in keys}
    _print("chunked vs sequential:", errs)
    for k, e in errs.items():
        assert e <= tol, f"{k}: chunked vs sequential {e:.3e} > {tol}"
    assert errs.get("ring", 0.0) == 0.0
    return errs


@pytest.mark.parametrize("T", [1, 32, 33, 37, 64, 65, 200])
@pytest.mark.parametrize("gdn", [False, True])
@pytest.mark.parametrize("B,H", [(2, 3), (1, 200), (2, 160)])
def test_small_vs_oracle(T, gdn, B, H):
    """Ragged T (partial chunks, T < K-1) and exact multiples of the 32-row chunk (the
    pipeline's one-, two- and seven-step runs), random state and ring."""
    cfg = CONFIGS["kda_decode"].with_(B=B, H=H, T=T, gdn=gdn)
    _print("case", cfg)
    inp, dev = inputs_for(cfg)
    got = run_gpu(cfg, dev, mode=CHK)
    torch.cuda.synchronize()
    heads = [0, H // 2, H - 1]
    ref, ch, rows, bsel, hh = oracle_run(inp, heads=heads, threads=16)
    errs = compare_to_oracle(cfg, got, ref, ch, rows, bsel, hh, tol=TOL)
    _print("errs", errs)


@pytest.mark.parametrize("gdn", [False, True])
def test_alternating_gates_vs_oracle(gdn):
    """Gates pushed to both ends of [-5, 0] on alternate heads (the long-prefill regime)
    exercise the rebased decay of the intra-chunk blocks."""
    cfg = CONFIGS["kda_long"].with_(B=2, T=300, H=8, gdn=gdn, random_init=True)
    inp, dev = inputs_for(cfg)
    got = run_gpu(cfg, dev, mode=CHK)
    torch.cuda.synchronize()
    ref, ch, rows, bsel, hh = oracle_run(inp, threads=16)
    errs = compare_to_oracle(cfg, got, ref, ch, rows, bsel, hh, tol=TOL)
    _print("errs", errs)


@pytest.mark.parametrize("gdn", [False, True])
def test_fp32_inputs_take_a_sequential_arm_at_the_fp32_bar(gdn):
    """fp32 activations at D = 128: the chunked and segmented modes refuse them (their
    bf16 MFMA operands cannot meet 1e-3) with nothing written, and AUTO runs them on a
    sequential arm, which meets the fp32 bar against the oracle."""
    cfg = CONFIGS["kda_decode"].with_(B=2, H=4, T=150, dtype="fp32", gdn=gdn)
    inp, dev = inputs_for(cfg)
    for mode in (CHK, kda.KDA_MODE_SEGMENTED):
        assert kda.prefill_arm(cfg.B, cfg.T, cfg.H, cfg.D, kda.KDA_DTYPE_F32, mode, gdn=gdn) == -1
        sentinel = torch.full_like(dev["state"], 7.0)
        with pytest.raises(kda.KdaError) as e:
            run_gpu(cfg, dev, mode=mode, state=sentinel, inplace=True)
        assert e.value.rc == 40008
        torch.cuda.synchronize()
        assert bool((sentinel == 7.0).all()), "a refused call wrote the state"
    arm = kda.prefill_arm(cfg.B, cfg.T, cfg.H, cfg.D, kda.KDA_DTYPE_F32, kda.KDA_MODE_AUTO, gdn=gdn)
    assert kda.ARM_NAMES[arm].startswith("seq"), arm
    got = run_gpu(cfg, dev, mode=kda.KDA_MODE_AUTO)
    torch.cuda.synchronize()
    ref, ch, rows, bsel, hh = oracle_run(inp, threads=16)
    errs = compare_to_oracle(cfg, got, ref, ch, rows, bsel, hh, tol=1e-3)
    _print("fp32 AUTO", kda.ARM_NAMES[arm], errs)


def test_prefill_full_size():
    """Single-sequence prefill T=4626, H=64 on the chunked arm (4 column splits):
    sampled heads against the oracle, everything against the sequential arm."""
    cfg = CONFIGS["kda_prefill"]
    inp, dev = inputs_for(cfg)
    assert kda.prefill_arm(cfg.B, cfg.T, cfg.H, cfg.D, 1, CHK) == 3
    got = run_gpu(cfg, dev, mode=CHK)
    torch.cuda.synchronize()
    ref, ch, rows, bsel, hh = oracle_run(inp, heads=[0, 33, 63])
    errs = compare_to_oracle(cfg, got, ref, ch, rows, bsel, hh, tol=TOL)
    _print("oracle errs", errs)
    _vs_sequential(cfg, dev, got)


def test_gdn_full_size():
    cfg = CONFIGS["gdn_prefill"]
    inp, dev = inputs_for(cfg)
    got = run_gpu(cfg, dev, mode=CHK)
    torch.cuda.synchronize()
    ref, ch, rows, bsel, hh = oracle_run(inp, heads=[7], batches=[1, 2])
    errs = compare_to_oracle(cfg, got, ref, ch, rows, bsel, hh, tol=TOL)
    _print("oracle errs", errs)
    _vs_sequential(cfg, dev, got)


def test_long_full_size():
    """B=8, T=16384, H=64 (one column split): outputs of tokens [0, 512) against the
    oracle, the full run against the sequential arm, and the state after 512 tokens
    (a separate run) against the oracle."""
    cfg = CONFIGS["kda_long"]
    pinp, dev = make_inputs(cfg, T=512), tiled_device_inputs(cfg, period=1024)
    got = run_gpu(cfg, dev, mode=CHK, o_core=True)
    torch.cuda.synchronize()
    ref, ch, rows, bsel, hh = oracle_run(pinp, heads=[0, 1, 62, 63], threads=16)
    P = 512
    out_err = oracle.rel_linf(to_f64(got["out"][:, :P])[bsel][:, :, ch], ref["out"])
    core_err = oracle.rel_linf(to_f64(got["o_core"][:, :P])[bsel][:, :, ch], ref["o_core"])
    _print("prefix errs out", out_err, "o_core", core_err)
    assert out_err <= TOL and core_err <= TOL
    short = run_gpu(cfg, dev, mode=CHK, T=P)
    st_err = oracle.rel_linf(to_f64(short["state"])[bsel][:, hh], ref["state"])
    _print("512-token state err", st_err)
    assert st_err <= TOL
    _vs_sequential(cfg, dev, got, keys=("out", "state", "ring"))


@pytest.mark.parametrize("split", [64, 100])
def test_split_prefill_close_to_one(split):
    cfg = CONFIGS["kda_decode"].with_(B=2, H=4, T=300)
    inp, dev = inputs_for(cfg)
    one = run_gpu(cfg, dev, mode=CHK)
    ring, state = dev["ring"].clone(), dev["state"].clone()
    a = run_gpu(cfg, dev, mode=CHK, T=split, ring=ring, state=state, inplace=True)
    b = run_gpu(cfg, dev, mode=CHK, t0=split, T=cfg.T - split, ring=ring, state=state, inplace=True)
    out = torch.cat([a["out"], b["out"]], 1)
    assert _rel(out, one["out"]) <= TOL
    assert _rel(state, one["state"]) <= TOL
    assert torch.equal(ring, one["ring"])


@pytest.mark.parametrize("K", [2, 3, 6, 8])
@pytest.mark.parametrize("mode", [SEQ, CHK])
def test_conv_kernel_widths(K, mode):
    """Conv kernels other than 4 (2..8 are allowed) on both arms, with a ragged chunk."""
    cfg = CONFIGS["kda_decode"].with_(B=2, H=3, T=70, K=K)
    inp, dev = inputs_for(cfg)
    got = run_gpu(cfg, dev, mode=mode)
    torch.cuda.synchronize()
    ref, ch, rows, bsel, hh = oracle_run(inp, threads=16)
    compare_to_oracle(cfg, got, ref, ch, rows, bsel, hh, tol=TOL)
