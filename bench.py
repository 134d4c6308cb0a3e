"""Benchmark of the KDA mixer hot path on one MI355X.

A step is one batched KDA decode step (B=64 sequences x 1 token, H=64, D=128, bf16
activations, fp32 state updated in place, conv kernel 4): conv + SiLU + l2, the
delta-rule scan, the gated RMSNorm and the ring roll, all in the library's one-token
decode kernel. Inputs are seeded synthetic data (gated_delta_rule_68_amd.synth)
already resident in HBM; NBUF independent copies of every buffer are cycled so
that the 268 MB of state cannot stay in the 256 MB last-level cache between steps.
The steps are replayed from a captured HIP graph of NBUF steps, as a serving loop
runs them (--eager: one launch per step); HIP events bracket each replay.

Prints ONE JSON line (rank 0). Extra legs: the prefill workloads on every arm, verify
and rollback, fused gates, grouped heads, packed batches, and the oracle's CPU rate on
a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "KDA tokens/s + achieved HBM GB/s (decode) / MFMA % (prefill), H=64 d=128"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
NBUF = 4
RMS_EPS = 1e-5


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def decode_bytes(cfg) -> int:
    """Algorithmic HBM bytes of one decode step: every input read once, every output
    written once (state and ring both ways)."""
    B, H, D, K, qkv = cfg.B, cfg.H, cfg.D, cfg.K, cfg.qkv
    es = 2 if cfg.dtype == "bf16" else 4
    state = 2 * B * H * D * D * 4
    ring = 2 * B * 3 * qkv * (K - 1) * 4
    acts_in = (5 * B * qkv + B * H) * es  # q, k, v, g, z + beta
    out = B * qkv * es
    params = 3 * qkv * K * 4 + D * 4
    return state + ring + acts_in + out + params


def prefill_bytes(cfg) -> int:
    B, T, H, D, K, qkv = cfg.B, cfg.T, cfg.H, cfg.D, cfg.K, cfg.qkv
    es = 2 if cfg.dtype == "bf16" else 4
    gate = B * T * (H if cfg.gdn else qkv)
    acts = (4 * B * T * qkv + gate + B * T * H) * es + B * T * qkv * es
    state = 2 * B * H * D * D * 4
    ring = 2 * B * 3 * qkv * (K - 1) * 4
    return acts + state + ring + 3 * qkv * K * 4 + D * 4


def chunk_flops(cfg, C=32) -> float:
    """Dense-tile contraction FLOPs of the chunked form: 2(5CD + 3D^2) per token-head
    (chunks of C = 32 rows: the kernel of every bf16 call with a conv of up to 4 taps)."""
    return 2.0 * (5 * C * cfg.D + 3 * cfg.D * cfg.D) * cfg.B * cfg.T * cfg.H


def profile_record(name: str) -> dict:
    """The committed rocprofv3 summary of a kernel (profiles/<name>_traffic.json: HBM
    bytes per launch from the counters, average duration from the kernel trace), if it
    was taken on the current kernel sources; else an empty dict."""
    path = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
    if not os.path.exists(path):
        return {}
    rec = json.load(open(path))
    h = hashlib.sha256()
    for f in rec.get("source_files", []):
        h.update(open(os.path.join(ROOT, "gated_delta_rule_68_amd", "csrc", f), "rb").read())
    if rec.get("source_sha256") != h.hexdigest():
        return {}
    return rec


COPY_BYTES = 1 << 30


def measure_copy(reps: int = 20) -> float:
    """A plain device copy of COPY_BYTES (torch's copy kernel): read + write GB/s.
    Also the calibration kernel for the HBM byte counters."""
    import torch

    x = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for a, b in ev:
        a.record()
        y.copy_(x)
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)[reps // 2]
    return 2 * COPY_BYTES / (ms * 1e-3) / 1e9


def measure_gemm(n: int = 8192, reps: int = 10) -> float:
    """A large dense bf16 GEMM (torch.mm, contiguous operands): the measured MFMA rate
    that the chunked arm's contraction fraction is also compared against."""
    import torch

    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    for _ in range(3):
        torch.mm(a, b)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for x, y in ev:
        x.record()
        torch.mm(a, b)
        y.record()
    torch.cuda.synchronize()
    ms = sorted(x.elapsed_time(y) for x, y in ev)[reps // 2]
    return 2.0 * n ** 3 / (ms * 1e-3) / 1e12


def cpu_baseline(cfg, inp, budget_s: float = 12.0):
    """The fp64 oracle on the host cores: whole decode steps of the same workload,
    repeated until the budget is spent."""
    import numpy as np
    import oracle

    threads = min(16, os.cpu_count() or 1)
    arrs = [np.ascontiguousarray(getattr(inp, n), np.float64)
            for n in ("q", "k", "v", "g", "beta", "conv_w", "ring", "state", "z", "norm_w")]
    scale = 1.0 / math.sqrt(cfg.D)
    oracle.mixer(*arrs, scale, RMS_EPS, gdn=cfg.gdn, threads=threads)  # warm
    steps, t0 = 0, time.perf_counter()
    while True:
        oracle.mixer(*arrs, scale, RMS_EPS, gdn=cfg.gdn, threads=threads)
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or steps >= 400:
            break
    return {"value": cfg.B * cfg.T * steps / el, "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "cpu_model": _cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"{steps} full decode steps (B={cfg.B}, H={cfg.H}, D={cfg.D}) of the "
                      f"same seeded inputs in {el:.1f} s, fp64, threads split the batch"}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# The oracle on every workload: (workload, rows timed, thread counts, runs). The oracle
# threads over whole sequences only, so a workload of B sequences uses at most B
# threads. The sequential definition costs the same per token at any position, so a
# leading slice of T rows gives the workload's tokens/s; the slices keep each leg to
# seconds.
CPU_LEGS = (("tiny_kda", None, (1,), 3),
            ("kda_decode", None, (1, 16), 3),
            ("kda_prefill", 512, (1,), 3),
            ("gdn_prefill", 1024, (4,), 1),
            ("kda_long", 512, (8,), 1))


def cpu_baselines() -> dict:
    """Time the fp64 oracle on each workload's seeded inputs (bounded slices)."""
    import numpy as np

    import oracle
    from gated_delta_rule_68_amd.synth import CONFIGS, make_inputs

    ncpu = os.cpu_count() or 1
    rec = {"cpu_model": _cpu_model(), "host_cpus": ncpu, "legs": []}
    for name, T, thread_counts, runs in CPU_LEGS:
        cfg = CONFIGS[name]
        inp = make_inputs(cfg, T=T)
        rows = T or cfg.T
        arrs = [np.ascontiguousarray(getattr(inp, n), np.float64)
                for n in ("q", "k", "v", "g", "beta", "conv_w", "ring", "state", "z", "norm_w")]
        scale = 1.0 / math.sqrt(cfg.D)
        for th in thread_counts:
            th = max(1, min(th, cfg.B, ncpu))
            times = []
            for _ in range(runs):
                t0 = time.perf_counter()
                oracle.mixer(*arrs, scale, RMS_EPS, gdn=cfg.gdn, threads=th)
                times.append(time.perf_counter() - t0)
            s = sorted(times)[len(times) // 2]
            leg = {"workload": name, "B": cfg.B, "T_timed": rows, "T_workload": cfg.T,
                   "H": cfg.H, "D": cfg.D, "threads": th, "runs": runs, "s": s,
                   "tokens_per_s": cfg.B * rows / s}
            log(f"oracle {leg}")
            rec["legs"].append(leg)
        del inp, arrs
    return rec


def run_decode(cfg, steps, warmup, graph=False):
    import torch

    import gated_delta_rule_68_amd as kda
    from gated_delta_rule_68_amd.synth import make_inputs
    from gated_delta_rule_68_amd.torch_io import alloc_outputs, to_device

    inp = make_inputs(cfg)
    base = to_device(inp, "cuda")
    sets = []
    for _ in range(NBUF):
        d = {n: t.clone() for n, t in base.items()}
        d.update(alloc_outputs(cfg, 1, "cuda", o_core=False))
        sets.append(d)
    del base
    scale = 1.0 / math.sqrt(cfg.D)

    def step(i):
        d = sets[i % NBUF]
        kda.kda_decode(d["q"], d["k"], d["v"], d["g"], d["beta"], d["conv_w"], d["ring"],
                       d["state"], d["state"], d["z"], d["norm_w"], d["out"], None,
                       scale=scale, rms_eps=RMS_EPS)

    if graph and steps % NBUF == 0:
        # A serving loop replays the decode step from a captured graph: one graph holds
        # NBUF steps (one per buffer set); HIP events bracket each replay, so a step's
        # kernel time is a replay's time / NBUF (the kernels plus the gaps between them).
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(NBUF):
                step(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(NBUF):
                step(i)
        for _ in range(max(1, -(-warmup // NBUF))):
            g.replay()
        torch.cuda.synchronize()
        reps = steps // NBUF
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(reps):
            ev[i][0].record()
            g.replay()
            ev[i][1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        kern_ms = sorted(a.elapsed_time(b) / NBUF for a, b in ev)
        return inp, wall, sum(kern_ms) / len(kern_ms), kern_ms[len(kern_ms) // 2]

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record()
        step(warmup + i)
        ev[i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = sorted(a.elapsed_time(b) for a, b in ev)
    return inp, wall, sum(kern_ms) / len(kern_ms), kern_ms[len(kern_ms) // 2]


def run_prefill(cfg, mode, reps=5, d=None):
    import torch

    import gated_delta_rule_68_amd as kda
    from gated_delta_rule_68_amd.torch_io import alloc_outputs, tiled_device_inputs

    d = dict(tiled_device_inputs(cfg) if d is None else d)
    d.update(alloc_outputs(cfg, cfg.T, "cuda", o_core=False))
    code = kda.KDA_DTYPE_BF16 if cfg.dtype == "bf16" else kda.KDA_DTYPE_F32
    nb = kda.workspace_bytes(cfg.B, cfg.T, cfg.H, cfg.D, code, mode, gdn=cfg.gdn)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
    ring0, s_out = d["ring"].clone(), torch.empty_like(d["state"])
    fn = kda.gdn_prefill if cfg.gdn else kda.kda_prefill
    scale = 1.0 / math.sqrt(cfg.D)

    def once():
        d["ring"].copy_(ring0)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn(d["q"], d["k"], d["v"], d["g"], d["beta"], d["conv_w"], d["ring"], d["state"], s_out,
           d["z"], d["norm_w"], d["out"], None, scale=scale, rms_eps=RMS_EPS, mode=mode,
           workspace=ws)
        b.record()
        return a, b

    for _ in range(3):  # warm-up runs
        once()
    torch.cuda.synchronize()
    evs = [once() for _ in range(reps)]
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in evs)[reps // 2]
    arm = kda.prefill_arm(cfg.B, cfg.T, cfg.H, cfg.D, code, mode, gdn=cfg.gdn)
    return ms, kda.ARM_NAMES.get(arm, str(arm))


def run_verify_leg(T_stash: int = 8, keep: int = 4, reps: int = 20) -> dict:
    """Speculative verify at the decode shape (B=64, H=64, D=128, bf16): one sequential
    prefill over T_stash draft rows, and the exact rollback of that round to `keep` rows
    (ring restore + replay from the pre-round state). HIP-event time of each call, and
    algorithmic HBM bytes (state both ways, ring both ways, rows read / written)."""
    import torch

    import gated_delta_rule_68_amd as kda
    from gated_delta_rule_68_amd.synth import CONFIGS
    from gated_delta_rule_68_amd.torch_io import alloc_outputs, tiled_device_inputs

    cfg = CONFIGS["kda_decode"].with_(T=T_stash)
    d = dict(tiled_device_inputs(cfg))
    d.update(alloc_outputs(cfg, T_stash, "cuda", o_core=False))
    ring_snap, state_snap = d["ring"].clone(), d["state"].clone()
    ring, state = d["ring"].clone(), d["state"].clone()
    scale = 1.0 / math.sqrt(cfg.D)

    def verify():
        kda.kda_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["conv_w"], ring, state, state,
                        d["z"], d["norm_w"], d["out"], None, scale=scale, rms_eps=RMS_EPS,
                        mode=kda.KDA_MODE_SEQUENTIAL)

    def rollback():
        kda.kda_rollback(d["q"], d["k"], d["v"], d["g"], d["beta"], d["conv_w"], ring_snap, state_snap,
                         ring, state, keep)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(b) for a, b in ev)[reps // 2]

    es = 2
    qkv, B, H = cfg.qkv, cfg.B, cfg.H
    state_b = 2 * B * H * cfg.D * cfg.D * 4
    ring_b = 2 * B * 3 * qkv * (cfg.K - 1) * 4
    row_in = (5 * qkv + H) * es  # q, k, v, g, z + beta
    ms_v = timed(verify)
    ms_r = timed(rollback)
    bytes_v = state_b + ring_b + B * T_stash * (row_in + qkv * es)
    bytes_r = state_b + 2 * ring_b + B * keep * (row_in - qkv * es)  # ring copy, no z / out
    rec = {"workload": f"KDA verify B={B} H={H} D={cfg.D} bf16, {T_stash} draft rows, rollback to {keep}",
           "verify_ms": ms_v, "verify_tokens_per_s": B * T_stash / (ms_v * 1e-3),
           "verify_hbm_gbs": bytes_v / (ms_v * 1e-3) / 1e9,
           "rollback_ms": ms_r, "rollback_hbm_gbs": bytes_r / (ms_r * 1e-3) / 1e9}
    log(f"verify/rollback: {rec}")
    return rec


def _timed(fn, reps):
    """Median HIP-event time (ms) of fn(i) over reps calls after one untimed call."""
    import torch

    fn(0)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i, (a, b) in enumerate(ev):
        a.record()
        fn(i)
        b.record()
    torch.cuda.synchronize()
    return sorted(a.elapsed_time(b) for a, b in ev)[reps // 2]


def _timed_graph(fn, nbuf, reps):
    """Median time (ms) per call of fn(0) .. fn(nbuf - 1) captured in one HIP graph:
    HIP events bracket each replay of the nbuf calls, and a call's time is a replay's
    time / nbuf (the kernels plus the gaps between them), as for the decode step."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(nbuf):
            fn(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(nbuf):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record()
        g.replay()
        b.record()
    torch.cuda.synchronize()
    return sorted(a.elapsed_time(b) / nbuf for a, b in ev)[reps // 2]


def _timed_pair(fa, fb, reps):
    """Median HIP-event times (ms) of fa(i) and fb(i), interleaved call by call (so that
    clock or cache drift affects both alike), after one untimed call of each."""
    import torch

    fa(0)
    fb(0)
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)] for _ in range(2)]
    for i in range(reps):
        for k, f in enumerate((fa, fb)):
            ev[k][i][0].record()
            f(i)
            ev[k][i][1].record()
    torch.cuda.synchronize()
    return tuple(sorted(a.elapsed_time(b) for a, b in e)[reps // 2] for e in ev)


def run_gated_leg(reps: int = 50) -> dict:
    """The fused gate activation (softplus form, g = max(-5, -e^A_log * softplus(x +
    dt_bias)), beta = sigmoid(b)): the gated decode step at the decode shape and the
    gated chunked prefill of the single-sequence KDA workload, each beside the same
    call on precomputed g / beta. Algorithmic bytes are the plain path's plus the gate
    parameters (A_log-derived factor per head, bias per gate column, fp32)."""
    import torch

    import gated_delta_rule_68_amd as kda
    from gated_delta_rule_68_amd.synth import CONFIGS
    from gated_delta_rule_68_amd.torch_io import alloc_outputs, tiled_device_inputs

    rec = {"form": "softplus, lower bound -5"}
    cfg = CONFIGS["kda_decode"]
    base = tiled_device_inputs(cfg)
    ga = -torch.exp(base["A_log"])
    sets = []
    for _ in range(NBUF):
        d = {n: t.clone() for n, t in base.items()}
        d.update(alloc_outputs(cfg, 1, "cuda", o_core=False))
        sets.append(d)
    del base
    scale = 1.0 / math.sqrt(cfg.D)

    # interleaved below: the gated call takes the even buffer sets, the plain one the
    # odd ones, so that no call finds its state left in the last-level cache
    def dec_gated(i=0):
        d = sets[(2 * i) % NBUF]
        kda.kda_decode_gated(d["q"], d["k"], d["v"], d["gate_x"], d["beta_x"], ga, d["dt_bias"],
                             d["conv_w"], d["ring"], d["state"], d["state"], d["z"], d["norm_w"],
                             d["out"], None, gate_form=kda.KDA_GATE_SOFTPLUS, gate_lb=-5.0,
                             scale=scale, rms_eps=RMS_EPS)

    def dec_plain(i=0):
        d = sets[(2 * i + 1) % NBUF]
        kda.kda_decode(d["q"], d["k"], d["v"], d["g"], d["beta"], d["conv_w"], d["ring"],
                       d["state"], d["state"], d["z"], d["norm_w"], d["out"], None,
                       scale=scale, rms_eps=RMS_EPS)

    nb = decode_bytes(cfg) + (cfg.H + cfg.qkv) * 4
    ms_g, ms_p = _timed_pair(dec_gated, dec_plain, reps)
    rec["decode"] = {"workload": f"KDA decode B={cfg.B} H={cfg.H} D={cfg.D} bf16",
                     "gated_ms": ms_g, "plain_ms": ms_p,
                     "gated_tokens_per_s": cfg.B / (ms_g * 1e-3),
                     "gated_hbm_gbs": nb / (ms_g * 1e-3) / 1e9,
                     "gated_hbm_frac": nb / (ms_g * 1e-3) / 1e9 / HBM_PEAK_GBS}
    del sets
    torch.cuda.empty_cache()

    for name in ("kda_prefill", "gdn_prefill"):
        cfg = CONFIGS[name]
        d = dict(tiled_device_inputs(cfg))
        d.update(alloc_outputs(cfg, cfg.T, "cuda", o_core=False))
        ga = -torch.exp(d["A_log"])
        mode = kda.KDA_MODE_CHUNKED
        ws = torch.empty(max(kda.workspace_bytes(cfg.B, cfg.T, cfg.H, cfg.D, kda.KDA_DTYPE_BF16, mode,
                                                 gdn=cfg.gdn), 1), dtype=torch.uint8, device="cuda")
        ring0, s_out = d["ring"].clone(), torch.empty_like(d["state"])
        gated = kda.gdn_prefill_gated if cfg.gdn else kda.kda_prefill_gated
        plain = kda.gdn_prefill if cfg.gdn else kda.kda_prefill

        def pre_gated(i=0):
            d["ring"].copy_(ring0)
            gated(d["q"], d["k"], d["v"], d["gate_x"], d["beta_x"], ga, d["dt_bias"], d["conv_w"],
                  d["ring"], d["state"], s_out, d["z"], d["norm_w"], d["out"], None,
                  gate_form=kda.KDA_GATE_SOFTPLUS, gate_lb=-5.0, scale=scale, rms_eps=RMS_EPS,
                  mode=mode, workspace=ws)

        def pre_plain(i=0):
            d["ring"].copy_(ring0)
            plain(d["q"], d["k"], d["v"], d["g"], d["beta"], d["conv_w"], d["ring"], d["state"], s_out,
                  d["z"], d["norm_w"], d["out"], None, scale=scale, rms_eps=RMS_EPS, mode=mode,
                  workspace=ws)

        ms_g, ms_p = _timed_pair(pre_gated, pre_plain, 7)
        rec[name] = {"workload": f"{'GDN' if cfg.gdn else 'KDA'} chunked prefill B={cfg.B} T={cfg.T} "
                                 f"H={cfg.H} D={cfg.D} bf16 (incl. a ring reset copy)",
                     "gated_ms": ms_g, "plain_ms": ms_p,
                     "gated_tokens_per_s": cfg.B * cfg.T / (ms_g * 1e-3)}
        del d, ws
        torch.cuda.empty_cache()
    log(f"gated: {rec}")
    return rec


def run_gqa_leg(reps: int = 50) -> dict:
    """GDN with grouped heads: 32 value heads over 16 query / key heads, D=128, bf16.
    The batched decode step (B=64, state in place, buffer sets cycled), timed like the
    decode step (a HIP graph of NBUF steps replayed, a replay's time / NBUF; the time of
    each eager call between HIP events beside it), and the chunked prefill of the GDN
    workload (B=4, T=8192, HIP-event time of each call); algorithmic HBM bytes (q / k
    rows are Hk*D wide)."""
    import torch

    import gated_delta_rule_68_amd as kda
    from gated_delta_rule_68_amd.synth import CONFIGS
    from gated_delta_rule_68_amd.torch_io import alloc_outputs, tiled_device_inputs

    rec = {}
    cfg = CONFIGS["kda_decode"].with_(gdn=True, H=32, Hk=16)
    base = tiled_device_inputs(cfg)
    sets = []
    for _ in range(NBUF):
        d = {n: t.clone() for n, t in base.items()}
        d.update(alloc_outputs(cfg, 1, "cuda", o_core=False))
        sets.append(d)
    del base
    scale = 1.0 / math.sqrt(cfg.D)

    def dec(i=0):
        d = sets[i % NBUF]
        kda.gdn_decode_gqa(d["q"], d["k"], d["v"], d["g"], d["beta"], d["conv_w"], d["ring"], d["state"],
                           d["state"], d["z"], d["norm_w"], d["out"], None, scale=scale, rms_eps=RMS_EPS)

    B, H, D, K, kw, vw = cfg.B, cfg.H, cfg.D, cfg.K, cfg.kw, cfg.qkv
    nb = (2 * B * H * D * D * 4 + 2 * B * cfg.conv_rows * (K - 1) * 4
          + (2 * B * kw + 3 * B * vw + 2 * B * H) * 2 + cfg.conv_rows * K * 4 + D * 4)
    eager_ms = _timed(dec, reps)
    ms = _timed_graph(dec, NBUF, reps)
    rec["decode"] = {"workload": f"GDN decode B={B} H={H} Hk={cfg.hk} D={D} bf16", "ms": ms,
                     "time": f"HIP graph of {NBUF} steps replayed, a replay / {NBUF} (median)",
                     "eager_ms": eager_ms, "tokens_per_s": B / (ms * 1e-3), "hbm_gbs": nb / (ms * 1e-3) / 1e9,
                     "hbm_frac": nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "algorithmic_bytes": nb}
    del sets
    torch.cuda.empty_cache()

    cfg = CONFIGS["gdn_prefill"].with_(Hk=16)
    d = dict(tiled_device_inputs(cfg))
    d.update(alloc_outputs(cfg, cfg.T, "cuda", o_core=False))
    mode = kda.KDA_MODE_CHUNKED
    ws = torch.empty(max(kda.gqa_workspace_bytes(cfg.B, cfg.T, cfg.H, cfg.hk, cfg.D, kda.KDA_DTYPE_BF16, mode),
                         1), dtype=torch.uint8, device="cuda")
    ring0, s_out = d["ring"].clone(), torch.empty_like(d["state"])

    def pre(i=0):
        d["ring"].copy_(ring0)
        kda.gdn_prefill_gqa(d["q"], d["k"], d["v"], d["g"], d["beta"], d["conv_w"], d["ring"], d["state"], s_out,
                            d["z"], d["norm_w"], d["out"], None, scale=scale, rms_eps=RMS_EPS, mode=mode,
                            workspace=ws)

    ms = _timed(pre, 5)
    B, T, H, kw, vw = cfg.B, cfg.T, cfg.H, cfg.kw, cfg.qkv
    nb = ((2 * kw + 3 * vw + 2 * H) * B * T * 2 + 2 * B * H * D * D * 4 + 2 * B * cfg.conv_rows * (K - 1) * 4
          + cfg.conv_rows * K * 4 + D * 4)
    tf = chunk_flops(cfg) / (ms * 1e-3) / 1e12
    rec["prefill"] = {"workload": f"GDN chunked prefill B={B} T={T} H={H} Hk={cfg.hk} D={D} bf16 "
                                  "(incl. a ring reset copy)", "ms": ms, "tokens_per_s": B * T / (ms * 1e-3),
                      "hbm_gbs": nb / (ms * 1e-3) / 1e9, "mfma_tflops": tf, "mfma_frac": tf / BF16_PEAK_TFLOPS}
    del d, ws
    torch.cuda.empty_cache()
    log(f"gqa: {rec}")
    return rec


def run_varlen_leg() -> dict:
    """Packed variable-length KDA prefill (H=64, D=128, bf16, chunked arm): 16 prompt
    lengths drawn log-uniformly from 64..4096 (numpy seed 7). One packed call, against
    the same work as a batch padded to the longest prompt and as one call per prompt;
    tokens/s counts the prompts' own tokens only."""
    import numpy as np
    import torch

    import gated_delta_rule_68_amd as kda
    from gated_delta_rule_68_amd.synth import CONFIGS
    from gated_delta_rule_68_amd.torch_io import ACTS, alloc_outputs, tiled_device_inputs

    lens = (2.0 ** np.random.default_rng(7).uniform(6, 12, 16)).astype(int)
    N, Tm = len(lens), int(lens.max())
    cfg = CONFIGS["kda_prefill"].with_(B=N, T=Tm)
    d = tiled_device_inputs(cfg)
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).to("cuda")
    T_total = int(lens.sum())
    p = {n: torch.cat([d[n][b, :L] for b, L in enumerate(lens)], 0).contiguous() for n in ACTS}
    mode, code = kda.KDA_MODE_CHUNKED, kda.KDA_DTYPE_BF16
    scale = 1.0 / math.sqrt(cfg.D)
    ring0 = d["ring"].clone()
    s_out = torch.empty_like(d["state"])
    out_p = torch.empty(T_total, cfg.qkv, dtype=torch.bfloat16, device="cuda")
    ws_p = torch.empty(max(kda.varlen_workspace_bytes(N, T_total, cfg.H, cfg.D, code, mode), 1),
                       dtype=torch.uint8, device="cuda")

    def packed(i=0):
        d["ring"].copy_(ring0)
        kda.prefill_varlen(p["q"], p["k"], p["v"], p["g"], p["beta"], d["conv_w"], d["ring"], d["state"], s_out,
                           p["z"], d["norm_w"], out_p, cu, None, scale=scale, rms_eps=RMS_EPS, mode=mode,
                           workspace=ws_p)

    out_b = alloc_outputs(cfg, Tm, "cuda", o_core=False)["out"]
    ws_b = torch.empty(max(kda.workspace_bytes(N, Tm, cfg.H, cfg.D, code, mode), 1), dtype=torch.uint8,
                       device="cuda")

    def padded(i=0):
        d["ring"].copy_(ring0)
        kda.kda_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["conv_w"], d["ring"], d["state"], s_out,
                        d["z"], d["norm_w"], out_b, None, scale=scale, rms_eps=RMS_EPS, mode=mode, workspace=ws_b)

    singles = []
    for b, L in enumerate(lens):
        one = {n: d[n][b:b + 1, :L].contiguous() for n in ("q", "k", "v", "g", "beta", "z")}
        one["ring"], one["state"] = d["ring"][b:b + 1].clone(), d["state"][b:b + 1]
        one["s_out"] = torch.empty_like(one["state"])
        one["out"] = torch.empty(1, int(L), cfg.qkv, dtype=torch.bfloat16, device="cuda")
        one["ws"] = torch.empty(max(kda.workspace_bytes(1, int(L), cfg.H, cfg.D, code, mode), 1),
                                dtype=torch.uint8, device="cuda")
        singles.append(one)

    def per_prompt(i=0):
        for o in singles:
            kda.kda_prefill(o["q"], o["k"], o["v"], o["g"], o["beta"], d["conv_w"], o["ring"], o["state"],
                            o["s_out"], o["z"], d["norm_w"], o["out"], None, scale=scale, rms_eps=RMS_EPS,
                            mode=mode, workspace=o["ws"])

    ms_p, ms_b = _timed_pair(packed, padded, 5)
    ms_s = _timed(per_prompt, 5)
    rec = {"workload": f"KDA chunked prefill H={cfg.H} D={cfg.D} bf16, {N} prompts of {int(lens.min())}.."
                       f"{Tm} tokens ({T_total} in all)", "lengths": [int(x) for x in lens],
           "packed_ms": ms_p, "packed_tokens_per_s": T_total / (ms_p * 1e-3),
           "padded_ms": ms_b, "padded_tokens_per_s": T_total / (ms_b * 1e-3),
           "per_prompt_ms": ms_s, "per_prompt_tokens_per_s": T_total / (ms_s * 1e-3)}
    del d, p, singles, ws_p, ws_b
    torch.cuda.empty_cache()
    log(f"varlen: {rec}")
    return rec


def run_prefill_legs() -> dict:
    """Each prefill workload on the chunked and the sequential arm, and on the segmented
    arm where AUTO takes it: time of the whole arm (every kernel it launches), tokens/s,
    algorithmic HBM GB/s and, for the chunked arms, the dense-tile contraction TFLOP/s
    of the unsegmented algorithm as a fraction of the bf16 peak."""
    import torch

    import gated_delta_rule_68_amd as kda
    from gated_delta_rule_68_amd.synth import CONFIGS
    from gated_delta_rule_68_amd.torch_io import tiled_device_inputs

    legs = {"measured_gemm_tflops": measure_gemm()}
    for name in ("kda_prefill", "gdn_prefill", "kda_long"):
        cfg = CONFIGS[name]
        d = tiled_device_inputs(cfg)
        rec = {"workload": f"{'GDN' if cfg.gdn else 'KDA'} prefill B={cfg.B} T={cfg.T} "
                           f"H={cfg.H} D={cfg.D} {cfg.dtype}",
               "algorithmic_bytes": prefill_bytes(cfg), "dense_tile_flops": chunk_flops(cfg)}
        auto = kda.prefill_arm(cfg.B, cfg.T, cfg.H, cfg.D, 1, kda.KDA_MODE_AUTO, gdn=cfg.gdn)
        for mode in (kda.KDA_MODE_CHUNKED, kda.KDA_MODE_SEGMENTED, kda.KDA_MODE_SEQUENTIAL):
            if kda.prefill_arm(cfg.B, cfg.T, cfg.H, cfg.D, 1, mode, gdn=cfg.gdn) < 0:
                continue
            if mode == kda.KDA_MODE_SEGMENTED and kda.ARM_NAMES.get(auto) != "segmented":
                continue  # timed where AUTO takes it
            ms, arm = run_prefill(cfg, mode, reps=10, d=d)
            r = {"ms": ms, "tokens_per_s": cfg.B * cfg.T / (ms * 1e-3),
                 "hbm_gbs": prefill_bytes(cfg) / (ms * 1e-3) / 1e9}
            if arm in ("chunked", "segmented"):
                tf = chunk_flops(cfg) / (ms * 1e-3) / 1e12
                r.update({"mfma_tflops": tf, "mfma_frac": tf / BF16_PEAK_TFLOPS,
                          "mfma_frac_of_measured_gemm": tf / legs["measured_gemm_tflops"],
                          "hbm_frac": r["hbm_gbs"] / HBM_PEAK_GBS})
            rec[arm] = r
            log(f"prefill {name} {arm}: {r}")
        legs[name] = rec
        del d
        torch.cuda.empty_cache()
    return legs


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-verify", action="store_true")
    ap.add_argument("--no-gated", action="store_true")
    ap.add_argument("--no-gqa", action="store_true")
    ap.add_argument("--no-varlen", action="store_true")
    ap.add_argument("--copy-only", action="store_true",
                    help="only run the 1 GiB device copy (counter calibration)")
    ap.add_argument("--prefill-only", metavar="WORKLOAD",
                    help="only run this prefill workload (kda_prefill, gdn_prefill, kda_long) on "
                         "the arm of --prefill-mode, --steps times after one warm-up (for profilers)")
    ap.add_argument("--prefill-mode", choices=("chunked", "segmented", "auto"), default="chunked",
                    help="prefill mode of --prefill-only (default: chunked)")
    ap.add_argument("--eager", action="store_true",
                    help="time the decode steps as separate launches instead of graph replays")
    ap.add_argument("--cpu-baselines", action="store_true",
                    help="only time the fp64 oracle on the host cores, on every workload "
                         "(bounded slices; no GPU used)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the mixer shards by (sequence, head) with no exchange)",
              file=sys.stderr)
        sys.exit(2)
    if args.cpu_baselines:
        print(json.dumps({"cpu_baselines": cpu_baselines()}), flush=True)
        return

    import torch

    from gated_delta_rule_68_amd import _lib
    from gated_delta_rule_68_amd.synth import CONFIGS

    if not os.path.exists(_lib.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_only:
        print(json.dumps({"copy_bytes": COPY_BYTES, "copy_gbs": measure_copy()}), flush=True)
        return
    if args.prefill_only:
        import gated_delta_rule_68_amd as kda

        cfg = CONFIGS[args.prefill_only]
        mode = {"chunked": kda.KDA_MODE_CHUNKED, "segmented": kda.KDA_MODE_SEGMENTED,
                "auto": kda.KDA_MODE_AUTO}[args.prefill_mode]
        ms, arm = run_prefill(cfg, mode, reps=max(1, args.steps))
        print(json.dumps({"workload": args.prefill_only, "arm": arm, "ms": ms,
                          "tokens_per_s": cfg.B * cfg.T / (ms * 1e-3)}), flush=True)
        return

    cfg = CONFIGS["kda_decode"]
    log(f"decode: {cfg}")
    graphed = not args.eager and args.steps % NBUF == 0
    inp, wall, kern_avg_ms, kern_med_ms = run_decode(cfg, args.steps, args.warmup, graph=graphed)
    ms_per_step = 1e3 * wall / args.steps
    tokens_per_step = cfg.B * cfg.T
    nbytes = decode_bytes(cfg)
    achieved = nbytes / (kern_avg_ms * 1e-3) / 1e9
    prof = profile_record("seq_short_kernel_kda_decode")
    line = {
        "metric": METRIC,
        "value": tokens_per_step / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded)",
        "config": {"workload": "KDA batched decode step", "activations": "bf16",
                   "B": cfg.B, "T": cfg.T, "H": cfg.H,
                   "D": cfg.D, "conv_kernel": cfg.K, "state": "fp32, in place",
                   "buffers_cycled": NBUF,
                   "arm": "seq_fused (kernel seq_short_kernel, one token per call)",
                   "launch": f"HIP graph of {NBUF} steps, replayed" if graphed else "one launch per step"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": prof.get("bytes_per_launch"),
                     "kernel": "seq_short_kernel<bf16,kda,1>",
                     # HIP events on the launch stream around each graph replay of NBUF
                     # launches, divided by NBUF: the kernel plus the gaps between launches
                     # (an upper bound of the kernel's own duration)
                     "launch_avg_us": kern_avg_ms * 1e3, "launch_median_us": kern_med_ms * 1e3,
                     "launch_time": (f"HIP events around each replay of {NBUF} launches, / {NBUF}" if graphed
                                     else "HIP events around each launch"),
                     "rocprof_kernel_avg_us": prof.get("avg_us_trace"),
                     "algorithmic_bytes": nbytes, "measured_copy_gbs": measure_copy()},
    }
    if not args.no_prefill:
        line["prefill"] = run_prefill_legs()
    if not args.no_verify:
        line["verify_rollback"] = run_verify_leg()
    if not args.no_gated:
        line["gated"] = run_gated_leg()
    if not args.no_gqa:
        line["gqa"] = run_gqa_leg()
    if not args.no_varlen:
        line["varlen"] = run_varlen_leg()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, inp)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
