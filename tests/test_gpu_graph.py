"""The decode step replayed from a captured HIP graph (torch.cuda.CUDAGraph over the
C ABI calls on the capturing stream), as a serving loop and bench.py run it: every
replay, with eager work and synchronisations between replays, equals the same steps run
eagerly, bit for bit (outputs, conv ring and state)."""
import math

import pytest
import torch

import gated_delta_rule_68_amd as kda
from gated_delta_rule_68_amd.synth import CONFIGS
from gated_delta_rule_68_amd.torch_io import alloc_outputs
from tests.gpu_util import DEV, RMS_EPS, assert_bitwise, inputs_for

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("gdn", [False, True])
def test_graph_replays_equal_eager_decode_steps(gdn):
    steps = 3
    cfg = CONFIGS["kda_decode"].with_(B=4, H=8, T=steps, gdn=gdn)
    inp, dev = inputs_for(cfg)
    scale = 1.0 / math.sqrt(cfg.D)
    rows = [{n: dev[n][:, t:t + 1].clone(memory_format=torch.contiguous_format)
             for n in ("q", "k", "v", "g", "beta", "z")} for t in range(steps)]
    fn = kda.gdn_decode if gdn else kda.kda_decode

    def run_steps(ring, state, outs):
        for t in range(steps):
            r = rows[t]
            fn(r["q"], r["k"], r["v"], r["g"], r["beta"], dev["conv_w"], ring, state, state, r["z"],
               dev["norm_w"], outs[t], None, scale=scale, rms_eps=RMS_EPS)

    # eager reference
    ring_e, state_e = dev["ring"].clone(), dev["state"].clone()
    outs_e = [alloc_outputs(cfg, 1, DEV, o_core=False)["out"] for _ in range(steps)]
    run_steps(ring_e, state_e, outs_e)
    torch.cuda.synchronize()

    # captured: static buffers, warmed on a side stream first
    ring_g, state_g = dev["ring"].clone(), dev["state"].clone()
    outs_g = [alloc_outputs(cfg, 1, DEV, o_core=False)["out"] for _ in range(steps)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run_steps(ring_g, state_g, outs_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_steps(ring_g, state_g, outs_g)
    torch.cuda.synchronize()

    x = torch.randn(256, 256, device=DEV)
    for rep in range(4):
        ring_g.copy_(dev["ring"])
        state_g.copy_(dev["state"])
        for o in outs_g:
            o.zero_()
        _ = x @ x  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        print("replay", rep, flush=True)
        for t in range(steps):
            assert_bitwise({"out": outs_g[t]}, {"out": outs_e[t]}, keys=("out",))
        assert_bitwise({"ring": ring_g, "state": state_g}, {"ring": ring_e, "state": state_e},
                       keys=("ring", "state"))
