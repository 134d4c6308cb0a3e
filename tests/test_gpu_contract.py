"""The C-ABI contract with real device buffers: every violation the host tests check
with fake addresses is rejected here too, before any launch (all outputs keep their
sentinel bytes), and valid calls still run afterwards.

Every pointer lies inside one device arena with room for the largest shape used, so a
call that got past validation by mistake would still only touch allocated memory. The
overflowing-shape case is left to the host test: it is rejected on the host only."""
import pytest
import torch

import gated_delta_rule_68_amd as kda
from tests.test_abi_host import (CASES, GATED_CASES, GATED_CHUNK_CASES, GATED_ROLLBACK_CASES, ROLLBACK_CASES,
                                 call_decode, call_gated, call_prefill, call_rollback, call_rollback_gated)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SLOT = 1 << 20  # bytes per argument slot (the shapes below need a few KB)
NAMES = ["q", "k", "v", "g", "beta", "conv_w", "ring", "state_in", "state_out", "z",
         "norm_w", "out", "o_core", "ws", "ring_snap", "state_snap", "gate_a", "gate_bias"]
OUTPUTS = ("ring", "state_out", "out", "o_core")
SENTINEL = 0x5A


@pytest.fixture(scope="module")
def arena():
    buf = torch.full((SLOT * (len(NAMES) + 1),), SENTINEL, dtype=torch.uint8, device=DEV)
    torch.cuda.synchronize()
    return buf


def real_args(arena, B=2, T=3, H=2, D=16, K=4, dtype=0, mode=1):
    base = arena.data_ptr()
    a = {n: base + i * SLOT for i, n in enumerate(NAMES)}
    a.update(B=B, T=T, H=H, D=D, K=K, dtype=dtype, mode=mode, ws_bytes=SLOT)
    return a


def rebase(arena, over):
    """The host cases name fake addresses BASE + i * 2^32 + off; map them to slot i."""
    from tests.test_abi_host import BASE
    base = arena.data_ptr()
    out = {}
    for k, v in over.items():
        if v is None:
            out[k] = 0
        elif isinstance(v, int) and v >= BASE:
            i, off = divmod(v - BASE, 1 << 32)
            out[k] = base + i * SLOT + off
        else:
            out[k] = v
    return out


def outputs_untouched(arena):
    torch.cuda.synchronize()
    for i, n in enumerate(NAMES):
        if n in OUTPUTS:
            sl = arena[i * SLOT:(i + 1) * SLOT]
            if not bool((sl == SENTINEL).all()):
                return n
    return None


GPU_CASES = [c for c in CASES if c[0] != "huge"]


@pytest.mark.parametrize("gdn", [False, True])
@pytest.mark.parametrize("what,over,rc", GPU_CASES, ids=[c[0] for c in GPU_CASES])
def test_prefill_rejected_before_launch(arena, what, over, rc, gdn):
    a = real_args(arena)
    a.update(rebase(arena, over))
    assert call_prefill(a, gdn) == rc
    assert outputs_untouched(arena) is None


@pytest.mark.parametrize("gdn", [False, True])
def test_decode_rejected_before_launch(arena, gdn):
    a = real_args(arena, T=2)
    assert call_decode(a, gdn) == 40005
    a = real_args(arena, T=1, D=64)
    assert call_decode(a, gdn) == 40002
    a = real_args(arena, T=1)
    a["z"] = 0
    assert call_decode(a, gdn) == 40001
    assert outputs_untouched(arena) is None


def test_workspace_too_small_rejected(arena):
    a = real_args(arena, B=1, T=100, H=2, D=16, mode=1)
    need = kda.workspace_bytes(1, 100, 2, 16, 0, 1)
    assert 0 < need <= SLOT
    a["ws_bytes"] = need - 1
    assert call_prefill(a) == 40006
    a["ws"], a["ws_bytes"] = 0, need
    assert call_prefill(a) == 40006
    assert outputs_untouched(arena) is None


@pytest.mark.parametrize("gdn", [False, True])
def test_valid_calls_after_rejections(gdn):
    """A small valid prefill and decode through the same raw C entry points (zero
    inputs give zero outputs and leave a zero state at zero) return 0."""
    B, T, H, D, K = 2, 3, 2, 16, 4
    qkv = H * D
    f32 = dict(dtype=torch.float32, device=DEV)
    t = {n: torch.zeros(B, T, qkv, **f32) for n in ("q", "k", "v", "z")}
    t["g"] = torch.zeros(B, T, H if gdn else qkv, **f32)
    t["beta"] = torch.zeros(B, T, H, **f32)
    t["conv_w"] = torch.zeros(3 * qkv, K, **f32)
    t["ring"] = torch.zeros(B, 3 * qkv, K - 1, **f32)
    t["state_in"] = torch.zeros(B, H, D, D, **f32)
    t["state_out"] = torch.full((B, H, D, D), 7.0, **f32)
    t["norm_w"] = torch.ones(D, **f32)
    t["out"] = torch.full((B, T, qkv), 7.0, **f32)
    t["o_core"] = torch.full((B, T, qkv), 7.0, **f32)
    a = {n: v.data_ptr() for n, v in t.items()}
    a.update(B=B, T=T, H=H, D=D, K=K, dtype=0, mode=1, ws=0, ws_bytes=0)
    assert call_prefill(a, gdn) == 0
    torch.cuda.synchronize()
    for n in ("state_out", "out", "o_core"):
        assert float(t[n].abs().max()) == 0.0, n
    a["T"] = 1
    t1 = {n: t[n][:, :1].contiguous() for n in ("q", "k", "v", "z", "g", "beta", "out", "o_core")}
    a.update({n: v.data_ptr() for n, v in t1.items()})
    assert call_decode(a, gdn) == 0
    torch.cuda.synchronize()
    assert float(t1["out"].abs().max()) == 0.0


@pytest.mark.parametrize("gdn", [False, True])
@pytest.mark.parametrize("what,over,kw,rc", ROLLBACK_CASES, ids=[c[0] for c in ROLLBACK_CASES])
def test_rollback_rejected_before_copy_or_launch(arena, what, over, kw, rc, gdn):
    a = real_args(arena)
    a.update(rebase(arena, over))
    assert call_rollback(a, gdn, **kw) == rc
    assert outputs_untouched(arena) is None


@pytest.mark.parametrize("decode", [False, True])
@pytest.mark.parametrize("gdn", [False, True])
@pytest.mark.parametrize("what,over,kw,rc", GATED_CASES, ids=[c[0] for c in GATED_CASES])
def test_gated_rejected_before_launch(arena, what, over, kw, rc, gdn, decode):
    a = real_args(arena, T=1 if decode else 3)
    a.update(rebase(arena, over))
    assert call_gated(a, gdn, decode, **kw) == rc
    assert outputs_untouched(arena) is None


@pytest.mark.parametrize("gdn", [False, True])
@pytest.mark.parametrize("what,over,kw,rc", GATED_ROLLBACK_CASES, ids=[c[0] for c in GATED_ROLLBACK_CASES])
def test_gated_rollback_rejected_before_copy_or_launch(arena, what, over, kw, rc, gdn):
    a = real_args(arena)
    a.update(rebase(arena, over))
    assert call_rollback_gated(a, gdn, **kw) == rc
    assert outputs_untouched(arena) is None


@pytest.mark.parametrize("gdn", [False, True])
@pytest.mark.parametrize("what,over,kw,rc", GATED_CHUNK_CASES, ids=[c[0] for c in GATED_CHUNK_CASES])
def test_gated_chunk_modes_refuse_unbounded_gates(arena, what, over, kw, rc, gdn):
    a = real_args(arena, T=100)
    a.update(over)
    assert call_gated(a, gdn, False, **kw) == rc
    assert outputs_untouched(arena) is None


def test_library_bound_before_torch_import():
    """A process that binds the library before importing torch itself still runs on
    one HIP runtime: the binding loads torch's runtime first. A fresh interpreter binds
    the library, then imports torch and runs a small decode (zero inputs, zero output)."""
    import os
    import subprocess
    import sys
    code = (
        "import gated_delta_rule_68_amd as kda\n"
        "kda.lib()\n"
        "import torch\n"
        "B, H, D, K = 2, 2, 16, 4\n"
        "f = dict(dtype=torch.float32, device='cuda:0')\n"
        "x = {n: torch.zeros(B, 1, H * D, **f) for n in ('q', 'k', 'v', 'g', 'z')}\n"
        "beta = torch.zeros(B, 1, H, **f)\n"
        "conv_w = torch.zeros(3 * H * D, K, **f)\n"
        "ring = torch.zeros(B, 3 * H * D, K - 1, **f)\n"
        "state = torch.zeros(B, H, D, D, **f)\n"
        "out = torch.full((B, 1, H * D), 7.0, **f)\n"
        "kda.kda_decode(x['q'], x['k'], x['v'], x['g'], beta, conv_w, ring, state, state, x['z'],\n"
        "               torch.ones(D, **f), out, None, scale=D ** -0.5, rms_eps=1e-5)\n"
        "torch.cuda.synchronize()\n"
        "assert float(out.abs().max()) == 0.0\n"
        "print('bound before torch: ok')\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=100)
    assert r.returncode == 0 and "ok" in r.stdout, r.stdout + r.stderr
