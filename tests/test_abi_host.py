"""C-ABI tests that need no GPU: the library loads, exports every function the
header declares, and rejects every contract violation before any launch.

The rejected calls pass fake (never dereferenced) device addresses. They are
skipped when a GPU is visible, where test_gpu_contract.py repeats them with real
buffers."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_68_amd as kda
from gated_delta_rule_68_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(?:int|size_t|const char\*)\s+(\w+)\s*\(", text)))


def test_library_exports_every_header_symbol():
    lib = kda.lib()
    names = header_functions()
    assert set(names) == set(_lib.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), f"libkda.so does not export {n}"


def test_status_strings():
    assert kda.status_string(0) == "ok"
    for rc in range(40001, 40011):
        s = kda.status_string(rc)
        assert s and s != "unknown status code", rc
    assert "HIP" in kda.status_string(10001)


def _gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


BASE = 1 << 40  # fake, 256-byte aligned, far-apart addresses; never dereferenced


def fake_args(B=2, T=3, H=2, D=16, K=4, dtype=0, mode=1):
    names = ["q", "k", "v", "g", "beta", "conv_w", "ring", "state_in", "state_out", "z",
             "norm_w", "out", "o_core", "ws", "ring_snap", "state_snap", "gate_a", "gate_bias"]
    a = {n: BASE + i * (1 << 32) for i, n in enumerate(names)}
    a.update(B=B, T=T, H=H, D=D, K=K, dtype=dtype, mode=mode, ws_bytes=1 << 31)
    return a


def call_prefill(a, gdn=False):
    f = kda.lib().gdn_prefill if gdn else kda.lib().kda_prefill
    return f(a["q"], a["k"], a["v"], a["g"], a["beta"], a["conv_w"], a["ring"], a["state_in"],
             a["state_out"], a["z"], a["norm_w"], a["out"], a["o_core"], a["B"], a["T"], a["H"],
             a["D"], a["K"], 0.25, 1e-5, a["dtype"], a["mode"], a["ws"], a["ws_bytes"], None)


def call_decode(a, gdn=False):
    f = kda.lib().gdn_decode if gdn else kda.lib().kda_decode
    return f(a["q"], a["k"], a["v"], a["g"], a["beta"], a["conv_w"], a["ring"], a["state_in"],
             a["state_out"], a["z"], a["norm_w"], a["out"], a["o_core"], a["B"], a["T"], a["H"],
             a["D"], a["K"], 0.25, 1e-5, a["dtype"], None)


CASES = [
    ("null q", dict(q=None), 40001),
    ("null state_out", dict(state_out=None), 40001),
    ("null norm_w", dict(norm_w=None), 40001),
    ("D=64", dict(D=64), 40002),
    ("D=0", dict(D=0), 40002),
    ("K=1", dict(K=1), 40003),
    ("K=9", dict(K=9), 40003),
    ("B=0", dict(B=0), 40004),
    ("T=0", dict(T=0), 40004),
    ("H=0", dict(H=0), 40004),
    ("huge", dict(B=1 << 20, T=1 << 20), 40004),
    ("misaligned q", dict(q=BASE + 8), 40007),
    ("misaligned ring", dict(ring=BASE + 6 * (1 << 32) + 4), 40007),
    ("dtype 2", dict(dtype=2), 40008),
    ("mode 7", dict(mode=7), 40008),
    ("chunked D=16", dict(mode=2, D=16), 40008),
    # the chunked and segmented arms take bf16 activations only (fp32 cannot meet its
    # 1e-3 bar through bf16 MFMA operands): fp32 through the explicit modes is refused
    ("chunked fp32", dict(mode=2, D=128, dtype=0), 40008),
    ("segmented fp32", dict(mode=3, D=128, dtype=0), 40008),
    ("out overlaps q", dict(out=BASE + 64), 40009),
    ("state partial overlap", dict(state_out=BASE + 7 * (1 << 32) + 256), 40009),
    ("ring overlaps conv_w", dict(ring=BASE + 5 * (1 << 32) + 16), 40009),
    ("o_core overlaps out", dict(o_core=BASE + 11 * (1 << 32) + 32), 40009),
]


@pytest.mark.skipif(_gpu_visible(), reason="fake pointers only where no GPU is visible")
@pytest.mark.parametrize("gdn", [False, True])
@pytest.mark.parametrize("what,over,rc", CASES, ids=[c[0] for c in CASES])
def test_prefill_contract(what, over, rc, gdn):
    a = fake_args()
    a.update({k: (0 if v is None else v) for k, v in over.items()})
    assert call_prefill(a, gdn) == rc


@pytest.mark.skipif(_gpu_visible(), reason="fake pointers only where no GPU is visible")
@pytest.mark.parametrize("what,over,rc", CASES, ids=[c[0] for c in CASES])
def test_prefill_noalloc_contract(what, over, rc):
    """The allocation-free prefill refuses every contract violation the plain prefill
    does, with the same code and before it looks up its scratch buffer."""
    a = fake_args()
    a.update({k: (0 if v is None else v) for k, v in over.items()})
    f = kda.lib().kda_prefill_noalloc
    assert f(a["q"], a["k"], a["v"], a["g"], a["beta"], a["conv_w"], a["ring"], a["state_in"], a["state_out"],
             a["z"], a["norm_w"], a["out"], a["o_core"], a["B"], a["T"], a["H"], a["D"], a["K"], 0.25, 1e-5,
             a["dtype"], a["mode"], None) == rc


@pytest.mark.skipif(_gpu_visible(), reason="fake pointers only where no GPU is visible")
@pytest.mark.parametrize("gdn", [False, True])
def test_decode_contract(gdn):
    a = fake_args(T=2)
    assert call_decode(a, gdn) == 40005
    a = fake_args(T=1, D=64)
    assert call_decode(a, gdn) == 40002
    a = fake_args(T=1)
    a["z"] = 0
    assert call_decode(a, gdn) == 40001


@pytest.mark.skipif(_gpu_visible(), reason="fake pointers only where no GPU is visible")
def test_workspace_too_small():
    # B*H small and T long: the split sequential arm, which needs a workspace.
    a = fake_args(B=1, T=100, H=2, D=16, mode=1)
    need = kda.workspace_bytes(1, 100, 2, 16, 0, 1)
    assert need > 0
    a["ws_bytes"] = need - 1
    assert call_prefill(a) == 40006
    a["ws"] = 0
    a["ws_bytes"] = need
    assert call_prefill(a) == 40006


def test_queries():
    assert kda.workspace_bytes(1, 1, 64, 128, 1, 1) == 0  # T = 1: fused arm
    assert kda.prefill_arm(64, 1, 64, 128, 1, 1) == 1
    assert kda.prefill_arm(1, 4626, 64, 128, 1, 1) == 2
    assert kda.prefill_arm(1, 64, 2, 64, 0, 1) == -1
    assert kda.workspace_bytes(0, 1, 1, 16, 0, 1) == ctypes.c_size_t(-1).value


def test_auto_arm_boundaries():
    # bf16 at D = 128: the short-call sequential kernel up to 16 tokens; the chunked arm
    # from 33 tokens, or from 17 with fewer than 1024 (b, h) pairs; fp32 and D = 16 stay
    # sequential (fused from 1024 pairs, else the column-split pipeline)
    assert kda.prefill_arm(64, 16, 64, 128, 1, 0) == 1
    assert kda.prefill_arm(64, 17, 64, 128, 1, 0) == 1
    assert kda.prefill_arm(64, 32, 64, 128, 1, 0) == 1
    assert kda.prefill_arm(64, 33, 64, 128, 1, 0) == 3
    assert kda.prefill_arm(8, 16, 32, 128, 1, 0) == 1
    assert kda.prefill_arm(8, 17, 32, 128, 1, 0) == 3
    assert kda.prefill_arm(16, 17, 64, 128, 1, 0) == 1  # 1024 pairs
    assert kda.prefill_arm(64, 64, 64, 128, 0, 0) == 1  # fp32
    assert kda.prefill_arm(8, 64, 32, 128, 0, 0) == 2
    assert kda.prefill_arm(8, 64, 32, 16, 1, 0) == 2  # D = 16
    # the explicit chunked and segmented modes refuse fp32 activations
    assert kda.prefill_arm(8, 64, 32, 128, 0, 2) == -1
    assert kda.prefill_arm(8, 64, 32, 128, 0, 3) == -1
    assert kda.workspace_bytes(8, 64, 32, 128, 0, 2) == ctypes.c_size_t(-1).value


def test_segmented_queries():
    # AUTO takes the segmented arm when its timed plan (segments of at least eight
    # 64-row units) shortens the critical path to 85% of the chunked arm's or less
    assert kda.prefill_arm(1, 4626, 64, 128, 1, 0) == 4  # 64 pairs, 73 chunks: 5 segments
    assert kda.prefill_arm(2, 4626, 64, 128, 1, 0) == 4  # 128 pairs: 3 segments
    assert kda.prefill_arm(4, 8192, 32, 128, 1, 0, gdn=True) == 4
    assert kda.prefill_arm(8, 16384, 64, 128, 1, 0) == 3  # 512 pairs fill the chip
    assert kda.prefill_arm(1, 1000, 64, 128, 1, 0) == 3  # 16 chunks: too short
    assert kda.prefill_arm(1, 4626, 64, 128, 0, 0) == 2  # fp32 activations: sequential
    assert kda.prefill_arm(1, 300, 2, 128, 1, 3) == 4
    assert kda.prefill_arm(1, 300, 2, 16, 1, 3) == -1
    # zero block (max(D*D, H*D) floats), identity, dummy row (H*D floats), then
    # (n-1) + 2(n-2) state blocks per pair: B*H = 2, T = 300 gives n = 5 segments
    blk = 128 * 128 * 4
    assert kda.workspace_bytes(1, 300, 2, 128, 1, 3) == blk + blk + 1024 + (4 + 6) * 2 * blk
    # the prefill workload: n = 5
    assert kda.workspace_bytes(1, 4626, 64, 128, 1, 0) == blk + blk + 64 * 128 * 4 + (4 + 6) * 64 * blk
    assert kda.workspace_bytes(1, 4626, 64, 128, 1, 0, gdn=True) == kda.workspace_bytes(1, 4626, 64, 128, 1, 0)
    # packed batches have no segmented arm
    assert kda.varlen_workspace_bytes(3, 500, 4, 128, 1, 3) == ctypes.c_size_t(-1).value


def _segments_from_workspace(B, T, H, mode):
    """The segment count n of a segmented call, read back from its workspace size:
    constant blocks, then (n-1) + 2(n-2) state blocks per pair."""
    blk, row = 128 * 128 * 4, H * 128 * 4
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    const = al(max(blk, row)) + al(blk) + al(row)
    ws = kda.workspace_bytes(B, T, H, 128, 1, mode)
    slots, rem = divmod(ws - const, B * H * blk)
    assert rem == 0 and slots >= 0
    return 1 if slots == 0 else (slots + 5) // 3


@pytest.mark.parametrize("B,H", [(1, 1), (1, 8), (1, 64), (2, 64), (4, 32), (1, 100), (3, 85), (2, 128)])
@pytest.mark.parametrize("T", [1, 64, 300, 4626, 70000])
def test_segment_plan_invariants(B, H, T):
    """Every plan fits pass 3 in one wave over 256 compute units, keeps at most 32
    segments of at least one chunk, and AUTO never picks the segmented arm with fewer
    than three segments or at 256 pairs and more."""
    P, nch = B * H, (T + 63) // 64
    n = _segments_from_workspace(B, T, H, 3)
    assert n == 1 or (3 <= n <= 32 and (n - 1) * P <= 256 and n <= nch), (n, P, nch)
    if kda.prefill_arm(B, T, H, 128, 1, 0) == 4:
        na = _segments_from_workspace(B, T, H, 0)
        assert 3 <= na <= 32 and (na - 1) * P <= 256 and P < 256 and nch > 8 * (na - 1)


def call_rollback(a, gdn=False, T_stash=3, keep=2):
    f = kda.lib().gdn_rollback if gdn else kda.lib().kda_rollback
    return f(a["q"], a["k"], a["v"], a["g"], a["beta"], a["conv_w"], a["ring_snap"], a["state_snap"],
             a["ring"], a["state_out"], a["B"], T_stash, keep, a["H"], a["D"], a["K"], a["dtype"],
             a["ws"], a["ws_bytes"], None)


ROLLBACK_CASES = [
    ("keep 0", dict(), dict(keep=0), 40004),
    ("keep past the stash", dict(), dict(keep=4), 40004),
    ("null ring_snap", dict(ring_snap=None), dict(), 40001),
    ("null state_out", dict(state_out=None), dict(), 40001),
    ("misaligned state_snap", dict(state_snap=BASE + 15 * (1 << 32) + 4), dict(), 40007),
    ("ring_snap partially over ring", dict(ring_snap=BASE + 6 * (1 << 32) + 16), dict(), 40009),
    ("state_out over q", dict(state_out=BASE + 256), dict(), 40009),
    ("state_snap over ring", dict(state_snap=BASE + 6 * (1 << 32) + 64), dict(), 40009),
    ("dtype 2", dict(dtype=2), dict(), 40008),
    ("D=64", dict(D=64), dict(), 40002),
    ("K=9", dict(K=9), dict(), 40003),
]


@pytest.mark.skipif(_gpu_visible(), reason="fake pointers only where no GPU is visible")
@pytest.mark.parametrize("gdn", [False, True])
@pytest.mark.parametrize("what,over,kw,rc", ROLLBACK_CASES, ids=[c[0] for c in ROLLBACK_CASES])
def test_rollback_contract(what, over, kw, rc, gdn):
    a = fake_args()
    a.update({k: (0 if v is None else v) for k, v in over.items()})
    assert call_rollback(a, gdn, **kw) == rc


@pytest.mark.skipif(_gpu_visible(), reason="fake pointers only where no GPU is visible")
def test_rollback_workspace_too_small():
    # few (b, h) pairs and keep > 16: the split arm, which needs a workspace
    a = fake_args(B=1, H=2, D=16)
    need = kda.rollback_workspace_bytes(1, 40, 2, 16, 0)
    assert need > 0
    a["ws_bytes"] = need - 1
    assert call_rollback(a, T_stash=50, keep=40) == 40006


def test_rollback_queries():
    assert kda.rollback_workspace_bytes(64, 8, 64, 128, 1) == 0  # short replay: fused arm
    assert kda.rollback_workspace_bytes(1, 40, 2, 16, 0) == kda.workspace_bytes(1, 40, 2, 16, 0, 1)
    assert kda.rollback_workspace_bytes(1, 40, 2, 64, 0) == ctypes.c_size_t(-1).value


def call_gated(a, gdn=False, decode=False, form=1, lb=-5.0):
    L = kda.lib()
    head = (a["q"], a["k"], a["v"], a["g"], a["beta"], a["gate_a"], a["gate_bias"], lb, form, a["conv_w"],
            a["ring"], a["state_in"], a["state_out"], a["z"], a["norm_w"], a["out"], a["o_core"], a["B"],
            a["T"], a["H"], a["D"], a["K"], 0.25, 1e-5, a["dtype"])
    if decode:
        return (L.gdn_decode_gated if gdn else L.kda_decode_gated)(*head, None)
    return (L.gdn_prefill_gated if gdn else L.kda_prefill_gated)(*head, a["mode"], a["ws"], a["ws_bytes"], None)


GATED_CASES = [
    ("form 0 (use the plain entry)", dict(), dict(form=0), 40008),
    ("form 3", dict(), dict(form=3), 40008),
    ("null gate_a", dict(gate_a=None), dict(), 40001),
    ("null gate_bias", dict(gate_bias=None), dict(), 40001),
    ("misaligned gate_bias", dict(gate_bias=BASE + 17 * (1 << 32) + 4), dict(), 40007),
    ("out over gate_bias", dict(out=BASE + 17 * (1 << 32)), dict(), 40009),
    ("state_out over gate_a", dict(state_out=BASE + 16 * (1 << 32)), dict(), 40009),
]


@pytest.mark.skipif(_gpu_visible(), reason="fake pointers only where no GPU is visible")
@pytest.mark.parametrize("decode", [False, True])
@pytest.mark.parametrize("gdn", [False, True])
@pytest.mark.parametrize("what,over,kw,rc", GATED_CASES, ids=[c[0] for c in GATED_CASES])
def test_gated_contract(what, over, kw, rc, gdn, decode):
    a = fake_args(T=1 if decode else 3)
    a.update({k: (0 if v is None else v) for k, v in over.items()})
    assert call_gated(a, gdn, decode, **kw) == rc


# The chunked arm's decay factorisation needs g >= -5; activated gates are bounded
# below by gate_lb, so the explicit chunked / segmented modes refuse a lower bound
# below -5 (AUTO runs such calls on the fused sequential arm instead).
GATED_CHUNK_CASES = [
    ("chunked lb -5.5", dict(mode=2, D=128, dtype=1), dict(lb=-5.5), 40008),
    ("segmented lb -inf", dict(mode=3, D=128, dtype=1), dict(lb=float("-inf")), 40008),
    ("chunked lb nan", dict(mode=2, D=128, dtype=1), dict(lb=float("nan"), form=2), 40008),
    ("chunked fp32 gated", dict(mode=2, D=128, dtype=0), dict(lb=-5.0), 40008),
]


@pytest.mark.skipif(_gpu_visible(), reason="fake pointers only where no GPU is visible")
@pytest.mark.parametrize("gdn", [False, True])
@pytest.mark.parametrize("what,over,kw,rc", GATED_CHUNK_CASES, ids=[c[0] for c in GATED_CHUNK_CASES])
def test_gated_chunk_modes_need_bounded_gates(what, over, kw, rc, gdn):
    a = fake_args(T=100)
    a.update(over)
    assert call_gated(a, gdn, False, **kw) == rc


def call_rollback_gated(a, gdn=False, T_stash=3, keep=2, form=2, lb=-5.0):
    L = kda.lib()
    f = L.gdn_rollback_gated if gdn else L.kda_rollback_gated
    return f(a["q"], a["k"], a["v"], a["g"], a["beta"], a["gate_a"], a["gate_bias"], lb, form, a["conv_w"],
             a["ring_snap"], a["state_snap"], a["ring"], a["state_out"], a["B"], T_stash, keep, a["H"], a["D"],
             a["K"], a["dtype"], a["ws"], a["ws_bytes"], None)


GATED_ROLLBACK_CASES = [
    ("form 0 (use the plain entry)", dict(), dict(form=0), 40008),
    ("form 3", dict(), dict(form=3), 40008),
    ("null gate_a", dict(gate_a=None), dict(), 40001),
    ("null gate_bias", dict(gate_bias=None), dict(), 40001),
    ("misaligned gate_a", dict(gate_a=BASE + 16 * (1 << 32) + 8), dict(), 40007),
    ("state_out over gate_bias", dict(state_out=BASE + 17 * (1 << 32)), dict(), 40009),
    ("ring over gate_a", dict(ring=BASE + 16 * (1 << 32)), dict(), 40009),
    ("keep past the stash", dict(), dict(keep=4), 40004),
]


@pytest.mark.skipif(_gpu_visible(), reason="fake pointers only where no GPU is visible")
@pytest.mark.parametrize("gdn", [False, True])
@pytest.mark.parametrize("what,over,kw,rc", GATED_ROLLBACK_CASES, ids=[c[0] for c in GATED_ROLLBACK_CASES])
def test_gated_rollback_contract(what, over, kw, rc, gdn):
    a = fake_args()
    a.update({k: (0 if v is None else v) for k, v in over.items()})
    assert call_rollback_gated(a, gdn, **kw) == rc


def call_gqa(a, Hk, decode=False, form=0, lb=0.0):
    L = kda.lib()
    head = (a["q"], a["k"], a["v"], a["g"], a["beta"], a["gate_a"], a["gate_bias"], lb, form, a["conv_w"],
            a["ring"], a["state_in"], a["state_out"], a["z"], a["norm_w"], a["out"], a["o_core"], a["B"],
            a["T"], a["H"], Hk, a["D"], a["K"], 0.25, 1e-5, a["dtype"])
    if decode:
        return L.gdn_decode_gqa(*head, None)
    return L.gdn_prefill_gqa(*head, a["mode"], a["ws"], a["ws_bytes"], None)


GQA_CASES = [
    ("Hk does not divide H", dict(H=4), 3, 40004),
    ("Hk above H", dict(H=2), 4, 40004),
    ("Hk 0", dict(H=4), 0, 40004),
    ("Hk negative", dict(H=4), -2, 40004),
    ("null q", dict(H=4, q=None), 2, 40001),
    ("gate form 5", dict(H=4), 2, 40008),
    ("misaligned k", dict(H=4, k=BASE + 1 * (1 << 32) + 2), 2, 40007),
    # q is [B][T][Hk*D] (here 2 x T x 32 floats): out 128 bytes after it overlaps it
    ("out over q", dict(H=4, out=BASE + 128), 2, 40009),
]


@pytest.mark.skipif(_gpu_visible(), reason="fake pointers only where no GPU is visible")
@pytest.mark.parametrize("decode", [False, True])
@pytest.mark.parametrize("what,over,Hk,rc", GQA_CASES, ids=[c[0] for c in GQA_CASES])
def test_gqa_contract(what, over, Hk, rc, decode):
    a = fake_args(T=1 if decode else 3, H=over.get("H", 2))
    a.update({k: (0 if v is None else v) for k, v in over.items() if k != "H"})
    form = 5 if what == "gate form 5" else 0
    assert call_gqa(a, Hk, decode, form=form) == rc


def test_gqa_queries():
    # grouped heads need less split-arm workspace (q / k staged once per key head)
    full = kda.workspace_bytes(1, 100, 4, 16, 0, 1, gdn=True)
    assert kda.gqa_workspace_bytes(1, 100, 4, 4, 16, 0, 1) == full
    assert 0 < kda.gqa_workspace_bytes(1, 100, 4, 2, 16, 0, 1) < full
    assert kda.gqa_workspace_bytes(1, 100, 4, 3, 16, 0, 1) == ctypes.c_size_t(-1).value
    assert kda.gqa_workspace_bytes(1, 100, 4, 0, 16, 0, 1) == ctypes.c_size_t(-1).value


def call_varlen(a, gdn=False, N=2, T_total=5, cu=None, mode=1, Hk=None):
    L = kda.lib()
    head = (a["q"], a["k"], a["v"], a["g"], a["beta"], a["gate_a"], a["gate_bias"], 0.0, 0, a["conv_w"],
            a["ring"], a["state_in"], a["state_out"], a["z"], a["norm_w"], a["out"], a["o_core"],
            BASE + 18 * (1 << 32) if cu is None else cu, N, T_total, a["H"])
    tail = (a["D"], a["K"], 0.25, 1e-5, a["dtype"], mode, a["ws"], a["ws_bytes"], None)
    if gdn:
        return L.gdn_prefill_varlen(*head, a["H"] if Hk is None else Hk, *tail)
    return L.kda_prefill_varlen(*head, *tail)


# the offsets table sits in a slot of its own (18) unless a case places it (cu=...)
VARLEN_CASES = [
    ("null cu_seqlens", dict(), dict(cu=0), 40001),
    ("misaligned cu_seqlens", dict(), dict(cu=BASE + 13 * (1 << 32) + 2), 40007),
    ("out over cu_seqlens", dict(out=BASE + 18 * (1 << 32)), dict(), 40009),
    ("workspace too small", dict(ws_bytes=255), dict(), 40006),
    ("T_total 0", dict(), dict(T_total=0), 40004),
    ("N 0", dict(), dict(N=0), 40004),
    ("chunked at D=16", dict(), dict(mode=2), 40008),
    ("mode 7", dict(), dict(mode=7), 40008),
]


@pytest.mark.skipif(_gpu_visible(), reason="fake pointers only where no GPU is visible")
@pytest.mark.parametrize("gdn", [False, True])
@pytest.mark.parametrize("what,over,kw,rc", VARLEN_CASES, ids=[c[0] for c in VARLEN_CASES])
def test_varlen_contract(what, over, kw, rc, gdn):
    a = fake_args()
    a.update(over)
    assert call_varlen(a, gdn, **kw) == rc


@pytest.mark.skipif(_gpu_visible(), reason="fake pointers only where no GPU is visible")
def test_varlen_gqa_heads_checked():
    a = fake_args(H=4)
    assert call_varlen(a, True, Hk=3) == 40004
    assert call_varlen(a, True, Hk=0) == 40004


def test_varlen_queries():
    # the longest-first order of the N sequences (256-byte aligned) heads the workspace;
    # the fused arm needs nothing more, the chunked arm with N*H < 256 the fp32 pre-norm
    # rows of all tokens
    assert kda.varlen_workspace_bytes(3, 500, 4, 16, 0, 1) == 256
    assert kda.varlen_workspace_bytes(3, 500, 4, 128, 1, 2) == 256 + 500 * 4 * 128 * 4
    assert kda.varlen_workspace_bytes(64, 500, 4, 128, 1, 2) == 256  # N*H = 256: one split
    assert kda.varlen_workspace_bytes(65, 500, 4, 128, 1, 2) == 512
    assert kda.varlen_workspace_bytes(3, 500, 4, 16, 0, 2) == ctypes.c_size_t(-1).value
    assert kda.varlen_workspace_bytes(3, 500, 4, 128, 1, 2, gdn=True, Hk=3) == ctypes.c_size_t(-1).value
