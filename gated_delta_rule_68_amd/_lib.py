"""ctypes binding of ``libkda.so`` (the C ABI in include/kda.h).

Argument marshalling only: shapes are read off the tensors, pointers and sizes are
passed through, and every step of the mixer runs in the HIP library. There is no
fallback: if the library is not built, loading it raises.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libkda.so")

KDA_DTYPE_F32, KDA_DTYPE_BF16 = 0, 1
KDA_MODE_AUTO, KDA_MODE_SEQUENTIAL, KDA_MODE_CHUNKED, KDA_MODE_SEGMENTED = 0, 1, 2, 3
ARM_NAMES = {1: "seq_fused", 2: "seq_split", 3: "chunked", 4: "segmented"}

_lib = None

_vp, _fp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_PREFILL_ARGS = [_vp] * 5 + [_fp, _fp, _fp, _fp, _vp, _fp, _vp, _fp] + [_i] * 5 + [_f, _f, _i, _i, _vp, _sz, _vp]
_DECODE_ARGS = [_vp] * 5 + [_fp, _fp, _fp, _fp, _vp, _fp, _vp, _fp] + [_i] * 5 + [_f, _f, _i, _vp]
_ROLLBACK_ARGS = [_vp] * 5 + [_fp] * 5 + [_i] * 7 + [_vp, _sz, _vp]
_GATE_ARGS = [_fp, _fp, _f, _i]
_GATED_PREFILL_ARGS = _PREFILL_ARGS[:5] + _GATE_ARGS + _PREFILL_ARGS[5:]
_GATED_DECODE_ARGS = _DECODE_ARGS[:5] + _GATE_ARGS + _DECODE_ARGS[5:]
_GATED_ROLLBACK_ARGS = _ROLLBACK_ARGS[:5] + _GATE_ARGS + _ROLLBACK_ARGS[5:]
# grouped heads: Hk follows H
_GQA_PREFILL_ARGS = _GATED_PREFILL_ARGS[:20] + [_i] + _GATED_PREFILL_ARGS[20:]
_GQA_DECODE_ARGS = _GATED_DECODE_ARGS[:20] + [_i] + _GATED_DECODE_ARGS[20:]
_GQA_ROLLBACK_ARGS = _GATED_ROLLBACK_ARGS[:18] + [_i] + _GATED_ROLLBACK_ARGS[18:]
KDA_GATE_GIVEN = 0
# packed batches: cu_seqlens, N, T_total in place of B, T
_VARLEN_KDA_ARGS = _GATED_PREFILL_ARGS[:17] + [_vp, _i, _i] + _GATED_PREFILL_ARGS[19:]
_VARLEN_GDN_ARGS = _GQA_PREFILL_ARGS[:17] + [_vp, _i, _i] + _GQA_PREFILL_ARGS[19:]
KDA_GATE_SIGMOID, KDA_GATE_SOFTPLUS = 1, 2
EXPORTS = ("kda_prefill", "kda_decode", "gdn_prefill", "gdn_decode",
           "kda_prefill_workspace_bytes", "gdn_prefill_workspace_bytes",
           "kda_prefill_arm", "gdn_prefill_arm", "kda_rollback", "gdn_rollback",
           "kda_rollback_workspace_bytes", "gdn_rollback_workspace_bytes", "kda_prefill_gated",
           "gdn_prefill_gated", "kda_decode_gated", "gdn_decode_gated", "kda_rollback_gated",
           "gdn_rollback_gated", "gdn_prefill_gqa", "gdn_decode_gqa", "gdn_rollback_gqa",
           "gdn_gqa_workspace_bytes", "kda_prefill_varlen", "gdn_prefill_varlen",
           "kda_prefill_varlen_workspace_bytes", "gdn_prefill_varlen_workspace_bytes", "kda_status_string",
           "kda_prefill_noalloc")
KDA_NOALLOC_SCRATCH_BYTES = 64 << 20


class KdaError(RuntimeError):
    def __init__(self, rc: int, what: str):
        self.rc = rc
        super().__init__(f"{what} failed: rc {rc} ({status_string(rc)})")


def lib() -> ctypes.CDLL:
    """The loaded library. Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(the mixer has no non-HIP fallback)")
        _lib = bind(LIB_PATH)
    return _lib


def bind(path: str) -> ctypes.CDLL:
    """Load the build of the library at `path` and declare every export's argument and
    result types."""
    # torch brings its own copy of the HIP runtime under another file name. Loaded
    # first, it is the one the library binds to; loaded after the library, it would be a
    # second runtime in the process, and calls through the library then fail (no device).
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    l = ctypes.CDLL(path)
    for n in ("kda_prefill", "gdn_prefill"):
        getattr(l, n).argtypes = _PREFILL_ARGS
        getattr(l, n).restype = _i
    for n in ("kda_decode", "gdn_decode"):
        getattr(l, n).argtypes = _DECODE_ARGS
        getattr(l, n).restype = _i
    l.kda_prefill_noalloc.argtypes = _PREFILL_ARGS[:-3] + [_vp]  # no workspace, its size
    l.kda_prefill_noalloc.restype = _i
    for n in ("kda_prefill_workspace_bytes", "gdn_prefill_workspace_bytes"):
        getattr(l, n).argtypes = [_i] * 6
        getattr(l, n).restype = _sz
    for n in ("kda_prefill_arm", "gdn_prefill_arm"):
        getattr(l, n).argtypes = [_i] * 6
        getattr(l, n).restype = _i
    for n in ("kda_prefill_gated", "gdn_prefill_gated"):
        getattr(l, n).argtypes = _GATED_PREFILL_ARGS
        getattr(l, n).restype = _i
    for n in ("kda_decode_gated", "gdn_decode_gated"):
        getattr(l, n).argtypes = _GATED_DECODE_ARGS
        getattr(l, n).restype = _i
    for n in ("kda_rollback", "gdn_rollback"):
        getattr(l, n).argtypes = _ROLLBACK_ARGS
        getattr(l, n).restype = _i
    for n in ("kda_rollback_gated", "gdn_rollback_gated"):
        getattr(l, n).argtypes = _GATED_ROLLBACK_ARGS
        getattr(l, n).restype = _i
    l.gdn_prefill_gqa.argtypes, l.gdn_prefill_gqa.restype = _GQA_PREFILL_ARGS, _i
    l.gdn_decode_gqa.argtypes, l.gdn_decode_gqa.restype = _GQA_DECODE_ARGS, _i
    l.gdn_rollback_gqa.argtypes, l.gdn_rollback_gqa.restype = _GQA_ROLLBACK_ARGS, _i
    l.gdn_gqa_workspace_bytes.argtypes, l.gdn_gqa_workspace_bytes.restype = [_i] * 7, _sz
    l.kda_prefill_varlen.argtypes, l.kda_prefill_varlen.restype = _VARLEN_KDA_ARGS, _i
    l.gdn_prefill_varlen.argtypes, l.gdn_prefill_varlen.restype = _VARLEN_GDN_ARGS, _i
    l.kda_prefill_varlen_workspace_bytes.argtypes = [_i] * 6
    l.kda_prefill_varlen_workspace_bytes.restype = _sz
    l.gdn_prefill_varlen_workspace_bytes.argtypes = [_i] * 7
    l.gdn_prefill_varlen_workspace_bytes.restype = _sz
    for n in ("kda_rollback_workspace_bytes", "gdn_rollback_workspace_bytes"):
        getattr(l, n).argtypes = [_i] * 5
        getattr(l, n).restype = _sz
    l.kda_status_string.argtypes = [_i]
    l.kda_status_string.restype = ctypes.c_char_p
    return l


def status_string(rc: int) -> str:
    return lib().kda_status_string(rc).decode()


def _ptr(t):
    return None if t is None else t.data_ptr()


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return KDA_DTYPE_BF16
    if t.dtype == torch.float32:
        return KDA_DTYPE_F32
    raise TypeError(f"activations must be float32 or bfloat16, got {t.dtype}")


def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _geometry(q, state, conv_w):
    B, T = q.shape[0], q.shape[1]
    H, D = state.shape[1], state.shape[2]
    return B, T, H, D, conv_w.shape[1]


def workspace_bytes(B, T, H, D, dtype_code, mode=KDA_MODE_AUTO, gdn=False) -> int:
    fn = lib().gdn_prefill_workspace_bytes if gdn else lib().kda_prefill_workspace_bytes
    return int(fn(B, T, H, D, dtype_code, mode))


def prefill_arm(B, T, H, D, dtype_code, mode=KDA_MODE_AUTO, gdn=False) -> int:
    fn = lib().gdn_prefill_arm if gdn else lib().kda_prefill_arm
    return int(fn(B, T, H, D, dtype_code, mode))


def _prefill(name, q, k, v, g, beta, conv_w, conv_ring, state_in, state_out, z, norm_w, out,
             o_core, scale, rms_eps, mode, workspace, stream, check):
    B, T, H, D, K = _geometry(q, state_in, conv_w)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = getattr(lib(), name)(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(conv_w), _ptr(conv_ring),
        _ptr(state_in), _ptr(state_out), _ptr(z), _ptr(norm_w), _ptr(out), _ptr(o_core),
        B, T, H, D, K, float(scale), float(rms_eps), _dtype_code(q), int(mode),
        _ptr(workspace), ws_bytes, _stream_handle(stream))
    if check and rc != 0:
        raise KdaError(rc, name)
    return rc


def kda_prefill_noalloc(q, k, v, g, beta, conv_w, conv_ring, state_in, state_out, z, norm_w, out,
                        o_core=None, *, scale, rms_eps, mode=KDA_MODE_AUTO, stream=None, check=True):
    """kda_prefill with its workspace taken from the library's static scratch buffer."""
    B, T, H, D, K = _geometry(q, state_in, conv_w)
    rc = lib().kda_prefill_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(conv_w), _ptr(conv_ring),
        _ptr(state_in), _ptr(state_out), _ptr(z), _ptr(norm_w), _ptr(out), _ptr(o_core),
        B, T, H, D, K, float(scale), float(rms_eps), _dtype_code(q), int(mode), _stream_handle(stream))
    if check and rc != 0:
        raise KdaError(rc, "kda_prefill_noalloc")
    return rc


def _decode(name, q, k, v, g, beta, conv_w, conv_ring, state_in, state_out, z, norm_w, out,
            o_core, scale, rms_eps, stream, check):
    B, T, H, D, K = _geometry(q, state_in, conv_w)
    rc = getattr(lib(), name)(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(conv_w), _ptr(conv_ring),
        _ptr(state_in), _ptr(state_out), _ptr(z), _ptr(norm_w), _ptr(out), _ptr(o_core),
        B, T, H, D, K, float(scale), float(rms_eps), _dtype_code(q), _stream_handle(stream))
    if check and rc != 0:
        raise KdaError(rc, name)
    return rc


def kda_prefill(q, k, v, g, beta, conv_w, conv_ring, state_in, state_out, z, norm_w, out,
                o_core=None, *, scale, rms_eps, mode=KDA_MODE_AUTO, workspace=None,
                stream=None, check=True):
    """Tensors in the layouts of include/kda.h (all on the GPU). Returns the status."""
    return _prefill("kda_prefill", q, k, v, g, beta, conv_w, conv_ring, state_in, state_out,
                    z, norm_w, out, o_core, scale, rms_eps, mode, workspace, stream, check)


def gdn_prefill(q, k, v, g, beta, conv_w, conv_ring, state_in, state_out, z, norm_w, out,
                o_core=None, *, scale, rms_eps, mode=KDA_MODE_AUTO, workspace=None,
                stream=None, check=True):
    return _prefill("gdn_prefill", q, k, v, g, beta, conv_w, conv_ring, state_in, state_out,
                    z, norm_w, out, o_core, scale, rms_eps, mode, workspace, stream, check)


def kda_decode(q, k, v, g, beta, conv_w, conv_ring, state_in, state_out, z, norm_w, out,
               o_core=None, *, scale, rms_eps, stream=None, check=True):
    return _decode("kda_decode", q, k, v, g, beta, conv_w, conv_ring, state_in, state_out, z,
                   norm_w, out, o_core, scale, rms_eps, stream, check)


def gdn_decode(q, k, v, g, beta, conv_w, conv_ring, state_in, state_out, z, norm_w, out,
               o_core=None, *, scale, rms_eps, stream=None, check=True):
    return _decode("gdn_decode", q, k, v, g, beta, conv_w, conv_ring, state_in, state_out, z,
                   norm_w, out, o_core, scale, rms_eps, stream, check)


def rollback_workspace_bytes(B, keep, H, D, dtype_code, gdn=False) -> int:
    fn = lib().gdn_rollback_workspace_bytes if gdn else lib().kda_rollback_workspace_bytes
    return int(fn(B, keep, H, D, dtype_code))


def _rollback(name, q, k, v, g, beta, conv_w, ring_snap, state_snap, conv_ring, state_out, keep,
              workspace, stream, check, gate=()):
    B, T, H, D, K = _geometry(q, state_snap, conv_w)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = getattr(lib(), name)(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), *gate, _ptr(conv_w), _ptr(ring_snap),
        _ptr(state_snap), _ptr(conv_ring), _ptr(state_out), B, T, int(keep), H, D, K,
        _dtype_code(q), _ptr(workspace), ws_bytes, _stream_handle(stream))
    if check and rc != 0:
        raise KdaError(rc, name)
    return rc


def kda_rollback(q, k, v, g, beta, conv_w, ring_snap, state_snap, conv_ring, state_out, keep, *,
                 workspace=None, stream=None, check=True):
    """Rebuild conv_ring / state_out as after the first `keep` rows of a verify round whose
    raw inputs are q, k, v, g, beta ([B][T_stash][...]) and whose pre-round ring and state
    were ring_snap and state_snap. Returns the status."""
    return _rollback("kda_rollback", q, k, v, g, beta, conv_w, ring_snap, state_snap, conv_ring,
                     state_out, keep, workspace, stream, check)


def gdn_rollback(q, k, v, g, beta, conv_w, ring_snap, state_snap, conv_ring, state_out, keep, *,
                 workspace=None, stream=None, check=True):
    return _rollback("gdn_rollback", q, k, v, g, beta, conv_w, ring_snap, state_snap, conv_ring,
                     state_out, keep, workspace, stream, check)


def kda_rollback_gated(q, k, v, gate_x, beta_x, gate_a, gate_bias, conv_w, ring_snap, state_snap,
                       conv_ring, state_out, keep, *, gate_form, gate_lb, workspace=None, stream=None,
                       check=True):
    """kda_rollback of a round verified with kda_prefill_gated (include/kda.h)."""
    return _rollback("kda_rollback_gated", q, k, v, gate_x, beta_x, conv_w, ring_snap, state_snap,
                     conv_ring, state_out, keep, workspace, stream, check,
                     (_ptr(gate_a), _ptr(gate_bias), float(gate_lb), int(gate_form)))


def gdn_rollback_gated(q, k, v, gate_x, beta_x, gate_a, gate_bias, conv_w, ring_snap, state_snap,
                       conv_ring, state_out, keep, *, gate_form, gate_lb, workspace=None, stream=None,
                       check=True):
    return _rollback("gdn_rollback_gated", q, k, v, gate_x, beta_x, conv_w, ring_snap, state_snap,
                     conv_ring, state_out, keep, workspace, stream, check,
                     (_ptr(gate_a), _ptr(gate_bias), float(gate_lb), int(gate_form)))


def _gated(name, decode, q, k, v, gate_x, beta_x, gate_a, gate_bias, conv_w, conv_ring, state_in,
           state_out, z, norm_w, out, o_core, gate_form, gate_lb, scale, rms_eps, mode, workspace,
           stream, check):
    B, T, H, D, K = _geometry(q, state_in, conv_w)
    head = (_ptr(q), _ptr(k), _ptr(v), _ptr(gate_x), _ptr(beta_x), _ptr(gate_a), _ptr(gate_bias),
            float(gate_lb), int(gate_form), _ptr(conv_w), _ptr(conv_ring), _ptr(state_in),
            _ptr(state_out), _ptr(z), _ptr(norm_w), _ptr(out), _ptr(o_core), B, T, H, D, K,
            float(scale), float(rms_eps), _dtype_code(q))
    if decode:
        rc = getattr(lib(), name)(*head, _stream_handle(stream))
    else:
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        rc = getattr(lib(), name)(*head, int(mode), _ptr(workspace), ws_bytes, _stream_handle(stream))
    if check and rc != 0:
        raise KdaError(rc, name)
    return rc


def kda_prefill_gated(q, k, v, gate_x, beta_x, gate_a, gate_bias, conv_w, conv_ring, state_in,
                      state_out, z, norm_w, out, o_core=None, *, gate_form, gate_lb, scale, rms_eps,
                      mode=KDA_MODE_AUTO, workspace=None, stream=None, check=True):
    """kda_prefill with the gate and beta pre-activations (include/kda.h, KDA_GATE_*)."""
    return _gated("kda_prefill_gated", False, q, k, v, gate_x, beta_x, gate_a, gate_bias, conv_w,
                  conv_ring, state_in, state_out, z, norm_w, out, o_core, gate_form, gate_lb, scale,
                  rms_eps, mode, workspace, stream, check)


def gdn_prefill_gated(q, k, v, gate_x, beta_x, gate_a, gate_bias, conv_w, conv_ring, state_in,
                      state_out, z, norm_w, out, o_core=None, *, gate_form, gate_lb, scale, rms_eps,
                      mode=KDA_MODE_AUTO, workspace=None, stream=None, check=True):
    return _gated("gdn_prefill_gated", False, q, k, v, gate_x, beta_x, gate_a, gate_bias, conv_w,
                  conv_ring, state_in, state_out, z, norm_w, out, o_core, gate_form, gate_lb, scale,
                  rms_eps, mode, workspace, stream, check)


def kda_decode_gated(q, k, v, gate_x, beta_x, gate_a, gate_bias, conv_w, conv_ring, state_in,
                     state_out, z, norm_w, out, o_core=None, *, gate_form, gate_lb, scale, rms_eps,
                     stream=None, check=True):
    return _gated("kda_decode_gated", True, q, k, v, gate_x, beta_x, gate_a, gate_bias, conv_w,
                  conv_ring, state_in, state_out, z, norm_w, out, o_core, gate_form, gate_lb, scale,
                  rms_eps, None, None, stream, check)


def gdn_decode_gated(q, k, v, gate_x, beta_x, gate_a, gate_bias, conv_w, conv_ring, state_in,
                     state_out, z, norm_w, out, o_core=None, *, gate_form, gate_lb, scale, rms_eps,
                     stream=None, check=True):
    return _gated("gdn_decode_gated", True, q, k, v, gate_x, beta_x, gate_a, gate_bias, conv_w,
                  conv_ring, state_in, state_out, z, norm_w, out, o_core, gate_form, gate_lb, scale,
                  rms_eps, None, None, stream, check)


# ---------------------------------------------------------------- grouped heads (GDN)
def gqa_workspace_bytes(B, T, H, Hk, D, dtype_code, mode=KDA_MODE_AUTO) -> int:
    return int(lib().gdn_gqa_workspace_bytes(B, T, H, Hk, D, dtype_code, mode))


def _gqa_head(q, k, v, g, beta, gate_a, gate_bias, gate_lb, gate_form, conv_w):
    return (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(gate_a), _ptr(gate_bias), float(gate_lb),
            int(gate_form), _ptr(conv_w))


def _gqa_dims(q, v, state, conv_w):
    """(B, T, H, Hk, D, K): H value heads from the state, Hk key heads from q's width."""
    B, T, H, D, K = _geometry(v, state, conv_w)
    return B, T, H, q.shape[2] // D, D, K


def gdn_prefill_gqa(q, k, v, g, beta, conv_w, conv_ring, state_in, state_out, z, norm_w, out, o_core=None,
                    *, scale, rms_eps, mode=KDA_MODE_AUTO, workspace=None, gate_a=None, gate_bias=None,
                    gate_form=KDA_GATE_GIVEN, gate_lb=0.0, stream=None, check=True):
    """gdn_prefill with Hk = q.shape[2] // D query / key heads (include/kda.h)."""
    B, T, H, Hk, D, K = _gqa_dims(q, v, state_in, conv_w)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib().gdn_prefill_gqa(
        *_gqa_head(q, k, v, g, beta, gate_a, gate_bias, gate_lb, gate_form, conv_w), _ptr(conv_ring),
        _ptr(state_in), _ptr(state_out), _ptr(z), _ptr(norm_w), _ptr(out), _ptr(o_core), B, T, H, Hk, D, K,
        float(scale), float(rms_eps), _dtype_code(v), int(mode), _ptr(workspace), ws_bytes,
        _stream_handle(stream))
    if check and rc != 0:
        raise KdaError(rc, "gdn_prefill_gqa")
    return rc


def gdn_decode_gqa(q, k, v, g, beta, conv_w, conv_ring, state_in, state_out, z, norm_w, out, o_core=None,
                   *, scale, rms_eps, gate_a=None, gate_bias=None, gate_form=KDA_GATE_GIVEN, gate_lb=0.0,
                   stream=None, check=True):
    B, T, H, Hk, D, K = _gqa_dims(q, v, state_in, conv_w)
    rc = lib().gdn_decode_gqa(
        *_gqa_head(q, k, v, g, beta, gate_a, gate_bias, gate_lb, gate_form, conv_w), _ptr(conv_ring),
        _ptr(state_in), _ptr(state_out), _ptr(z), _ptr(norm_w), _ptr(out), _ptr(o_core), B, T, H, Hk, D, K,
        float(scale), float(rms_eps), _dtype_code(v), _stream_handle(stream))
    if check and rc != 0:
        raise KdaError(rc, "gdn_decode_gqa")
    return rc


def gdn_rollback_gqa(q, k, v, g, beta, conv_w, ring_snap, state_snap, conv_ring, state_out, keep, *,
                     workspace=None, gate_a=None, gate_bias=None, gate_form=KDA_GATE_GIVEN, gate_lb=0.0,
                     stream=None, check=True):
    B, T, H, Hk, D, K = _gqa_dims(q, v, state_snap, conv_w)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib().gdn_rollback_gqa(
        *_gqa_head(q, k, v, g, beta, gate_a, gate_bias, gate_lb, gate_form, conv_w), _ptr(ring_snap),
        _ptr(state_snap), _ptr(conv_ring), _ptr(state_out), B, T, int(keep), H, Hk, D, K, _dtype_code(v),
        _ptr(workspace), ws_bytes, _stream_handle(stream))
    if check and rc != 0:
        raise KdaError(rc, "gdn_rollback_gqa")
    return rc


# ---------------------------------------------------------------- packed batches
def varlen_workspace_bytes(N, T_total, H, D, dtype_code, mode=KDA_MODE_AUTO, gdn=False, Hk=None) -> int:
    if gdn:
        return int(lib().gdn_prefill_varlen_workspace_bytes(N, T_total, H, Hk or H, D, dtype_code, mode))
    return int(lib().kda_prefill_varlen_workspace_bytes(N, T_total, H, D, dtype_code, mode))


def prefill_varlen(q, k, v, g, beta, conv_w, conv_ring, state_in, state_out, z, norm_w, out, cu_seqlens,
                   o_core=None, *, gdn=False, scale, rms_eps, mode=KDA_MODE_AUTO, workspace=None, gate_a=None,
                   gate_bias=None, gate_form=KDA_GATE_GIVEN, gate_lb=0.0, stream=None, check=True):
    """Packed variable-length prefill (include/kda.h): activations [T_total][...], the
    int32 device tensor cu_seqlens [N+1], ring / state [N][...]. Hk (GDN) is read off
    q's width."""
    import torch

    N, H, D = state_in.shape[0], state_in.shape[1], state_in.shape[2]
    T_total, K = v.shape[-2], conv_w.shape[1]
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.numel() != N + 1 or not cu_seqlens.is_contiguous():
        raise ValueError(f"cu_seqlens must be a contiguous int32 tensor of N + 1 = {N + 1} offsets")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    head = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(gate_a), _ptr(gate_bias), float(gate_lb),
            int(gate_form), _ptr(conv_w), _ptr(conv_ring), _ptr(state_in), _ptr(state_out), _ptr(z),
            _ptr(norm_w), _ptr(out), _ptr(o_core), _ptr(cu_seqlens), N, T_total, H)
    tail = (D, K, float(scale), float(rms_eps), _dtype_code(v), int(mode), _ptr(workspace), ws_bytes,
            _stream_handle(stream))
    if gdn:
        rc = lib().gdn_prefill_varlen(*head, q.shape[-1] // D, *tail)
    else:
        rc = lib().kda_prefill_varlen(*head, *tail)
    if check and rc != 0:
        raise KdaError(rc, "gdn_prefill_varlen" if gdn else "kda_prefill_varlen")
    return rc

