"""ctypes wrapper around the fp64 C oracle (``kda_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library. Every array argument is a
C-contiguous float64 numpy array in the layouts documented in ``kda_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_D = ctypes.POINTER(ctypes.c_double)


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc, -O2, no fast-math."""
    subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", out, src, "-lm"],
                   check=True)
    return out


def _bind(lib):
    i, l, d = ctypes.c_int, ctypes.c_long, ctypes.c_double
    lib.orc_conv_silu_plane.argtypes = [i, i, i, i, i, _D, _D, _D, _D, _D]
    lib.orc_l2norm_rows.argtypes = [l, i, _D, _D]
    lib.orc_scan.argtypes = [i, i, i, i, i, _D, _D, _D, _D, _D, d, _D, _D, _D]
    lib.orc_chunked_scan.argtypes = [i, i, i, i, i, i, _D, _D, _D, _D, _D, d, _D, _D, _D]
    lib.orc_gated_rmsnorm.argtypes = [l, i, _D, _D, _D, d, i, _D]
    lib.orc_mixer.argtypes = [i, i, i, i, i, i] + [_D] * 14 + [d, d]
    for f in ("orc_conv_silu_plane", "orc_l2norm_rows", "orc_scan", "orc_chunked_scan",
              "orc_gated_rmsnorm", "orc_mixer"):
        getattr(lib, f).restype = None
    return lib


def load(path: str | None = None):
    """Load (building first if needed) the oracle library. ``path`` loads another
    build of it, e.g. a deliberately mutated copy in a test."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _p(a: np.ndarray):
    assert a.dtype == np.float64 and a.flags.c_contiguous
    return a.ctypes.data_as(_D)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def conv_silu_plane(x, conv_w, ring_in, plane, ring_out=None, lib=None):
    """x [B,T,qkv] -> (y [B,T,qkv], ring_out [B,3qkv,K-1] with this plane's rows rolled)."""
    lib = lib or load()
    x, conv_w, ring_in = _f64(x), _f64(conv_w), _f64(ring_in)
    B, T, qkv = x.shape
    K = conv_w.shape[1]
    y = np.empty_like(x)
    ring_out = ring_in.copy() if ring_out is None else ring_out
    lib.orc_conv_silu_plane(B, T, qkv, K, plane, _p(x), _p(conv_w), _p(ring_in), _p(y),
                            _p(ring_out))
    return y, ring_out


def l2norm_rows(x, D, lib=None):
    lib = lib or load()
    x = _f64(x)
    y = np.empty_like(x)
    lib.orc_l2norm_rows(x.size // D, D, _p(x), _p(y))
    return y


def scan(q, k, v, g, beta, state, scale, gdn=False, lib=None):
    """Sequential definition. Returns (o [B,T,H*D], state_out [B,H,D,D])."""
    lib = lib or load()
    q, k, v, g, beta, state = map(_f64, (q, k, v, g, beta, state))
    B, H, D, _ = state.shape
    T = q.shape[1]
    o = np.empty_like(q)
    s_out = np.empty_like(state)
    lib.orc_scan(B, T, H, D, int(gdn), _p(q), _p(k), _p(v), _p(g), _p(beta), scale,
                 _p(state), _p(s_out), _p(o))
    return o, s_out


def chunked_scan(q, k, v, g, beta, state, scale, C, gdn=False, lib=None):
    """Chunked form (chunk C). Returns (o, state_out)."""
    lib = lib or load()
    q, k, v, g, beta, state = map(_f64, (q, k, v, g, beta, state))
    B, H, D, _ = state.shape
    T = q.shape[1]
    o = np.empty_like(q)
    s_out = np.empty_like(state)
    lib.orc_chunked_scan(B, T, H, D, int(gdn), C, _p(q), _p(k), _p(v), _p(g), _p(beta),
                         scale, _p(state), _p(s_out), _p(o))
    return o, s_out


def gated_rmsnorm(o, z, w, eps, gdn=False, lib=None):
    lib = lib or load()
    o, z, w = _f64(o), _f64(z), _f64(w)
    D = w.shape[0]
    out = np.empty_like(o)
    lib.orc_gated_rmsnorm(o.size // D, D, _p(o), _p(z), _p(w), eps, int(gdn), _p(out))
    return out


def mixer(q, k, v, g, beta, conv_w, ring, state, z, norm_w, scale, rms_eps, gdn=False,
          threads: int = 1, lib=None):
    """The whole path. Returns dict(out, o_core, ring, state). ``threads`` > 1 splits the
    batch across threads (each sequence is independent)."""
    lib = lib or load()
    q, k, v, g, beta, conv_w, ring, state, z, norm_w = map(
        _f64, (q, k, v, g, beta, conv_w, ring, state, z, norm_w))
    B, H, D, _ = state.shape
    T = q.shape[1]
    K = conv_w.shape[1]
    out = np.empty_like(q)
    o_core = np.empty_like(q)
    ring_out = np.empty_like(ring)
    state_out = np.empty_like(state)

    def run(b0, b1):
        sl = slice(b0, b1)
        lib.orc_mixer(int(gdn), b1 - b0, T, H, D, K,
                      _p(q[sl]), _p(k[sl]), _p(v[sl]), _p(g[sl]), _p(beta[sl]), _p(conv_w),
                      _p(ring[sl]), _p(ring_out[sl]), _p(state[sl]), _p(state_out[sl]),
                      _p(z[sl]), _p(norm_w), _p(out[sl]), _p(o_core[sl]), scale, rms_eps)

    threads = max(1, min(threads, B))
    if threads == 1:
        run(0, B)
    else:
        bounds = np.linspace(0, B, threads + 1).astype(int)
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(lambda ab: run(*ab), zip(bounds[:-1], bounds[1:])))
    return {"out": out, "o_core": o_core, "ring": ring_out, "state": state_out}


def rel_linf(x, y) -> float:
    """max|x - y| / max|y| — the comparison metric (y is the oracle)."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    den = float(np.max(np.abs(y))) if y.size else 0.0
    num = float(np.max(np.abs(x - y))) if y.size else 0.0
    return num / den if den > 0 else num
