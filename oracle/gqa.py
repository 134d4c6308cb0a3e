"""Grouped query / key heads for GDN in fp64, written as their definition.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle``): the grouped-head entry points
of the library are checked against this.

aprender-serve gdn_ops.rs, the gated delta-rule recurrence wrapper: q and k carry
num_k_heads heads, v, beta and the gate num_v_heads heads, and value head h reads
query / key head h % num_k_heads (the tiled order). The conv, its ring and the l2
norm act per channel, so each value head is handed the query / key channels of its key
head together with their conv taps and ring rows, and the plain GDN mixer runs on that
problem. The rolled q / k ring rows of key head j are read back from value head j
(j < Hk reads key head j itself); they depend only on the raw q / k rows, which every
value head of key head j shares.

Layouts: q, k [B][T][Hk*D]; v, z [B][T][H*D]; g, beta [B][T][H]; conv_w
[(2*Hk + H)*D][K] and ring [B][(2*Hk + H)*D][K-1] with planes q, k, v; state
[B][H][D][D].
"""
from __future__ import annotations

import numpy as np

from . import mixer


def key_channels(heads, H: int, Hk: int, D: int) -> np.ndarray:
    """The query / key channels the value heads `heads` read: (h % Hk) * D + i."""
    heads = np.asarray(heads)
    return ((heads % Hk)[:, None] * D + np.arange(D)).ravel()


def value_head_problem(q, k, v, g, beta, conv_w, ring, state, z, heads):
    """The plain GDN problem of the value heads `heads`: each handed its key head's
    query / key channels with their conv taps and ring rows. Returns (the keyword
    arrays of oracle.mixer but norm_w, and the row of the grouped conv weight / ring
    that each row of the problem's conv weight / ring is)."""
    H, D = state.shape[1], state.shape[2]
    kw = q.shape[2]
    assert kw % D == 0 and H % (kw // D) == 0, "Hk must divide H"
    heads = np.asarray(heads)
    kc = key_channels(heads, H, kw // D, D)
    vc = (heads[:, None] * D + np.arange(D)).ravel()
    rows = np.concatenate([kc, kw + kc, 2 * kw + vc])
    d = dict(q=q[:, :, kc], k=k[:, :, kc], v=v[:, :, vc], g=g[:, :, heads], beta=beta[:, :, heads],
             conv_w=conv_w[rows], ring=ring[:, rows], state=state[:, heads], z=z[:, :, vc])
    return d, rows


def mixer_gqa(q, k, v, g, beta, conv_w, ring, state, z, norm_w, scale, rms_eps, threads=1,
              lib=None):
    """The GDN mixer with Hk = q.shape[2] // D query / key heads. Returns dict(out,
    o_core, ring, state) in the grouped layouts above."""
    H = state.shape[1]
    d, rows = value_head_problem(q, k, v, g, beta, conv_w, ring, state, z, np.arange(H))
    r = mixer(**d, norm_w=norm_w, scale=scale, rms_eps=rms_eps, gdn=True, threads=threads, lib=lib)
    ring_out = np.array(ring, dtype=np.float64)
    ring_out[:, rows] = r["ring"]  # the copies of a q / k row all hold the same values
    return {**r, "ring": ring_out}
