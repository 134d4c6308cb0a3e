"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each ``pin_*`` takes an oracle library handle (``oracle.load()`` or a deliberately
mutated build) and raises AssertionError when the oracle disagrees with:
a hand-derived worked example, a closed form, an invariant, an independent
restatement built from numpy/scipy primitives, or brute-force equivalence of the
chunked and sequential forms. The mutation tests reuse them to show that each
planted mistake is caught.
"""
from __future__ import annotations

import json
import os

import numpy as np
from scipy.special import expit

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _unit_rows(x, D):
    sh = x.shape
    r = x.reshape(-1, D)
    return (r / np.linalg.norm(r, axis=1, keepdims=True)).reshape(sh)


def _rand_scan_inputs(rng, B, T, H, D, gdn=False, gmin=-5.0):
    q = _unit_rows(rng.standard_normal((B, T, H * D)), D)
    k = _unit_rows(rng.standard_normal((B, T, H * D)), D)
    v = rng.standard_normal((B, T, H * D))
    g = rng.uniform(gmin, 0.0, (B, T, H) if gdn else (B, T, H * D))
    beta = rng.uniform(0.0, 1.0, (B, T, H))
    s0 = 0.1 * rng.standard_normal((B, H, D, D))
    return q, k, v, g, beta, s0


def _close(a, b, tol, what):
    err = oracle.rel_linf(a, b)
    assert err <= tol, f"{what}: rel L-inf {err:.3e} > {tol:.1e}"


# ---------------------------------------------------------------- scan -----------
def pin_three_token(lib, D_embed=2):
    """Hand-derived worked example (golden/three_token.json), optionally zero-padded
    into a wider head: the padding channels must not change anything."""
    with open(os.path.join(GOLDEN, "three_token.json")) as f:
        gd = json.load(f)
    D = D_embed
    T = 3

    def pad(rows):
        a = np.zeros((1, T, D))
        a[0, :, :2] = np.asarray(rows)
        return a

    q, k, v = pad(gd["q"]), pad(gd["k"]), pad(gd["v"])
    g = np.zeros((1, T, D))
    g[0, :, :2] = np.log(np.asarray(gd["gate_decay"]))
    beta = np.asarray(gd["beta"]).reshape(1, T, 1)
    o, s = oracle.scan(q, k, v, g, beta, np.zeros((1, 1, D, D)), gd["scale"], lib=lib)
    want_o = np.asarray(gd["expected_o"])
    assert np.allclose(o[0, :, :2], want_o, rtol=0, atol=1e-12), f"o {o[0, :, :2]} != {want_o}"
    assert np.all(o[0, :, 2:] == 0)
    s_key_rows = s[0, 0].T  # stored [value j][key i]
    want_s = np.asarray(gd["expected_S_key_rows"])
    assert np.allclose(s_key_rows[:2, :2], want_s, rtol=0, atol=1e-12), f"S {s_key_rows[:2, :2]}"
    assert np.all(s_key_rows[2:, :] == 0) and np.all(s_key_rows[:, 2:] == 0)


def pin_beta0_g0(lib):
    """beta = 0, g = 0: the state is untouched bit for bit and o_t = scale * S0^T q_t."""
    rng = _rng(1)
    B, T, H, D = 2, 7, 2, 8
    q, k, v, g, beta, s0 = _rand_scan_inputs(rng, B, T, H, D)
    g[:] = 0.0
    beta[:] = 0.0
    o, s = oracle.scan(q, k, v, g, beta, s0, 0.37, lib=lib)
    assert np.array_equal(s, s0), "state changed with beta=0, g=0"
    for h in range(H):
        S = s0[:, h].transpose(0, 2, 1)  # [b][key i][value j]
        want = 0.37 * np.einsum("bij,bti->btj", S, q[:, :, h * D:(h + 1) * D])
        _close(o[:, :, h * D:(h + 1) * D], want, 1e-13, "beta=0 readout")


def pin_beta1_unit_k(lib):
    """beta = 1, g = 0, unit-norm k: after each token S_t^T k_t = v_t."""
    rng = _rng(2)
    B, T, H, D = 1, 6, 2, 8
    q, k, v, g, beta, s = _rand_scan_inputs(rng, B, T, H, D)
    g[:] = 0.0
    beta[:] = 1.0
    for t in range(T):
        sl = slice(t, t + 1)
        _, s = oracle.scan(q[:, sl], k[:, sl], v[:, sl], g[:, sl], beta[:, sl], s, 1.0, lib=lib)
        for h in range(H):
            kt = k[0, t, h * D:(h + 1) * D]
            got = s[0, h] @ kt  # rows of the stored state are value columns j
            _close(got, v[0, t, h * D:(h + 1) * D], 1e-13, "S^T k = v")


def pin_decay_closed_form(lib, gdn=False):
    """beta = 0, arbitrary g: S_T[i][j] = exp(sum_t g_t[i]) * S_0[i][j]. Pins the decay
    axis to the key index (the fastest axis of the stored state)."""
    rng = _rng(3)
    B, T, H, D = 2, 9, 2, 8
    q, k, v, g, beta, s0 = _rand_scan_inputs(rng, B, T, H, D, gdn=gdn)
    beta[:] = 0.0
    _, s = oracle.scan(q, k, v, g, beta, s0, 1.0, gdn=gdn, lib=lib)
    G = g.sum(axis=1)  # [B, H*D] or [B, H]
    if gdn:
        want = np.exp(G)[:, :, None, None] * s0
    else:
        want = np.exp(G.reshape(B, H, 1, D)) * s0  # key index i is the last axis
    _close(s, want, 1e-13, "decay closed form")


def pin_transition_form(lib, gdn=False):
    """Brute force: the recurrence restated as S_t = (I - beta k k^T) diag(e^g) S_{t-1}
    + beta k v^T with o_t = scale S_t^T q_t, built from numpy matrix products."""
    rng = _rng(4)
    B, T, H, D = 2, 11, 3, 6
    q, k, v, g, beta, s0 = _rand_scan_inputs(rng, B, T, H, D, gdn=gdn)
    k = k * rng.uniform(0.5, 1.5, (B, T, H * D))  # not unit-norm on purpose
    scale = 0.41
    o, s = oracle.scan(q, k, v, g, beta, s0, scale, gdn=gdn, lib=lib)
    for b in range(B):
        for h in range(H):
            cs = slice(h * D, (h + 1) * D)
            S = s0[b, h].T.copy()  # [key][value]
            for t in range(T):
                gt = np.full(D, g[b, t, h]) if gdn else g[b, t, cs]
                kt, bt = k[b, t, cs], beta[b, t, h]
                A = (np.eye(D) - bt * np.outer(kt, kt)) @ np.diag(np.exp(gt))
                S = A @ S + bt * np.outer(kt, v[b, t, cs])
                _close(o[b, t, cs], scale * S.T @ q[b, t, cs], 1e-12, "transition-form o")
            _close(s[b, h].T, S, 1e-12, "transition-form state")


def pin_gdn_is_broadcast_kda(lib):
    """GDN equals KDA with the per-head gate broadcast over the head's channels."""
    rng = _rng(5)
    B, T, H, D = 1, 8, 2, 8
    q, k, v, g, beta, s0 = _rand_scan_inputs(rng, B, T, H, D, gdn=True)
    o1, s1 = oracle.scan(q, k, v, g, beta, s0, 0.5, gdn=True, lib=lib)
    o2, s2 = oracle.scan(q, k, v, np.repeat(g, D, axis=2), beta, s0, 0.5, gdn=False, lib=lib)
    _close(o1, o2, 1e-15, "gdn vs broadcast kda o")
    _close(s1, s2, 1e-15, "gdn vs broadcast kda state")


def pin_chunked_equals_sequential(lib, Ts=(1, 5, 17, 64, 65, 130), Cs=(4, 16, 64), D=8,
                                  gdn=False, gmin=-5.0, tol=1e-12):
    """The chunked form reproduces the sequential definition to fp64 rounding."""
    rng = _rng(6 + int(gdn))
    for T in Ts:
        q, k, v, g, beta, s0 = _rand_scan_inputs(rng, 1, T, 2, D, gdn=gdn, gmin=gmin)
        o_s, s_s = oracle.scan(q, k, v, g, beta, s0, 0.3, gdn=gdn, lib=lib)
        for C in Cs:
            o_c, s_c = oracle.chunked_scan(q, k, v, g, beta, s0, 0.3, C, gdn=gdn, lib=lib)
            _close(o_c, o_s, tol, f"chunked o T={T} C={C}")
            _close(s_c, s_s, tol, f"chunked state T={T} C={C}")


# ---------------------------------------------------------------- conv -----------
def _conv_case(rng, B=2, T=9, qkv=6, K=4):
    x = [rng.standard_normal((B, T, qkv)) for _ in range(3)]
    w = rng.standard_normal((3 * qkv, K))
    ring = rng.standard_normal((B, 3 * qkv, K - 1))
    return x, w, ring


def pin_conv_identity_taps(lib):
    """Tap K-1 alone gives y = SiLU(x); tap 0 alone gives y_t = SiLU(x_{t-K+1}) with the
    ring supplying t < K-1 (slot 0 = oldest). Pins tap order and ring order."""
    rng = _rng(7)
    x, w, ring = _conv_case(rng)
    B, T, qkv = x[0].shape
    K = w.shape[1]
    for plane in range(3):
        w_last = np.zeros_like(w)
        w_last[:, K - 1] = 1.0
        y, _ = oracle.conv_silu_plane(x[plane], w_last, ring, plane, lib=lib)
        _close(y, x[plane] * expit(x[plane]), 1e-15, "tap K-1")
        w_first = np.zeros_like(w)
        w_first[:, 0] = 1.0
        y, _ = oracle.conv_silu_plane(x[plane], w_first, ring, plane, lib=lib)
        rows = slice(plane * qkv, (plane + 1) * qkv)
        xt = np.concatenate([ring[:, rows, :].transpose(0, 2, 1), x[plane]], axis=1)
        shifted = xt[:, :T]  # x_{t-K+1}
        _close(y, shifted * expit(shifted), 1e-15, "tap 0")


def pin_conv_bruteforce(lib):
    """Against numpy.convolve over [ring ++ x] per channel (plane offset plane*qkv for both
    the fused weight and the fused ring), and the rolled ring = last K-1 raw inputs,
    including T < K-1 where old ring slots and new rows mix."""
    rng = _rng(8)
    for T in (1, 2, 3, 9):
        x, w, ring = _conv_case(rng, T=T)
        B, _, qkv = x[0].shape
        K = w.shape[1]
        ring_out = ring.copy()
        for plane in range(3):
            y, ring_out = oracle.conv_silu_plane(x[plane], w, ring, plane, ring_out=ring_out,
                                                 lib=lib)
            for b in range(B):
                for c in range(qkv):
                    cf = plane * qkv + c
                    xt = np.concatenate([ring[b, cf], x[plane][b, :, c]])
                    pre = np.convolve(xt, w[cf][::-1], mode="valid")
                    _close(y[b, :, c], pre * expit(pre), 1e-14, "conv brute force")
                    _close(ring_out[b, cf], xt[-(K - 1):], 0.0, "ring roll")


# ----------------------------------------------------------- norms ---------------
def pin_l2_closed_forms(lib):
    D = 16
    c = 0.3
    y = oracle.l2norm_rows(np.full((3, D), c), D, lib=lib)
    _close(y, np.full((3, D), c / np.sqrt(D * c * c + 1e-6)), 1e-15, "l2 constant row")
    y = oracle.l2norm_rows(np.zeros((2, D)), D, lib=lib)
    assert np.all(y == 0)
    x = _rng(9).standard_normal((5, D)) * 1e-3  # small rows make the eps placement visible
    want = x / np.sqrt(np.linalg.norm(x, axis=1, keepdims=True) ** 2 + 1e-6)
    _close(oracle.l2norm_rows(x, D, lib=lib), want, 1e-14, "l2 eps inside sqrt")


def pin_rmsnorm_closed_forms(lib):
    D = 8
    eps = 1e-5
    c = 0.7
    o = np.full((2, D), c)
    w = np.ones(D)
    z0 = np.zeros((2, D))
    _close(oracle.gated_rmsnorm(o, z0, w, eps, gdn=False, lib=lib),
           np.full((2, D), 0.5 * c / np.sqrt(c * c + eps)), 1e-15, "kda gate sigmoid(0)")
    assert np.all(oracle.gated_rmsnorm(o, z0, w, eps, gdn=True, lib=lib) == 0), "SiLU(0) = 0"
    rng = _rng(10)
    o = rng.standard_normal((4, D))
    z = rng.standard_normal((4, D))
    w = rng.standard_normal(D)
    rms = np.sqrt(np.mean(o * o, axis=1, keepdims=True) + eps)
    _close(oracle.gated_rmsnorm(o, z, w, eps, gdn=False, lib=lib), o / rms * w * expit(z),
           1e-14, "kda rmsnorm")
    _close(oracle.gated_rmsnorm(o, z, w, eps, gdn=True, lib=lib), o / rms * w * z * expit(z),
           1e-14, "gdn rmsnorm")


# ----------------------------------------------------------- whole path ----------
def brute_mixer(inp_q, inp_k, inp_v, g, beta, conv_w, ring, state, z, norm_w, scale, eps, gdn):
    """Independent restatement of the whole path from numpy/scipy primitives:
    numpy.convolve for the conv, numpy.linalg.norm for l2, the transition-matrix
    form of the recurrence, expit for the gates. q and k may have fewer heads than v
    (grouped heads, GDN): value head h then reads query / key head h % Hk, and the
    conv weight and ring planes are q, k (Hk*D rows each), v (H*D)."""
    B, T, kw = inp_q.shape
    H, D = state.shape[1], state.shape[2]
    Hk = kw // D
    K = conv_w.shape[1]
    convd = []
    base = 0
    for x in (inp_q, inp_k, inp_v):
        y = np.empty_like(x)
        for b in range(B):
            for c in range(x.shape[2]):
                cf = base + c
                xt = np.concatenate([ring[b, cf], x[b, :, c]])
                pre = np.convolve(xt, conv_w[cf][::-1], mode="valid")
                y[b, :, c] = pre * expit(pre)
        convd.append(y)
        base += x.shape[2]
    qc, kc, vc = convd
    out = np.empty_like(inp_v)
    s_out = np.empty_like(state)
    for b in range(B):
        for h in range(H):
            cs = slice(h * D, (h + 1) * D)
            ks = slice((h % Hk) * D, (h % Hk + 1) * D)
            S = state[b, h].T.copy()
            for t in range(T):
                qt = qc[b, t, ks] / np.sqrt(np.linalg.norm(qc[b, t, ks]) ** 2 + 1e-6)
                kt = kc[b, t, ks] / np.sqrt(np.linalg.norm(kc[b, t, ks]) ** 2 + 1e-6)
                gt = np.full(D, g[b, t, h]) if gdn else g[b, t, cs]
                bt = beta[b, t, h]
                S = (np.eye(D) - bt * np.outer(kt, kt)) @ np.diag(np.exp(gt)) @ S \
                    + bt * np.outer(kt, vc[b, t, cs])
                o = scale * S.T @ qt
                zz = z[b, t, cs]
                gate = zz * expit(zz) if gdn else expit(zz)
                out[b, t, cs] = o / np.sqrt(np.mean(o * o) + eps) * norm_w * gate
            s_out[b, h] = S.T
    xt_all = np.concatenate([ring, np.concatenate([inp_q, inp_k, inp_v], axis=2)
                             .transpose(0, 2, 1)], axis=2)
    ring_out = xt_all[:, :, -(K - 1):]
    return out, s_out, ring_out


def _mixer_case(rng, B=2, T=7, H=2, D=8, K=4, gdn=False):
    qkv = H * D
    a = dict(
        q=rng.standard_normal((B, T, qkv)), k=rng.standard_normal((B, T, qkv)),
        v=rng.standard_normal((B, T, qkv)),
        g=rng.uniform(-5, 0, (B, T, H) if gdn else (B, T, qkv)),
        beta=rng.uniform(0, 1, (B, T, H)), conv_w=0.5 * rng.standard_normal((3 * qkv, K)),
        ring=rng.standard_normal((B, 3 * qkv, K - 1)),
        state=0.05 * rng.standard_normal((B, H, D, D)), z=rng.standard_normal((B, T, qkv)),
        norm_w=1 + 0.1 * rng.standard_normal(D))
    return a


def pin_mixer_bruteforce(lib, gdn=False):
    rng = _rng(11 + int(gdn))
    for T in (1, 2, 7):
        a = _mixer_case(rng, T=T, gdn=gdn)
        scale, eps = 0.35, 1e-5
        r = oracle.mixer(**a, scale=scale, rms_eps=eps, gdn=gdn, lib=lib)
        out, s_out, ring_out = brute_mixer(a["q"], a["k"], a["v"], a["g"], a["beta"],
                                           a["conv_w"], a["ring"], a["state"], a["z"],
                                           a["norm_w"], scale, eps, gdn)
        _close(r["out"], out, 1e-11, f"mixer out T={T}")
        _close(r["state"], s_out, 1e-11, f"mixer state T={T}")
        _close(r["ring"], ring_out, 0.0, f"mixer ring T={T}")


def pin_resume(lib, gdn=False):
    """prefill(T1) then prefill(T2) with ring and state carried == prefill(T1 + T2)."""
    rng = _rng(13)
    a = _mixer_case(rng, T=11, gdn=gdn)
    full = oracle.mixer(**a, scale=0.3, rms_eps=1e-5, gdn=gdn, lib=lib)
    t1 = 4
    first = {n: (x[:, :t1] if n in ("q", "k", "v", "g", "beta", "z") else x) for n, x in a.items()}
    r1 = oracle.mixer(**first, scale=0.3, rms_eps=1e-5, gdn=gdn, lib=lib)
    second = {n: (x[:, t1:] if n in ("q", "k", "v", "g", "beta", "z") else x) for n, x in a.items()}
    second["ring"], second["state"] = r1["ring"], r1["state"]
    r2 = oracle.mixer(**second, scale=0.3, rms_eps=1e-5, gdn=gdn, lib=lib)
    _close(np.concatenate([r1["out"], r2["out"]], axis=1), full["out"], 1e-14, "resume out")
    _close(r2["state"], full["state"], 1e-14, "resume state")
    _close(r2["ring"], full["ring"], 0.0, "resume ring")


ALL_PINS = {
    "three_token": pin_three_token,
    "three_token_padded": lambda lib: pin_three_token(lib, D_embed=16),
    "beta0_g0": pin_beta0_g0,
    "beta1_unit_k": pin_beta1_unit_k,
    "decay_kda": pin_decay_closed_form,
    "decay_gdn": lambda lib: pin_decay_closed_form(lib, gdn=True),
    "transition_kda": pin_transition_form,
    "transition_gdn": lambda lib: pin_transition_form(lib, gdn=True),
    "gdn_broadcast": pin_gdn_is_broadcast_kda,
    "chunked_kda": pin_chunked_equals_sequential,
    "chunked_gdn": lambda lib: pin_chunked_equals_sequential(lib, gdn=True),
    "conv_taps": pin_conv_identity_taps,
    "conv_brute": pin_conv_bruteforce,
    "l2": pin_l2_closed_forms,
    "rmsnorm": pin_rmsnorm_closed_forms,
    "mixer_kda": pin_mixer_bruteforce,
    "mixer_gdn": lambda lib: pin_mixer_bruteforce(lib, gdn=True),
    "resume": pin_resume,
}
