"""Pins of the grouped-head GDN oracle (oracle/gqa.py), independent of its index
arithmetic: Hk = H is the plain mixer; physically tiling q / k (numpy.tile) and
running the plain mixer gives the same result; zeroing one key head's queries
silences exactly the value heads h with h % Hk equal to it (the tiled order, not
blocks of consecutive heads); the independent numpy restatement with explicit
key-head indexing agrees; the ring holds the last raw inputs of each plane."""
import numpy as np
import pytest

import oracle
from oracle import gqa
from tests.pins import brute_mixer

SCALE, EPS = 0.3, 1e-5


def _case(seed, B=2, T=6, H=4, Hk=2, D=8, K=4):
    rng = np.random.default_rng(seed)
    kw, vw = Hk * D, H * D
    return dict(
        q=rng.standard_normal((B, T, kw)), k=rng.standard_normal((B, T, kw)),
        v=rng.standard_normal((B, T, vw)), g=rng.uniform(-5, 0, (B, T, H)),
        beta=rng.uniform(0, 1, (B, T, H)), conv_w=0.5 * rng.standard_normal((2 * kw + vw, K)),
        ring=rng.standard_normal((B, 2 * kw + vw, K - 1)),
        state=0.05 * rng.standard_normal((B, H, D, D)), z=rng.standard_normal((B, T, vw)),
        norm_w=1 + 0.1 * rng.standard_normal(D))


def test_equal_heads_is_the_plain_mixer():
    a = _case(1, H=3, Hk=3)
    r = gqa.mixer_gqa(**a, scale=SCALE, rms_eps=EPS)
    p = oracle.mixer(**a, scale=SCALE, rms_eps=EPS, gdn=True)
    for n in ("out", "o_core", "state", "ring"):
        assert np.array_equal(r[n], p[n]), n


@pytest.mark.parametrize("H,Hk", [(4, 2), (6, 2), (6, 3), (4, 1)])
def test_tiled_copies_give_the_same_result(H, Hk):
    a = _case(2, H=H, Hk=Hk)
    D, G = 8, H // Hk
    kw = Hk * D

    def tile_heads(x):  # [..., Hk*D] -> [..., H*D] in the order h -> h % Hk
        return np.tile(x.reshape(*x.shape[:-1], Hk, D), (1,) * (x.ndim - 1) + (G, 1)).reshape(
            *x.shape[:-1], H * D)

    def tile_rows(x):  # planes q, k of [.., Hk*D, K'] rows -> [.., H*D, K'], v as is
        parts = []
        for j in (0, 1):
            blk = x[..., j * kw:(j + 1) * kw, :]
            blk = blk.reshape(*blk.shape[:-2], Hk, D, blk.shape[-1])
            blk = np.tile(blk, (1,) * (blk.ndim - 3) + (G, 1, 1))
            parts.append(blk.reshape(*x.shape[:-2], H * D, x.shape[-1]))
        parts.append(x[..., 2 * kw:, :])
        return np.concatenate(parts, axis=-2)

    plain = dict(a, q=tile_heads(a["q"]), k=tile_heads(a["k"]), conv_w=tile_rows(a["conv_w"]),
                 ring=tile_rows(a["ring"]))
    p = oracle.mixer(**plain, scale=SCALE, rms_eps=EPS, gdn=True)
    r = gqa.mixer_gqa(**a, scale=SCALE, rms_eps=EPS)
    for n in ("out", "o_core", "state"):
        assert np.array_equal(r[n], p[n]), n
    # every tiled copy of a q / k ring row rolls to the same values
    assert np.array_equal(tile_rows(r["ring"]), p["ring"])


def test_zero_queries_of_one_key_head_silence_its_value_heads():
    a = _case(3, H=4, Hk=2)
    D = 8
    a["q"][:, :, D:2 * D] = 0.0   # key head 1 ...
    a["conv_w"][D:2 * D] = 0.0    # ... and its q conv rows: its conv output is SiLU(0) = 0
    r = gqa.mixer_gqa(**a, scale=SCALE, rms_eps=EPS)
    for h in range(4):
        o = r["o_core"][:, :, h * D:(h + 1) * D]
        if h % 2 == 1:
            assert np.all(o == 0.0), h
        else:
            assert np.abs(o).max() > 1e-3, h


@pytest.mark.parametrize("H,Hk,T", [(4, 2, 1), (4, 2, 5), (6, 3, 4), (4, 1, 3)])
def test_independent_restatement(H, Hk, T):
    a = _case(4, H=H, Hk=Hk, T=T)
    r = gqa.mixer_gqa(**a, scale=SCALE, rms_eps=EPS)
    out, s_out, ring_out = brute_mixer(a["q"], a["k"], a["v"], a["g"], a["beta"], a["conv_w"], a["ring"],
                                       a["state"], a["z"], a["norm_w"], SCALE, EPS, True)
    np.testing.assert_allclose(r["out"], out, rtol=0, atol=1e-11 * np.abs(out).max())
    np.testing.assert_allclose(r["state"], s_out, rtol=0, atol=1e-11 * np.abs(s_out).max())
    assert np.array_equal(r["ring"], ring_out)


def test_blocked_head_order_is_caught(monkeypatch):
    """A planted mistake: value head h reading key head h // (H / Hk) (consecutive
    blocks) instead of h % Hk fails the restatement and the zero-query pins."""
    def blocked(heads, H, Hk, D):
        return ((np.asarray(heads) // (H // Hk))[:, None] * D + np.arange(D)).ravel()

    monkeypatch.setattr(gqa, "key_channels", blocked)
    with pytest.raises(AssertionError):
        test_independent_restatement(4, 2, 5)
    with pytest.raises(AssertionError):
        test_zero_queries_of_one_key_head_silence_its_value_heads()
