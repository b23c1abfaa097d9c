"""Pins of the pre-attention normalization + 3-D RoPE oracle (oracle/prenorm.py)
against hand-worked values, closed forms and an independent complex-number
formulation of the rotation."""
import numpy as np
import pytest

from oracle import prenorm as pn


def test_split_sizes():
    assert pn.split_sizes(128) == (44, 42, 42)
    assert pn.split_sizes(64) == (24, 20, 20)
    for d in range(12, 260, 2):
        t, h, w = pn.split_sizes(d)
        assert t + h + w == d and t % 2 == h % 2 == w % 2 == 0 and t >= h == w


def test_rms_norm_hand_value():
    # x = (3, 4): mean square 12.5, rms 3.5355339...; gamma = (1, 2)
    y = pn.rms_norm(np.array([3.0, 4.0]), np.array([1.0, 2.0]), eps=0.0)
    assert np.allclose(y, [3 / np.sqrt(12.5), 8 / np.sqrt(12.5)], rtol=0, atol=1e-15)


def test_rms_norm_properties():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 7, 64))
    y = pn.rms_norm(x, np.ones(64), eps=0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, atol=1e-14)
    assert np.allclose(pn.rms_norm(3.7 * x, np.ones(64), eps=0.0), y, atol=1e-14)
    assert np.all(pn.rms_norm(np.zeros((2, 64)), np.ones(64)) == 0.0)


def test_rope_hand_value():
    # d = 12: groups t, h, w of 4 channels; pair i of a group turns by
    # pos * 10000^(-2i/4) = pos * (1, 0.01); token (t, h, w) = (1, 2, 3)
    grid = (2, 3, 4)
    n = (1 * 3 + 2) * 4 + 3
    x = np.zeros((1, 24, 12))
    x[0, n, 0::2] = 1.0
    y = pn.rope3d(x, grid)[0, n]
    ang = [1.0, 0.01, 2.0, 0.02, 3.0, 0.03]
    want = np.ravel([[np.cos(a), np.sin(a)] for a in ang])
    assert np.allclose(y, want, atol=1e-15)


def test_rope_origin_is_identity_and_norms_are_kept():
    rng = np.random.default_rng(1)
    grid = (3, 5, 6)
    x = rng.standard_normal((2, 90, 64))
    y = pn.rope3d(x, grid)
    assert np.array_equal(y[:, 0], x[:, 0])               # token (0, 0, 0)
    pair = lambda z: z[..., 0::2] ** 2 + z[..., 1::2] ** 2
    assert np.allclose(pair(y), pair(x), atol=1e-13)


def test_rope_matches_complex_rotation():
    rng = np.random.default_rng(2)
    grid = (4, 6, 5)
    d = 128
    x = rng.standard_normal((3, 120, d))
    # independent form: pair (x0, x1) as the complex x0 + i x1 times e^{i a},
    # with the angles rebuilt group by group from the coordinates
    T, H, W = grid
    t, h, w = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    coords = [t.ravel(), h.ravel(), w.ravel()]
    angles = []
    for axis, g in enumerate((44, 42, 42)):
        for i in range(g // 2):
            angles.append(coords[axis] * 10000.0 ** (-2.0 * i / g))
    a = np.stack(angles, axis=1)
    z = (x[..., 0::2] + 1j * x[..., 1::2]) * np.exp(1j * a)
    y = pn.rope3d(x, grid)
    assert np.allclose(y[..., 0::2], z.real, atol=1e-13)
    assert np.allclose(y[..., 1::2], z.imag, atol=1e-13)


def test_rope_scores_depend_on_relative_position():
    # <R(p) q, R(p') k> = <R(p - p') q, k> along every axis
    rng = np.random.default_rng(3)
    grid = (9, 9, 9)
    d = 64
    q, k = rng.standard_normal((2, d))
    pos = pn.positions(grid)
    X = np.broadcast_to(q, (729, d))
    Y = np.broadcast_to(k, (729, d))
    rq, rk = pn.rope3d(X[None], grid)[0], pn.rope3d(Y[None], grid)[0]
    idx = {tuple(p): n for n, p in enumerate(pos)}
    for a, b in [((5, 2, 7), (3, 1, 4)), ((8, 8, 8), (2, 5, 0)), ((4, 4, 4), (0, 0, 0))]:
        lhs = rq[idx[a]] @ rk[idx[b]]
        rel = tuple(x - y for x, y in zip(a, b))
        rhs = rq[idx[rel]] @ k
        assert abs(lhs - rhs) < 1e-12


@pytest.mark.parametrize("d", [64, 128])
def test_norm_then_rope_order(d):
    rng = np.random.default_rng(4)
    grid = (2, 3, 4)
    x = rng.standard_normal((1, 24, d))
    g = rng.uniform(0.5, 1.5, d)
    y = pn.norm_rope(x, g, grid)
    # rotation keeps pair norms, so the rms of the output equals the rms of
    # the normalized (pre-rotation) vector
    pre = pn.rms_norm(x, g)
    assert np.allclose(np.sum(y * y, -1), np.sum(pre * pre, -1), atol=1e-12)
    assert not np.allclose(y, pn.rms_norm(pn.rope3d(x, grid), g))  # order matters (gamma)
