"""Pins of the A2V cross-attention layer oracle (oracle/crossattn.py).

The backward is pinned to central finite differences of the exact (unrounded)
forward; the forward to closed forms (one audio token, constant logits), to
the zone scorer's A2V feature (identity projections, one head), and to
symmetries; the bf16 rounding to hand values and to the input generator's
float32 route."""
import numpy as np
import pytest

import synth
from oracle import crossattn as oca
from oracle import zones as ozon


def _weights(rng, C, D, scale=None):
    s = scale if scale is not None else 1 / np.sqrt(C)
    return [rng.normal(size=(D, C)) * s for _ in range(3)] + [rng.normal(size=(C, D)) / np.sqrt(D)]


def test_round_bf16_hand_values():
    r = oca.round_bf16
    assert r(1.0) == 1.0
    assert r(1 + 2 ** -8) == 1.0                      # tie -> even (1.0)
    assert r(1 + 3 * 2 ** -8) == 1 + 2 ** -6          # tie -> even (1 + 2^-6)
    assert r(1 + 2 ** -8 + 2 ** -20) == 1 + 2 ** -7   # above the tie
    assert r(-3.0) == -3.0 and r(0.0) == 0.0
    assert r(255.5) == 256.0 and r(2 ** -133) == 2 ** -133
    assert r(2 ** -134 * 1.5) == 2 ** -133            # subnormal spacing


def test_round_bf16_matches_the_float32_route():
    x = np.random.default_rng(0).normal(size=20000).astype(np.float32) * 10.0 ** \
        np.random.default_rng(1).integers(-20, 20, 20000)
    want = synth.bf16_bits_to_f64(synth.f32_to_bf16_bits(x))
    assert np.array_equal(oca.round_bf16(x.astype(np.float64)), want)


@pytest.mark.parametrize("heads,d", [(1, 4), (2, 3)])
def test_backward_matches_finite_differences(heads, d):
    rng = np.random.default_rng(2)
    N, Na, C = 5, 4, 6
    D = heads * d
    X, A = rng.normal(size=(N, C)), rng.normal(size=(Na, C))
    W = _weights(rng, C, D, scale=0.7)
    dY = rng.normal(size=(N, C))
    f = oca.forward(X, A, *W, heads, rounding=False)
    g = oca.backward(X, A, *W, heads, f, dY)

    def loss(X_, A_, Wq, Wk, Wv, Wo):
        return float((oca.forward(X_, A_, Wq, Wk, Wv, Wo, heads, rounding=False)["y"] * dY).sum())

    args = [X, A] + W
    for ai, name in enumerate(("dx", "da", "dwq", "dwk", "dwv", "dwo")):
        num = np.zeros_like(args[ai])
        for idx in np.ndindex(args[ai].shape):
            h = 1e-6
            plus = [a.copy() for a in args]
            minus = [a.copy() for a in args]
            plus[ai][idx] += h
            minus[ai][idx] -= h
            num[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        assert np.abs(num - g[name]).max() <= 1e-7 * max(1.0, np.abs(num).max()), name


def test_one_audio_token_copies_its_value():
    rng = np.random.default_rng(3)
    N, C, heads, d = 6, 8, 2, 4
    X, A = rng.normal(size=(N, C)), rng.normal(size=(1, C))
    W = _weights(rng, C, heads * d)
    f = oca.forward(X, A, *W, heads, rounding=False)
    assert np.allclose(f["o"], np.repeat(A @ W[2].T, N, axis=0), atol=1e-14)
    for h in range(heads):                       # lse = the only logit
        c = slice(h * d, (h + 1) * d)
        assert np.allclose(f["lse"][h], f["q"][:, c] @ f["k"][0, c] / np.sqrt(d), atol=1e-13)


def test_zero_queries_average_the_values():
    rng = np.random.default_rng(4)
    N, Na, C, heads, d = 5, 7, 8, 2, 4
    X, A = rng.normal(size=(N, C)), rng.normal(size=(Na, C))
    Wq, Wk, Wv, Wo = _weights(rng, C, heads * d)
    f = oca.forward(X, A, np.zeros_like(Wq), Wk, Wv, Wo, heads, rounding=False)
    assert np.allclose(f["o"], np.repeat((A @ Wv.T).mean(0, keepdims=True), N, axis=0), atol=1e-14)
    assert np.allclose(f["lse"], np.log(Na), atol=1e-14)


def test_identity_projections_give_the_zone_scorers_a2v_feature():
    rng = np.random.default_rng(5)
    N, Na, C = 9, 6, 16
    X, A = rng.normal(size=(N, C)), rng.normal(size=(Na, C))
    eye = np.eye(C)
    f = oca.forward(X, A, eye, eye, eye, eye, 1, rounding=False)
    assert np.allclose(np.linalg.norm(f["y"], axis=1), ozon.a2v_norm(X, A), rtol=1e-12)


def test_audio_order_does_not_matter_and_heads_are_independent():
    rng = np.random.default_rng(6)
    N, Na, C, heads, d = 6, 5, 8, 2, 4
    X, A = rng.normal(size=(N, C)), rng.normal(size=(Na, C))
    Wq, Wk, Wv, Wo = _weights(rng, C, heads * d)
    f = oca.forward(X, A, Wq, Wk, Wv, Wo, heads, rounding=False)
    g = oca.forward(X, A[::-1].copy(), Wq, Wk, Wv, Wo, heads, rounding=False)
    assert np.allclose(f["y"], g["y"], atol=1e-13)
    Wq2 = Wq.copy()
    Wq2[d:] = rng.normal(size=(d, C))                  # change head 1's query weights only
    g = oca.forward(X, A, Wq2, Wk, Wv, Wo, heads, rounding=False)
    assert np.array_equal(f["o"][:, :d], g["o"][:, :d])
    assert not np.allclose(f["o"][:, d:], g["o"][:, d:])


def test_rounding_points_store_bf16_values():
    rng = np.random.default_rng(7)
    N, Na, C, heads, d = 6, 5, 8, 2, 4
    X, A = rng.normal(size=(N, C)), rng.normal(size=(Na, C))
    W = _weights(rng, C, heads * d)
    f = oca.forward(X, A, *W, heads)
    for name in ("q", "k", "v", "o", "y"):
        assert np.array_equal(oca.round_bf16(f[name]), f[name]), name
    # the backward rounds nothing: its gradients are the exact ones of the
    # rounded forward's stored tensors (dO = dY Wo exactly)
    dY = rng.normal(size=(N, C))
    g = oca.backward(X, A, *W, heads, f, dY)
    assert np.array_equal(g["do"], dY @ W[3])
    exact = oca.forward(X, A, *W, heads, rounding=False)
    assert np.abs(f["y"] - exact["y"]).max() < 0.05 * np.abs(exact["y"]).max()
