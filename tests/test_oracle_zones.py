"""Pins of the oracle's zone scoring and block-shape rule (oracle/zones.py).

Closed forms of linear ramps, fields for which a signal must vanish, a
library evaluation of the A2V attention, and the monotonicity of the rule.
"""
import numpy as np
import pytest
import torch

from oracle import layout as lay
from oracle import zones as zon

ZONE = (4, 16, 16)


def _ramp(grid, axis, slope, C=3, offset=0.0):
    T, H, W = grid
    t, h, w = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    coord = (t, h, w)[axis].astype(np.float64).reshape(-1, 1)
    return offset + slope * coord * np.ones((1, C))


def test_constant_field_has_zero_variance():
    L = lay.make_layout((8, 32, 32), "dynamic", ZONE)
    X = np.full((L.n_tokens, 5), 2.5)
    V, G, nz = zon.zone_stats(L, X, np.full(L.n_tokens, 1.0))
    assert np.all(V == 0) and np.all(G == 0) and np.all(nz == 4 * 16 * 16)


@pytest.mark.parametrize("axis", [0, 1, 2])
def test_ramp_variance_closed_form(axis):
    """A ramp of slope s along an axis of extent Z (every line complete):
    the variance of s*{0..Z-1} is s^2 (Z^2 - 1)/12 on that axis, 0 elsewhere."""
    grid = (8, 32, 32)
    L = lay.make_layout(grid, "dynamic", ZONE)
    s = 0.37
    X = _ramp(grid, axis, s, offset=1.0)
    V, G, nz = zon.zone_stats(L, X, None)
    Z = ZONE[axis]
    want = s * s * (Z * Z - 1) / 12.0
    for a in range(3):
        np.testing.assert_allclose(V[:, a], want if a == axis else 0.0, rtol=1e-12, atol=1e-12)


def test_ragged_zone_lines_use_their_real_length():
    """Grid 5x20x36: the last w-zone holds 36-32 = 4 real columns, so a w-ramp
    of slope s gives s^2 (4^2-1)/12 there and s^2 (16^2-1)/12 in full zones."""
    grid = (5, 20, 36)
    L = lay.make_layout(grid, "dynamic", ZONE)
    s = 1.5
    V, _, nz = zon.zone_stats(L, _ramp(grid, 2, s), None)
    gz = L.zone_grid
    for z in range(L.n_zones):
        wz = z % gz[2]
        Lw = 16 if wz < 2 else 4
        np.testing.assert_allclose(V[z, 2], s * s * (Lw * Lw - 1) / 12.0, rtol=1e-12)
        assert V[z, 0] == pytest.approx(0.0, abs=1e-12)


@pytest.mark.parametrize("axis,expect", [
    (0, 2),   # fast change along t  -> 1x8x16 (one frame per block)
    (1, 1),   # fast change along h  -> 4x4x8 (finest along h)
    (2, 0),   # fast change along w  -> 2x8x8 and 4x4x8 tie exactly -> canonical 2x8x8
])
def test_ramp_picks_the_shape_finest_along_the_ramp(axis, expect):
    grid = (8, 32, 32)
    L = lay.make_layout(grid, "dynamic", ZONE)
    shape, V, G, cost, gap = zon.score_zones(L, _ramp(grid, axis, 0.2), None)
    assert np.all(shape == expect)
    if axis == 2:
        assert np.all(gap == 0.0)
        # the hand values: r_w = 3 (mean over 3 axes), factors 63/255, 63/255, 255/255
        np.testing.assert_allclose(cost[0], [3 * 63 / 255, 3 * 63 / 255, 3.0], rtol=1e-12)


def test_shape_factors_are_the_exact_rationals():
    L = lay.make_layout((4, 16, 16), "dynamic", ZONE)
    f = zon.shape_factors(L)
    want = np.array([[3 / 15, 63 / 255, 63 / 255],     # 2x8x8
                     [15 / 15, 15 / 255, 63 / 255],    # 4x4x8
                     [0 / 15, 63 / 255, 255 / 255]])   # 1x8x16
    np.testing.assert_allclose(f, want, rtol=0, atol=1e-15)


def test_single_audio_token_gives_constant_norm():
    rng = np.random.default_rng(1)
    X = rng.standard_normal((50, 16))
    A = rng.standard_normal((1, 16))
    g = zon.a2v_norm(X, A)
    np.testing.assert_allclose(g, np.linalg.norm(A[0]), rtol=1e-13)


def test_zero_video_gives_mean_audio_norm():
    rng = np.random.default_rng(2)
    A = rng.standard_normal((7, 16))
    g = zon.a2v_norm(np.zeros((30, 16)), A)
    np.testing.assert_allclose(g, np.linalg.norm(A.mean(axis=0)), rtol=1e-13)
    L = lay.make_layout((4, 16, 16), "dynamic", ZONE)
    X = np.zeros((L.n_tokens, 16))
    _, G, _ = zon.zone_stats(L, X, zon.a2v_norm(X, A))
    assert np.all(np.abs(G) < 1e-24)


def test_dominant_audio_token_gives_its_norm():
    """Orthogonal audio rows and X_n = 40 * A_j: the softmax is one-hot up to
    exp(-40^2 |A|^2/sqrt(C)) and g_n = |A_j|."""
    C = 16
    A = np.eye(C)[:4] * 3.0
    X = 40.0 * A[[0, 1, 2, 3, 2]]
    g = zon.a2v_norm(X, A)
    np.testing.assert_allclose(g, 3.0, rtol=1e-12)


def test_a2v_norm_matches_library_attention():
    """torch's scaled_dot_product_attention (fp64, CPU) with query X, key A and
    value A computes F; its row norm must equal g."""
    rng = np.random.default_rng(3)
    X = rng.standard_normal((40, 24))
    A = rng.standard_normal((9, 24))
    F = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(X)[None], torch.from_numpy(A)[None], torch.from_numpy(A)[None])
    np.testing.assert_allclose(zon.a2v_norm(X, A), F[0].norm(dim=1).numpy(), rtol=1e-12)
    np.testing.assert_allclose(zon.a2v_norm_gram(X, A), zon.a2v_norm(X, A), rtol=1e-12)


def test_growing_t_variance_moves_choice_to_frame_blocks():
    """Add an increasing t-ramp to a w-ramp: once r_t grows the choice must
    move to 1x8x16 and never back."""
    grid = (4, 16, 16)
    L = lay.make_layout(grid, "dynamic", ZONE)
    base = _ramp(grid, 2, 0.1) + _ramp(grid, 1, 0.05)
    picks = []
    for s in np.linspace(0.0, 2.0, 21):
        shape, *_ = zon.score_zones(L, base + _ramp(grid, 0, s), None)
        picks.append(int(shape[0]))
    first = picks.index(2)
    assert all(p == 2 for p in picks[first:]) and picks[0] != 2


def test_zero_cost_zone_ties_to_first_candidate():
    """A zone whose costs are all 0 (no variation at all) is an exact tie and
    goes to shape 0. (Padding to zone multiples leaves every zone at least one
    real token, so all-pad zones do not occur; the zero row is forced.)"""
    L = lay.make_layout((5, 16, 16), "dynamic", ZONE)   # zones t0=0 (full), t0=4 (1 frame)
    X = np.random.default_rng(0).standard_normal((L.n_tokens, 4))
    shape, V, G, cost, gap = zon.score_zones(L, X, None)
    assert shape.shape == (2,)
    cost2 = np.vstack([cost, np.zeros((1, 3))])
    s2, g2 = zon.choose_shapes(cost2)
    assert s2[-1] == 0 and g2[-1] == 0.0


def test_tie_window_prefers_canonical_order():
    s, g = zon.choose_shapes(np.array([[1.0 + 5e-7, 1.0, 2.0],
                                       [1.0 + 2e-6, 1.0, 2.0],
                                       [3.0, 2.0, 2.0]]))
    assert s.tolist() == [0, 1, 1]
    assert g[0] == pytest.approx(5e-7, rel=1e-6) and g[2] == 0.0


def test_a2v_term_acts_per_axis():
    """Constant video and an audio-driven g that varies along h only: the A2V
    term alone must pick the shape finest along h (4x4x8)."""
    grid = (4, 16, 16)
    L = lay.make_layout(grid, "dynamic", ZONE)
    T, H, W = grid
    g = np.repeat(np.arange(H, dtype=np.float64)[None, :, None], T, 0).repeat(W, 2).reshape(-1)
    X = np.zeros((L.n_tokens, 4))
    V, G, nz = zon.zone_stats(L, X, g)
    assert G[0, 1] > 0 and G[0, 0] == 0 and G[0, 2] == 0
    r = zon.zone_signal(V, G, nz, use_audio=True)
    shape, _ = zon.choose_shapes(zon.shape_costs(L, r))
    assert shape[0] == 1


def test_two_signals_pulling_apart_hand_values():
    """Both terms non-zero and pulling toward different shapes. Worked by hand:

    zone 0: V = (8, 0, 1), G = (0, 8, 1); zone 1: V = (5, 5, 5), G = (1, 1, 1);
    zone 2 is empty (n_z = 0, V = G = 0) and must not enter the means.
    Means over the six non-empty (zone, axis) pairs: Vbar = 24/6 = 4,
    Gbar = 12/6 = 2. So r = V/4 + G/2:
      zone 0: (2 + 0, 0 + 4, 1/4 + 1/2) = (2, 4, 3/4);  zone 1: (7/4, 7/4, 7/4).
    Shape factors (b^2-1)/(Z^2-1), Z = (4, 16, 16):
      2x8x8: (3/15, 63/255, 63/255); 4x4x8: (1, 15/255, 63/255);
      1x8x16: (0, 63/255, 1).
    Zone 0 costs: 2x8x8: 2/5 + 4.75*63/255 = 401.25/255;
                  4x4x8: 2 + (60 + 47.25)/255 = 617.25/255;
                  1x8x16: 252/255 + 3/4 = 443.25/255  -> 2x8x8.
    The video term alone (r = (2, 0, 1/4)) picks 1x8x16 (costs 0.4 + 15.75/255,
    2 + 15.75/255, 1/4), the audio term alone (r = (0, 4, 1/2)) picks 4x4x8
    (costs 283.5/255, 91.5/255, 379.5/255), and the sum without the
    normalisation (r = (8, 8, 2)) picks 1x8x16 (costs 1.6 + 630/255,
    8 + 246/255, 504/255 + 2): only the normalised sum of both gives 2x8x8.
    Zone 1: 7/4 (177/255, 333/255, 318/255) -> 2x8x8."""
    L = lay.make_layout((12, 16, 16), "dynamic", ZONE)   # three zones along t
    V = np.array([[8.0, 0.0, 1.0], [5.0, 5.0, 5.0], [0.0, 0.0, 0.0]])
    G = np.array([[0.0, 8.0, 1.0], [1.0, 1.0, 1.0], [0.0, 0.0, 0.0]])
    nz = np.array([1024, 1024, 0])
    r = zon.zone_signal(V, G, nz, use_audio=True)
    np.testing.assert_allclose(r, [[2.0, 4.0, 0.75], [1.75, 1.75, 1.75], [0.0, 0.0, 0.0]],
                               rtol=1e-15)
    cost = zon.shape_costs(L, r)
    np.testing.assert_allclose(cost[0], np.array([401.25, 617.25, 443.25]) / 255, rtol=1e-14)
    np.testing.assert_allclose(cost[1], 1.75 * np.array([177.0, 333.0, 318.0]) / 255, rtol=1e-14)
    shape, _ = zon.choose_shapes(cost)
    assert shape.tolist() == [0, 0, 0]
    # each signal alone, and the unnormalised sum, choose differently
    rv = zon.zone_signal(V, G, nz, use_audio=False)
    np.testing.assert_allclose(rv[0], [2.0, 0.0, 0.25], rtol=1e-15)
    assert zon.choose_shapes(zon.shape_costs(L, rv))[0][0] == 2
    ra = zon.zone_signal(np.zeros_like(V), G, nz, use_audio=True)
    np.testing.assert_allclose(ra[0], [0.0, 4.0, 0.5], rtol=1e-15)
    assert zon.choose_shapes(zon.shape_costs(L, ra))[0][0] == 1
    assert zon.choose_shapes(zon.shape_costs(L, V + G))[0][0] == 2
