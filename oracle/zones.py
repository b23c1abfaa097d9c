"""Per-zone scoring and block-shape choice (oracle, dynamic mode only).

[Prism §Blocks]: in every macro-zone the method computes (i) the channel-wise
variance of the video features, telling in which direction and how fast the
content changes, and (ii) the feature norm of the audio-to-video (A2V)
cross-attention, telling how strongly audio drives that region. Both signals
together set the zone's block shape; axes with fast video change or strong
audio-video coupling are split more finely.

The page gives no formula. Readings taken here (parity against Prism's own
code is unpinned for all of them):

1. A2V feature: one head, identity projections, scale 1/sqrt(C):
   p_n = softmax_j(X_n . A_j / sqrt(C)) over the audio tokens,
   F_n = sum_j p_nj A_j, g_n = ||F_n||_2 (equivalently g_n^2 = p_n^T (A A^T) p_n).
2. Per axis a in (t, h, w) of zone z, a *line* is the set of the zone's real
   tokens sharing the other two coordinates;
   V_a(z) = sum_lines sum_{n in line} ||X_n - mean_line X||^2 / (C n_z),
   G_a(z) = sum_lines sum_{n in line} (g_n - mean_line g)^2 / n_z,
   with n_z the zone's real-token count (V = G = 0 for an all-pad zone).
3. r_a(z) = V_a(z)/Vbar + G_a(z)/Gbar, Vbar and Gbar the means over all
   (non-empty zone, axis) pairs; a term whose mean is 0, or the A2V term when
   there is no audio, is dropped. Equal weights: the page says both signals are
   used together.
4. Shape: argmin over candidates B of cost(z,B) = sum_a r_a(z) (b_a^2-1)/(Z_a^2-1),
   Z the zone extent. For a locally linear field of slope s along an axis, a
   run of length L has variance s^2 (L^2-1)/12, so (b^2-1)/(Z^2-1) converts a
   zone-line variance into the expected within-block variance: the chosen
   shape is the one whose blocks are predicted to be most homogeneous, i.e.
   it is finest along the axes that vary most.
   Ties: every candidate within a relative 1e-6 of the lowest cost is tied and
   the first of them in canonical order (2x8x8, 4x4x8, 1x8x16) wins.
"""
from __future__ import annotations

import numpy as np

from .layout import Layout, zone_origin

TIE_REL = 1e-6


def softmax_rows(x: np.ndarray) -> np.ndarray:
    m = x.max(axis=-1, keepdims=True)
    e = np.exp(x - m)
    return e / e.sum(axis=-1, keepdims=True)


def a2v_norm(X: np.ndarray, A: np.ndarray) -> np.ndarray:
    """g_n = || sum_j softmax_j(X_n.A_j/sqrt(C)) A_j ||, formed through F."""
    C = X.shape[1]
    p = softmax_rows(X @ A.T / np.sqrt(C))
    F = p @ A
    return np.sqrt((F * F).sum(axis=1))


def a2v_norm_gram(X: np.ndarray, A: np.ndarray) -> np.ndarray:
    """The same g_n through the Gram matrix: g_n^2 = p_n^T (A A^T) p_n."""
    C = X.shape[1]
    p = softmax_rows(X @ A.T / np.sqrt(C))
    gram = A @ A.T
    return np.sqrt(np.einsum("nj,jk,nk->n", p, gram, p))


def _line_sq_dev(box: np.ndarray, axis: int) -> float:
    """Sum over lines along ``axis`` of squared deviations from the line mean."""
    dev = box - box.mean(axis=axis, keepdims=True)
    return float((dev * dev).sum())


def zone_stats(L: Layout, X: np.ndarray, g: np.ndarray | None):
    """V [nZ,3], G [nZ,3] (zeros when g is None), n_z [nZ].

    X is [N, C] video features in raster order, g is [N] or None.
    """
    T, H, W = L.grid
    C = X.shape[1]
    Xg = X.reshape(T, H, W, C)
    gg = None if g is None else g.reshape(T, H, W)
    nZ = L.n_zones
    V = np.zeros((nZ, 3))
    G = np.zeros((nZ, 3))
    nz = np.zeros(nZ, dtype=np.int64)
    zt, zh, zw = L.zone
    for z in range(nZ):
        t0, h0, w0 = zone_origin(L, z)
        t1, h1, w1 = min(t0 + zt, T), min(h0 + zh, H), min(w0 + zw, W)
        if t1 <= t0 or h1 <= h0 or w1 <= w0:
            continue                      # all-pad zone
        box = Xg[t0:t1, h0:h1, w0:w1, :]
        n = box.shape[0] * box.shape[1] * box.shape[2]
        nz[z] = n
        for a in range(3):
            V[z, a] = _line_sq_dev(box, a) / (C * n)
        if gg is not None:
            gb = gg[t0:t1, h0:h1, w0:w1]
            for a in range(3):
                G[z, a] = _line_sq_dev(gb, a) / n
    return V, G, nz


def zone_signal(V: np.ndarray, G: np.ndarray, nz: np.ndarray, use_audio: bool) -> np.ndarray:
    """r_a(z): each signal divided by its mean over non-empty (zone, axis) pairs."""
    ne = nz > 0
    r = np.zeros_like(V)
    if ne.any():
        vbar = V[ne].mean()
        if vbar > 0:
            r += V / vbar
        if use_audio:
            gbar = G[ne].mean()
            if gbar > 0:
                r += G / gbar
    return r


def shape_factors(L: Layout) -> np.ndarray:
    """f[s, a] = (b_a^2 - 1) / (Z_a^2 - 1) (0 where the zone extent is 1)."""
    f = np.zeros((len(L.shapes), 3))
    for s, shp in enumerate(L.shapes):
        for a in range(3):
            Z = L.zone[a]
            f[s, a] = 0.0 if Z == 1 else (shp[a] ** 2 - 1) / (Z ** 2 - 1)
    return f


def shape_costs(L: Layout, r: np.ndarray) -> np.ndarray:
    """cost[z, s] = sum_a r_a(z) f[s, a]."""
    return r @ shape_factors(L).T


def choose_shapes(cost: np.ndarray, tie_rel: float = TIE_REL):
    """Shape id per zone, and each zone's gap (c2 - c1)/c1 between its two lowest
    costs (0 for an exact tie, inf when c1 = 0 < c2).

    Candidates within ``tie_rel`` (relative) of the minimum are tied; the first
    of them in canonical order wins. The gap is reported so that callers can
    flag near-ties (gap 0 for an exact tie)."""
    nZ, nS = cost.shape
    shape = np.zeros(nZ, dtype=np.int32)
    gap = np.full(nZ, np.inf)
    for z in range(nZ):
        c = cost[z]
        cmin = c.min()
        tied = [s for s in range(nS) if c[s] <= cmin + tie_rel * cmin]
        shape[z] = tied[0]
        if nS > 1:
            c1, c2 = np.sort(c)[:2]
            gap[z] = 0.0 if c2 == c1 else ((c2 - c1) / c1 if c1 > 0 else np.inf)
    return shape, gap


def score_zones(L: Layout, X: np.ndarray, A: np.ndarray | None):
    """Whole zone-scoring step: (shape ids, V, G, cost, gap)."""
    g = None if A is None else a2v_norm(X, A)
    V, G, nz = zone_stats(L, X, g)
    r = zone_signal(V, G, nz, A is not None)
    cost = shape_costs(L, r)
    shape, gap = choose_shapes(cost)
    return shape, V, G, cost, gap
