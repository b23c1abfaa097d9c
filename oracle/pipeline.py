"""The whole selection side of the path, chained in the order it runs (oracle).

zone scoring (dynamic mode) -> permutation -> block-mean pooling -> hybrid
selection. Attention is evaluated separately (``oracle.attention``) because
its cost is what the tests sample.
"""
from __future__ import annotations

import numpy as np

from . import layout as lay
from . import select as sel
from . import zones as zon


def run_selection(grid, mode, block, q, k, sparsity_1e4, tau, video=None, audio=None,
                  zone_shape=None):
    """q, k: [H, N, d] float arrays (raster). video [N, C], audio [Na, C] or None.

    ``zone_shape`` forces the shapes (skips scoring). Returns a dict with the
    layout, shapes, permutation, block counts, pooled features and lists."""
    L = lay.make_layout(grid, mode, block)
    out = {"layout": L}
    if zone_shape is None:
        if mode == "dynamic" and video is not None:
            X = np.asarray(video, dtype=np.float64)
            A = None if audio is None else np.asarray(audio, dtype=np.float64)
            zone_shape, V, G, cost, gap = zon.score_zones(L, X, A)
            out.update(V=V, G=G, cost=cost, gap=gap)
        else:
            zone_shape = np.zeros(L.n_zones, dtype=np.int32)
    zone_shape = np.asarray(zone_shape, dtype=np.int32)
    perm = lay.permutation(L, zone_shape)
    counts = lay.block_counts(L, perm)
    qbar = sel.pool(L, lay.permute(q, perm), perm)
    kbar = sel.pool(L, lay.permute(k, perm), perm)
    lists, n, m, kk = sel.select(L, qbar, kbar, counts, sparsity_1e4, tau)
    out.update(zone_shape=zone_shape, perm=perm, counts=counts, qbar=qbar, kbar=kbar,
               lists=lists, n=n, m=m, k=kk)
    return out
