"""Pins of the oracle's pooling and hybrid selection (oracle/select.py).

Hand-worked rows (tests/golden/select_rows.json), brute force over all subsets
for small rows, the invariants of the top-k U CDF-prefix set, and pooling
special cases.
"""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import layout as lay
from oracle import select as sel

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "select_rows.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


@pytest.mark.parametrize("row", _golden()["rows"], ids=lambda r: r["why"][:40])
def test_hand_worked_rows(row):
    lst, n, m, _ = sel.select_row(np.array(row["logits"]), np.array(row["ids"]),
                                  row["k"], row["tau"])
    assert lst.tolist() == row["expect"]


@pytest.mark.parametrize("mv,S,k", _golden()["topk"]["cases"])
def test_top_k_size_hand_values(mv, S, k):
    assert sel.top_k_size(mv, S) == k


def _brute_force(p, k, tau):
    """Enumerate every subset: the top-k set is the size-k subset of largest
    mass; the CDF set is, for the smallest size m whose best subset reaches
    tau, that best subset. Returns their union (sorted)."""
    idx = range(len(p))

    def best(r):
        return max(itertools.combinations(idx, r), key=lambda c: (sum(p[j] for j in c), [-j for j in c]))

    topk = set(best(k))
    for r in range(1, len(p) + 1):
        b = best(r)
        if sum(p[j] for j in b) >= tau:
            return sorted(topk | set(b))
    return sorted(idx)


@pytest.mark.parametrize("seed", range(40))
def test_brute_force_subsets(seed):
    rng = np.random.default_rng(seed)
    M = int(rng.integers(2, 11))
    spread = [0.05, 0.5, 2.0][seed % 3]          # flat rows exercise the CDF branch
    logits = rng.standard_normal(M) * spread
    k = int(rng.integers(1, M + 1))
    tau = float(rng.choice([0.2, 0.35, 0.6, 0.9]))
    p = np.exp(logits - logits.max())
    p /= p.sum()
    lst, n, m, _ = sel.select_row(logits, np.arange(M), k, tau)
    assert lst.tolist() == _brute_force(p, k, tau)


@pytest.mark.parametrize("seed", range(20))
def test_selected_set_invariants(seed):
    rng = np.random.default_rng(100 + seed)
    M = 300
    logits = rng.standard_normal(M) * [0.02, 0.3, 3.0][seed % 3]
    ids = np.arange(M) * 2 + 1                     # arbitrary block ids
    for S in (7500, 8000, 8500, 9300):
        k = sel.top_k_size(M, S)
        lst, n, m, _ = sel.select_row(logits, ids, k, 0.2)
        p = np.exp(logits - logits.max())
        p /= p.sum()
        rank = np.argsort(-logits, kind="stable")
        mass = dict(zip(ids, p))
        assert len(lst) == max(k, m) == n
        assert set(ids[rank[:k]]) <= set(lst.tolist())             # contains its top-k
        assert sum(mass[j] for j in lst) >= 0.2 - 1e-12            # reaches tau
        if n > k:                                                  # CDF prefix is minimal
            assert p[rank[:n - 1]].sum() < 0.2
        assert np.all(np.diff(lst) > 0)                            # ascending, unique


def _workload(grid, mode, block, H=2, d=16, seed=0):
    L = lay.make_layout(grid, mode, block)
    rng = np.random.default_rng(seed)
    zs = rng.integers(0, len(L.shapes), L.n_zones).astype(np.int32)
    perm = lay.permutation(L, zs)
    q = rng.standard_normal((H, L.n_tokens, d))
    k = rng.standard_normal((H, L.n_tokens, d))
    return L, zs, perm, q, k


def test_sparsity_zero_selects_every_nonempty_block():
    L, zs, perm, q, k = _workload((5, 20, 36), "dynamic", (4, 16, 16))
    counts = lay.block_counts(L, perm)
    qb = sel.pool(L, lay.permute(q, perm), perm)
    kb = sel.pool(L, lay.permute(k, perm), perm)
    lists, n, m, kk = sel.select(L, qb, kb, counts, 0, 0.2)
    ne = np.nonzero(counts > 0)[0]
    assert kk == len(ne)
    for h in range(q.shape[0]):
        for i in range(L.n_blocks):
            want = ne if counts[i] > 0 else np.zeros(0, int)
            assert np.array_equal(lists[h][i], want)


def test_empty_blocks_never_selected_and_have_empty_lists():
    L, zs, perm, q, k = _workload((5, 20, 36), "dynamic", (4, 16, 16), seed=4)
    counts = lay.block_counts(L, perm)
    assert (counts == 0).any()
    qb = sel.pool(L, lay.permute(q, perm), perm)
    kb = sel.pool(L, lay.permute(k, perm), perm)
    lists, n, m, kk = sel.select(L, qb, kb, counts, 9300, 0.2)
    empty = set(np.nonzero(counts == 0)[0].tolist())
    for h in range(q.shape[0]):
        for i in range(L.n_blocks):
            assert not (set(lists[h][i].tolist()) & empty)
            if counts[i] == 0:
                assert lists[h][i].size == 0 and n[h, i] == 0


def test_pool_is_the_mean_of_real_tokens():
    """Brute force: average the raster tokens of each block box by hand."""
    L, zs, perm, q, k = _workload((5, 20, 36), "dynamic", (4, 16, 16), seed=2)
    qb = sel.pool(L, lay.permute(q, perm), perm)
    T, H, W = L.grid
    for b in range(L.n_blocks):
        t0, h0, w0, bt, bh, bw = lay.block_box(L, zs, b)
        ids = [(t * H + h) * W + w for t in range(t0, min(t0 + bt, T))
               for h in range(h0, min(h0 + bh, H)) for w in range(w0, min(w0 + bw, W))]
        want = q[:, ids].mean(axis=1) if ids else np.zeros((q.shape[0], q.shape[2]))
        np.testing.assert_allclose(qb[:, b], want, rtol=1e-13, atol=1e-14)


def test_pool_constant_and_linear():
    L, zs, perm, q, k = _workload((4, 16, 16), "dynamic", (4, 16, 16))
    c = np.full_like(q, 3.25)
    assert np.all(sel.pool(L, lay.permute(c, perm), perm) == 3.25)
    a = sel.pool(L, lay.permute(2 * q - k, perm), perm)
    b = 2 * sel.pool(L, lay.permute(q, perm), perm) - sel.pool(L, lay.permute(k, perm), perm)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


def test_flat_rows_take_more_than_k_blocks():
    """At s = 0.93 with M_v = 100 (k = 7), a row of near-equal pooled logits
    holds about 7% of the mass in its top-7, so the CDF prefix (tau = 0.2)
    must extend the list to about 20 blocks."""
    logits = np.linspace(0.0, 0.01, 100)
    lst, n, m, _ = sel.select_row(logits, np.arange(100), sel.top_k_size(100, 9300), 0.2)
    assert n == m and 19 <= n <= 21


def test_block_mask_rows_by_brute_force():
    """The one-block mask row against a per-token walk over the permutation
    (slot p of block b holds raster token perm[p]): on a ragged dynamic grid
    with forced shapes, key token m is allowed for block i exactly when the
    slot holding m lies in a block of i's list."""
    L = lay.make_layout((5, 20, 36), "dynamic", (4, 16, 16))
    rng = np.random.default_rng(3)
    zs = rng.integers(0, len(L.shapes), L.n_zones).astype(np.int32)
    perm = lay.permutation(L, zs)
    B = L.block_tokens
    for _ in range(5):
        lst = np.sort(rng.choice(L.n_blocks, 7, replace=False))
        row = sel.block_mask_rows(L, lst, perm)
        want = np.zeros(L.n_tokens, dtype=bool)
        for p in range(L.n_padded):
            if perm[p] >= 0 and (p // B) in set(lst.tolist()):
                want[perm[p]] = True
        assert np.array_equal(row, want)
