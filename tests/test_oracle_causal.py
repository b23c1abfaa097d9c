"""Pins of the frame-chunk causal selection oracle (oracle/causal.py).

Each check is independent of the function's own arithmetic: the reduction to
the non-causal selection (every block visible), hand-counted visible sets and
top-k sizes, and a token-level brute force of the mask built from the
permutation (frames of the real tokens), not from block boxes."""
import numpy as np
import pytest

import synth
from oracle import causal as ocau
from oracle import layout as olay
from oracle import select as osel


def _case(grid, mode, block, seed=7, H=2, d=64):
    L = olay.make_layout(grid, mode, block)
    rng = np.random.default_rng(seed)
    zs = rng.integers(0, len(L.shapes), L.n_zones).astype(np.int32)
    perm = olay.permutation(L, zs)
    counts = olay.block_counts(L, perm)
    q = synth.smooth_field(H, grid, d, 1)
    k = synth.smooth_field(H, grid, d, 2)
    qbar = osel.pool(L, olay.permute(synth.bf16_bits_to_f64(q), perm), perm)
    kbar = osel.pool(L, olay.permute(synth.bf16_bits_to_f64(k), perm), perm)
    return L, zs, perm, counts, qbar, kbar


CASES = [((8, 16, 16), "fixed", (2, 8, 8)), ((13, 20, 36), "dynamic", (4, 16, 16)),
         ((9, 16, 32), "dynamic", (4, 16, 16))]


@pytest.mark.parametrize("grid,mode,block", CASES)
def test_all_frames_in_one_chunk_is_the_plain_selection(grid, mode, block):
    L, zs, perm, counts, qbar, kbar = _case(grid, mode, block)
    F = L.padded[0]
    lists, n, m, k = ocau.select_causal(L, zs, qbar, kbar, counts, 8500, 0.2, F)
    lists0, n0, m0, k0 = osel.select(L, qbar, kbar, counts, 8500, 0.2)
    assert all(np.array_equal(a, b) for ra, rb in zip(lists, lists0) for a, b in zip(ra, rb))
    assert np.array_equal(n, n0) and np.array_equal(m, m0)
    assert np.all(k[counts > 0] == k0)


@pytest.mark.parametrize("grid,mode,block", CASES)
def test_last_chunk_rows_equal_the_plain_selection(grid, mode, block):
    L, zs, perm, counts, qbar, kbar = _case(grid, mode, block)
    F = L.zone[0]
    ch = ocau.block_chunks(L, zs, F)
    lists, n, m, k = ocau.select_causal(L, zs, qbar, kbar, counts, 8000, 0.2, F)
    lists0, n0, m0, _ = osel.select(L, qbar, kbar, counts, 8000, 0.2)
    last = ch == ch[counts > 0].max()
    for h in range(qbar.shape[0]):
        for i in np.nonzero(last & (counts > 0))[0]:
            assert np.array_equal(lists[h][i], lists0[h][i])


def _token_frames_of_blocks(L, perm):
    """(min frame, max frame) of each block's real tokens, from the permutation."""
    B = L.block_tokens
    T, Hh, W = L.grid
    fr = np.where(perm >= 0, perm // (Hh * W), -1).reshape(L.n_blocks, B)
    lo = np.array([r[r >= 0].min() if (r >= 0).any() else -1 for r in fr])
    hi = np.array([r[r >= 0].max() if (r >= 0).any() else -1 for r in fr])
    return lo, hi


@pytest.mark.parametrize("grid,mode,block", CASES)
@pytest.mark.parametrize("mult", [1, 2])
def test_no_token_attends_to_a_later_chunk(grid, mode, block, mult):
    L, zs, perm, counts, qbar, kbar = _case(grid, mode, block)
    F = mult * L.zone[0]
    lists, n, m, k = ocau.select_causal(L, zs, qbar, kbar, counts, 7500, 0.2, F)
    frame = np.arange(L.n_tokens) // (L.grid[1] * L.grid[2])
    for h in range(qbar.shape[0]):
        mask = osel.block_mask(L, lists, h, perm)        # [N, N] raster order
        qn, kn = np.nonzero(mask)
        assert np.all(frame[kn] // F <= frame[qn] // F)
    # every block's real tokens sit in one chunk
    lo, hi = _token_frames_of_blocks(L, perm)
    ne = counts > 0
    assert np.all(lo[ne] // F == hi[ne] // F)


@pytest.mark.parametrize("grid,mode,block", CASES)
def test_visible_counts_from_token_frames(grid, mode, block):
    L, zs, perm, counts, qbar, kbar = _case(grid, mode, block)
    F = L.zone[0]
    lo, _ = _token_frames_of_blocks(L, perm)
    ne = counts > 0
    vis = ocau.visible(L, zs, counts, F)
    for i in np.nonzero(ne)[0]:
        want = np.nonzero(ne & (lo // F <= lo[i] // F))[0]
        assert np.array_equal(np.nonzero(vis[i])[0], want)


def test_hand_counted_sizes_fixed_grid():
    # 8 x 16 x 16 with 2x8x8 blocks: 4 block rows in time, 4 blocks per row; F = 2
    # puts block row c in chunk c, so a row of chunk c sees V = 4 (c + 1) blocks and
    # k = ceil(V (1 - s)): s = 0.75 -> 1, 2, 3, 4
    L, zs, perm, counts, qbar, kbar = _case((8, 16, 16), "fixed", (2, 8, 8))
    assert L.n_blocks == 16 and np.all(counts == 128)
    lists, n, m, k = ocau.select_causal(L, zs, qbar, kbar, counts, 7500, 0.2, 2)
    assert k.tolist() == [1] * 4 + [2] * 4 + [3] * 4 + [4] * 4
    assert np.all(n >= k[None, :])
    for h in range(2):
        for i in range(4):                                 # first chunk: blocks 0..3 only
            assert set(lists[h][i].tolist()) <= {0, 1, 2, 3}
        for i in range(16):
            assert lists[h][i].max() < 4 * (i // 4 + 1)
            assert np.all(np.diff(lists[h][i]) > 0)


def test_single_visible_block_gives_that_block():
    # a 1 x 8 x 16 shape per zone and F = 4: the first zone-row's blocks see only
    # the first chunk; with one zone in h and w and one frame, chunk 0 holds the
    # 8 blocks of zone 0, of which only the first (frame 0, 8 x 16 tokens) is real
    L = olay.make_layout((1, 8, 16), "dynamic", (4, 16, 16))
    zs = np.array([2], dtype=np.int32)
    perm = olay.permutation(L, zs)
    counts = olay.block_counts(L, perm)
    assert counts.tolist() == [128] + [0] * 7
    rng = np.random.default_rng(0)
    qbar = rng.normal(size=(1, 8, 64))
    kbar = rng.normal(size=(1, 8, 64))
    lists, n, m, k = ocau.select_causal(L, zs, qbar, kbar, counts, 9900, 0.2, 4)
    assert lists[0][0].tolist() == [0] and k[0] == 1
    assert all(lists[0][i].size == 0 for i in range(1, 8))


def test_rejects_chunks_that_split_blocks():
    L = olay.make_layout((8, 16, 16), "dynamic", (4, 16, 16))
    zs = np.zeros(L.n_zones, dtype=np.int32)
    for F in (0, 2, 6):
        with pytest.raises(ValueError):
            ocau.block_chunks(L, zs, F)
