"""Pins of the oracle's layout: permutation, padding and block boxes.

The rules pinned here are the readings stated in oracle/layout.py (token order
raster, t slowest; zones raster; blocks raster inside a zone; tokens raster
inside a block; pad to the zone extent). Each test checks them against an
independent brute-force construction or hand-counted sizes.
"""
import numpy as np
import pytest

from oracle import layout as lay

CASES = [
    ((3, 8, 8), "fixed", (1, 8, 8)),
    ((13, 45, 80), "fixed", (2, 8, 8)),
    ((5, 20, 36), "dynamic", (4, 16, 16)),     # ragged on every axis
    ((4, 16, 16), "dynamic", (4, 16, 16)),     # exactly one zone
    ((1, 3, 5), "dynamic", (4, 16, 16)),       # mostly padding
]


def _shapes_for(L, seed):
    rng = np.random.default_rng(seed)
    return rng.integers(0, len(L.shapes), size=L.n_zones).astype(np.int32)


@pytest.mark.parametrize("grid,mode,block", CASES)
def test_permute_unpermute_identity(grid, mode, block):
    L = lay.make_layout(grid, mode, block)
    zs = _shapes_for(L, 7)
    perm = lay.permutation(L, zs)
    rng = np.random.default_rng(0)
    x = rng.standard_normal((2, L.n_tokens, 4)).astype(np.float32)
    xp = lay.permute(x, perm)
    assert xp.shape == (2, L.n_padded, 4)
    assert np.array_equal(lay.unpermute(xp, perm, L.n_tokens), x)      # bitwise
    assert np.all(xp[:, perm < 0] == 0)                                # pad slots zero


@pytest.mark.parametrize("grid,mode,block", CASES)
def test_real_slots_are_a_bijection(grid, mode, block):
    L = lay.make_layout(grid, mode, block)
    perm = lay.permutation(L, _shapes_for(L, 3))
    real = perm[perm >= 0]
    assert real.size == L.n_tokens
    assert np.array_equal(np.sort(real), np.arange(L.n_tokens))


def _brute_force_perm(L, zone_shape):
    """Independent construction: visit every padded grid point, compute its
    (zone, block, position) by integer division, and place it."""
    T, H, W = L.grid
    PT, PH, PW = L.padded
    zt, zh, zw = L.zone
    gz_h, gz_w = PH // zh, PW // zw
    B = L.block_tokens
    perm = np.full(L.n_padded, -2, dtype=np.int64)
    for t in range(PT):
        for h in range(PH):
            for w in range(PW):
                z = ((t // zt) * gz_h + h // zh) * gz_w + w // zw
                bt, bh, bw = L.shapes[zone_shape[z]]
                rt, rh, rw = t % zt, h % zh, w % zw            # offset in zone
                local = ((rt // bt) * (zh // bh) + rh // bh) * (zw // bw) + rw // bw
                pos = ((rt % bt) * bh + rh % bh) * bw + rw % bw
                slot = (z * L.blocks_per_zone + local) * B + pos
                assert perm[slot] == -2
                perm[slot] = (t * H + h) * W + w if (t < T and h < H and w < W) else -1
    return perm


@pytest.mark.parametrize("grid,mode,block", CASES[:1] + CASES[2:])
def test_matches_brute_force_box_construction(grid, mode, block):
    L = lay.make_layout(grid, mode, block)
    for seed in range(3):
        zs = _shapes_for(L, seed)
        assert np.array_equal(lay.permutation(L, zs), _brute_force_perm(L, zs))


def test_block_real_tokens_form_their_box():
    L = lay.make_layout((5, 20, 36), "dynamic", (4, 16, 16))
    zs = _shapes_for(L, 11)
    perm = lay.permutation(L, zs)
    T, H, W = L.grid
    for b in range(L.n_blocks):
        t0, h0, w0, bt, bh, bw = lay.block_box(L, zs, b)
        want = sorted((t * H + h) * W + w
                      for t in range(t0, min(t0 + bt, T))
                      for h in range(h0, min(h0 + bh, H))
                      for w in range(w0, min(w0 + bw, W)))
        got = perm[b * L.block_tokens:(b + 1) * L.block_tokens]
        assert sorted(got[got >= 0].tolist()) == want


def test_sizes_of_the_measured_workloads():
    """Hand counts. 720p fixed 2x8x8: 13x45x80 pads to 14x48x80, blocks
    7*6*10 = 420, all non-empty. 720p dynamic: pads to 16x48x80, 4*3*5 = 60
    zones of 8 blocks = 480 blocks. Non-empty blocks with one shape everywhere:
    per axis, the number of non-empty blocks in a zone is ceil(real extent / b)
    with real extents t: 4,4,4,1; h: 16,16,13; w: 16 (x5):
      2x8x8  -> (2+2+2+1)*(2+2+2)*(2*5) = 7*6*10 = 420
      4x4x8  -> (1+1+1+1)*(4+4+4)*(2*5) = 4*12*10 = 480
      1x8x16 -> (4+4+4+1)*(2+2+2)*(1*5) = 13*6*5 = 390."""
    L = lay.make_layout((13, 45, 80), "fixed", (2, 8, 8))
    assert (L.n_tokens, L.padded, L.n_blocks, L.n_padded) == (46800, (14, 48, 80), 420, 53760)
    c = lay.block_counts(L, lay.permutation(L, np.zeros(L.n_zones, np.int32)))
    assert (c > 0).sum() == 420 and c.sum() == 46800
    L = lay.make_layout((13, 45, 80), "dynamic", (4, 16, 16))
    assert (L.n_zones, L.n_blocks, L.n_padded) == (60, 480, 61440)
    for sid, want in [(0, 420), (1, 480), (2, 390)]:
        c = lay.block_counts(L, lay.permutation(L, np.full(L.n_zones, sid, np.int32)))
        assert (c > 0).sum() == want and c.sum() == 46800
    # 1080p: 13x68x120 pads to 16x80x128: 4*5*8 = 160 zones, 1280 blocks
    L = lay.make_layout((13, 68, 120), "dynamic", (4, 16, 16))
    assert (L.n_zones, L.n_blocks, L.n_padded) == (160, 1280, 163840)
    # 2K: 13x90x160 pads to 16x96x160: 4*6*10 = 240 zones, 1920 blocks
    L = lay.make_layout((13, 90, 160), "dynamic", (4, 16, 16))
    assert (L.n_zones, L.n_blocks, L.n_padded) == (240, 1920, 245760)


def test_tiny_fixed_layout_is_frame_blocks():
    """3x8x8 with 1x8x8 blocks: block t is exactly frame t, raster inside."""
    L = lay.make_layout((3, 8, 8), "fixed", (1, 8, 8))
    perm = lay.permutation(L, np.zeros(L.n_zones, np.int32))
    assert np.array_equal(perm, np.arange(192))


def test_shape_must_tile_zone():
    with pytest.raises(ValueError):
        lay.make_layout((4, 16, 16), "dynamic", (4, 16, 16), candidates=((3, 8, 8),))
