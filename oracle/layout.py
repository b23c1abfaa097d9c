"""Token -> macro-zone -> shaped-block layout (oracle).

[Prism §Blocks] partitions the latent tokens into spatio-temporal macro-zones
and gives every zone its own block shape, so that tokens inside one block are
semantically close. The page fixes neither the token order, the padding, nor
the order of blocks. Readings taken here:

- Token order: Q/K/V are [heads, tokens, d] with raster token id
  n = (t*H + h)*W + w (t slowest).
- Padding: every axis is padded up to a multiple of the zone extent (in fixed
  mode the zone is the block itself). A slot is real iff t<T, h<H and w<W.
  Pad slots carry zeros and are never attended to.
- Order: zones in raster order over the zone grid; inside a zone, blocks in
  raster order over its (zt/bt, zh/bh, zw/bw) sub-grid; inside a block, tokens
  in raster order. Block id = zone * blocks_per_zone + local block.
- Candidate block shapes (dynamic mode), canonical order and shape ids:
  0 = 2x8x8, 1 = 4x4x8, 2 = 1x8x16, each 128 tokens, zone 4x16x16.
"""
from __future__ import annotations

import dataclasses

import numpy as np

CANDIDATES = ((2, 8, 8), (4, 4, 8), (1, 8, 16))
ZONE = (4, 16, 16)


@dataclasses.dataclass(frozen=True)
class Layout:
    grid: tuple      # (T, H, W) latent grid
    zone: tuple      # zone extent (zt, zh, zw); equals the block in fixed mode
    shapes: tuple    # candidate block shapes; shape id = index

    @property
    def n_tokens(self) -> int:
        return int(np.prod(self.grid))

    @property
    def padded(self) -> tuple:
        return tuple(-(-g // z) * z for g, z in zip(self.grid, self.zone))

    @property
    def zone_grid(self) -> tuple:
        return tuple(p // z for p, z in zip(self.padded, self.zone))

    @property
    def n_zones(self) -> int:
        return int(np.prod(self.zone_grid))

    @property
    def block_tokens(self) -> int:
        return int(np.prod(self.shapes[0]))

    @property
    def blocks_per_zone(self) -> int:
        return int(np.prod(self.zone)) // self.block_tokens

    @property
    def n_blocks(self) -> int:
        return self.n_zones * self.blocks_per_zone

    @property
    def n_padded(self) -> int:
        return self.n_blocks * self.block_tokens


def make_layout(grid, mode: str, block, candidates=CANDIDATES) -> Layout:
    """Fixed mode: ``block`` is the one block shape (and the zone).
    Dynamic mode: ``block`` is the zone extent and ``candidates`` the shapes."""
    grid = tuple(int(g) for g in grid)
    block = tuple(int(b) for b in block)
    if mode == "fixed":
        L = Layout(grid, block, (block,))
    elif mode == "dynamic":
        L = Layout(grid, block, tuple(tuple(c) for c in candidates))
    else:
        raise ValueError(mode)
    for s in L.shapes:
        if any(z % b for z, b in zip(L.zone, s)):
            raise ValueError(f"shape {s} does not tile zone {L.zone}")
        if int(np.prod(s)) != L.block_tokens:
            raise ValueError("candidate shapes must hold equally many tokens")
    return L


def zone_origin(L: Layout, z: int) -> tuple:
    """Grid coordinates of the first token of zone z (zones raster-ordered)."""
    gt, gh, gw = L.zone_grid
    zt, zh, zw = L.zone
    return ((z // (gh * gw)) * zt, ((z // gw) % gh) * zh, (z % gw) * zw)


def block_box(L: Layout, zone_shape, b: int) -> tuple:
    """(t0, h0, w0, bt, bh, bw) of block b: its box in the padded grid."""
    bpz = L.blocks_per_zone
    z, local = divmod(b, bpz)
    bt, bh, bw = L.shapes[int(zone_shape[z])]
    zt, zh, zw = L.zone
    nh, nw = zh // bh, zw // bw
    lt, lh, lw = local // (nh * nw), (local // nw) % nh, local % nw
    t0, h0, w0 = zone_origin(L, z)
    return (t0 + lt * bt, h0 + lh * bh, w0 + lw * bw, bt, bh, bw)


def permutation(L: Layout, zone_shape) -> np.ndarray:
    """perm[p] = raster id of slot p, or -1 for a pad slot. int64 [Np]."""
    T, H, W = L.grid
    B = L.block_tokens
    perm = np.empty(L.n_padded, dtype=np.int64)
    for b in range(L.n_blocks):
        t0, h0, w0, bt, bh, bw = block_box(L, zone_shape, b)
        t, h, w = np.meshgrid(np.arange(t0, t0 + bt), np.arange(h0, h0 + bh),
                              np.arange(w0, w0 + bw), indexing="ij")
        t, h, w = t.ravel(), h.ravel(), w.ravel()   # raster order inside the block
        real = (t < T) & (h < H) & (w < W)
        perm[b * B:(b + 1) * B] = np.where(real, (t * H + h) * W + w, -1)
    return perm


def inverse(perm: np.ndarray, n_tokens: int) -> np.ndarray:
    """inv[n] = slot of raster id n."""
    inv = np.full(n_tokens, -1, dtype=np.int64)
    slots = np.nonzero(perm >= 0)[0]
    inv[perm[slots]] = slots
    return inv


def block_counts(L: Layout, perm: np.ndarray) -> np.ndarray:
    """c_b: number of real tokens in each block."""
    return (perm.reshape(L.n_blocks, L.block_tokens) >= 0).sum(axis=1)


def permute(x: np.ndarray, perm: np.ndarray) -> np.ndarray:
    """[H, N, d] -> [H, Np, d]; pad slots are zero."""
    out = np.zeros((x.shape[0], perm.shape[0]) + x.shape[2:], dtype=x.dtype)
    real = perm >= 0
    out[:, real] = x[:, perm[real]]
    return out


def unpermute(xp: np.ndarray, perm: np.ndarray, n_tokens: int) -> np.ndarray:
    """[H, Np, d] -> [H, N, d]; reads real slots only."""
    return xp[:, inverse(perm, n_tokens)]
