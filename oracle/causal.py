"""Frame-chunk causal block selection (oracle; test infrastructure, imported
only by tests and the benchmark's oracle timing).

[Post-training page (gist.science, paper 2604.25427, "A Systematic Post-Train
Framework for Video Generation"), section 2 (method), stage 4: autoregressive
distillation] distils the bidirectional model into a causal student that
generates frames conditioned on its own earlier output through a KV cache,
after a switch to a causal attention mask. The page gives no chunk size and no
mask formula; the readings taken here, on top of the hybrid selection of
``select`` ([Prism §Blocks]):

- Latent frames are grouped into chunks of F consecutive frames: frame t lies
  in chunk t // F.
- A block lies in the chunk of its first frame. F must be a multiple of the
  zone's time extent (in fixed mode: of the block's), so that no block spans
  two chunks and the mask is exact at block granularity.
- Query block i sees key block j iff chunk(j) <= chunk(i) (its own chunk in
  full, every earlier chunk, no later one).
- The hybrid selection runs over each row's visible non-empty key blocks:
  softmax over them, the same order, k_i = max(1, ceil(V_i (1 - s))) with V_i
  the number of those blocks, the CDF prefix m_i over them, and the list is
  the first max(k_i, m_i) of the order, ascending. With F at least the padded
  frame count every block is visible and this is ``select.select``.
"""
from __future__ import annotations

import numpy as np

from .layout import Layout, block_box
from .select import select_row, top_k_size


def block_chunks(L: Layout, zone_shape, frames_per_chunk: int) -> np.ndarray:
    """Chunk index of every block (its first frame // F). int64 [M]."""
    F = int(frames_per_chunk)
    if F < 1 or F % L.zone[0]:
        raise ValueError(f"frames per chunk {F} must be a positive multiple of {L.zone[0]}")
    return np.array([block_box(L, zone_shape, b)[0] // F for b in range(L.n_blocks)],
                    dtype=np.int64)


def visible(L: Layout, zone_shape, counts: np.ndarray, frames_per_chunk: int) -> np.ndarray:
    """vis[i, j]: key block j is a candidate of query block i (non-empty, chunk(j) <= chunk(i))."""
    ch = block_chunks(L, zone_shape, frames_per_chunk)
    return (ch[None, :] <= ch[:, None]) & (counts[None, :] > 0)


def select_causal(L: Layout, zone_shape, qbar: np.ndarray, kbar: np.ndarray,
                  counts: np.ndarray, sparsity_1e4: int, tau: float, frames_per_chunk: int):
    """Hybrid selection restricted to each row's visible blocks.

    Returns (lists, n [H, M], m [H, M], k [M]) as ``select.select`` does, with
    k per query block."""
    H, M, d = qbar.shape
    vis = visible(L, zone_shape, counts, frames_per_chunk)
    lists = [[np.zeros(0, dtype=np.int64) for _ in range(M)] for _ in range(H)]
    n = np.zeros((H, M), dtype=np.int64)
    m = np.zeros((H, M), dtype=np.int64)
    k = np.zeros(M, dtype=np.int64)
    scale = 1.0 / np.sqrt(d)
    for i in range(M):
        if counts[i] == 0:
            continue
        cand = np.nonzero(vis[i])[0]
        k[i] = top_k_size(len(cand), sparsity_1e4)
        for h in range(H):
            logits = (kbar[h, cand] @ qbar[h, i]) * scale
            lists[h][i], n[h, i], m[h, i], _ = select_row(logits, cand, int(k[i]), tau)
    return lists, n, m, k
