"""Block-mean pooling and hybrid block selection (oracle).

[Prism §Blocks] builds block-level features and selects key blocks per query
with a hybrid strategy that sets each query's sparsity dynamically; the
configuration examples are a sparsity of 0.75/0.80/0.85/0.93 and a CDF
threshold of 0.20 for the hybrid selection. The page gives no formula.
Readings taken here (parity against Prism's own code is unpinned):

- Block feature = mean of the block's real tokens (pad slots excluded), for Q
  and for K. Only non-empty blocks are candidates.
- Pooled logits l_ij = qbar_i . kbar_j / sqrt(d); Pbar_ij = softmax_j(l_ij) over
  the M_v non-empty key blocks. No block-size correction.
- Order pi_i: candidates by l descending, ties to the lower block id.
- Sparsity is the skipped fraction: k = max(1, ceil(M_v (1 - s))) computed in
  integers with S = round(1e4 s): k = max(1, (M_v (10000 - S) + 9999) // 10000).
- CDF size m = smallest m >= 1 with sum_{r<=m} Pbar_{i,pi_i(r)} >= tau
  (M_v if the rounded sum never reaches tau).
- Hybrid set = top-k U CDF-prefix. Both are prefixes of pi_i, so the union is
  the first n_i = max(k, m) entries of pi_i.
- Granularity is the query block (one list per (head, query block)); an empty
  query block gets an empty list; no block is forced in (no diagonal rule).
- Emitted list: the n_i block ids in ascending order.
"""
from __future__ import annotations

import numpy as np

from .layout import Layout


def pool(L: Layout, xp: np.ndarray, perm: np.ndarray) -> np.ndarray:
    """Block means over real tokens: [H, Np, d] (permuted) -> [H, M, d] fp64.
    Empty blocks get zeros."""
    H, Np, d = xp.shape
    B = L.block_tokens
    real = (perm >= 0).reshape(L.n_blocks, B)
    x = xp.astype(np.float64).reshape(H, L.n_blocks, B, d)
    s = (x * real[None, :, :, None]).sum(axis=2)
    c = real.sum(axis=1)
    out = np.zeros_like(s)
    ne = c > 0
    out[:, ne] = s[:, ne] / c[ne][None, :, None]
    return out


def top_k_size(m_valid: int, sparsity_1e4: int) -> int:
    return max(1, (m_valid * (10000 - sparsity_1e4) + 9999) // 10000)


def select_row(logits: np.ndarray, cand: np.ndarray, k: int, tau: float):
    """One query block: (sorted list of block ids, n, m, probabilities in pi order).

    ``logits`` are the pooled logits of the candidate blocks ``cand`` (same order)."""
    ex = np.exp(logits - logits.max())
    p = ex / ex.sum()
    order = np.lexsort((cand, -logits))      # l descending, then block id ascending
    cum = np.cumsum(p[order])
    reach = np.nonzero(cum >= tau)[0]
    m = int(reach[0]) + 1 if reach.size else len(cand)
    n = min(max(k, m), len(cand))
    return np.sort(cand[order[:n]]), n, m, p[order]


def select(L: Layout, qbar: np.ndarray, kbar: np.ndarray, counts: np.ndarray,
           sparsity_1e4: int, tau: float):
    """Hybrid selection for every (head, query block).

    Returns (lists, n [H, M], m [H, M], k) where lists[h][i] is an ascending
    int array of selected key-block ids (empty for an empty query block)."""
    H, M, d = qbar.shape
    cand = np.nonzero(counts > 0)[0]
    k = top_k_size(len(cand), sparsity_1e4)
    lists = [[np.zeros(0, dtype=np.int64) for _ in range(M)] for _ in range(H)]
    n = np.zeros((H, M), dtype=np.int64)
    m = np.zeros((H, M), dtype=np.int64)
    scale = 1.0 / np.sqrt(d)
    for h in range(H):
        logits = (qbar[h] @ kbar[h, cand].T) * scale
        for i in range(M):
            if counts[i] == 0:
                continue
            lst, n[h, i], m[h, i], _ = select_row(logits[i], cand, k, tau)
            lists[h][i] = lst
    return lists, n, m, k


def pooled_logits(qbar: np.ndarray, kbar: np.ndarray, counts: np.ndarray) -> np.ndarray:
    """l[h, i, j] for all blocks (-inf where key block j is empty)."""
    d = qbar.shape[-1]
    l = np.einsum("hid,hjd->hij", qbar, kbar) / np.sqrt(d)
    l[:, :, counts == 0] = -np.inf
    return l


def block_mask(L: Layout, lists, h: int, perm: np.ndarray) -> np.ndarray:
    """Dense boolean mask [N, N] in raster order for head h:
    mask[n, m] = block(m) is in the list of block(n), and m is real."""
    N = L.n_tokens
    B = L.block_tokens
    blk = np.full(N, -1, dtype=np.int64)
    slots = np.nonzero(perm >= 0)[0]
    blk[perm[slots]] = slots // B
    sel = np.zeros((L.n_blocks, L.n_blocks), dtype=bool)
    for i, lst in enumerate(lists[h]):
        sel[i, lst] = True
    return sel[blk[:, None], blk[None, :]]


def block_mask_rows(L: Layout, lst, perm: np.ndarray) -> np.ndarray:
    """One row of ``block_mask`` for the queries of a block whose list is
    ``lst``: [N] bool in raster order, key m allowed iff block(m) is listed
    (pad slots are not tokens, so every raster key is real). Every query of
    the block shares this row."""
    N = L.n_tokens
    B = L.block_tokens
    blk = np.full(N, -1, dtype=np.int64)
    slots = np.nonzero(perm >= 0)[0]
    blk[perm[slots]] = slots // B
    sel = np.zeros(L.n_blocks, dtype=bool)
    sel[np.asarray(lst, dtype=np.int64)] = True
    return sel[blk]
