"""Softmax attention restricted to the selected blocks (oracle), fwd and bwd.

[Prism §Blocks] replaces full self-attention by Prism Block Sparse Attention:
every query attends only to the key blocks selected for its query block. The
page gives no formula; the reading taken here (parity against Prism's own
code unpinned) is the plain one:

  O[n] = sum_{m in K(n)} softmax_m(Q_n . K_m * scale) V_m,
  lse[n] = ln sum_{m in K(n)} exp(Q_n . K_m * scale),

with K(n) the real tokens of the blocks listed for block(n), scale = 1/sqrt(d)
by default, non-causal, no dropout, no bias, and the softmax normalised over
the selected keys only (no correction for the dropped mass).

Backward (same pairs, forward lists reused), with P the probabilities above:
  D_n = dO_n . O_n,  dV_m = sum_n P_nm dO_n,  dP_nm = dO_n . V_m,
  dS_nm = P_nm (dP_nm - D_n),  dQ_n = scale sum_m dS_nm K_m,
  dK_m = scale sum_n dS_nm Q_n.

Two evaluators:
- ``*_dense_masked``: dense [N, N] logits with an explicit boolean mask in
  raster order (the definition; small N only);
- ``*_gathered``: per (head, query block), only the selected keys (the same
  sums, fast enough for sampled rows of the large workloads).
"""
from __future__ import annotations

import numpy as np

from .layout import Layout


def attn_fwd_dense_masked(q, k, v, mask, scale):
    """One head. q,k,v [N, d] fp64, mask [N, N] bool. Returns (O [N,d], lse [N])."""
    s = (q @ k.T) * scale
    s = np.where(mask, s, -np.inf)
    mx = s.max(axis=1, keepdims=True)
    e = np.where(mask, np.exp(s - mx), 0.0)
    z = e.sum(axis=1, keepdims=True)
    p = e / z
    return p @ v, (mx + np.log(z))[:, 0]


def attn_bwd_dense_masked(q, k, v, do, mask, scale):
    """One head. Returns (dQ, dK, dV), each [N, d]."""
    s = np.where(mask, (q @ k.T) * scale, -np.inf)
    mx = s.max(axis=1, keepdims=True)
    e = np.where(mask, np.exp(s - mx), 0.0)
    p = e / e.sum(axis=1, keepdims=True)
    o = p @ v
    D = (do * o).sum(axis=1, keepdims=True)
    dv = p.T @ do
    dp = do @ v.T
    ds = p * (dp - D)
    dq = (ds @ k) * scale
    dk = (ds.T @ q) * scale
    return dq, dk, dv


def _block_tokens(L: Layout, perm: np.ndarray):
    """Raster ids of the real tokens of every block."""
    B = L.block_tokens
    pb = perm.reshape(L.n_blocks, B)
    return [row[row >= 0] for row in pb]


def attn_fwd_gathered_pair(toks, q, k, v, lst, scale, i):
    """One (head, query block): q, k, v [N, d] of that head (raster), ``lst``
    the block's key-block list, ``toks`` the raster ids of every block's real
    tokens. Returns (raster rows, O rows [n, d], lse rows [n]) in fp64."""
    rows = toks[i]
    if rows.size == 0:
        return rows, np.zeros((0, q.shape[1])), np.zeros(0)
    keys = np.concatenate([toks[j] for j in lst])
    qi = q[rows].astype(np.float64)
    kj = k[keys].astype(np.float64)
    vj = v[keys].astype(np.float64)
    s = (qi @ kj.T) * scale
    mx = s.max(axis=1, keepdims=True)
    e = np.exp(s - mx)
    z = e.sum(axis=1, keepdims=True)
    return rows, (e / z) @ vj, (mx + np.log(z))[:, 0]


def block_tokens(L: Layout, perm):
    """Raster ids of the real tokens of every block (list of int arrays)."""
    return _block_tokens(L, perm)


def attn_fwd_gathered(L: Layout, perm, q, k, v, lists, scale, pairs=None):
    """All heads, raster layout. q,k,v [H, N, d] (any float dtype, upcast to fp64).

    ``pairs``: iterable of (head, query block) to evaluate (default: all).
    Returns (O [H,N,d], lse [H,N]); rows not evaluated are NaN."""
    H, N, d = q.shape
    toks = _block_tokens(L, perm)
    O = np.full((H, N, d), np.nan)
    lse = np.full((H, N), np.nan)
    if pairs is None:
        pairs = [(h, i) for h in range(H) for i in range(L.n_blocks)]
    for h, i in pairs:
        rows, o_rows, l_rows = attn_fwd_gathered_pair(toks, q[h], k[h], v[h], lists[h][i],
                                                      scale, i)
        O[h, rows] = o_rows
        lse[h, rows] = l_rows
    return O, lse


def attn_bwd_gathered(L: Layout, perm, q, k, v, do, lists, scale, heads=None, o=None):
    """All (or the given) heads, raster layout. Returns dQ, dK, dV [H, N, d] fp64
    (zeros for heads not evaluated).

    ``o``: the forward output handed to the backward ([H, N, d]); D = rowsum(dO * O)
    then uses it, as a backward that receives O as an input does. By default O
    is recomputed exactly."""
    H, N, d = q.shape
    toks = _block_tokens(L, perm)
    dQ = np.zeros((H, N, d))
    dK = np.zeros((H, N, d))
    dV = np.zeros((H, N, d))
    for h in (range(H) if heads is None else heads):
        qh = q[h].astype(np.float64)
        kh = k[h].astype(np.float64)
        vh = v[h].astype(np.float64)
        doh = do[h].astype(np.float64)
        for i in range(L.n_blocks):
            rows = toks[i]
            if rows.size == 0:
                continue
            keys = np.concatenate([toks[j] for j in lists[h][i]])
            s = (qh[rows] @ kh[keys].T) * scale
            e = np.exp(s - s.max(axis=1, keepdims=True))
            p = e / e.sum(axis=1, keepdims=True)
            oo = p @ vh[keys] if o is None else o[h, rows].astype(np.float64)
            D = (doh[rows] * oo).sum(axis=1, keepdims=True)
            dV[h, keys] += p.T @ doh[rows]
            ds = p * (doh[rows] @ vh[keys].T - D)
            dQ[h, rows] += (ds @ kh[keys]) * scale
            dK[h, keys] += (ds.T @ qh[rows]) * scale
    return dQ, dK, dV


def attn_bwd_gathered_blocks(L: Layout, perm, q, k, v, do, lists, scale, h, q_blocks=(),
                             k_blocks=(), o=None):
    """Gradients of one head restricted to chosen blocks (the same sums as
    ``attn_bwd_gathered``, evaluated only where asked):

    dQ rows of the query blocks ``q_blocks`` and dK/dV rows of the key blocks
    ``k_blocks`` (which need every query block whose list holds them).
    ``o`` as in ``attn_bwd_gathered``.
    Returns dicts block -> (raster rows, dQ) and block -> (raster rows, dK, dV)."""
    toks = _block_tokens(L, perm)
    qh = q[h].astype(np.float64)
    kh = k[h].astype(np.float64)
    vh = v[h].astype(np.float64)
    doh = do[h].astype(np.float64)
    want_k = set(int(j) for j in k_blocks)
    need_q = set(int(i) for i in q_blocks)
    for i in range(L.n_blocks):
        if want_k & set(int(j) for j in lists[h][i]):
            need_q.add(i)
    out_q = {}
    acc_k = {j: (toks[j], np.zeros((toks[j].size, q.shape[2])), np.zeros((toks[j].size, q.shape[2])))
             for j in want_k}
    for i in sorted(need_q):
        rows = toks[i]
        if rows.size == 0:
            continue
        lst = [int(j) for j in lists[h][i]]
        keys = np.concatenate([toks[j] for j in lst])
        s = (qh[rows] @ kh[keys].T) * scale
        e = np.exp(s - s.max(axis=1, keepdims=True))
        p = e / e.sum(axis=1, keepdims=True)
        oo = p @ vh[keys] if o is None else o[h, rows].astype(np.float64)
        D = (doh[rows] * oo).sum(axis=1, keepdims=True)
        ds = p * (doh[rows] @ vh[keys].T - D)
        if i in q_blocks:
            out_q[i] = (rows, (ds @ kh[keys]) * scale)
        off = 0
        for j in lst:
            n = toks[j].size
            if j in acc_k:
                _, dk, dv = acc_k[j]
                dv += p[:, off:off + n].T @ doh[rows]
                dk += (ds[:, off:off + n].T @ qh[rows]) * scale
            off += n
    return out_q, acc_k


def attn_bwd_key_blocks_from_lse(L: Layout, perm, q, k, v, do, o, lse, lists, scale, h, k_blocks):
    """dK and dV rows of the key blocks ``k_blocks`` of head h, with the
    softmax weights formed from the forward's log-sum-exp, P = exp(S - lse),
    and D = rowsum(dO * O) from the forward's output: the quantities a flash
    backward receives from its forward. Same sums as ``attn_bwd_gathered``
    restricted to those key blocks, at the cost of one pass over the queries
    that list them (no per-row softmax over whole lists).

    o [H, N, d] and lse [H, N] in raster order. Returns block -> (raster rows,
    dK, dV)."""
    toks = _block_tokens(L, perm)
    out = {}
    for j in k_blocks:
        j = int(j)
        keys = toks[j]
        qb = [i for i in range(L.n_blocks) if toks[i].size and np.any(np.asarray(lists[h][i]) == j)]
        if not qb or keys.size == 0:
            out[j] = (keys, np.zeros((keys.size, q.shape[2])), np.zeros((keys.size, q.shape[2])))
            continue
        rows = np.concatenate([toks[i] for i in qb])
        qr = q[h, rows].astype(np.float64)
        dor = do[h, rows].astype(np.float64)
        kj = k[h, keys].astype(np.float64)
        vj = v[h, keys].astype(np.float64)
        p = np.exp((qr @ kj.T) * scale - lse[h, rows].astype(np.float64)[:, None])
        D = (dor * o[h, rows].astype(np.float64)).sum(axis=1, keepdims=True)
        ds = p * (dor @ vj.T - D)
        out[j] = (keys, (ds.T @ qr) * scale, p.T @ dor)
    return out

