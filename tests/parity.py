"""Helpers of the GPU parity tests: tensor conversion, the oracle side of each
comparison, and the comparison rules.

Comparison rules (the bar every GPU test applies):
- permutation, unpermutation, zone shapes and block lists: exact, except
  documented near-ties (zone costs within a relative ZONE_TIE; pooled logits
  within LIST_TIE of the cut, or a CDF prefix sum within LIST_TIE of tau);
- fp32 outputs: max-abs <= 1e-5;
- bf16 outputs: evaluated under the GPU's own lists, max-abs <= 2e-2 and
  sum|diff| / sum|ref| <= 5e-3.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch
from threadpoolctl import threadpool_limits

import synth
from oracle import attention as oatt
from oracle import layout as olay
from oracle import select as osel

LIST_TIE = 1e-6
# Zone costs within a relative 1e-6 of each other are a tie (the shape rule's
# own tie window); a zone whose two lowest oracle costs are that close may
# legitimately differ.
ZONE_TIE = 1e-6
F32_TOL = 1e-5
BF16_MAX_ABS = 2e-2
BF16_L1_REL = 5e-3
# lse of the bf16 attention kernels: the softmax denominator is the sum of the
# bf16-rounded weights that the PV product uses, each within 2^-9 (relative)
# of the exact weight, so the sum is too and ln of it moves by at most
# -ln(1 - 2^-9) = 1.955e-3; the sum runs in fp32 over up to 17 536 weights
# (137 blocks of 128 keys at the 2K workload), which adds at most about
# n 2^-24 = 1.05e-3 relative in the worst case. lse max-abs <= 3e-3.
LSE_TOL = 3e-3


def to_dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    """numpy (float32, or uint16 bf16 bits) -> contiguous cuda tensor."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.cuda()


def to_f64(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return synth.bf16_bits_to_f64(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
    return t.detach().cpu().numpy().astype(np.float64)


def host_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    return synth.bf16_bits_to_f64(x) if dtype == "bf16" else np.asarray(x, dtype=np.float64)


def oracle_layout(wl) -> olay.Layout:
    return olay.make_layout(wl.grid, wl.mode, wl.block)


def gpu_lists(counts: torch.Tensor, idx: torch.Tensor):
    c = counts.cpu().numpy()
    ix = idx.cpu().numpy()
    H, M = c.shape
    return [[ix[h, i, :c[h, i]].astype(np.int64) for i in range(M)] for h in range(H)]


def compare_lists(L, qbar, kbar, counts_np, sparsity_1e4, tau, gpu, oracle, visible=None):
    """Exact list equality per (head, query block), except near-ties.
    ``visible`` (bool [M, M], optional): row i's candidate key blocks (the
    causal selection); by default every non-empty block.

    Returns (exact rows, tie-exempt rows, list of failures)."""
    cand_all = np.nonzero(counts_np > 0)[0]
    d = qbar.shape[-1]
    exact = exempt = 0
    failures = []
    for h in range(len(gpu)):
        for i in range(len(gpu[h])):
            a, b = gpu[h][i], oracle[h][i]
            if a.shape == b.shape and np.array_equal(a, b):
                exact += 1
                continue
            if counts_np[i] == 0:
                failures.append((h, i, "empty query block got a list"))
                continue
            cand = cand_all if visible is None else np.nonzero(visible[i])[0]
            k = osel.top_k_size(len(cand), sparsity_1e4)
            logits = (qbar[h, i] @ kbar[h, cand].T) / np.sqrt(d)
            order = np.lexsort((cand, -logits))
            srt = logits[order]
            p = np.exp(logits - logits.max())
            p /= p.sum()
            cum = np.cumsum(p[order])
            n = len(b)
            cdf_tie = bool(np.any(np.abs(cum[max(0, n - 2):n + 1] - tau) < LIST_TIE))
            cut = srt[n - 1]
            diff = set(a.tolist()) ^ set(b.tolist())
            pos = {int(c): r for r, c in enumerate(cand[order])}
            near_cut = all(abs(logits[np.searchsorted(cand, j)] - cut) < LIST_TIE
                           for j in diff if j in pos)
            ascending = np.all(np.diff(a) > 0) and np.all(counts_np[a] > 0) and \
                np.all(np.isin(a, cand))
            if ascending and (cdf_tie or (near_cut and len(a) == len(b))):
                exempt += 1
            else:
                failures.append((h, i, f"gpu {a.tolist()[:8]}.. ({len(a)}) vs oracle "
                                       f"{b.tolist()[:8]}.. ({len(b)}), k={k}"))
    return exact, exempt, failures


def bf16_close(got: np.ndarray, ref: np.ndarray):
    diff = np.abs(got - ref)
    mx = float(diff.max()) if diff.size else 0.0
    rel = float(diff.sum() / max(np.abs(ref).sum(), 1e-300))
    return mx, rel


def assert_grad_close(got, ref, what=""):
    """The bar of the backward's gradients (fp32 outputs computed from bf16
    MFMA operands: the kernel rounds P and dS to bf16, within 2^-9 relative,
    for its products). A gradient row sums as many terms as the key or query
    rows that reach it, so its rounding error grows with its magnitude: on the
    4096-block case a key block reached by all 524 288 query rows has
    max |dK| = 33, and rounding dS alone (every other step exact) moves it by
    0.062 max-abs at an L1 ratio of 1.7e-3. So max-abs <= 2e-2 max(1, max|ref|)
    (the bf16 bar wherever |ref| <= 1) and sum|diff| / sum|ref| <= 5e-3: the
    rule the cross-attention layer's gradients use."""
    mx, rel = bf16_close(got, ref)
    scale = max(1.0, float(np.abs(ref).max()) if ref.size else 1.0)
    assert mx <= BF16_MAX_ABS * scale and rel <= BF16_L1_REL, \
        f"{what}: max-abs {mx:.3g} (max |ref| {scale:.3g}), L1-rel {rel:.3g}"
    return mx, rel


def assert_bf16_close(got, ref, what=""):
    mx, rel = bf16_close(got, ref)
    assert mx <= BF16_MAX_ABS and rel <= BF16_L1_REL, f"{what}: max-abs {mx:.3g}, L1-rel {rel:.3g}"
    return mx, rel


def oracle_fwd_rows(L, perm, q, k, v, lists, scale, pairs):
    """Oracle O and lse (raster) on the given (head, query block) pairs."""
    return oatt.attn_fwd_gathered(L, perm, q, k, v, lists, scale, pairs=pairs)


def block_rows(L, perm, i):
    """Raster ids of the real tokens of block i."""
    row = perm[i * L.block_tokens:(i + 1) * L.block_tokens]
    return row[row >= 0]


def host_threads() -> int:
    """Host threads the oracle checks may use (the GPU machine gives a process 16)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def parallel_map(fn, items, threads=None):
    """fn over items on a thread pool, one BLAS thread per worker (numpy
    releases the GIL inside its kernels). Results in item order."""
    threads = threads or host_threads()
    with threadpool_limits(limits=1):
        with ThreadPoolExecutor(threads) as ex:
            return list(ex.map(fn, items))


def check_fwd_pairs(L, perm, q, k, v, lists, scale, pairs, o_gpu, lse_gpu, dense=False,
                    keep=None):
    """The GPU's O (raster, [H, N, d] fp64 on the host) and lse (raster [H, N])
    on every listed (head, query block) pair against the oracle: the gathered
    evaluator, or (dense=True) the dense evaluator over all N keys under the
    block's explicit mask row. Each pair must meet the bf16 bar (max-abs and
    sum|diff| / sum|ref| over its rows) and lse max-abs <= LSE_TOL. Returns the
    worst max-abs, the overall L1 ratio and the worst lse error. ``keep``: a
    dict that receives the oracle's rows, "o" [H, N, d] and "lse" [H, N]."""
    toks = oatt.block_tokens(L, perm)

    def one(pair):
        h, i = pair
        rows = toks[i]
        if dense:
            mask = osel.block_mask_rows(L, lists[h][i], perm)[None, :]
            o_ref, l_ref = oatt.attn_fwd_dense_masked(q[h, rows], k[h], v[h], mask, scale)
        else:
            _, o_ref, l_ref = oatt.attn_fwd_gathered_pair(toks, q[h], k[h], v[h], lists[h][i],
                                                          scale, i)
        diff = np.abs(o_gpu[h, rows] - o_ref)
        if keep is not None:
            keep["o"][h, rows] = o_ref
            keep["lse"][h, rows] = l_ref
        return (h, i, float(diff.max()), float(diff.sum()), float(np.abs(o_ref).sum()),
                float(np.abs(lse_gpu[h, rows] - l_ref).max()))

    if keep is not None:
        keep["o"] = np.full(o_gpu.shape, np.nan)
        keep["lse"] = np.full(lse_gpu.shape, np.nan)

    res = parallel_map(one, [p for p in pairs if toks[p[1]].size])
    bad = [(h, i, mx, sd / sr) for h, i, mx, sd, sr, _ in res
           if mx > BF16_MAX_ABS or sd > BF16_L1_REL * sr]
    assert not bad, f"{len(bad)} pairs fail the bf16 bar, e.g. {bad[:3]}"
    lbad = [(h, i, le) for h, i, _, _, _, le in res if le > LSE_TOL]
    assert not lbad, f"{len(lbad)} pairs fail the lse bar, e.g. {lbad[:3]}"
    return (max(r[2] for r in res), sum(r[3] for r in res) / sum(r[4] for r in res),
            max(r[5] for r in res))


def sample_pairs(rng, heads, nonempty, n, must=()):
    """n distinct seeded (head, query block) pairs, the ``must`` ones first."""
    pairs = list(dict.fromkeys((int(h), int(i)) for h, i in must))
    seen = set(pairs)
    while len(pairs) < n:
        p = (int(rng.integers(0, heads)), int(rng.choice(nonempty)))
        if p not in seen:
            seen.add(p)
            pairs.append(p)
    return pairs


def grad_stats(got, ref):
    """(max-abs, sum|diff| / sum|ref|) of a gradient comparison."""
    diff = np.abs(got - ref)
    return float(diff.max()), float(diff.sum() / max(np.abs(ref).sum(), 1e-300))
