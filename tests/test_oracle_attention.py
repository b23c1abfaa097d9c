"""Pins of the oracle's block-sparse attention, forward and backward.

Library routines (torch's scaled_dot_product_attention with a boolean mask,
torch.logsumexp, torch autograd, all fp64 on the CPU) for the masked softmax
attention; exact probes (V = 1, V = one-hot); central finite differences; and
exact gradient invariants.
"""
import numpy as np
import pytest
import torch

from oracle import attention as att
from oracle import layout as lay
from oracle import pipeline as pipe
from oracle import select as sel


def _case(grid=(3, 8, 8), mode="fixed", block=(1, 8, 8), H=2, d=64, S=5000, tau=0.2, seed=0,
          random_shapes=False):
    rng = np.random.default_rng(seed)
    N = int(np.prod(grid))
    q, k, v = (rng.standard_normal((H, N, d)) for _ in range(3))
    zs = None
    if random_shapes:
        L = lay.make_layout(grid, mode, block)
        zs = rng.integers(0, len(L.shapes), L.n_zones).astype(np.int32)
    r = pipe.run_selection(grid, mode, block, q, k, S, tau, zone_shape=zs)
    return r, q, k, v


def _sdpa(q, k, v, mask):
    t = [torch.from_numpy(x)[None] for x in (q, k, v)]
    return torch.nn.functional.scaled_dot_product_attention(
        *t, attn_mask=torch.from_numpy(mask)[None])[0].numpy()


CASES = [dict(), dict(grid=(5, 20, 36), mode="dynamic", block=(4, 16, 16), d=16, S=9300,
                      random_shapes=True, seed=1)]


@pytest.mark.parametrize("kw", CASES)
def test_masked_forward_matches_library_sdpa(kw):
    r, q, k, v = _case(**kw)
    L = r["layout"]
    scale = 1 / np.sqrt(q.shape[2])
    for h in range(q.shape[0]):
        mask = sel.block_mask(L, r["lists"], h, r["perm"])
        o, lse = att.attn_fwd_dense_masked(q[h], k[h], v[h], mask, scale)
        np.testing.assert_allclose(o, _sdpa(q[h], k[h], v[h], mask), rtol=1e-12, atol=1e-13)
        logits = torch.from_numpy(q[h] @ k[h].T * scale).masked_fill(
            ~torch.from_numpy(mask), float("-inf"))
        np.testing.assert_allclose(lse, torch.logsumexp(logits, dim=1).numpy(), rtol=1e-13)


def test_sparsity_zero_is_full_attention():
    r, q, k, v = _case(S=0)
    L = r["layout"]
    for h in range(2):
        o, _ = att.attn_fwd_gathered(L, r["perm"], q, k, v, r["lists"], 1 / 8.0)
        full = _sdpa(q[h], k[h], v[h], np.ones((L.n_tokens, L.n_tokens), bool))
        np.testing.assert_allclose(o[h], full, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("kw", CASES)
def test_gathered_equals_dense_masked(kw):
    r, q, k, v = _case(**kw)
    L = r["layout"]
    scale = 1 / np.sqrt(q.shape[2])
    O, lse = att.attn_fwd_gathered(L, r["perm"], q, k, v, r["lists"], scale)
    for h in range(q.shape[0]):
        mask = sel.block_mask(L, r["lists"], h, r["perm"])
        o, l = att.attn_fwd_dense_masked(q[h], k[h], v[h], mask, scale)
        np.testing.assert_allclose(O[h], o, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[h], l, rtol=1e-13)


def test_constant_values_give_constant_output():
    r, q, k, v = _case(S=5000)
    O, _ = att.attn_fwd_gathered(r["layout"], r["perm"], q, k, np.ones_like(v), r["lists"], 0.125)
    np.testing.assert_allclose(O, 1.0, rtol=0, atol=1e-14)


def test_one_hot_values_expose_the_probabilities():
    """V = identity over keys: O = P, so every masked entry is exactly 0 and
    every row is a probability vector over its selected keys."""
    r, q, k, _ = _case(grid=(5, 20, 36), mode="dynamic", block=(4, 16, 16), d=16, S=9300,
                       random_shapes=True, seed=3)
    L = r["layout"]
    N = L.n_tokens
    for h in range(2):
        mask = sel.block_mask(L, r["lists"], h, r["perm"])
        P, _ = att.attn_fwd_dense_masked(q[h], k[h], np.eye(N), mask, 0.25)
        assert np.all(P[~mask] == 0.0)
        assert np.all(P[mask] > 0.0)
        np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=1e-13)
        s = q[h] @ k[h].T * 0.25
        i = 17
        sel_keys = np.nonzero(mask[i])[0]
        e = np.exp(s[i, sel_keys] - s[i, sel_keys].max())
        np.testing.assert_allclose(P[i, sel_keys], e / e.sum(), rtol=1e-12)


def test_backward_matches_library_autograd():
    r, q, k, v = _case(grid=(5, 20, 36), mode="dynamic", block=(4, 16, 16), d=16, S=9300,
                       random_shapes=True, seed=5)
    L = r["layout"]
    do = np.random.default_rng(9).standard_normal(q.shape)
    for h in range(2):
        mask = sel.block_mask(L, r["lists"], h, r["perm"])
        tq, tk, tv = (torch.from_numpy(x[h]).requires_grad_() for x in (q, k, v))
        o = torch.nn.functional.scaled_dot_product_attention(
            tq[None], tk[None], tv[None], attn_mask=torch.from_numpy(mask)[None])[0]
        o.backward(torch.from_numpy(do[h]))
        dq, dk, dv = att.attn_bwd_dense_masked(q[h], k[h], v[h], do[h], mask, 0.25)
        for a, b in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
            np.testing.assert_allclose(a, b.numpy(), rtol=1e-10, atol=1e-12)


def test_backward_finite_differences():
    """Central differences (step 1e-6) of <dO, O(Q,K,V)> on the tiny layout."""
    r, q, k, v = _case(H=1, d=8)
    L = r["layout"]
    mask = sel.block_mask(L, r["lists"], 0, r["perm"])
    do = np.random.default_rng(1).standard_normal(q[0].shape)
    scale = 0.3

    def f(qq, kk, vv):
        return float((att.attn_fwd_dense_masked(qq, kk, vv, mask, scale)[0] * do).sum())

    dq, dk, dv = att.attn_bwd_dense_masked(q[0], k[0], v[0], do, mask, scale)
    rng = np.random.default_rng(2)
    eps = 1e-6
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        for _ in range(12):
            n, c = int(rng.integers(0, q.shape[1])), int(rng.integers(0, 8))
            args = [q[0].copy(), k[0].copy(), v[0].copy()]
            args[which][n, c] += eps
            fp = f(*args)
            args[which][n, c] -= 2 * eps
            fm = f(*args)
            num = (fp - fm) / (2 * eps)
            assert abs(num - grad[n, c]) <= 1e-6 * max(1.0, abs(num))


@pytest.mark.parametrize("kw", CASES)
def test_backward_invariants_and_gathered(kw):
    """sum_m dV_m = sum_n dO_n (each row of P sums to 1) and sum_m dK_m = 0
    (softmax is invariant to a shift of the logits); the gathered evaluator
    equals the dense one; dO = 0 gives zero gradients."""
    r, q, k, v = _case(**kw)
    L = r["layout"]
    scale = 1 / np.sqrt(q.shape[2])
    do = np.random.default_rng(4).standard_normal(q.shape)
    dQ, dK, dV = att.attn_bwd_gathered(L, r["perm"], q, k, v, do, r["lists"], scale)
    for h in range(q.shape[0]):
        np.testing.assert_allclose(dV[h].sum(axis=0), do[h].sum(axis=0), rtol=1e-11, atol=1e-11)
        np.testing.assert_allclose(dK[h].sum(axis=0), 0.0, atol=1e-11)
        mask = sel.block_mask(L, r["lists"], h, r["perm"])
        dq, dk, dv = att.attn_bwd_dense_masked(q[h], k[h], v[h], do[h], mask, scale)
        np.testing.assert_allclose(dQ[h], dq, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(dK[h], dk, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(dV[h], dv, rtol=1e-11, atol=1e-12)
    z = att.attn_bwd_gathered(L, r["perm"], q, k, v, np.zeros_like(do), r["lists"], scale)
    assert all(np.all(g == 0) for g in z)
    # handing the exact forward output to the backward changes nothing
    O, _ = att.attn_fwd_gathered(L, r["perm"], q, k, v, r["lists"], scale)
    withO = att.attn_bwd_gathered(L, r["perm"], q, k, v, do, r["lists"], scale, o=O)
    for a, b in zip(withO, (dQ, dK, dV)):
        np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("kw", CASES)
def test_key_blocks_from_lse_equal_the_gathered_backward(kw):
    """The lse form of the key-side gradients equals the per-row softmax form
    (itself pinned to autograd and finite differences above) when it is given
    the exact forward output and log-sum-exp, on every non-empty key block;
    a key block no query lists gets zero gradients."""
    r, q, k, v = _case(**kw)
    L = r["layout"]
    scale = 1 / np.sqrt(q.shape[2])
    do = np.random.default_rng(5).standard_normal(q.shape)
    dQ, dK, dV = att.attn_bwd_gathered(L, r["perm"], q, k, v, do, r["lists"], scale)
    O, lse = att.attn_fwd_gathered(L, r["perm"], q, k, v, r["lists"], scale)
    O, lse = np.nan_to_num(O), np.nan_to_num(lse)
    for h in range(q.shape[0]):
        blocks = [j for j in range(L.n_blocks) if r["counts"][j] > 0]
        got = att.attn_bwd_key_blocks_from_lse(L, r["perm"], q, k, v, do, O, lse, r["lists"],
                                               scale, h, blocks)
        for j, (rows, dk, dv) in got.items():
            np.testing.assert_allclose(dk, dK[h, rows], rtol=1e-10, atol=1e-11)
            np.testing.assert_allclose(dv, dV[h, rows], rtol=1e-10, atol=1e-11)
    lists = [[np.array([0]) for _ in range(L.n_blocks)] for _ in range(q.shape[0])]
    nz = [j for j in range(1, L.n_blocks) if r["counts"][j] > 0][:1]
    (rows, dk, dv), = att.attn_bwd_key_blocks_from_lse(L, r["perm"], q, k, v, do, O, lse, lists,
                                                       scale, 0, nz).values()
    assert rows.size > 0 and np.all(dk == 0) and np.all(dv == 0)



def test_bf16_storage_of_o_alone_moves_dq_past_the_bf16_bar():
    """The backward takes the forward's O as an input (D = rowsum(dO * O)),
    and a bf16 forward stores O rounded to bf16. On the ragged dynamic case of
    the GPU tests (5 x 20 x 36 grid, 2 heads, d = 128, forced zone shapes,
    sparsity 0.93), with every other step exact in fp64, rounding O alone moves
    dQ by more than 2e-2 (max-abs; dK by about 1e-2, dV not at all, since dV
    does not depend on D). So against the exact oracle no bf16 backward can
    meet a 2e-2 max-abs bar on dQ end to end; its parity is judged given the O
    it receives, and the end-to-end figure is reported beside it."""
    import synth
    from oracle import crossattn as oca
    from oracle import pipeline as opipe

    wl = synth.Workload("ragged-dyn", (5, 20, 36), 2, 128, "bf16", "dynamic", (4, 16, 16), 9300,
                        0.2)
    inp = synth.make_inputs(wl, parts=("q", "k", "v", "do"))
    L = lay.make_layout(wl.grid, wl.mode, wl.block)
    rng = np.random.default_rng(5)
    zs = rng.integers(0, len(L.shapes), L.n_zones).astype(np.int32)
    zs[0] = len(L.shapes) - 1
    q, k, v, do = (synth.bf16_bits_to_f64(inp[p]) for p in ("q", "k", "v", "do"))
    r = opipe.run_selection(wl.grid, wl.mode, wl.block, q, k, wl.sparsity_1e4, wl.tau,
                            zone_shape=zs)
    scale = 1 / np.sqrt(wl.d)
    O, _ = att.attn_fwd_gathered(L, r["perm"], q, k, v, r["lists"], scale)
    O = np.nan_to_num(O)                       # (no empty query blocks here; pads are not rows)
    exact = att.attn_bwd_gathered(L, r["perm"], q, k, v, do, r["lists"], scale)
    stored = att.attn_bwd_gathered(L, r["perm"], q, k, v, do, r["lists"], scale,
                                   o=oca.round_bf16(O))
    shift = [np.abs(a - b).max() for a, b in zip(stored, exact)]
    assert shift[0] > 2e-2          # dQ
    assert 5e-3 < shift[1] < 2e-2   # dK
    assert shift[2] == 0.0          # dV
