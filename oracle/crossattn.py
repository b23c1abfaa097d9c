"""Audio-to-video cross-attention layer, forward and backward (oracle; test
infrastructure, imported only by tests and the benchmark's oracle timing).

[Prism page (trawling.dev/post/2299), §Blocks]: the zone's block shape uses
the feature norm of the audio-to-video (A2V) cross-attention, the layer in
which video tokens attend to the audio tokens. The page gives no layer
definition; the readings taken here (the plainest multi-head form):

- Video features X [N, C], audio features A [Na, C]; H heads of d channels
  (H d = D). Weights in [out, in] layout: Wq [D, C], Wk [D, C], Wv [D, C],
  Wo [C, D]; no biases, no normalization, no positional terms.
- Q = X Wq^T, K = A Wk^T, V = A Wv^T; per head h (columns h d .. h d + d - 1):
  O_h = softmax(Q_h K_h^T / sqrt(d)) V_h over all Na audio tokens; lse_h the
  natural log of the softmax denominator; Y = O Wo^T.
- Backward from dY: dO = dY Wo, dWo = dY^T O; per head P = exp(S - lse),
  dP = dO_h V_h^T, D = rowsum(dO_h * O_h), dS = P (dP - D),
  dQ_h = dS K_h / sqrt(d), dK_h = dS^T Q_h / sqrt(d), dV_h = P^T dO_h;
  dX = dQ Wq, dWq = dQ^T X, dA = dK Wk + dV Wv, dWk = dK^T A, dWv = dV^T A.
- Storage precision: the layer hands back its activations as bf16 tensors
  (Q, K, V, O and Y, the forward's outputs, which its backward takes as
  inputs), so with ``rounding=True`` the forward rounds each of those to bf16
  (nearest, ties to even) where it is stored. Nothing else is rounded: every
  product and sum is fp64, and the backward is the exact fp64 gradient of the
  layer given the forward's stored tensors (whatever a kernel keeps inside its
  backward, such as dO, dQ, dK and dV, is its own affair and not part of the
  layer's interface). ``rounding=False`` gives the exact fp64 function (used by
  the finite-difference pins).
"""
from __future__ import annotations

import numpy as np


def round_bf16(x) -> np.ndarray:
    """Round fp64 values to the nearest bfloat16 value (ties to even), as fp64."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                  # x = m 2^e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)             # below 2^-126 the spacing stays 2^-133
    return np.ldexp(np.rint(np.ldexp(x, 8 - e)), e - 8)


def _r(x, rounding):
    return round_bf16(x) if rounding else x


def forward(X, A, Wq, Wk, Wv, Wo, heads: int, rounding: bool = True) -> dict:
    """Returns q, k, v, o [*, D], lse [H, N], y [N, C] (fp64 arrays)."""
    D = Wq.shape[0]
    d = D // heads
    q = _r(X @ Wq.T, rounding)
    k = _r(A @ Wk.T, rounding)
    v = _r(A @ Wv.T, rounding)
    N = X.shape[0]
    o = np.empty((N, D))
    lse = np.empty((heads, N))
    for h in range(heads):
        c = slice(h * d, (h + 1) * d)
        s = (q[:, c] @ k[:, c].T) / np.sqrt(d)
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        den = p.sum(axis=1, keepdims=True)
        o[:, c] = (p / den) @ v[:, c]
        lse[h] = (m + np.log(den))[:, 0]
    o = _r(o, rounding)
    y = _r(o @ Wo.T, rounding)
    return {"q": q, "k": k, "v": v, "o": o, "lse": lse, "y": y}


def backward(X, A, Wq, Wk, Wv, Wo, heads: int, fwd: dict, dY) -> dict:
    """Exact gradients of sum(Y * dY) given the forward's stored tensors ``fwd``
    (fp64 throughout)."""
    D = Wq.shape[0]
    d = D // heads
    q, k, v, o, lse = fwd["q"], fwd["k"], fwd["v"], fwd["o"], fwd["lse"]
    dO = dY @ Wo
    dWo = dY.T @ o
    dQ = np.empty_like(q)
    dK = np.empty_like(k)
    dV = np.empty_like(v)
    scale = 1.0 / np.sqrt(d)
    for h in range(heads):
        c = slice(h * d, (h + 1) * d)
        s = (q[:, c] @ k[:, c].T) * scale
        p = np.exp(s - lse[h][:, None])
        dp = dO[:, c] @ v[:, c].T
        Dr = (dO[:, c] * o[:, c]).sum(axis=1, keepdims=True)
        ds = p * (dp - Dr)
        dQ[:, c] = (ds @ k[:, c]) * scale
        dK[:, c] = (ds.T @ q[:, c]) * scale
        dV[:, c] = p.T @ dO[:, c]
    return {"dx": dQ @ Wq, "da": dK @ Wk + dV @ Wv, "dwq": dQ.T @ X, "dwk": dK.T @ A,
            "dwv": dV.T @ A, "dwo": dWo, "do": dO, "dq": dQ, "dk": dK, "dv": dV}
