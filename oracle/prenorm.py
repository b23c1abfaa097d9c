"""Pre-attention normalization and 3-D rotary position embedding of Q and K
(oracle; test infrastructure, imported only by tests and the benchmark's
oracle timing).

[Helios page (suanlab.com, Helios review), core contributions: fused
normalization and RoPE kernels raise throughput] and [Kaleido page
(gist.science, paper 2607.13770), methodology, channel-wise reuse: the video
DiT's rotary embedding splits a head's channels into three groups, for the
time axis and the two spatial axes, each encoding its axis at its own
frequencies]. Neither page gives a formula; the readings taken here:

- Normalization: RMSNorm of each token's head vector over its d channels,
  y = x / sqrt(mean_c x_c^2 + eps) * gamma, gamma a per-channel weight [d].
- Channel groups, in the order t, h, w: d_t = d - 4 floor(d/6) and
  d_h = d_w = 2 floor(d/6) (d = 128: 44, 42, 42; d = 64: 24, 20, 20): as equal
  as possible in even sizes, the remainder to t.
- Rotation: inside a group of g channels, the pair (2i, 2i+1) of the group
  turns by the angle pos * base^(-2i/g), pos the token's coordinate on the
  group's axis (raster token n = (t H + h) W + w), base 10000:
  (x0, x1) -> (x0 cos a - x1 sin a, x0 sin a + x1 cos a).
- Q and K are normalized, then rotated; V is untouched.

Everything is fp64 on exactly upcast inputs.
"""
from __future__ import annotations

import numpy as np

ROPE_BASE = 10000.0
EPS = 1e-6


def split_sizes(d: int) -> tuple:
    """Channels of the t, h and w groups."""
    s = 2 * (d // 6)
    return d - 2 * s, s, s


def rms_norm(x: np.ndarray, gamma: np.ndarray, eps: float = EPS) -> np.ndarray:
    """RMSNorm over the last axis (the head channels)."""
    x = np.asarray(x, np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gamma, np.float64)


def positions(grid) -> np.ndarray:
    """[N, 3] (t, h, w) of every raster token."""
    T, H, W = grid
    n = np.arange(T * H * W)
    return np.stack([n // (H * W), (n // W) % H, n % W], axis=1)


def rope_angles(grid, d: int, base: float = ROPE_BASE) -> np.ndarray:
    """[N, d/2] rotation angle of every channel pair of every raster token."""
    pos = positions(grid).astype(np.float64)
    cols = []
    for axis, g in enumerate(split_sizes(d)):
        i = np.arange(g // 2, dtype=np.float64)
        theta = base ** (-2.0 * i / g)
        cols.append(pos[:, axis:axis + 1] * theta[None, :])
    return np.concatenate(cols, axis=1)


def rope3d(x: np.ndarray, grid, base: float = ROPE_BASE) -> np.ndarray:
    """Rotate the channel pairs of x [..., N, d] (raster token order)."""
    x = np.asarray(x, np.float64)
    a = rope_angles(grid, x.shape[-1], base)
    c, s = np.cos(a), np.sin(a)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def norm_rope(x: np.ndarray, gamma: np.ndarray, grid, eps: float = EPS,
              base: float = ROPE_BASE) -> np.ndarray:
    """The pre-attention transform of Q or K [heads, N, d]."""
    return rope3d(rms_norm(x, gamma, eps), grid, base)
