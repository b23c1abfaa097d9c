"""Seeded, synthetic stand-ins for video-DiT latent tokens.

The pages train on Wan VAE latents of real clips at 720p/1080p/2K (Prism page,
section on data preparation and the training procedure). Those clips and the
VAE are not available, so these generators produce inputs of the same shapes
with the property the method acts on: low-frequency spatio-temporal structure
plus per-token noise.

Recipe of the smooth field (every draw comes from numpy's PCG64):

1. white N(0,1) noise in float32, one independent stream per leading index
   (head, or the single video "head"), spawned from ``SeedSequence(seed)``;
2. a separable Gaussian blur with sigma = 3 tokens (taps at offsets -12..12,
   weights proportional to exp(-x^2/18), normalised) along t, h and w, with
   symmetric (edge-repeating mirror) boundaries;
3. standardisation of each (leading index, channel) field to mean 0, std 1
   over the grid;
4. plus 0.3 x N(0,1) from a second set of spawned streams;
5. rounding to bfloat16, round-to-nearest-even (stored as uint16 bits).

Token order is raster over the latent grid, t slowest: n = (t*H + h)*W + w,
and tensors are [heads, tokens, d] (or [tokens, channels] for video/audio
features).
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

SIGMA = 3.0
RADIUS = 12
NOISE_AMPLITUDE = 0.3

# Seeds of the individual tensors of one workload.
SEED_Q, SEED_K, SEED_V, SEED_VIDEO, SEED_AUDIO, SEED_DO = 1, 2, 3, 4, 5, 6


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and parameters of one synthetic workload (no arithmetic)."""

    name: str
    grid: tuple          # latent grid (T, H, W)
    heads: int
    d: int
    dtype: str           # "f32" or "bf16"
    mode: str            # "fixed" or "dynamic"
    block: tuple         # block shape (fixed mode) or zone extent (dynamic mode)
    sparsity_1e4: int    # sparsity x 1e4 (0.85 -> 8500)
    tau: float           # CDF threshold of the hybrid selection
    video_channels: int = 0   # 0: no video features (no zone scoring)
    n_audio: int = 0          # 0: no audio tokens (no A2V term)
    backward: bool = False
    smooth: bool = True       # False: plain N(0,1) Q/K/V (the tiny fp32 case)

    @property
    def n_tokens(self) -> int:
        t, h, w = self.grid
        return t * h * w


# The five workloads of the measurement plan, named by what they are.
WORKLOADS = {
    "tiny": Workload("tiny", (3, 8, 8), 2, 64, "f32", "fixed", (1, 8, 8), 5000, 0.20,
                     smooth=False),
    "720p": Workload("720p", (13, 45, 80), 40, 128, "bf16", "fixed", (2, 8, 8), 8500, 0.20),
    "720p-dyn": Workload("720p-dyn", (13, 45, 80), 40, 128, "bf16", "dynamic", (4, 16, 16),
                         8000, 0.20, video_channels=1536, n_audio=200),
    "1080p": Workload("1080p", (13, 68, 120), 10, 128, "bf16", "dynamic", (4, 16, 16),
                      9300, 0.20, video_channels=1536, n_audio=200),
    "2k": Workload("2k", (13, 90, 160), 4, 128, "bf16", "dynamic", (4, 16, 16),
                   9300, 0.20, video_channels=1536, n_audio=200, backward=True),
}


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(b).astype(np.float64)


def gaussian_noise(shape, seed: int) -> np.ndarray:
    """N(0,1) float32; one PCG64 stream per leading index, spawned from ``seed``."""
    shape = tuple(int(s) for s in shape)
    lead = shape[0]
    rest = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    out = np.empty((lead, rest), dtype=np.float32)
    seqs = np.random.SeedSequence(seed).spawn(lead)

    def fill(i):
        np.random.Generator(np.random.PCG64(seqs[i])).standard_normal(
            rest, dtype=np.float32, out=out[i])

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(lead)))
    return out.reshape(shape)


def _mirror(i: int, n: int) -> int:
    """Symmetric boundary: ... 1 0 | 0 1 ... n-1 | n-1 n-2 ..."""
    i %= 2 * n
    return i if i < n else 2 * n - 1 - i


def _blur_operator(n: int) -> np.ndarray:
    """n x n matrix of the 1-D Gaussian blur with symmetric boundaries."""
    taps = np.arange(-RADIUS, RADIUS + 1, dtype=np.float64)
    w = np.exp(-taps * taps / (2.0 * SIGMA * SIGMA))
    w /= w.sum()
    op = np.zeros((n, n), dtype=np.float64)
    for i in range(n):
        for k, wk in zip(taps.astype(int), w):
            op[i, _mirror(i + k, n)] += wk
    return op.astype(np.float32)


def smooth_field(lead: int, grid, channels: int, seed: int) -> np.ndarray:
    """Smooth field + noise, rounded to bf16: uint16 [lead, T*H*W, channels]."""
    t, h, w = grid
    sub = np.random.SeedSequence(seed).generate_state(2)
    x = gaussian_noise((lead, t, h, w, channels), int(sub[0]))
    # separable blur along t, h, w (matrix products, batched over the rest)
    x = np.matmul(_blur_operator(t), x.reshape(lead, t, h * w * channels))
    x = np.matmul(_blur_operator(h), x.reshape(lead * t, h, w * channels))
    x = np.matmul(_blur_operator(w), x.reshape(lead * t * h, w, channels))
    x = x.reshape(lead, t * h * w, channels)
    mean = x.mean(axis=1, dtype=np.float64, keepdims=True)
    std = x.std(axis=1, dtype=np.float64, keepdims=True)
    std[std == 0] = 1.0
    x -= mean.astype(np.float32)
    x /= std.astype(np.float32)
    x += np.float32(NOISE_AMPLITUDE) * gaussian_noise(x.shape, int(sub[1]))
    return f32_to_bf16_bits(x)


def make_inputs(wl: Workload, parts=("q", "k", "v"), heads: int | None = None) -> dict:
    """Inputs of a workload as numpy arrays.

    bf16 tensors are uint16 bit patterns; the tiny fp32 workload returns float32.
    ``heads`` limits the smooth Q/K/V and dO to their first heads: each head has
    its own spawned stream and its own standardisation, so these are exactly
    the first heads of the full draw.
    """
    H = wl.heads if heads is None else heads
    N = wl.n_tokens
    out = {}
    seeds = {"q": SEED_Q, "k": SEED_K, "v": SEED_V}
    for p in parts:
        if p in seeds:
            if wl.smooth:
                out[p] = smooth_field(H, wl.grid, wl.d, seeds[p])
            else:
                g = np.random.Generator(np.random.PCG64(seeds[p]))
                x = g.standard_normal((H, N, wl.d), dtype=np.float32)
                out[p] = x if wl.dtype == "f32" else f32_to_bf16_bits(x)
        elif p == "do":
            x = gaussian_noise((H, N, wl.d), SEED_DO)
            out[p] = x if wl.dtype == "f32" else f32_to_bf16_bits(x)
        elif p == "video":
            out[p] = smooth_field(1, wl.grid, wl.video_channels, SEED_VIDEO)[0]
        elif p == "audio":
            x = gaussian_noise((wl.n_audio, wl.video_channels), SEED_AUDIO)
            out[p] = f32_to_bf16_bits(x)
        else:
            raise KeyError(p)
    return out
