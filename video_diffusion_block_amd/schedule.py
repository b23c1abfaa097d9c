"""Reuse of zone shapes and block lists across diffusion steps.

[PAB page (nubint.ai review of "Real-Time Video Generation with Pyramid
Attention Broadcast"), proposed method and main results]: attention outputs
change little between consecutive diffusion steps over the middle 70% of the
schedule (the difference is U-shaped over the steps), so they can be computed
once and reused over a range of steps. Applied here to Prism's selection
([Prism page, trawling.dev/post/2299, §Blocks]) rather than to the attention
output: inside the middle segment the zone shapes and block lists are
recomputed every ``every`` steps and reused in between; outside it, every step
recomputes them. A reuse step still gathers the step's own Q, K, V (under the
cached zone shapes) and runs the attention; only zone scoring, pooling and
selection are skipped.

Host-side scheduling only: every computation is a call into libbsa through
``ops``.
"""
from __future__ import annotations

import math

from . import ops

MIDDLE = (0.15, 0.85)  # the stable middle 70% of the schedule


def refresh_steps(total_steps: int, every: int, middle=MIDDLE) -> list:
    """For each step 0..total_steps-1: True if it recomputes shapes and lists.

    Steps before ceil(middle[0] * total) and from ceil(middle[1] * total) on
    always recompute; inside [lo, hi) the steps lo, lo + every, ... recompute
    and the rest reuse the last lists. Step 0 always recomputes."""
    if total_steps < 1:
        raise ValueError(f"total_steps = {total_steps} must be >= 1")
    if every < 1:
        raise ValueError(f"every = {every} must be >= 1")
    if not (0.0 <= middle[0] <= middle[1] <= 1.0):
        raise ValueError(f"middle = {middle} must satisfy 0 <= lo <= hi <= 1")
    lo = math.ceil(middle[0] * total_steps)
    hi = math.ceil(middle[1] * total_steps)
    out = []
    for s in range(total_steps):
        inside = lo <= s < hi
        out.append(s == 0 or not inside or (s - lo) % every == 0)
    return out


class ReusedSelection:
    """One attention layer's forward over a diffusion schedule, with its zone
    shapes and block lists reused per ``refresh_steps``.

    ``layer(step, q, k, v, video, audio)`` returns (O [H, N, d], lse [H, N])
    in raster order; ``layer.refreshed`` says whether the last call
    recomputed the selection. ``frames_per_chunk`` > 0 selects with the
    frame-chunk causal rule (bsa_select_causal). Where bsa_attn_fwd_gather
    takes the configuration, no block-ordered copy is made: a refresh step
    pools the block means from the token-order Q, K, and every step's
    attention gathers Q, K, V itself (same results as the gather +
    bsa_attn_fwd_raster sequence used otherwise)."""

    def __init__(self, layout: "ops.BSALayout", sparsity_1e4: int, tau: float,
                 total_steps: int, every: int, middle=MIDDLE, frames_per_chunk: int = 0):
        self.layout = layout
        self.sparsity_1e4 = int(sparsity_1e4)
        self.tau = float(tau)
        self.frames_per_chunk = int(frames_per_chunk)
        self.plan = refresh_steps(total_steps, every, middle)
        self.zone_shape = self.counts = self.idx = None
        self.refreshed = False

    def __call__(self, step: int, q, k, v, video=None, audio=None):
        lay = self.layout
        gather = ops.gather_supported(lay, q.dtype, q.shape[2])
        if self.plan[step] or self.idx is None:
            zs = ops.zone_score(lay, video, audio)
            if gather:
                _, (qbar, kbar) = ops.permute_pool(lay, zs, [q, k], npool=2, store=False)
            else:
                (qp, kp, vp), (qbar, kbar) = ops.permute_pool(lay, zs, [q, k, v], npool=2)
            if self.frames_per_chunk:
                counts, idx = ops.select_causal(lay, zs, qbar, kbar, self.sparsity_1e4, self.tau,
                                                self.frames_per_chunk)
            else:
                counts, idx = ops.select(lay, zs, qbar, kbar, self.sparsity_1e4, self.tau)
            self.zone_shape, self.counts, self.idx = zs, counts, idx
            self.refreshed = True
        else:
            if not gather:
                qp, kp, vp = ops.permute(lay, self.zone_shape, [q, k, v])
            self.refreshed = False
        if gather:
            return ops.attn_fwd_gather(lay, self.zone_shape, q, k, v, self.counts, self.idx)
        return ops.attn_fwd_raster(lay, self.zone_shape, qp, kp, vp, self.counts, self.idx)
