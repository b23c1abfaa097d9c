"""Plain fp64 CPU oracle of Prism-style block-sparse attention (BSA).

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The GPU library
(``video_diffusion_block_amd``) never imports it, and this package imports
nothing from the GPU library: the two share no code.

Sources. The method is described on the page "Prism: 2K 공동 영상·오디오 생성
학습을 위한 동적 희소 어텐션" (Prism: dynamic sparse attention for training 2K
joint video-audio generation; trawling.dev/post/2299), section "지역별 정보에
맞춘 블록 구성" (block composition matched to regional information), cited
below as [Prism §Blocks]. The page gives the ingredients in prose and no
formulas; every step below that the page leaves open states the reading it
takes, and the module docstrings list them.

Modules, in the order the hot path runs them:

- ``layout``    token -> macro-zone -> shaped block permutation, padding
- ``zones``     per-zone video channel variance and A2V feature norm, per axis;
                block-shape choice
- ``select``    block-mean pooling and hybrid (top-k U CDF-prefix) selection
- ``attention`` dense softmax attention under an explicit block mask, forward
                and backward, plus a gathered evaluator of the same sums
- ``prenorm``   RMSNorm + 3-D RoPE of Q and K before the gather
- ``causal``    the hybrid selection under a frame-chunk causal block mask
- ``crossattn`` the A2V cross-attention layer (projections, multi-head
                attention over the audio tokens), forward and backward

All arithmetic is float64 on inputs upcast exactly from bf16/fp32.

Parity pins (tests/test_oracle_*.py): closed forms, invariants, brute force on
tiny inputs, and special cases that reduce to library routines. The page prints
no worked example, so agreement with Prism's own implementation is unpinned for
the readings listed in each module; the oracle itself is pinned to mathematics.
"""
from . import attention, layout, pipeline, select, zones  # noqa: F401
