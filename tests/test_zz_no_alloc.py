"""bsa_attn_fwd_noalloc (the forward for callers that cannot allocate: its
block table lives in the library's static per-GPU scratch) against
bsa_attn_fwd with a caller workspace: bitwise-equal O and lse on two calls in
a row, the second on a smaller layout (fewer blocks, so the scratch holds the
first call's larger table when the second starts)."""
import numpy as np
import pytest
import torch

import synth
from parity import to_dev
from video_diffusion_block_amd import ops

pytestmark = pytest.mark.gpu


def _case(wl):
    inp = synth.make_inputs(wl)
    lay = (ops.BSALayout.fixed(wl.grid, wl.block) if wl.mode == "fixed"
           else ops.BSALayout.dynamic(wl.grid, wl.block))
    zs = torch.as_tensor(np.arange(lay.sizes()["n_zones"], dtype=np.int32) % len(lay.shapes)).cuda()
    q, k, v = (to_dev(inp[p], wl.dtype) for p in "qkv")
    (qp, kp, vp), (qbar, kbar) = ops.permute_pool(lay, zs, [q, k, v], npool=2)
    counts, idx = ops.select(lay, zs, qbar, kbar, wl.sparsity_1e4, wl.tau)
    return lay, zs, qp, kp, vp, counts, idx


@pytest.mark.parametrize("order", ["large-then-small", "dynamic-then-fixed"])
def test_noalloc_matches_workspace_call(order):
    if order == "large-then-small":
        wls = [synth.Workload("big", (13, 45, 80), 3, 128, "bf16", "fixed", (2, 8, 8), 8500, 0.2),
               synth.Workload("small", (4, 16, 24), 2, 128, "bf16", "fixed", (2, 8, 8), 7000, 0.2)]
    else:
        wls = [synth.Workload("dyn", (9, 40, 52), 2, 128, "bf16", "dynamic", (4, 16, 16), 8000, 0.2),
               synth.Workload("fix", (3, 17, 20), 2, 128, "bf16", "fixed", (1, 8, 16), 6000, 0.2)]
    for wl in wls:
        lay, zs, qp, kp, vp, counts, idx = _case(wl)
        o_ref, lse_ref = ops.attn_fwd(lay, zs, qp, kp, vp, counts, idx)
        o, lse = ops.attn_fwd_noalloc(lay, zs, qp, kp, vp, counts, idx)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), wl.name
        assert torch.equal(lse, lse_ref), wl.name
        assert torch.isfinite(o.float()).all()
