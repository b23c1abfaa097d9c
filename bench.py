"""Benchmark of the block-sparse attention hot path on one GPU.

One step = one BSA attention layer forward on the 720p workload (13x45x80 =
46 800 latent tokens, 40 heads, d = 128, bf16, fixed 2x8x8 blocks, sparsity
0.85, tau = 0.20): zone scoring (a no-op fill for a fixed layout), the block
means of Q and K pooled from the token-order tensors, hybrid selection, and the
block-sparse attention forward, whose tile loads gather Q, K, V into block
order from the token-order tensors and which writes O in raster order (no
block-ordered copy of Q, K or V is stored). Inputs are seeded synthetic
latents (smooth field + noise), resident in HBM before timing starts.

Prints one JSON line: value = executed attention TFLOP/s over the whole layer
time (the layer's executed attention FLOPs / ms per layer), plus ms per layer,
per-stage times, the roofline of the dominant kernel (attention forward, bf16
MFMA) measured with HIP events on the launch stream, and the fp64 CPU oracle's
rate on the same layer (the whole layer; --cpu-sample times a bounded sample
and scales it).

Options: --workload NAME runs another workload of the measurement plan
(720p-dyn, 1080p, 2k; 2k adds the backward, which needs block-ordered copies
and so gathers them, and which writes the gradients in raster order); --copy-calib runs only a plain 1 GiB device copy (the
calibration kernel for HBM byte counters); --permuted (block-ordered copies of
Q, K, V gathered with the pooling, then the attention on them), --unfused
(separate gather and pool+select calls), --norm-rope (RMSNorm + 3-D RoPE of Q
and K in the gather), --causal-frames F (frame-chunk causal selection) and
--reuse-every R (zone shapes and lists recomputed every R steps, reused in
between) time the variants of the same layer.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="720p")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", action="store_true",
                    help="time the oracle on a bounded sample (6 heads) instead of the whole layer")
    ap.add_argument("--copy-calib", action="store_true")
    ap.add_argument("--norm-rope", action="store_true",
                    help="fuse RMSNorm + 3-D RoPE of Q and K into the gather (bsa_permute_norm_rope)")
    ap.add_argument("--causal-frames", type=int, default=0, metavar="F",
                    help="frame-chunk causal selection (bsa_select_causal) with chunks of F frames")
    ap.add_argument("--reuse-every", type=int, default=1, metavar="R",
                    help="recompute zone shapes and block lists every R steps and reuse them in "
                         "between (forward-only; ms/layer is the average over the steps)")
    ap.add_argument("--xattn", action="store_true",
                    help="time the A2V cross-attention layer (forward + backward) at the "
                         "workload's token count instead of the BSA layer")
    ap.add_argument("--unfused", action="store_true",
                    help="time bsa_permute + bsa_pool_select instead of bsa_permute_pool + bsa_select")
    ap.add_argument("--permuted", action="store_true",
                    help="store block-ordered Q, K, V (bsa_permute_pool) and run "
                         "bsa_attn_fwd_raster on them instead of bsa_attn_fwd_gather; with "
                         "the backward, bsa_attn_bwd + bsa_unpermute of the gradients instead "
                         "of bsa_attn_bwd_raster")
    return ap.parse_args()


def device_copy_gbps():
    """Read + write rate of a plain 1 GiB device-to-device copy (event-timed),
    the practical ceiling of a stage that reads and writes every byte once."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 10
    del a, b
    return 2 * n / (ms * 1e-3) / 1e9


def hbm_stages(wl, sizes, stage_ms, copy_gbps):
    """Algorithmic HBM bytes of the data-movement stages and the rate they reach
    in the event-timed stage time, against the 8 TB/s HBM peak and against the
    measured rate of a plain device copy."""
    N, Np, H, d = sizes["n_tokens"], sizes["n_padded"], wl.heads, wl.d
    e = 2  # bf16
    M = sizes["n_blocks"]
    alg = {}
    if "unpermute" in stage_ms:
        alg["unpermute"] = 2 * H * N * d * e           # O: read real slots, write raster rows
    if "pool" in stage_ms:                             # Q, K read; fp64 block means written
        alg["pool"] = 2 * H * N * d * e + 2 * H * M * d * 8
    elif "permute" in stage_ms:
        alg["permute"] = 3 * H * (N + Np) * d * e      # Q, K, V: read real rows, write padded
        alg["pool_select"] = 2 * H * N * d * e         # pooling reads the real rows of Qp, Kp
    else:                                              # + the fp64 block means of Q and K
        name = "permute_norm_rope" if "permute_norm_rope" in stage_ms else "permute_pool"
        alg[name] = 3 * H * (N + Np) * d * e + 2 * H * M * d * 8
    if "reuse_permute" in stage_ms:                    # reuse steps: gather without pooling
        alg["reuse_permute"] = 3 * H * (N + Np) * d * e
    if wl.mode == "dynamic":
        alg["zone_score"] = N * wl.video_channels * e + wl.n_audio * wl.video_channels * e
    if wl.backward:
        alg["permute_dO"] = H * (N + Np) * d * e
    if "unpermute_grads" in stage_ms:
        alg["unpermute_grads"] = 3 * 2 * H * N * d * 4  # fp32 dQ, dK, dV
    out = {}
    for stage, nbytes in alg.items():
        ms = stage_ms[stage]
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[stage] = {"ms": round(ms, 4), "alg_GB": round(nbytes / 1e9, 4), "alg_GBps": round(gbs, 1),
                      "frac_of_8TBps": round(gbs / PEAK_HBM_GBS, 3),
                      "frac_of_copy": round(gbs / copy_gbps, 3)}
    out["device_copy_GBps"] = round(copy_gbps, 1)
    return out


def measured_traffic(workload):
    """HBM bytes per attention-forward launch from the committed counter runs
    (profiles/attn_fwd_720p_traffic.md), or None when they do not apply: another
    workload, or kernel sources changed since the counters were taken."""
    import hashlib
    if workload != "720p":
        return None
    path = os.path.join(ROOT, "profiles", "attn_fwd_720p_traffic.md")
    try:
        fields = dict(line.split(": ", 1) for line in open(path).read().splitlines()
                      if line.startswith(("traffic_bytes_per_launch: ", "source_sha256: ")))
    except OSError:
        return None
    h = hashlib.sha256()
    for src in ("attn_fwd.hip", "attn_common.hpp", "kernels.hpp"):
        with open(os.path.join(ROOT, "video_diffusion_block_amd", "csrc", src), "rb") as f:
            h.update(f.read())
    if fields.get("source_sha256", "").strip() != h.hexdigest():
        return None
    return int(fields["traffic_bytes_per_launch"])


def skipped_pair_products(pad_hi, counts, idx):
    """Number of half-block products (B^2 d FLOPs each) of the selected pairs
    that the forward kernel does not issue. pad_hi[j]: key block j's upper 64
    keys are all pad. For such a listed block the upper key-half wave skips
    that half's S product (not for the first list entry, which every wave
    computes before its loop) and, when the next listed block is such a block
    too or it is the last one, that half's PV product."""
    import torch
    M = counts.shape[1]
    n = counts.long()
    j = torch.arange(M, device=counts.device)
    valid = j[None, None, :] < n[..., None]
    p = pad_hi[idx.long().clamp(0, M - 1)] & valid
    nxt = torch.zeros_like(p)
    nxt[..., :-1] = p[..., 1:]
    last = j[None, None, :] == (n[..., None] - 1)
    skip_s = p.clone()
    skip_s[..., 0] = False
    skip_pv = p & (nxt | last)
    return int(skip_s.sum()) + int(skip_pv.sum())


def skipped_pad_half_flops(lay, zs, counts, idx, B, d):
    """FLOPs of the selected block pairs that the forward kernel does not
    issue (skipped_pair_products x B^2 d). Pad slots are found by permuting a
    tensor of ones."""
    import torch
    from video_diffusion_block_amd import ops
    N = lay.sizes()["n_tokens"]
    ones = torch.ones((1, N, d), dtype=torch.bfloat16, device=counts.device)
    (perm,) = ops.permute(lay, zs, [ones])
    M = counts.shape[1]
    pad_hi = ~(perm[0, :, 0] != 0).view(M, B)[:, B // 2:].any(dim=1)
    return float(skipped_pair_products(pad_hi, counts, idx)) * B * B * d


def copy_calib():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(10):
        b.copy_(a)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / 10
    print(json.dumps({"copy_bytes": n, "copy_GBps": 2 * n / dt / 1e9}))


def xattn_bench(args, wl):
    """The A2V cross-attention layer at the workload's video token count:
    C = 1536 channels, 200 audio tokens, 12 heads of 128; seeded synthetic
    features, weights N(0, 1/fan_in) and output gradient (no trained weights)."""
    import numpy as np
    import torch
    import synth
    from video_diffusion_block_amd import ops
    dev = torch.device("cuda:0")
    grid = wl.grid
    N, C, Na, H = int(np.prod(grid)), 1536, 200, 12
    D = 128 * H
    rng = np.random.default_rng(11)

    def bf(x):
        return torch.from_numpy(synth.f32_to_bf16_bits(np.asarray(x, np.float32))
                                .view(np.int16)).view(torch.bfloat16).to(dev)

    x = bf(synth.bf16_bits_to_f32(synth.smooth_field(1, grid, C, 4)[0]))
    a = bf(synth.gaussian_noise((Na, C), 5))
    w = [bf(rng.normal(size=(D, C)) / np.sqrt(C)) for _ in range(3)] + \
        [bf(rng.normal(size=(C, D)) / np.sqrt(D))]
    g = torch.Generator(device=dev).manual_seed(6)
    dy = torch.randn((N, C), generator=g, device=dev).to(torch.bfloat16)
    evs = []
    for it in range(args.warmup + args.steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        y, saved = ops.xattn_fwd(x, a, *w, H)
        e[1].record()
        ops.xattn_bwd(x, a, *w, H, saved, dy)
        e[2].record()
        if it >= args.warmup:
            evs.append(e)
    torch.cuda.synchronize()
    fwd_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    bwd_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    proj = 2.0 * N * C * D                       # one video-side projection GEMM
    audio = 2.0 * Na * C * D                     # one audio-side projection GEMM
    core = 2.0 * N * Na * D                      # one attention product (S, PV, ...)
    fwd_fl = 2 * proj + 2 * audio + 2 * core     # Q, Y; K, V; S, PV
    bwd_fl = 4 * proj + 4 * audio + 7 * core     # dO, dWo, dX, dWq; dA x2, dWk, dWv;
    #                                              dQ pass: S, dP, dQ; dK/dV pass: S, dP, dV, dK
    res = {
        "metric": "A2V cross-attention layer ms (forward + backward) and executed TFLOP/s",
        "value": round((fwd_fl + bwd_fl) / ((fwd_ms + bwd_ms) * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s (executed FLOPs per layer time)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(fwd_ms + bwd_ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded features, weights, dY)",
        "config": {"workload": f"xattn-{wl.name}", "video_tokens": N, "audio_tokens": Na,
                   "channels": C, "heads": H, "d": 128},
        "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
        "fwd_TFLOPs": round(fwd_fl / (fwd_ms * 1e-3) / 1e12, 2),
        "bwd_TFLOPs": round(bwd_fl / (bwd_ms * 1e-3) / 1e12, 2),
        "pct_bf16_peak": round(100 * (fwd_fl + bwd_fl) / ((fwd_ms + bwd_ms) * 1e-3) / 1e12
                               / PEAK_BF16_TFLOPS, 2),
    }
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: measures one GPU only; the path shards by head "
              "across GPUs but no multi-GPU run is provided (use --gpus 1).", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import synth
    from video_diffusion_block_amd import ops

    if args.copy_calib:
        copy_calib()
        return

    wl = synth.WORKLOADS[args.workload]
    if args.xattn:
        xattn_bench(args, wl)
        return
    if args.causal_frames and args.unfused:
        sys.exit("--causal-frames selects from the gather's block means; it does not combine "
                 "with --unfused")
    if args.reuse_every < 1:
        sys.exit("--reuse-every must be >= 1")
    if args.reuse_every > 1 and (wl.backward or args.unfused or args.norm_rope):
        sys.exit("--reuse-every applies to the default forward-only sequence")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t_gen = time.perf_counter()
    parts = ("q", "k", "v") + (("video", "audio") if wl.mode == "dynamic" else ()) + \
            (("do",) if wl.backward else ())
    inp = synth.make_inputs(wl, parts=parts)

    def to_dev(x):
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = (to_dev(inp[p]) for p in "qkv")
    video = to_dev(inp["video"]) if "video" in inp else None
    audio = to_dev(inp["audio"]) if "audio" in inp else None
    do = to_dev(inp["do"]) if "do" in inp else None
    t_gen = time.perf_counter() - t_gen
    lay = (ops.BSALayout.fixed(wl.grid, wl.block) if wl.mode == "fixed"
           else ops.BSALayout.dynamic(wl.grid, wl.block))
    sizes = lay.sizes()
    # synthetic RMSNorm channel weights of Q and K (seeded; no trained weights)
    grng = np.random.default_rng(7)
    gammas = [torch.from_numpy(grng.uniform(0.5, 1.5, wl.d).astype(np.float32)).to(dev)
              for _ in range(2)]

    # forward-only sequences write O in raster order from the attention kernel
    # (bsa_attn_fwd_raster); the backward needs the permuted O, so a backward
    # workload keeps bsa_attn_fwd + bsa_unpermute. The default forward-only
    # sequence also reads Q, K, V in token order (bsa_attn_fwd_gather: every
    # block shape of these layouts is a multiple of 4 tokens wide)
    raster = not wl.backward and not args.unfused
    gather = (raster and not args.permuted and not args.norm_rope and
              ops.gather_supported(lay, q.dtype, wl.d))
    state = {"step": 0}

    def step(record):
        s = torch.cuda.current_stream()
        marks = []

        def mark(name):
            if record:
                e = torch.cuda.Event(enable_timing=True)
                e.record(s)
                marks.append((name, e))

        reuse = args.reuse_every > 1 and state["step"] % args.reuse_every != 0
        state["step"] += 1
        mark(None)
        if reuse:   # zone shapes and lists of the last refresh; this step's Q, K, V
            zs, counts, idx = state["zs"], state["counts"], state["idx"]
            if gather:
                o, lse = ops.attn_fwd_gather(lay, zs, q, k, v, counts, idx)
            else:
                qp, kp, vp = ops.permute(lay, zs, [q, k, v])
                mark("reuse_permute")
                o, lse = ops.attn_fwd_raster(lay, zs, qp, kp, vp, counts, idx)
            mark("reuse_attn_fwd")
            if record:
                ev_marks.append(marks)
            return
        zs = ops.zone_score(lay, video, audio)
        mark("zone_score")
        if gather:
            _, (qbar, kbar) = ops.permute_pool(lay, zs, [q, k], npool=2, store=False)
            mark("pool")
            if args.causal_frames:
                counts, idx = ops.select_causal(lay, zs, qbar, kbar, wl.sparsity_1e4, wl.tau,
                                                args.causal_frames)
            else:
                counts, idx = ops.select(lay, zs, qbar, kbar, wl.sparsity_1e4, wl.tau)
            mark("select")
        elif args.unfused:
            qp, kp, vp = ops.permute(lay, zs, [q, k, v])
            mark("permute")
            counts, idx = ops.pool_select(lay, zs, qp, kp, wl.sparsity_1e4, wl.tau)
            mark("pool_select")
        else:
            if args.norm_rope:
                (qp, kp, vp), (qbar, kbar) = ops.permute_norm_rope(lay, zs, [q, k, v], gammas)
                mark("permute_norm_rope")
            else:
                (qp, kp, vp), (qbar, kbar) = ops.permute_pool(lay, zs, [q, k, v], npool=2)
                mark("permute_pool")
            if args.causal_frames:
                counts, idx = ops.select_causal(lay, zs, qbar, kbar, wl.sparsity_1e4, wl.tau,
                                                args.causal_frames)
            else:
                counts, idx = ops.select(lay, zs, qbar, kbar, wl.sparsity_1e4, wl.tau)
            mark("select")
        if gather:
            o, lse = ops.attn_fwd_gather(lay, zs, q, k, v, counts, idx)
            mark("attn_fwd")
        elif raster:
            o, lse = ops.attn_fwd_raster(lay, zs, qp, kp, vp, counts, idx)
            mark("attn_fwd")
        else:
            op, lse = ops.attn_fwd(lay, zs, qp, kp, vp, counts, idx)
            mark("attn_fwd")
            (o,) = ops.unpermute(lay, zs, [op])
            mark("unpermute")
        if wl.backward:
            (dop,) = ops.permute(lay, zs, [do])
            mark("permute_dO")
            if args.permuted or args.unfused:
                grads = ops.attn_bwd(lay, zs, qp, kp, vp, op, dop, lse, counts, idx)
                mark("attn_bwd")
                ops.unpermute(lay, zs, list(grads))
                mark("unpermute_grads")
            else:  # gradients written in raster order by the backward kernels
                grads = ops.attn_bwd_raster(lay, zs, qp, kp, vp, op, dop, lse, counts, idx)
                mark("attn_bwd")
        state.update(zs=zs, counts=counts, idx=idx)
        if record:
            ev_marks.append(marks)

    ev_marks = []
    for _ in range(args.warmup):
        step(False)
    state["step"] = 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # stage times: refresh steps under their stage names, reuse steps (which
    # skip zone scoring, pooling and selection) under "reuse_<stage>"
    ev = {}
    for marks in ev_marks:
        for (_, a), (name, b) in zip(marks, marks[1:]):
            ev.setdefault(name, []).append(a.elapsed_time(b))
    stage_ms = {s: float(np.mean(v)) for s, v in ev.items()}
    ms_per_step = wall * 1e3 / args.steps

    counts = state["counts"].cpu().numpy().astype(np.int64)
    B, d = sizes["block_tokens"], wl.d
    pairs = int(counts.sum())
    fwd_flops = pairs * 4.0 * B * B * d               # QK^T and PV per (query block, key block)
    bwd_flops = pairs * 10.0 * B * B * d if wl.backward else 0.0
    N, H = sizes["n_tokens"], wl.heads
    eff_flops = 4.0 * N * N * d * H * (3.5 if wl.backward else 1.0)
    layer_flops = fwd_flops + bwd_flops
    attn_ms = stage_ms["attn_fwd"]
    value = layer_flops / (ms_per_step * 1e-3) / 1e12
    # the forward kernel's issued matrix-unit work: the pair FLOPs minus the
    # products it skips on key halves that are all pad (reported beside the
    # roofline, whose figure is the per-pair executed work)
    fwd_issued = fwd_flops - skipped_pad_half_flops(lay, state["zs"], state["counts"],
                                                    state["idx"], B, d)

    result = {
        "metric": "BSA ms/layer + executed TFLOP/s (% bf16 MFMA peak), 720p s=0.85",
        "value": round(value, 2),
        "unit": "TFLOP/s (executed attention FLOPs per layer time)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_layer": round(ms_per_step, 4),
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "effective_TFLOPs": round(eff_flops / (ms_per_step * 1e-3) / 1e12, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded smooth field + noise latents)",
        "config": {"workload": wl.name, "grid": list(wl.grid), "tokens": N, "heads": H, "d": d,
                   "blocks": sizes["n_blocks"], "sparsity": wl.sparsity_1e4 / 1e4, "tau": wl.tau,
                   "mode": wl.mode, "backward": wl.backward,
                   "sequence": ("unfused" if args.unfused else
                                "norm_rope+pool" if args.norm_rope else
                                "pool, gathering attention" if gather else "pool") +
                               (", raster O" if raster else "") +
                               (", raster gradients" if wl.backward and not (args.permuted or
                                                                           args.unfused) else "") +
                               (f", causal chunks of {args.causal_frames} frames"
                                if args.causal_frames else "") +
                               (f", lists reused for {args.reuse_every} steps"
                                if args.reuse_every > 1 else ""),
                   "mean_list": round(pairs / max(1, int((counts > 0).sum())), 2)},
        "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "roofline": {
            "kernel": "attn_fwd_mfma<true>" if gather else "attn_fwd_mfma<false>",
            "bound": "mfma",
            "achieved": round(fwd_flops / (attn_ms * 1e-3) / 1e12, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(fwd_flops / (attn_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "work": "4 B^2 d FLOPs per selected (query block, key block) pair",
            "issued_of_pair_flops": round(fwd_issued / max(fwd_flops, 1.0), 4),
            "issued_achieved": round(fwd_issued / (attn_ms * 1e-3) / 1e12, 2),
            "issued_frac": round(fwd_issued / (attn_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "traffic": None if args.causal_frames else measured_traffic(wl.name),
        },
        "hbm_stages": hbm_stages(wl, sizes, stage_ms, device_copy_gbps()),
        "input_gen_s": round(t_gen, 1),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, inp, counts, sample=args.cpu_sample)
    print(json.dumps(result), flush=True)


def cpu_baseline(wl, inp, counts_gpu, sample: bool = False):
    """The fp64 oracle on the host cores, in the same unit (executed attention
    TFLOP/s over the layer): by default the whole layer (selection for every
    head, gathered attention for every (head, query block) pair); with
    ``sample`` a bounded sample (6 heads, 420 query blocks each) scaled up."""
    import numpy as np

    import synth
    from oracle import attention as oatt
    from oracle import pipeline as opipe

    threads = len(os.sched_getaffinity(0))
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():  # numpy's BLAS pool size
        threads = min(threads, int(os.environ["OMP_NUM_THREADS"]))
    hs = 6 if sample else wl.heads
    q = synth.bf16_bits_to_f64(inp["q"][:hs])
    k = synth.bf16_bits_to_f64(inp["k"][:hs])
    v = synth.bf16_bits_to_f64(inp["v"][:hs])
    t0 = time.perf_counter()
    r = opipe.run_selection(wl.grid, wl.mode, wl.block, q, k, wl.sparsity_1e4, wl.tau)
    t_sel = time.perf_counter() - t0
    L = r["layout"]
    B = L.block_tokens
    total_pairs = int(counts_gpu.sum())
    flops = total_pairs * 4.0 * B * B * wl.d
    if sample:
        rng = np.random.default_rng(0)
        nonempty = np.nonzero(r["counts"] > 0)[0]
        per_head = min(420, len(nonempty))
        pairs = [(h, int(i)) for h in range(hs) for i in rng.choice(nonempty, per_head, replace=False)]
    else:
        pairs = None  # every (head, query block)
    t0 = time.perf_counter()
    oatt.attn_fwd_gathered(L, r["perm"], q, k, v, r["lists"], 1 / np.sqrt(wl.d), pairs=pairs)
    t_att = time.perf_counter() - t0
    if not sample:
        oracle_pairs = int(sum(len(r["lists"][h][i]) for h in range(hs) for i in range(L.n_blocks)))
        layer_s = t_sel + t_att
        return {"value": round(flops / layer_s / 1e12, 5),
                "unit": "TFLOP/s (executed attention FLOPs per layer time)",
                "cores": threads, "kind": "oracle",
                "layer_s": round(layer_s, 1),
                "sample": f"whole layer: oracle selection for all {wl.heads} heads "
                          f"({t_sel:.1f} s) and gathered fp64 attention for every "
                          f"(head, query block) ({oracle_pairs} block pairs, {t_att:.1f} s)"}
    sample_pairs = sum(len(r["lists"][h][i]) for h, i in pairs)
    per_pair = t_att / sample_pairs
    layer_s = t_sel * wl.heads / hs + per_pair * total_pairs
    return {"value": round(flops / layer_s / 1e12, 5),
            "unit": "TFLOP/s (executed attention FLOPs per layer time)",
            "cores": threads, "kind": "oracle",
            "layer_s_est": round(layer_s, 1),
            "sample": f"oracle selection for {hs} of {wl.heads} heads ({t_sel:.1f} s) and "
                      f"gathered fp64 attention on {len(pairs)} (head, query block) pairs "
                      f"({sample_pairs} block pairs, {t_att:.1f} s), scaled to all "
                      f"{wl.heads} heads and {total_pairs} block pairs"}


if __name__ == "__main__":
    main()
