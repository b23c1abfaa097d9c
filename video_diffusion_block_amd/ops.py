"""Thin torch-facing wrappers of the C ABI (argument marshalling only).

Every step runs in the HIP kernels of ``libbsa.so``; these functions only
allocate outputs/workspaces with torch (device memory) and pass pointers and
the current HIP stream. Names follow the C entry points (``bsa_<name>``).
Inputs must be contiguous device tensors (torch.float32 or torch.bfloat16).
"""
from __future__ import annotations

import ctypes
import dataclasses
import math

import torch

from . import _lib

CANDIDATES = ((2, 8, 8), (4, 4, 8), (1, 8, 16))
ZONE = (4, 16, 16)


@dataclasses.dataclass(frozen=True)
class BSALayout:
    """Token layout: grid, mode, zone extent and candidate block shapes."""

    grid: tuple
    mode: int
    zone: tuple
    shapes: tuple

    @staticmethod
    def fixed(grid, block) -> "BSALayout":
        return BSALayout(tuple(grid), _lib.BSA_MODE_FIXED, tuple(block), (tuple(block),))

    @staticmethod
    def dynamic(grid, zone=ZONE, shapes=CANDIDATES) -> "BSALayout":
        return BSALayout(tuple(grid), _lib.BSA_MODE_DYNAMIC, tuple(zone),
                         tuple(tuple(s) for s in shapes))

    def c(self) -> _lib.Layout:
        L = _lib.Layout()
        for a in range(3):
            L.grid[a] = int(self.grid[a])
            L.zone[a] = int(self.zone[a])
        L.mode = int(self.mode)
        L.n_shapes = len(self.shapes)
        for s, shp in enumerate(self.shapes):
            for a in range(3):
                L.shapes[s][a] = int(shp[a])
        return L

    def sizes(self) -> dict:
        lib = _lib.load()
        n, npad = ctypes.c_int64(), ctypes.c_int64()
        m, nz, b = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        L = self.c()
        _lib.check("bsa_layout_sizes", lib.bsa_layout_sizes(
            ctypes.byref(L), ctypes.byref(n), ctypes.byref(npad), ctypes.byref(m),
            ctypes.byref(nz), ctypes.byref(b)))
        return dict(n_tokens=n.value, n_padded=npad.value, n_blocks=m.value, n_zones=nz.value,
                    block_tokens=b.value)


_POISON = False


def poison_outputs(enable: bool = True) -> None:
    """Fill every output and workspace this module allocates with 0xFF bytes
    before the call (NaN in floating point, -1 in int32), so that a kernel that
    leaves part of its output unwritten, or reads workspace it did not write,
    is seen by the caller. A testing aid; off by default."""
    global _POISON
    _POISON = bool(enable)


def _empty(shape, dtype, device) -> torch.Tensor:
    t = torch.empty(shape, dtype=dtype, device=device)
    if _POISON:
        t.view(torch.uint8).fill_(0xFF)
    return t


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return _lib.BSA_BF16
    if t.dtype == torch.float32:
        return _lib.BSA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("tensors must live on the GPU")
            if not t.is_contiguous():
                raise ValueError("tensors must be contiguous")


def _workspace(call: int, layout: BSALayout, heads: int, d: int, device) -> torch.Tensor:
    L = layout.c()
    n = _lib.load().bsa_workspace_size(call, ctypes.byref(L), heads, d)
    return _empty(max(int(n), 256), torch.uint8, device)


def zone_score(layout: BSALayout, video: torch.Tensor | None, audio: torch.Tensor | None,
               with_stats: bool = False):
    """bsa_zone_score: shape id per zone (int32 [n_zones]) and optionally the
    per-zone (V_a, G_a) statistics (float64 [n_zones, 3, 2])."""
    lib = _lib.load()
    sz = layout.sizes()
    dev = video.device if video is not None else torch.device("cuda")
    _dev(video, audio)
    zs = _empty(sz["n_zones"], torch.int32, dev)
    stats = _empty((sz["n_zones"], 3, 2), torch.float64, dev) if with_stats else None
    C = 0 if video is None else video.shape[1]
    na = 0 if audio is None else audio.shape[0]
    ws = _workspace(_lib.BSA_CALL_ZONE_SCORE, layout, 1, max(C, 1), dev)
    L = layout.c()
    _lib.check("bsa_zone_score", lib.bsa_zone_score(
        ctypes.byref(L), _ptr(video), C, _ptr(audio), na, _ptr(zs), _ptr(stats), _ptr(ws),
        ws.numel(), _stream()))
    return (zs, stats) if with_stats else zs


def _permute_call(name, layout, zone_shape, srcs, dsts):
    lib = _lib.load()
    H, _, d = srcs[0].shape
    n = len(srcs)
    src_arr = (ctypes.c_void_p * n)(*[t.data_ptr() for t in srcs])
    dst_arr = (ctypes.c_void_p * n)(*[t.data_ptr() for t in dsts])
    L = layout.c()
    fn = getattr(lib, name)
    _lib.check(name, fn(ctypes.byref(L), _ptr(zone_shape), n, src_arr, dst_arr, H, d,
                        _dtype(srcs[0]), _stream()))


def permute(layout: BSALayout, zone_shape, tensors):
    """bsa_permute: list of [H, N, d] -> list of [H, Np, d] (one launch)."""
    _dev(zone_shape, *tensors)
    npad = layout.sizes()["n_padded"]
    outs = [_empty((t.shape[0], npad, t.shape[2]), t.dtype, t.device)
            for t in tensors]
    _permute_call("bsa_permute", layout, zone_shape, list(tensors), outs)
    return outs


def permute_pool(layout: BSALayout, zone_shape, tensors, npool: int = 2, store: bool = True):
    """bsa_permute_pool: the gathered tensors (as permute) and the fp64 block
    means [H, M, d] of the first npool of them, from one launch. store=False
    (pooled tensors only, ntensors == npool): the means alone, no gathered
    copies (outs is then a list of None)."""
    lib = _lib.load()
    _dev(zone_shape, *tensors)
    sz = layout.sizes()
    if not store and npool != len(tensors):
        raise ValueError("store=False pools every tensor it is given (npool == len(tensors))")
    outs = [_empty((t.shape[0], sz["n_padded"], t.shape[2]), t.dtype, t.device) if store else None
            for t in tensors]
    means = [_empty((t.shape[0], sz["n_blocks"], t.shape[2]), torch.float64, t.device)
             for t in tensors[:npool]]
    H, _, d = tensors[0].shape
    n = len(tensors)
    src_arr = (ctypes.c_void_p * n)(*[t.data_ptr() for t in tensors])
    dst_arr = (ctypes.c_void_p * n)(*[t.data_ptr() if t is not None else None for t in outs])
    mean_arr = (ctypes.c_void_p * max(npool, 1))(*[t.data_ptr() for t in means])
    L = layout.c()
    _lib.check("bsa_permute_pool", lib.bsa_permute_pool(
        ctypes.byref(L), _ptr(zone_shape), n, src_arr, dst_arr, H, d, _dtype(tensors[0]), npool,
        mean_arr, _stream()))
    return outs, means


def permute_norm_rope(layout: BSALayout, zone_shape, tensors, gammas=None, eps: float = 1e-6,
                      rope_base: float = 10000.0, nrope: int = 2, npool: int = 2):
    """bsa_permute_norm_rope: the gathered tensors, the first nrope of them
    RMS-normalized (channel weights gammas[t], float32 [d] tensors or None) and
    rotated by the 3-D RoPE, plus the fp64 block means [H, M, d] of the first
    npool stored tensors, from one launch."""
    lib = _lib.load()
    _dev(zone_shape, *tensors)
    gammas = list(gammas) if gammas is not None else [None] * nrope
    for g in gammas:
        if g is not None:
            _dev(g)
            if g.dtype != torch.float32 or g.numel() != tensors[0].shape[2]:
                raise ValueError("gamma must be a float32 tensor of d elements")
    sz = layout.sizes()
    outs = [_empty((t.shape[0], sz["n_padded"], t.shape[2]), t.dtype, t.device)
            for t in tensors]
    means = [_empty((t.shape[0], sz["n_blocks"], t.shape[2]), torch.float64, t.device)
             for t in tensors[:npool]]
    H, _, d = tensors[0].shape
    n = len(tensors)
    src_arr = (ctypes.c_void_p * n)(*[t.data_ptr() for t in tensors])
    dst_arr = (ctypes.c_void_p * n)(*[t.data_ptr() for t in outs])
    mean_arr = (ctypes.c_void_p * max(npool, 1))(*[t.data_ptr() for t in means])
    gam_arr = (ctypes.c_void_p * max(nrope, 1))(*[(g.data_ptr() if g is not None else None)
                                                  for g in gammas[:nrope]])
    L = layout.c()
    _lib.check("bsa_permute_norm_rope", lib.bsa_permute_norm_rope(
        ctypes.byref(L), _ptr(zone_shape), n, src_arr, dst_arr, H, d, _dtype(tensors[0]), nrope,
        gam_arr, float(eps), float(rope_base), npool, mean_arr, _stream()))
    return outs, means


def select(layout: BSALayout, zone_shape, qbar, kbar, sparsity_1e4: int, tau: float,
           return_logits: bool = False):
    """bsa_select: counts [H, M] int32, idx [H, M, M] int32 from fp64 block
    means (and the fp64 pooled logits when asked)."""
    lib = _lib.load()
    _dev(zone_shape, qbar, kbar)
    H, M, d = qbar.shape
    counts = _empty((H, M), torch.int32, qbar.device)
    idx = _empty((H, M, M), torch.int32, qbar.device)
    logits = _empty((H, M, M), torch.float64, qbar.device) if return_logits else None
    ws = _workspace(_lib.BSA_CALL_SELECT, layout, H, d, qbar.device)
    L = layout.c()
    _lib.check("bsa_select", lib.bsa_select(
        ctypes.byref(L), _ptr(zone_shape), _ptr(qbar), _ptr(kbar), H, d, int(sparsity_1e4),
        float(tau), _ptr(counts), _ptr(idx), _ptr(logits), _ptr(ws), ws.numel(), _stream()))
    return (counts, idx, logits) if return_logits else (counts, idx)


def select_causal(layout: BSALayout, zone_shape, qbar, kbar, sparsity_1e4: int, tau: float,
                  frames_per_chunk: int):
    """bsa_select_causal: bsa_select with each query block restricted to the
    key blocks of its own and earlier chunks of frames_per_chunk frames."""
    lib = _lib.load()
    _dev(zone_shape, qbar, kbar)
    H, M, d = qbar.shape
    counts = _empty((H, M), torch.int32, qbar.device)
    idx = _empty((H, M, M), torch.int32, qbar.device)
    ws = _workspace(_lib.BSA_CALL_SELECT, layout, H, d, qbar.device)
    L = layout.c()
    _lib.check("bsa_select_causal", lib.bsa_select_causal(
        ctypes.byref(L), _ptr(zone_shape), _ptr(qbar), _ptr(kbar), H, d, int(sparsity_1e4),
        float(tau), int(frames_per_chunk), _ptr(counts), _ptr(idx), None, _ptr(ws), ws.numel(),
        _stream()))
    return counts, idx


def unpermute(layout: BSALayout, zone_shape, tensors):
    """bsa_unpermute: list of [H, Np, d] -> list of [H, N, d] (one launch)."""
    _dev(zone_shape, *tensors)
    n = layout.sizes()["n_tokens"]
    outs = [_empty((t.shape[0], n, t.shape[2]), t.dtype, t.device)
            for t in tensors]
    _permute_call("bsa_unpermute", layout, zone_shape, list(tensors), outs)
    return outs


def pool_select(layout: BSALayout, zone_shape, qp, kp, sparsity_1e4: int, tau: float,
                return_logits: bool = False):
    """bsa_pool_select: counts [H, M] int32, idx [H, M, M] int32 (and the fp64
    pooled logits when asked)."""
    lib = _lib.load()
    _dev(zone_shape, qp, kp)
    H, _, d = qp.shape
    M = layout.sizes()["n_blocks"]
    counts = _empty((H, M), torch.int32, qp.device)
    idx = _empty((H, M, M), torch.int32, qp.device)
    logits = _empty((H, M, M), torch.float64, qp.device) if return_logits else None
    ws = _workspace(_lib.BSA_CALL_POOL_SELECT, layout, H, d, qp.device)
    L = layout.c()
    _lib.check("bsa_pool_select", lib.bsa_pool_select(
        ctypes.byref(L), _ptr(zone_shape), _ptr(qp), _ptr(kp), H, d, _dtype(qp),
        int(sparsity_1e4), float(tau), _ptr(counts), _ptr(idx), _ptr(logits), _ptr(ws),
        ws.numel(), _stream()))
    return (counts, idx, logits) if return_logits else (counts, idx)


def attn_fwd(layout: BSALayout, zone_shape, qp, kp, vp, counts, idx, scale: float = 0.0):
    """bsa_attn_fwd: op [H, Np, d] (input dtype) and lse [H, Np] float32."""
    lib = _lib.load()
    _dev(zone_shape, qp, kp, vp, counts, idx)
    H, Np, d = qp.shape
    op = _empty(qp.shape, qp.dtype, qp.device)
    lse = _empty((H, Np), torch.float32, qp.device)
    ws = _workspace(_lib.BSA_CALL_ATTN_FWD, layout, H, d, qp.device)
    L = layout.c()
    _lib.check("bsa_attn_fwd", lib.bsa_attn_fwd(
        ctypes.byref(L), _ptr(zone_shape), _ptr(qp), _ptr(kp), _ptr(vp), _ptr(counts),
        _ptr(idx), H, d, _dtype(qp), float(scale), _ptr(op), _ptr(lse), _ptr(ws), ws.numel(),
        _stream()))
    return op, lse


def attn_fwd_noalloc(layout: BSALayout, zone_shape, qp, kp, vp, counts, idx,
                     scale: float = 0.0, out=None):
    """bsa_attn_fwd_noalloc: bsa_attn_fwd with the library's static scratch
    instead of a workspace (the C call allocates nothing). ``out``: (op, lse)
    to write into, else they are allocated here like bsa_attn_fwd's."""
    lib = _lib.load()
    _dev(zone_shape, qp, kp, vp, counts, idx)
    H, Np, d = qp.shape
    if out is None:
        op = _empty(qp.shape, qp.dtype, qp.device)
        lse = _empty((H, Np), torch.float32, qp.device)
    else:
        op, lse = out
        _dev(op, lse)
    L = layout.c()
    _lib.check("bsa_attn_fwd_noalloc", lib.bsa_attn_fwd_noalloc(
        ctypes.byref(L), _ptr(zone_shape), _ptr(qp), _ptr(kp), _ptr(vp), _ptr(counts),
        _ptr(idx), H, d, _dtype(qp), float(scale), _ptr(op), _ptr(lse), _stream()))
    return op, lse


def attn_fwd_raster(layout: BSALayout, zone_shape, qp, kp, vp, counts, idx, scale: float = 0.0):
    """bsa_attn_fwd_raster: o [H, N, d] (raster token order, input dtype) and
    lse [H, N] float32."""
    lib = _lib.load()
    _dev(zone_shape, qp, kp, vp, counts, idx)
    H, Np, d = qp.shape
    N = layout.sizes()["n_tokens"]
    o = _empty((H, N, d), qp.dtype, qp.device)
    lse = _empty((H, N), torch.float32, qp.device)
    ws = _workspace(_lib.BSA_CALL_ATTN_FWD, layout, H, d, qp.device)
    L = layout.c()
    _lib.check("bsa_attn_fwd_raster", lib.bsa_attn_fwd_raster(
        ctypes.byref(L), _ptr(zone_shape), _ptr(qp), _ptr(kp), _ptr(vp), _ptr(counts),
        _ptr(idx), H, d, _dtype(qp), float(scale), _ptr(o), _ptr(lse), _ptr(ws), ws.numel(),
        _stream()))
    return o, lse


def gather_supported(layout: BSALayout, dtype, d: int) -> bool:
    """Whether bsa_attn_fwd_gather takes this configuration: bf16, d = 128,
    128-token blocks, every candidate block shape a multiple of 4 tokens wide."""
    return (dtype == torch.bfloat16 and d == 128 and layout.sizes()["block_tokens"] == 128
            and all(int(shp[2]) % 4 == 0 for shp in layout.shapes))


def attn_fwd_gather(layout: BSALayout, zone_shape, q, k, v, counts, idx, scale: float = 0.0):
    """bsa_attn_fwd_gather: q, k, v in raster token order [H, N, d] (bf16);
    o [H, N, d] and lse [H, N] float32 in the same order."""
    lib = _lib.load()
    _dev(zone_shape, q, k, v, counts, idx)
    H, N, d = q.shape
    if N != layout.sizes()["n_tokens"]:
        raise ValueError(f"q has {N} tokens, the layout {layout.sizes()['n_tokens']}")
    o = _empty((H, N, d), q.dtype, q.device)
    lse = _empty((H, N), torch.float32, q.device)
    ws = _workspace(_lib.BSA_CALL_ATTN_FWD, layout, H, d, q.device)
    L = layout.c()
    _lib.check("bsa_attn_fwd_gather", lib.bsa_attn_fwd_gather(
        ctypes.byref(L), _ptr(zone_shape), _ptr(q), _ptr(k), _ptr(v), _ptr(counts),
        _ptr(idx), H, d, _dtype(q), float(scale), _ptr(o), _ptr(lse), _ptr(ws), ws.numel(),
        _stream()))
    return o, lse


def attn_bwd(layout: BSALayout, zone_shape, qp, kp, vp, op, dop, lse, counts, idx,
             scale: float = 0.0):
    """bsa_attn_bwd: dqp, dkp, dvp [H, Np, d], float32 for any input dtype."""
    lib = _lib.load()
    _dev(zone_shape, qp, kp, vp, op, dop, lse, counts, idx)
    H, Np, d = qp.shape
    dq, dk, dv = (_empty(qp.shape, torch.float32, qp.device) for _ in range(3))
    ws = _workspace(_lib.BSA_CALL_ATTN_BWD, layout, H, d, qp.device)
    L = layout.c()
    _lib.check("bsa_attn_bwd", lib.bsa_attn_bwd(
        ctypes.byref(L), _ptr(zone_shape), _ptr(qp), _ptr(kp), _ptr(vp), _ptr(op), _ptr(dop),
        _ptr(lse), _ptr(counts), _ptr(idx), H, d, _dtype(qp), float(scale), _ptr(dq), _ptr(dk),
        _ptr(dv), _ptr(ws), ws.numel(), _stream()))
    return dq, dk, dv


def attn_bwd_raster(layout: BSALayout, zone_shape, qp, kp, vp, op, dop, lse, counts, idx,
                    scale: float = 0.0):
    """bsa_attn_bwd_raster: dq, dk, dv [H, N, d] float32 in raster token order
    (inputs in block order, as bsa_attn_bwd)."""
    lib = _lib.load()
    _dev(zone_shape, qp, kp, vp, op, dop, lse, counts, idx)
    H, Np, d = qp.shape
    N = layout.sizes()["n_tokens"]
    dq, dk, dv = (_empty((H, N, d), torch.float32, qp.device) for _ in range(3))
    ws = _workspace(_lib.BSA_CALL_ATTN_BWD, layout, H, d, qp.device)
    L = layout.c()
    _lib.check("bsa_attn_bwd_raster", lib.bsa_attn_bwd_raster(
        ctypes.byref(L), _ptr(zone_shape), _ptr(qp), _ptr(kp), _ptr(vp), _ptr(op), _ptr(dop),
        _ptr(lse), _ptr(counts), _ptr(idx), H, d, _dtype(qp), float(scale), _ptr(dq), _ptr(dk),
        _ptr(dv), _ptr(ws), ws.numel(), _stream()))
    return dq, dk, dv


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def xattn_fwd(x, a, wq, wk, wv, wo, heads: int):
    """bsa_xattn_fwd: the A2V cross-attention layer forward. x [N, C], a [Na, C],
    wq/wk/wv [128 heads, C], wo [C, 128 heads] (bf16). Returns y [N, C] and the
    tensors the backward takes: dict(q, k, v, o, lse)."""
    lib = _lib.load()
    _dev(x, a, wq, wk, wv, wo)
    N, C = x.shape
    Na = a.shape[0]
    D = wq.shape[0]
    dev = x.device
    bf = torch.bfloat16
    q = _empty((N, D), bf, dev)
    k = _empty((Na, D), bf, dev)
    v = _empty((Na, D), bf, dev)
    o = _empty((N, D), bf, dev)
    lse = _empty((heads, N), torch.float32, dev)
    y = _empty((N, C), bf, dev)
    _lib.check("bsa_xattn_fwd", lib.bsa_xattn_fwd(
        N, Na, C, heads, D // max(1, heads), _ptr(x), _ptr(a), _ptr(wq), _ptr(wk), _ptr(wv),
        _ptr(wo), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(y), _stream()))
    return y, {"q": q, "k": k, "v": v, "o": o, "lse": lse}


def xattn_bwd(x, a, wq, wk, wv, wo, heads: int, saved: dict, dy):
    """bsa_xattn_bwd: fp32 gradients dict(dx, da, dwq, dwk, dwv, dwo) of
    sum(Y * dy), from the forward's saved tensors."""
    lib = _lib.load()
    _dev(x, a, wq, wk, wv, wo, dy)
    N, C = x.shape
    Na = a.shape[0]
    D = wq.shape[0]
    dev = x.device
    f = torch.float32
    out = {"dx": _empty((N, C), f, dev),
           "da": _empty((Na, C), f, dev),
           "dwq": _empty((D, C), f, dev),
           "dwk": _empty((D, C), f, dev),
           "dwv": _empty((D, C), f, dev),
           "dwo": _empty((C, D), f, dev)}
    nbytes = lib.bsa_xattn_bwd_workspace_size(N, Na, C, heads)
    if nbytes == 0:
        raise _lib.BSAError("bsa_xattn_bwd_workspace_size", _lib.BSA_INVALID_ARG)
    ws = _empty(nbytes, torch.uint8, dev)
    _lib.check("bsa_xattn_bwd", lib.bsa_xattn_bwd(
        N, Na, C, heads, D // max(1, heads), _ptr(x), _ptr(a), _ptr(wq), _ptr(wk), _ptr(wv),
        _ptr(wo), _ptr(saved["q"]), _ptr(saved["k"]), _ptr(saved["v"]), _ptr(saved["o"]),
        _ptr(saved["lse"]), _ptr(dy), _ptr(out["dx"]), _ptr(out["da"]), _ptr(out["dwq"]),
        _ptr(out["dwk"]), _ptr(out["dwv"]), _ptr(out["dwo"]), _ptr(ws), nbytes, _stream()))
    return out
