"""Host-side checks of the C ABI (no GPU needed, no kernel is launched).

The library must load, export every entry point declared in include/bsa.h,
report layout sizes, and reject every invalid argument with the documented
status before touching the device. Every call below is built to fail
validation; the fake device pointers are never dereferenced.
"""
import ctypes
import os
import re

import pytest

from video_diffusion_block_amd import _lib
from video_diffusion_block_amd.ops import BSALayout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsa.h")
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bsa_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 11
    for name in names:
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, f"binding lacks {name}"


def test_abi_version_matches_header(lib):
    m = re.search(r"#define BSA_ABI_VERSION (\d+)", open(HEADER).read())
    assert lib.bsa_abi_version() == int(m.group(1))


def test_status_strings(lib):
    for s, name in enumerate(["BSA_OK", "BSA_INVALID_ARG", "BSA_UNSUPPORTED",
                              "BSA_WORKSPACE_TOO_SMALL", "BSA_LAYOUT", "BSA_HIP_ERROR"]):
        assert lib.bsa_status_string(s).decode() == name


@pytest.mark.parametrize("grid,mode,block,want", [
    ((3, 8, 8), "fixed", (1, 8, 8), (192, 192, 3, 3, 64)),
    ((13, 45, 80), "fixed", (2, 8, 8), (46800, 53760, 420, 420, 128)),
    ((13, 45, 80), "dynamic", (4, 16, 16), (46800, 61440, 480, 60, 128)),
    ((13, 68, 120), "dynamic", (4, 16, 16), (106080, 163840, 1280, 160, 128)),
    ((13, 90, 160), "dynamic", (4, 16, 16), (187200, 245760, 1920, 240, 128)),
])
def test_layout_sizes(grid, mode, block, want):
    L = BSALayout.fixed(grid, block) if mode == "fixed" else BSALayout.dynamic(grid, block)
    s = L.sizes()
    assert (s["n_tokens"], s["n_padded"], s["n_blocks"], s["n_zones"], s["block_tokens"]) == want


def _status_of_layout(lib, L):
    c = L.c()
    return lib.bsa_layout_sizes(ctypes.byref(c), None, None, None, None, None)


def test_invalid_layouts(lib):
    assert _status_of_layout(lib, BSALayout.fixed((0, 8, 8), (1, 8, 8))) == _lib.BSA_INVALID_ARG
    assert _status_of_layout(lib, BSALayout.dynamic((4, 16, 16), (4, 16, 16), ((3, 8, 8),))) == _lib.BSA_LAYOUT
    assert _status_of_layout(lib, BSALayout.dynamic((4, 16, 16), (4, 16, 16),
                                                    ((2, 8, 8), (2, 4, 8)))) == _lib.BSA_LAYOUT
    assert _status_of_layout(lib, BSALayout.fixed((4, 16, 16), (2, 4, 4))) == _lib.BSA_UNSUPPORTED
    assert _status_of_layout(lib, BSALayout.fixed((64, 256, 256), (2, 8, 8))) == _lib.BSA_LAYOUT
    bad = BSALayout(grid=(4, 16, 16), mode=0, zone=(4, 16, 16), shapes=((2, 8, 8),))
    assert _status_of_layout(lib, bad) == _lib.BSA_LAYOUT          # fixed: zone != shape
    bad = BSALayout(grid=(4, 16, 16), mode=7, zone=(2, 8, 8), shapes=((2, 8, 8),))
    assert _status_of_layout(lib, bad) == _lib.BSA_INVALID_ARG
    assert "mode" in lib.bsa_last_error().decode()


def test_workspace_sizes_positive(lib):
    L = BSALayout.dynamic((13, 90, 160)).c()
    for call in range(4):
        assert lib.bsa_workspace_size(call, ctypes.byref(L), 4, 128) > 0
    # the forward needs only its per-block table: 32 bytes per block
    assert lib.bsa_workspace_size(_lib.BSA_CALL_ATTN_FWD, ctypes.byref(L), 4, 128) == 1920 * 32
    bad = BSALayout.fixed((0, 1, 1), (1, 8, 8)).c()
    assert lib.bsa_workspace_size(1, ctypes.byref(bad), 4, 128) == 0


LAY = BSALayout.fixed((13, 45, 80), (2, 8, 8))
DYN = BSALayout.dynamic((13, 45, 80))


def _pool_select(lib, L=LAY, zs=FAKE, q=FAKE, k=FAKE, H=2, d=128, dt=1, S=8500, tau=0.2,
                 counts=FAKE, idx=FAKE, ws=FAKE, wsb=1 << 40):
    c = L.c()
    return lib.bsa_pool_select(ctypes.byref(c), zs, q, k, H, d, dt, S, tau, counts, idx, None,
                               ws, wsb, None)


def test_pool_select_validation(lib):
    assert _pool_select(lib, q=None) == _lib.BSA_INVALID_ARG
    assert _pool_select(lib, S=10000) == _lib.BSA_INVALID_ARG
    assert _pool_select(lib, S=-1) == _lib.BSA_INVALID_ARG
    assert _pool_select(lib, tau=0.0) == _lib.BSA_INVALID_ARG
    assert _pool_select(lib, tau=1.5) == _lib.BSA_INVALID_ARG
    assert _pool_select(lib, tau=float("nan")) == _lib.BSA_INVALID_ARG
    assert _pool_select(lib, d=96) == _lib.BSA_UNSUPPORTED
    assert _pool_select(lib, dt=7) == _lib.BSA_INVALID_ARG
    assert _pool_select(lib, H=0) == _lib.BSA_INVALID_ARG
    assert _pool_select(lib, wsb=16) == _lib.BSA_WORKSPACE_TOO_SMALL
    assert _pool_select(lib, ws=None) == _lib.BSA_WORKSPACE_TOO_SMALL
    assert _pool_select(lib, L=DYN, zs=None) == _lib.BSA_INVALID_ARG
    assert _pool_select(lib, S=12000) == _lib.BSA_INVALID_ARG
    assert "sparsity" in lib.bsa_last_error().decode()


def _attn_fwd(lib, L=LAY, q=FAKE, d=128, dt=1, scale=0.0, lse=FAKE, zs=FAKE):
    c = L.c()
    return lib.bsa_attn_fwd(ctypes.byref(c), zs, q, FAKE, FAKE, FAKE, FAKE, 2, d, dt, scale,
                            FAKE, lse, None, 0, None)


def test_attn_fwd_validation(lib):
    assert _attn_fwd(lib, q=None) == _lib.BSA_INVALID_ARG
    assert _attn_fwd(lib, lse=None) == _lib.BSA_INVALID_ARG
    assert _attn_fwd(lib, d=32) == _lib.BSA_UNSUPPORTED
    assert _attn_fwd(lib, dt=3) == _lib.BSA_INVALID_ARG
    assert _attn_fwd(lib, scale=-1.0) == _lib.BSA_INVALID_ARG
    assert _attn_fwd(lib, scale=float("inf")) == _lib.BSA_INVALID_ARG
    assert _attn_fwd(lib, scale=float("nan")) == _lib.BSA_INVALID_ARG
    assert _attn_fwd(lib, L=DYN, zs=None) == _lib.BSA_INVALID_ARG


def _attn_fwd_gather(lib, L=LAY, q=FAKE, o=FAKE, d=128, dt=1, zs=FAKE, wsb=1 << 40):
    c = L.c()
    return lib.bsa_attn_fwd_gather(ctypes.byref(c), zs, q, FAKE, FAKE, FAKE, FAKE, 2, d, dt, 0.0,
                                   o, FAKE, FAKE, wsb, None)


def test_attn_fwd_gather_validation(lib):
    assert _attn_fwd_gather(lib, q=None) == _lib.BSA_INVALID_ARG
    assert _attn_fwd_gather(lib, o=ctypes.c_void_p(0x1008)) == _lib.BSA_INVALID_ARG
    assert _attn_fwd_gather(lib, dt=0) == _lib.BSA_UNSUPPORTED     # fp32: the MFMA kernel only
    assert _attn_fwd_gather(lib, d=64) == _lib.BSA_UNSUPPORTED
    assert _attn_fwd_gather(lib, wsb=16) == _lib.BSA_WORKSPACE_TOO_SMALL
    assert _attn_fwd_gather(lib, L=DYN, zs=None) == _lib.BSA_INVALID_ARG
    # a block two tokens wide: its rows do not come in runs of four tokens
    narrow = BSALayout.fixed((13, 45, 80), (2, 32, 2))
    assert _attn_fwd_gather(lib, L=narrow) == _lib.BSA_UNSUPPORTED
    assert "multiples of 4" in lib.bsa_last_error().decode()
    # dynamic layouts: every candidate shape must qualify
    mixed = BSALayout.dynamic((13, 45, 80), zone=(4, 16, 16), shapes=((2, 8, 8), (4, 16, 2)))
    assert mixed.sizes()["n_blocks"] > 0
    assert _attn_fwd_gather(lib, L=mixed) == _lib.BSA_UNSUPPORTED


def test_attn_fwd_rejects_misaligned_tensors(lib):
    assert _attn_fwd(lib, q=ctypes.c_void_p(0x1008)) == _lib.BSA_INVALID_ARG
    assert "aligned" in lib.bsa_last_error().decode()


def test_attn_fwd_noalloc_validation(lib):
    """The allocation-free forward validates like bsa_attn_fwd before it
    touches the device (no GPU here: a valid call would fail at the device
    lookup, never before)."""
    c = LAY.c()

    def call(q=FAKE, d=128, dt=1, scale=0.0, zs=FAKE, L=c):
        return lib.bsa_attn_fwd_noalloc(ctypes.byref(L), zs, q, FAKE, FAKE, FAKE, FAKE, 2, d, dt,
                                        scale, FAKE, FAKE, None)

    assert call(q=None) == _lib.BSA_INVALID_ARG
    assert call(q=ctypes.c_void_p(0x1008)) == _lib.BSA_INVALID_ARG
    assert call(d=32) == _lib.BSA_UNSUPPORTED
    assert call(dt=3) == _lib.BSA_INVALID_ARG
    assert call(scale=float("nan")) == _lib.BSA_INVALID_ARG
    assert call(L=DYN.c(), zs=None) == _lib.BSA_INVALID_ARG
    assert call() == _lib.BSA_HIP_ERROR and "scratch" in lib.bsa_last_error().decode()


def test_attn_fwd_raster_validation(lib):
    c = LAY.c()

    def call(d=128, dt=1, q=FAKE):
        return lib.bsa_attn_fwd_raster(ctypes.byref(c), FAKE, q, FAKE, FAKE, FAKE, FAKE, 2, d, dt,
                                       0.0, FAKE, FAKE, FAKE, 1 << 40, None)

    assert call(d=64) == _lib.BSA_UNSUPPORTED     # the raster output needs the MFMA kernel
    assert call(dt=0) == _lib.BSA_UNSUPPORTED     # fp32
    assert call(q=None) == _lib.BSA_INVALID_ARG
    assert "raster" in (call(d=64) and lib.bsa_last_error().decode())


def test_attn_bwd_validation(lib):
    c = LAY.c()

    def call(dq=FAKE, wsb=1 << 40, d=128, op=FAKE):
        return lib.bsa_attn_bwd(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, op, FAKE, FAKE, FAKE,
                                FAKE, 2, d, 1, 0.0, dq, FAKE, FAKE, FAKE, wsb, None)

    assert call(dq=None) == _lib.BSA_INVALID_ARG
    assert call(op=ctypes.c_void_p(0x1004)) == _lib.BSA_INVALID_ARG   # misaligned
    assert call(wsb=1) == _lib.BSA_WORKSPACE_TOO_SMALL
    assert call(d=48) == _lib.BSA_UNSUPPORTED


def test_attn_bwd_raster_validation(lib):
    c = LAY.c()

    def call(d=128, dt=1, ptr=FAKE, wsb=1 << 40, L=c):
        return lib.bsa_attn_bwd_raster(ctypes.byref(L), FAKE, ptr, *([FAKE] * 7), 2, d, dt, 0.0,
                                       FAKE, FAKE, FAKE, FAKE, wsb, None)

    assert call(ptr=None) == _lib.BSA_INVALID_ARG
    assert call(d=64) == _lib.BSA_UNSUPPORTED       # raster gradients: the MFMA kernels only
    assert "raster" in lib.bsa_last_error().decode()
    assert call(dt=0) == _lib.BSA_UNSUPPORTED       # fp32
    assert call(wsb=16) == _lib.BSA_WORKSPACE_TOO_SMALL


def test_permute_validation(lib):
    c = LAY.c()
    arr = (ctypes.c_void_p * 4)(FAKE, FAKE, FAKE, FAKE)
    nul = (ctypes.c_void_p * 2)(FAKE, None)
    assert lib.bsa_permute(ctypes.byref(c), None, 5, arr, arr, 2, 128, 1, None) == _lib.BSA_INVALID_ARG
    assert lib.bsa_permute(ctypes.byref(c), None, 0, arr, arr, 2, 128, 1, None) == _lib.BSA_INVALID_ARG
    assert lib.bsa_permute(ctypes.byref(c), None, 2, nul, arr, 2, 128, 1, None) == _lib.BSA_INVALID_ARG
    assert lib.bsa_permute(ctypes.byref(c), None, 1, None, arr, 2, 128, 1, None) == _lib.BSA_INVALID_ARG
    assert lib.bsa_unpermute(ctypes.byref(c), None, 1, arr, arr, 2, 4, 1, None) == _lib.BSA_UNSUPPORTED
    assert lib.bsa_unpermute(ctypes.byref(c), None, 1, arr, arr, 2, 512, 1, None) == _lib.BSA_UNSUPPORTED
    d = DYN.c()
    assert lib.bsa_permute(ctypes.byref(d), None, 1, arr, arr, 2, 128, 1, None) == _lib.BSA_INVALID_ARG


def test_permute_pool_validation(lib):
    c = LAY.c()
    arr = (ctypes.c_void_p * 3)(FAKE, FAKE, FAKE)
    means = (ctypes.c_void_p * 2)(FAKE, FAKE)
    half = (ctypes.c_void_p * 2)(FAKE, None)

    def call(nt=3, npool=2, m=means, d=128, dt=1):
        return lib.bsa_permute_pool(ctypes.byref(c), None, nt, arr, arr, 2, d, dt, npool, m, None)

    assert call(npool=4) == _lib.BSA_INVALID_ARG         # more than ntensors
    assert call(npool=-1) == _lib.BSA_INVALID_ARG
    assert call(m=None) == _lib.BSA_INVALID_ARG
    assert call(m=half) == _lib.BSA_INVALID_ARG
    assert call(d=96) == _lib.BSA_UNSUPPORTED             # pooling needs d in {64, 128}
    assert call(dt=5) == _lib.BSA_INVALID_ARG
    assert "npool" in (call(npool=4) and lib.bsa_last_error().decode())
    # a missing dst is allowed only for a pooled tensor (pool without storing)
    nodst = (ctypes.c_void_p * 3)(None, None, None)
    assert lib.bsa_permute_pool(ctypes.byref(c), None, 3, arr, nodst, 2, 128, 1, 2, means,
                                None) == _lib.BSA_INVALID_ARG   # tensor 2 is not pooled
    assert "tensor 2" in lib.bsa_last_error().decode()
    assert lib.bsa_permute(ctypes.byref(c), None, 1, arr, nodst, 2, 128, 1,
                           None) == _lib.BSA_INVALID_ARG        # nothing pooled: dst required


def test_permute_norm_rope_validation(lib):
    c = LAY.c()
    arr = (ctypes.c_void_p * 3)(FAKE, FAKE, FAKE)
    means = (ctypes.c_void_p * 2)(FAKE, FAKE)

    def call(nrope=2, gamma=None, eps=1e-6, base=10000.0, d=128, npool=2):
        return lib.bsa_permute_norm_rope(ctypes.byref(c), None, 3, arr, arr, 2, d, 1, nrope,
                                         gamma, eps, base, npool, means, None)

    assert call(nrope=4) == _lib.BSA_INVALID_ARG
    assert call(nrope=-1) == _lib.BSA_INVALID_ARG
    assert call(d=96, npool=0) == _lib.BSA_UNSUPPORTED
    assert call(eps=0.0) == _lib.BSA_INVALID_ARG
    assert call(eps=float("inf")) == _lib.BSA_INVALID_ARG
    assert call(eps=float("nan")) == _lib.BSA_INVALID_ARG
    assert call(base=1.0) == _lib.BSA_INVALID_ARG
    assert call(base=float("inf")) == _lib.BSA_INVALID_ARG
    assert "rope_base" in lib.bsa_last_error().decode()


def test_select_validation(lib):
    c = LAY.c()

    def call(qbar=FAKE, d=128, S=8500, tau=0.2, wsb=1 << 40, ws=FAKE, counts=FAKE, L=c, zs=FAKE):
        return lib.bsa_select(ctypes.byref(L), zs, qbar, FAKE, 2, d, S, tau, counts, FAKE, None,
                              ws, wsb, None)

    assert call(qbar=None) == _lib.BSA_INVALID_ARG
    assert call(counts=None) == _lib.BSA_INVALID_ARG
    assert call(d=96) == _lib.BSA_UNSUPPORTED
    assert call(S=10000) == _lib.BSA_INVALID_ARG
    assert call(tau=0.0) == _lib.BSA_INVALID_ARG
    assert call(wsb=16) == _lib.BSA_WORKSPACE_TOO_SMALL
    assert call(ws=None) == _lib.BSA_WORKSPACE_TOO_SMALL
    dyn = DYN.c()
    assert call(L=dyn, zs=None) == _lib.BSA_INVALID_ARG
    need = lib.bsa_workspace_size(4, ctypes.byref(c), 2, 128)  # BSA_CALL_SELECT
    assert 0 < need < lib.bsa_workspace_size(1, ctypes.byref(c), 2, 128)


def test_select_causal_validation(lib):
    c = LAY.c()   # fixed 2x8x8 blocks: chunks must be whole multiples of 2 frames
    dyn = DYN.c()  # zones 4 frames deep

    def call(F, L=c, S=8500, wsb=1 << 40, zs=FAKE):
        return lib.bsa_select_causal(ctypes.byref(L), zs, FAKE, FAKE, 2, 128, S, 0.2, F, FAKE,
                                     FAKE, None, FAKE, wsb, None)

    for F in (0, -2, 3):
        assert call(F) == _lib.BSA_INVALID_ARG, F
    assert "frames_per_chunk" in lib.bsa_last_error().decode()
    for F in (2, 6):
        assert call(F, L=dyn) == _lib.BSA_INVALID_ARG, F
    assert call(4, S=10000) == _lib.BSA_INVALID_ARG
    assert call(4, wsb=16) == _lib.BSA_WORKSPACE_TOO_SMALL
    assert call(8, L=dyn, zs=None) == _lib.BSA_INVALID_ARG


def test_zone_score_validation(lib):
    c = DYN.c()

    def call(video=FAKE, C=1536, audio=FAKE, na=200, zs=FAKE, wsb=1 << 40):
        return lib.bsa_zone_score(ctypes.byref(c), video, C, audio, na, zs, None, FAKE, wsb, None)

    assert call(zs=None) == _lib.BSA_INVALID_ARG
    assert call(video=None) == _lib.BSA_INVALID_ARG
    assert call(C=100) == _lib.BSA_INVALID_ARG
    assert call(audio=None) == _lib.BSA_INVALID_ARG            # n_audio given without audio
    assert call(na=0) == _lib.BSA_INVALID_ARG                  # audio given without n_audio
    assert call(na=300) == _lib.BSA_INVALID_ARG
    assert call(wsb=8) == _lib.BSA_WORKSPACE_TOO_SMALL
    big = BSALayout.dynamic((16, 64, 64), (8, 16, 16), ((2, 8, 8),)).c()
    assert lib.bsa_zone_score(ctypes.byref(big), FAKE, 1536, None, 0, FAKE, None, FAKE, 1 << 40,
                              None) == _lib.BSA_UNSUPPORTED


def test_zone_score_rejects_zone_offsets_past_32_bits(lib):
    # zt*H*W*C*2 = 4*256*512*2048*2 = 2^31: one zone's row offsets would not fit
    wide = BSALayout.dynamic((4, 256, 512)).c()
    assert lib.bsa_zone_score(ctypes.byref(wide), FAKE, 2048, None, 0, FAKE, None, FAKE, 1 << 40,
                              None) == _lib.BSA_UNSUPPORTED
    assert "2^31" in lib.bsa_last_error().decode()


def test_xattn_fwd_validation(lib):
    def call(N=100, Na=200, C=256, H=2, d=128, ptr=FAKE):
        return lib.bsa_xattn_fwd(N, Na, C, H, d, ptr, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                 FAKE, FAKE, FAKE, FAKE, None)

    assert call(N=0) == _lib.BSA_INVALID_ARG
    assert call(Na=0) == _lib.BSA_INVALID_ARG
    assert call(Na=257) == _lib.BSA_INVALID_ARG
    assert call(C=100) == _lib.BSA_INVALID_ARG
    assert call(H=0) == _lib.BSA_INVALID_ARG
    assert call(d=64) == _lib.BSA_UNSUPPORTED
    assert call(ptr=None) == _lib.BSA_INVALID_ARG
    assert call(ptr=ctypes.c_void_p(0x1008)) == _lib.BSA_INVALID_ARG   # misaligned


def test_xattn_bwd_validation(lib):
    need = lib.bsa_xattn_bwd_workspace_size(1000, 200, 256, 2)
    assert need > 0
    assert lib.bsa_xattn_bwd_workspace_size(1000, 300, 256, 2) == 0

    def call(Na=200, d=128, wsb=need, ptr=FAKE, ws=FAKE):
        return lib.bsa_xattn_bwd(1000, Na, 256, 2, d, ptr, *([FAKE] * 9), FAKE, FAKE,
                                 *([FAKE] * 6), ws, wsb, None)

    assert call(Na=0) == _lib.BSA_INVALID_ARG
    assert call(d=96) == _lib.BSA_UNSUPPORTED
    assert call(ptr=None) == _lib.BSA_INVALID_ARG
    assert call(wsb=need - 1) == _lib.BSA_WORKSPACE_TOO_SMALL
    assert call(ws=ctypes.c_void_p(0x1008)) == _lib.BSA_INVALID_ARG   # misaligned workspace
    assert "workspace" in lib.bsa_last_error().decode()
