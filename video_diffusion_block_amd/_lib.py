"""ctypes loader of ``libbsa.so`` (the C ABI declared in include/bsa.h).

There is no fallback: if the library has not been built, ``load()`` raises.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbsa.so")

BSA_OK, BSA_INVALID_ARG, BSA_UNSUPPORTED, BSA_WORKSPACE_TOO_SMALL, BSA_LAYOUT, BSA_HIP_ERROR = range(6)
BSA_F32, BSA_BF16 = 0, 1
BSA_MODE_FIXED, BSA_MODE_DYNAMIC = 0, 1
BSA_CALL_ZONE_SCORE, BSA_CALL_POOL_SELECT, BSA_CALL_ATTN_FWD, BSA_CALL_ATTN_BWD, BSA_CALL_SELECT = range(5)
MAX_SHAPES = 4

c_i32p = ctypes.POINTER(ctypes.c_int32)
c_i64p = ctypes.POINTER(ctypes.c_int64)
vp = ctypes.c_void_p


class Layout(ctypes.Structure):
    """Mirror of ``bsa_layout``."""

    _fields_ = [
        ("grid", ctypes.c_int32 * 3),
        ("mode", ctypes.c_int32),
        ("zone", ctypes.c_int32 * 3),
        ("n_shapes", ctypes.c_int32),
        ("shapes", (ctypes.c_int32 * 3) * MAX_SHAPES),
    ]


LayoutP = ctypes.POINTER(Layout)

# name -> (restype, argtypes)
SIGNATURES = {
    "bsa_abi_version": (ctypes.c_int, []),
    "bsa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "bsa_last_error": (ctypes.c_char_p, []),
    "bsa_layout_sizes": (ctypes.c_int, [LayoutP, c_i64p, c_i64p, c_i32p, c_i32p, c_i32p]),
    "bsa_workspace_size": (ctypes.c_size_t, [ctypes.c_int, LayoutP, ctypes.c_int, ctypes.c_int]),
    "bsa_zone_score": (ctypes.c_int, [LayoutP, vp, ctypes.c_int, vp, ctypes.c_int, vp, vp, vp,
                                      ctypes.c_size_t, vp]),
    "bsa_permute": (ctypes.c_int, [LayoutP, vp, ctypes.c_int, ctypes.POINTER(vp),
                                   ctypes.POINTER(vp), ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   vp]),
    "bsa_permute_pool": (ctypes.c_int, [LayoutP, vp, ctypes.c_int, ctypes.POINTER(vp),
                                        ctypes.POINTER(vp), ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, ctypes.POINTER(vp), vp]),
    "bsa_permute_norm_rope": (ctypes.c_int, [LayoutP, vp, ctypes.c_int, ctypes.POINTER(vp),
                                             ctypes.POINTER(vp), ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_int, ctypes.POINTER(vp),
                                             ctypes.c_float, ctypes.c_float, ctypes.c_int,
                                             ctypes.POINTER(vp), vp]),
    "bsa_select": (ctypes.c_int, [LayoutP, vp, vp, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int32,
                                  ctypes.c_double, vp, vp, vp, vp, ctypes.c_size_t, vp]),
    "bsa_xattn_fwd": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int] + [vp] * 6 + [vp] * 4 + [vp, vp, vp]),
    "bsa_xattn_bwd_workspace_size": (ctypes.c_size_t, [ctypes.c_int] * 4),
    "bsa_xattn_bwd": (ctypes.c_int, [ctypes.c_int] * 5 + [vp] * 10 + [vp, vp] + [vp] * 6 +
                      [vp, ctypes.c_size_t, vp]),
    "bsa_select_causal": (ctypes.c_int, [LayoutP, vp, vp, vp, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int32, ctypes.c_double, ctypes.c_int, vp, vp,
                                         vp, vp, ctypes.c_size_t, vp]),
    "bsa_unpermute": (ctypes.c_int, [LayoutP, vp, ctypes.c_int, ctypes.POINTER(vp),
                                     ctypes.POINTER(vp), ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, vp]),
    "bsa_pool_select": (ctypes.c_int, [LayoutP, vp, vp, vp, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int32, ctypes.c_double, vp, vp, vp,
                                       vp, ctypes.c_size_t, vp]),
    "bsa_attn_fwd": (ctypes.c_int, [LayoutP, vp, vp, vp, vp, vp, vp, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_float, vp, vp, vp, ctypes.c_size_t,
                                    vp]),
    "bsa_attn_fwd_noalloc": (ctypes.c_int, [LayoutP, vp, vp, vp, vp, vp, vp, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_int, ctypes.c_float, vp, vp,
                                            vp]),
    "bsa_attn_fwd_raster": (ctypes.c_int, [LayoutP, vp, vp, vp, vp, vp, vp, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_int, ctypes.c_float, vp, vp, vp,
                                           ctypes.c_size_t, vp]),
    "bsa_attn_fwd_gather": (ctypes.c_int, [LayoutP, vp, vp, vp, vp, vp, vp, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_int, ctypes.c_float, vp, vp, vp,
                                           ctypes.c_size_t, vp]),
    "bsa_attn_bwd": (ctypes.c_int, [LayoutP, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_float, vp, vp, vp, vp,
                                    ctypes.c_size_t, vp]),
    "bsa_attn_bwd_raster": (ctypes.c_int, [LayoutP, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                           ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_float, vp, vp, vp, vp, ctypes.c_size_t, vp]),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load the built library (raises if it is missing: there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -m video_diffusion_block_amd.build)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class BSAError(RuntimeError):
    def __init__(self, call: str, status: int):
        lib = load()
        self.status = status
        name = lib.bsa_status_string(status).decode()
        msg = lib.bsa_last_error().decode()
        super().__init__(f"{call}: {name}: {msg}")


def check(call: str, status: int) -> None:
    if status != BSA_OK:
        raise BSAError(call, status)
