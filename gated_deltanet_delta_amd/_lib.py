"""ctypes declarations of libgdn's C ABI (include/gdn.h).  Loading fails loudly if the library
has not been built: there is no fallback path."""
from __future__ import annotations

import ctypes
import os

LIBRARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdn.so")

GDN_SUCCESS = 0
GDN_ERROR_INVALID_VALUE = 1
GDN_ERROR_NOT_SUPPORTED = 2
GDN_ERROR_WORKSPACE = 3
GDN_ERROR_LAUNCH_FAILURE = 4

GDN_F32 = 0
GDN_BF16 = 1

EXPORTED = ("gdn_status_string", "gdn_version", "gdn_chunk_fwd_workspace_size", "gdn_chunk_fwd",
            "gdn_chunk_fwd_prepare", "gdn_chunk_fwd_scan", "gdn_recurrent_step",
            "gdn_chunk_fwd_gating", "gdn_recurrent_step_gating", "gdn_chunk_fwd_indexed",
            "gdn_recurrent_step_indexed", "gdn_gated_rmsnorm", "gdn_causal_conv1d",
            "gdn_chunk_fwd_ex", "gdn_recurrent_step_ex", "gdn_chunk_bwd_workspace_size",
            "gdn_chunk_bwd", "gdn_chunk_bwd_ex_workspace_size", "gdn_chunk_bwd_ex",
            "gdn_chunk_fwd_noalloc_max_bytes", "gdn_chunk_fwd_noalloc",
            "gdn_chunk_fwd_gated_norm_workspace_size", "gdn_chunk_fwd_gated_norm")

GDN_FLAG_QK_L2NORM = 1

_lib = None


class GdnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBRARY):
        raise RuntimeError(
            f"libgdn.so is not built ({LIBRARY} missing); build it with "
            "`python -m gated_deltanet_delta_amd.build` (or __graft_entry__.build())")
    lib = ctypes.CDLL(LIBRARY)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_status_string.argtypes = [i32]
    lib.gdn_version.restype = i32
    lib.gdn_version.argtypes = []
    lib.gdn_chunk_fwd_workspace_size.restype = sz
    lib.gdn_chunk_fwd_workspace_size.argtypes = [i32] * 7 + [i32]
    for name in ("gdn_chunk_fwd", "gdn_chunk_fwd_prepare", "gdn_chunk_fwd_scan"):
        fn = getattr(lib, name)
        fn.restype = i32
        fn.argtypes = [vp] * 7 + [i32] * 7 + [i32, i32] + [vp, vp, vp, sz, vp]
    lib.gdn_chunk_fwd_noalloc_max_bytes.restype = sz
    lib.gdn_chunk_fwd_noalloc_max_bytes.argtypes = []
    lib.gdn_chunk_fwd_noalloc.restype = i32
    lib.gdn_chunk_fwd_noalloc.argtypes = [vp] * 7 + [i32] * 7 + [i32, i32] + [vp, vp, vp]
    lib.gdn_recurrent_step.restype = i32
    lib.gdn_recurrent_step.argtypes = [vp] * 6 + [i32] * 6 + [i32, i32] + [vp, vp]
    lib.gdn_chunk_fwd_gating.restype = i32
    lib.gdn_chunk_fwd_gating.argtypes = [vp] * 9 + [i32] * 7 + [i32, i32] + [vp, vp, vp, sz, vp]
    lib.gdn_recurrent_step_gating.restype = i32
    lib.gdn_recurrent_step_gating.argtypes = [vp] * 8 + [i32] * 6 + [i32, i32] + [vp, vp]
    lib.gdn_chunk_fwd_indexed.restype = i32
    lib.gdn_chunk_fwd_indexed.argtypes = [vp] * 7 + [i32] + [vp] + [i32] * 7 + [i32, i32] + [vp, vp, sz, vp]
    lib.gdn_recurrent_step_indexed.restype = i32
    lib.gdn_recurrent_step_indexed.argtypes = [vp] * 7 + [i32] + [i32] * 6 + [i32, i32] + [vp, vp]
    lib.gdn_gated_rmsnorm.restype = i32
    lib.gdn_gated_rmsnorm.argtypes = [vp, vp, vp, ctypes.c_float, ctypes.c_int64, i32, i32, i32, vp, vp]
    lib.gdn_causal_conv1d.restype = i32
    lib.gdn_causal_conv1d.argtypes = [vp] * 5 + [i32] + [vp] + [i32] * 5 + [i32, i32] + [vp, vp]
    u32 = ctypes.c_uint
    lib.gdn_chunk_fwd_ex.restype = i32
    lib.gdn_chunk_fwd_ex.argtypes = [vp] * 10 + [i32] + [vp] + [i32] * 7 + [i32, i32] + [u32] + [vp, vp, sz, vp]
    lib.gdn_chunk_fwd_gated_norm_workspace_size.restype = sz
    lib.gdn_chunk_fwd_gated_norm_workspace_size.argtypes = [i32] * 7 + [i32]
    lib.gdn_chunk_fwd_gated_norm.restype = i32
    lib.gdn_chunk_fwd_gated_norm.argtypes = ([vp] * 10 + [i32] + [vp] + [vp, vp, ctypes.c_float] + [i32] * 7
                                             + [i32] * 4 + [u32] + [vp, vp, sz, vp])
    lib.gdn_chunk_bwd_workspace_size.restype = sz
    lib.gdn_chunk_bwd_workspace_size.argtypes = [i32] * 7
    lib.gdn_chunk_bwd.restype = i32
    lib.gdn_chunk_bwd.argtypes = [vp] * 9 + [i32] * 7 + [i32, i32] + [vp] * 6 + [vp, sz, vp]
    lib.gdn_chunk_bwd_ex_workspace_size.restype = sz
    lib.gdn_chunk_bwd_ex_workspace_size.argtypes = [i32] * 7 + [i32, i32, i32, u32]
    lib.gdn_chunk_bwd_ex.restype = i32
    lib.gdn_chunk_bwd_ex.argtypes = ([vp] * 9 + [i32] + [vp] * 3 + [i32] * 7 + [i32, i32, u32] + [vp] * 8
                                     + [vp, sz, vp])
    lib.gdn_recurrent_step_ex.restype = i32
    lib.gdn_recurrent_step_ex.argtypes = [vp] * 9 + [i32] + [i32] * 6 + [i32, i32] + [u32] + [vp, vp]
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().gdn_status_string(int(status)).decode()
