"""ctypes loader for libgdn.so (the C ABI declared in include/gdn.h).

The library is built in-tree by ``gated_deltanet_chunked_prefill_amd.build``.
There is no fallback: if it is missing or cannot be loaded, every entry point
raises immediately.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdn.so")

GDN_OK = 0
GDN_ERR_INVALID_ARG = 1
GDN_ERR_UNSUPPORTED = 2
GDN_ERR_WORKSPACE = 3
GDN_ERR_HIP = 4
GDN_F32 = 0
GDN_BF16 = 1

#: every function include/gdn.h declares
EXPORTS = ("gdn_default_options", "gdn_plan_segments", "gdn_chunk_fwd_workspace_size",
           "gdn_chunk_fwd", "gdn_chunk_bwd_workspace_size", "gdn_chunk_bwd",
           "gdn_gate_scan_workspace_size", "gdn_gate_scan", "gdn_profile_events",
           "gdn_last_error", "gdn_chunk_fwd_plan_info", "gdn_chunk_fwd_varlen",
           "gdn_chunk_bwd_varlen_workspace_size", "gdn_chunk_bwd_varlen", "gdn_chunk_fwd_noalloc", "gdn_kda_fwd",
           "gdn_kda_plan_segments", "gdn_kda_fwd_workspace_size", "gdn_chunk_bwd_plan_segments", "gdn_stream_probe", "gdn_profile_kinds")
#: bytes of the fixed scratch array of gdn_chunk_fwd_noalloc (GDN_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 << 20

LAUNCH_KINDS = {0: "gate_sums", 1: "gate_flags", 2: "fwd_single", 3: "fwd_windows",
                4: "fwd_queue", 5: "bwd_states", 6: "bwd_dh", 7: "bwd_local", 8: "fwd_sums",
                9: "kda_fwd", 10: "stream_probe", 11: "kda_pass1", 12: "kda_chain", 13: "bwd_chain"}


class Options(ctypes.Structure):
    _fields_ = [("split_mode", ctypes.c_int), ("n_segments", ctypes.c_int),
                ("use_window", ctypes.c_int), ("window_chunks", ctypes.c_int),
                ("log_eps", ctypes.c_float), ("window_levels", ctypes.c_int)]


_lib = None
_vp = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t


def load():
    """Load libgdn.so once and declare the signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with gated_deltanet_chunked_prefill_amd.build.build() "
            "(hipcc --offload-arch=gfx950); there is no CPU fallback")
    lib = ctypes.CDLL(LIB_PATH)
    op = ctypes.POINTER(Options)
    lib.gdn_default_options.argtypes = [op]
    lib.gdn_default_options.restype = None
    lib.gdn_plan_segments.argtypes = [_i, _i, _i, _i, op]
    lib.gdn_plan_segments.restype = _i
    lib.gdn_chunk_fwd_workspace_size.argtypes = [_i, _i, _i, _i, _i, _i, op]
    lib.gdn_chunk_fwd_workspace_size.restype = _sz
    lib.gdn_chunk_fwd.argtypes = [_vp] * 8 + [_i] * 6 + [ctypes.c_float, op, _vp, _sz, _vp]
    lib.gdn_chunk_fwd.restype = _i
    lib.gdn_chunk_fwd_noalloc.argtypes = [_vp] * 8 + [_i] * 6 + [ctypes.c_float, op, _vp]
    lib.gdn_chunk_fwd_noalloc.restype = _i
    lib.gdn_kda_fwd.argtypes = [_vp] * 8 + [_i] * 6 + [ctypes.c_float, _i, _vp, _sz, _vp]
    lib.gdn_kda_fwd.restype = _i
    lib.gdn_profile_kinds.argtypes = [ctypes.c_uint32]
    lib.gdn_profile_kinds.restype = ctypes.c_uint32
    lib.gdn_kda_plan_segments.argtypes = [_i] * 5
    lib.gdn_kda_plan_segments.restype = _i
    lib.gdn_chunk_bwd_plan_segments.argtypes = [_i] * 4
    lib.gdn_chunk_bwd_plan_segments.restype = _i
    lib.gdn_kda_fwd_workspace_size.argtypes = [_i] * 6
    lib.gdn_kda_fwd_workspace_size.restype = _sz
    lib.gdn_stream_probe.argtypes = [_vp] * 4 + [_i] * 3 + [_vp]
    lib.gdn_stream_probe.restype = _i
    lib.gdn_chunk_fwd_varlen.argtypes = [_vp] * 9 + [_i] * 6 + [ctypes.c_float, _vp]
    lib.gdn_chunk_fwd_varlen.restype = _i
    lib.gdn_chunk_bwd_varlen_workspace_size.argtypes = [_i] * 6
    lib.gdn_chunk_bwd_varlen_workspace_size.restype = _sz
    lib.gdn_chunk_bwd_varlen.argtypes = [_vp] * 15 + [_i] * 6 + [ctypes.c_float, _vp, _sz, _vp]
    lib.gdn_chunk_bwd_varlen.restype = _i
    lib.gdn_chunk_fwd_plan_info.argtypes = [_i, _i, _i, op, _vp, _vp, _vp]
    lib.gdn_chunk_fwd_plan_info.restype = _i
    lib.gdn_chunk_bwd_workspace_size.argtypes = [_i] * 6
    lib.gdn_chunk_bwd_workspace_size.restype = _sz
    lib.gdn_chunk_bwd.argtypes = [_vp] * 14 + [_i] * 6 + [ctypes.c_float, _vp, _sz, _vp]
    lib.gdn_chunk_bwd.restype = _i
    lib.gdn_gate_scan_workspace_size.argtypes = [_i, _i, _i]
    lib.gdn_gate_scan_workspace_size.restype = _sz
    lib.gdn_gate_scan.argtypes = [_vp, _i, _i, _i, _i, ctypes.c_float, _vp, _vp, _vp, _sz, _vp]
    lib.gdn_gate_scan.restype = _i
    lib.gdn_profile_events.argtypes = [_vp, _vp, _i]
    lib.gdn_profile_events.restype = _i
    lib.gdn_last_error.argtypes = []
    lib.gdn_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def last_error() -> str:
    return load().gdn_last_error().decode()


class GDNError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"gdn status {status}: {msg}")
        self.status = status


def check(status: int) -> None:
    if status != GDN_OK:
        raise GDNError(status, last_error())
