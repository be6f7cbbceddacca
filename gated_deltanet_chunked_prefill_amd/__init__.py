"""MI355X-native Gated DeltaNet chunked-prefill operator.

A thin Python binding over the C ABI in include/gdn.h (libgdn.so, built for
gfx950).  These functions only marshal arguments: they check tensors, allocate
outputs and the workspace with torch, and pass raw device pointers plus the
current HIP stream to the library.  Every step of the computation runs in the
library's HIP kernels; there is no fallback path.

    gdn_chunk_fwd(q, k, v, g, beta, h0=None, scale=1.0, ...) -> (o, ht)
    gdn_chunk_fwd_varlen(q, k, v, g, beta, cu_seqlens, h0=None, ...) -> (o, ht)
    gdn_kda_fwd(q, k, v, g, beta, h0=None, scale=1.0, n_segments=0) -> (o, ht)   (g per key channel)
    gdn_chunk_bwd(q, k, v, g, beta, dout, h0=None, dht=None, scale=1.0) -> dict
    gdn_chunk_bwd_varlen(q, k, v, g, beta, dout, cu_seqlens, h0=None, ...) -> dict
    gdn_gate_scan(g, window_chunks=8, log_eps=log(2^-24)) -> (flags, max_window_logdecay)

Layouts: q, k [B,T,H,128]; v [B,T,H,128]; g = log(alpha) and beta [B,T,H]
float32; h0 / ht [B,H,128,128] float32; q, k, v in bfloat16 or float32.
"""
from __future__ import annotations

import ctypes
import math

from . import _lib

DEFAULT_LOG_EPS = math.log(2.0 ** -24)

__all__ = ["gdn_chunk_fwd", "gdn_chunk_fwd_noalloc", "gdn_kda_fwd",
           "gdn_kda_plan_segments", "gdn_kda_fwd_workspace_size", "gdn_chunk_bwd_plan_segments", "gdn_chunk_fwd_varlen", "gdn_chunk_bwd", "gdn_chunk_bwd_varlen", "gdn_gate_scan",
           "gdn_plan_segments",
           "gdn_chunk_fwd_plan_info", "gdn_chunk_fwd_workspace_size", "gdn_chunk_bwd_workspace_size",
           "gdn_chunk_bwd_varlen_workspace_size", "options"]


def options(split_mode=0, n_segments=1, use_window=True, window_chunks=8,
            log_eps=DEFAULT_LOG_EPS, window_levels=4) -> _lib.Options:
    """Build a gdn_options struct (split_mode 0 auto, 1 off, 2 forced n_segments;
    window lengths window_chunks * (1 .. window_levels) are tried per head)."""
    return _lib.Options(int(split_mode), int(n_segments), int(bool(use_window)),
                        int(window_chunks), float(log_eps), int(window_levels))


def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return _lib.GDN_BF16
    if t.dtype == torch.float32:
        return _lib.GDN_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _dev(t, name, dtype=None):
    torch = _torch()
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _shape(t, name, shape, device):
    """Raise ValueError unless tensor t (or None) has exactly `shape` and lives on
    `device`: a tensor the library would index past its end never reaches it."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def _workspace_arg(ws, device):
    torch = _torch()
    if ws is None:
        return
    _dev(ws, "workspace")
    if ws.dtype != torch.uint8 or ws.dim() != 1:
        raise ValueError("workspace must be a 1-D uint8 tensor")
    _shape(ws, "workspace", ws.shape, device)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def gdn_plan_segments(B, T, H, num_cus, **opts) -> int:
    """Segments per head the forward uses for these shapes on num_cus compute units."""
    o = options(**opts)
    return _lib.load().gdn_plan_segments(int(B), int(T), int(H), int(num_cus), ctypes.byref(o))


def gdn_chunk_fwd_workspace_size(B, T, H, dk=128, dv=128, bf16=True, **opts) -> int:
    o = options(**opts)
    n = _lib.load().gdn_chunk_fwd_workspace_size(int(B), int(T), int(H), int(dk), int(dv),
                                                 _lib.GDN_BF16 if bf16 else _lib.GDN_F32,
                                                 ctypes.byref(o))
    if n == ctypes.c_size_t(-1).value:
        raise _lib.GDNError(_lib.GDN_ERR_INVALID_ARG, _lib.last_error())
    return int(n)


def gdn_chunk_bwd_varlen_workspace_size(n_seqs, T, H, dk=128, dv=128, bf16=True) -> int:
    n = _lib.load().gdn_chunk_bwd_varlen_workspace_size(n_seqs, T, H, dk, dv,
                                                        _lib.GDN_BF16 if bf16 else _lib.GDN_F32)
    if n == ctypes.c_size_t(-1).value:
        raise _lib.GDNError(_lib.GDN_ERR_INVALID_ARG, _lib.last_error())
    return int(n)


def gdn_chunk_bwd_workspace_size(B, T, H, dk=128, dv=128, bf16=True) -> int:
    n = _lib.load().gdn_chunk_bwd_workspace_size(int(B), int(T), int(H), int(dk), int(dv),
                                                 _lib.GDN_BF16 if bf16 else _lib.GDN_F32)
    if n == ctypes.c_size_t(-1).value:
        raise _lib.GDNError(_lib.GDN_ERR_INVALID_ARG, _lib.last_error())
    return int(n)


def _workspace(nbytes, device):
    torch = _torch()
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def gdn_chunk_fwd(q, k, v, g, beta, h0=None, scale=1.0, *, output_final_state=True, out=None,
                  out_ht=None, workspace=None, **opts):
    """Fused chunked forward.  Returns (o, ht) (ht is None when not requested).
    ``opts`` are the gdn_options fields (split_mode, n_segments, use_window,
    window_chunks, log_eps, window_levels).  ``out`` / ``out_ht`` may supply preallocated
    outputs and ``workspace`` a preallocated uint8 workspace."""
    torch = _torch()
    lib = _lib.load()
    _dev(q, "q")
    dt = q.dtype
    _dev(k, "k", dt), _dev(v, "v", dt)
    _dev(g, "g", torch.float32), _dev(beta, "beta", torch.float32)
    _dev(h0, "h0", torch.float32)
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, T, H, d]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    _shape(k, "k", (B, T, H, dk), dev)
    _shape(v, "v", (B, T, H, dv), dev)
    _shape(g, "g", (B, T, H), dev)
    _shape(beta, "beta", (B, T, H), dev)
    _shape(h0, "h0", (B, H, dk, dv), dev)
    o = out if out is not None else torch.empty((B, T, H, dv), dtype=dt, device=q.device)
    _dev(o, "o", dt)
    _shape(o, "out", (B, T, H, dv), dev)
    if out_ht is not None:
        ht = _dev(out_ht, "out_ht", torch.float32)
        _shape(ht, "out_ht", (B, H, dk, dv), dev)
    else:
        ht = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device) if output_final_state else None
    _workspace_arg(workspace, dev)
    opt = options(**opts)
    code = _dtype_code(q)
    if workspace is None:
        n = lib.gdn_chunk_fwd_workspace_size(B, T, H, dk, dv, code, ctypes.byref(opt))
        if n == ctypes.c_size_t(-1).value:
            raise _lib.GDNError(_lib.GDN_ERR_INVALID_ARG, _lib.last_error())
        workspace = _workspace(int(n), q.device)
    wsz = 0 if workspace is None else workspace.numel()
    _lib.check(lib.gdn_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0),
                                 _ptr(o), _ptr(ht), B, T, H, dk, dv, code, float(scale),
                                 ctypes.byref(opt), _ptr(workspace), wsz, _stream(q.device)))
    return o, ht


def _varlen_shapes(q, k, v, g, beta, cu_seqlens):
    """Packed-batch shapes: q, k [T, H, dk] or [1, T, H, dk], v like q with dv,
    g, beta q's shape without the last axis, cu_seqlens 1-D with S + 1 >= 2
    entries, all on q's device.  Returns (T, H, dk, dv, S)."""
    if q.dim() not in (3, 4) or (q.dim() == 4 and q.shape[0] != 1):
        raise ValueError("q, k, v must be [T, H, d] or [1, T, H, d]")
    T, H, dk = q.shape[-3], q.shape[-2], q.shape[-1]
    dv = v.shape[-1]
    dev = q.device
    _shape(k, "k", q.shape, dev)
    _shape(v, "v", tuple(q.shape[:-1]) + (dv,), dev)
    _shape(g, "g", q.shape[:-1], dev)
    _shape(beta, "beta", q.shape[:-1], dev)
    if cu_seqlens.dim() != 1:
        raise ValueError("cu_seqlens must be 1-D")
    _shape(cu_seqlens, "cu_seqlens", cu_seqlens.shape, dev)
    S = cu_seqlens.numel() - 1
    if S < 1:
        raise ValueError("cu_seqlens needs at least two entries")
    return T, H, dk, dv, S


def gdn_chunk_fwd_noalloc(q, k, v, g, beta, h0=None, scale=1.0, *, out, out_ht=None, **opts):
    """gdn_chunk_fwd without a workspace: the library's fixed per-GPU scratch
    array holds the split forward's state (no allocation inside the call, so it
    can run under graph capture).  ``out`` (and ``out_ht`` when the final state is
    wanted) must be preallocated; returns (out, out_ht).  Calls that overlap in
    time on one GPU share the scratch and race."""
    torch = _torch()
    lib = _lib.load()
    _dev(q, "q")
    dt = q.dtype
    _dev(k, "k", dt), _dev(v, "v", dt)
    _dev(g, "g", torch.float32), _dev(beta, "beta", torch.float32)
    _dev(h0, "h0", torch.float32)
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, T, H, d]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    _shape(k, "k", (B, T, H, dk), dev)
    _shape(v, "v", (B, T, H, dv), dev)
    _shape(g, "g", (B, T, H), dev)
    _shape(beta, "beta", (B, T, H), dev)
    _shape(h0, "h0", (B, H, dk, dv), dev)
    _dev(out, "out", dt)
    _shape(out, "out", (B, T, H, dv), dev)
    if out_ht is not None:
        _dev(out_ht, "out_ht", torch.float32)
        _shape(out_ht, "out_ht", (B, H, dk, dv), dev)
    opt = options(**opts)
    _lib.check(lib.gdn_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0),
                                         _ptr(out), _ptr(out_ht), B, T, H, dk, dv, _dtype_code(q), float(scale),
                                         ctypes.byref(opt), _stream(dev)))
    return out, out_ht


def gdn_chunk_bwd_plan_segments(B, T, H, num_cus) -> int:
    """Segments per head of gdn_chunk_bwd's state-gradient sweep on a device with
    num_cus compute units (1 = unsplit, 0 = invalid arguments)."""
    return _lib.load().gdn_chunk_bwd_plan_segments(int(B), int(T), int(H), int(num_cus))


def gdn_kda_plan_segments(B, T, H, num_cus, n_segments=0) -> int:
    """Segments per head gdn_kda_fwd uses for these shapes on num_cus compute units."""
    return _lib.load().gdn_kda_plan_segments(int(B), int(T), int(H), int(num_cus), int(n_segments))


def gdn_kda_fwd_workspace_size(B, T, H, dk=128, dv=128, n_segments=0) -> int:
    n = _lib.load().gdn_kda_fwd_workspace_size(int(B), int(T), int(H), int(dk), int(dv), int(n_segments))
    if n == ctypes.c_size_t(-1).value:
        raise _lib.GDNError(_lib.GDN_ERR_INVALID_ARG, _lib.last_error())
    return int(n)


def gdn_kda_fwd(q, k, v, g, beta, h0=None, scale=1.0, *, output_final_state=True, out=None, out_ht=None,
                n_segments=0, workspace=None):
    """Chunked forward of the per-key-channel-decay variant (KDA): as
    gdn_chunk_fwd, with g [B, T, H, dk] float32 (one log-decay per key channel)
    and bf16 q, k, v.  n_segments: 0 automatic sequence split, 1 unsplit, k >= 2
    that many segments per head.  Returns (o, ht)."""
    torch = _torch()
    lib = _lib.load()
    _dev(q, "q", torch.bfloat16)
    _dev(k, "k", torch.bfloat16), _dev(v, "v", torch.bfloat16)
    _dev(g, "g", torch.float32), _dev(beta, "beta", torch.float32)
    _dev(h0, "h0", torch.float32)
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, T, H, d]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    _shape(k, "k", (B, T, H, dk), dev)
    _shape(v, "v", (B, T, H, dv), dev)
    _shape(g, "g", (B, T, H, dk), dev)
    _shape(beta, "beta", (B, T, H), dev)
    _shape(h0, "h0", (B, H, dk, dv), dev)
    o = out if out is not None else torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev)
    _dev(o, "o", torch.bfloat16)
    _shape(o, "out", (B, T, H, dv), dev)
    if out_ht is not None:
        ht = _dev(out_ht, "out_ht", torch.float32)
        _shape(ht, "out_ht", (B, H, dk, dv), dev)
    else:
        ht = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev) if output_final_state else None
    _workspace_arg(workspace, dev)
    if workspace is None:
        n = lib.gdn_kda_fwd_workspace_size(B, T, H, dk, dv, int(n_segments))
        if n == ctypes.c_size_t(-1).value:
            raise _lib.GDNError(_lib.GDN_ERR_INVALID_ARG, _lib.last_error())
        workspace = _workspace(int(n), dev)
    wsz = 0 if workspace is None else workspace.numel()
    _lib.check(lib.gdn_kda_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(o), _ptr(ht),
                               B, T, H, dk, dv, _lib.GDN_BF16, float(scale), int(n_segments), _ptr(workspace),
                               wsz, _stream(dev)))
    return o, ht


def gdn_stream_probe(k, q, v, o, segments):
    """Measurement aid: stream k, q, v ([T, H, 128] bf16, T a multiple of
    64 * segments) into LDS chunk by chunk in the fused forward's layout and write
    o, with no arithmetic (one workgroup per head and segment).  Returns None."""
    torch = _torch()
    lib = _lib.load()
    for t, nm in ((k, "k"), (q, "q"), (v, "v"), (o, "o")):
        _dev(t, nm, torch.bfloat16)
    if k.dim() != 3 or k.shape[-1] != 128:
        raise ValueError("k, q, v, o must be [T, H, 128]")
    T, H, _ = k.shape
    for t, nm in ((q, "q"), (v, "v"), (o, "o")):
        _shape(t, nm, (T, H, 128), k.device)
    _lib.check(lib.gdn_stream_probe(_ptr(k), _ptr(q), _ptr(v), _ptr(o), T, H, int(segments), _stream(k.device)))


def gdn_chunk_fwd_varlen(q, k, v, g, beta, cu_seqlens, h0=None, scale=1.0, *,
                         output_final_state=True, out=None, out_ht=None):
    """Fused forward over packed variable-length sequences.  q, k, v: [T, H, d]
    (or [1, T, H, d]) in bf16 or float32, g, beta: [T, H] (or [1, T, H]) float32,
    cu_seqlens: int32 [S + 1] on the same device (token offsets of the S
    sequences), h0: [S, H, dk, dv] float32 or None.  Returns (o, ht) with o
    shaped like v and ht [S, H, dk, dv] (None when not requested)."""
    torch = _torch()
    lib = _lib.load()
    _dev(q, "q")
    dt = q.dtype
    _dev(k, "k", dt), _dev(v, "v", dt)
    _dev(g, "g", torch.float32), _dev(beta, "beta", torch.float32)
    _dev(cu_seqlens, "cu_seqlens", torch.int32)
    _dev(h0, "h0", torch.float32)
    T, H, dk, dv, S = _varlen_shapes(q, k, v, g, beta, cu_seqlens)
    dev = q.device
    _shape(h0, "h0", (S, H, dk, dv), dev)
    o = out if out is not None else torch.empty_like(v)
    _dev(o, "o", dt)
    _shape(o, "out", v.shape, dev)
    if out_ht is not None:
        ht = _dev(out_ht, "out_ht", torch.float32)
        _shape(ht, "out_ht", (S, H, dk, dv), dev)
    else:
        ht = torch.empty((S, H, dk, dv), dtype=torch.float32, device=q.device) if output_final_state else None
    _lib.check(lib.gdn_chunk_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0),
                                        _ptr(o), _ptr(ht), _ptr(cu_seqlens), S, T, H, dk, dv,
                                        _dtype_code(q), float(scale), _stream(q.device)))
    return o, ht


def gdn_chunk_fwd_plan_info(B, T, H, workspace=None, device=None, **opts) -> dict:
    """The plan the last split forward with these shapes, options and workspace
    used (synchronises the device's current stream)."""
    lib = _lib.load()
    info = (ctypes.c_int32 * 8)()
    opt = options(**opts)
    dev = workspace.device if workspace is not None else device
    _lib.check(lib.gdn_chunk_fwd_plan_info(int(B), int(T), int(H), ctypes.byref(opt), _ptr(workspace),
                                           info, _stream(dev) if dev is not None else None))
    keys = ("P_exact", "P_window", "n_exact", "n_window", "n_jobs", "handed_out", "error")
    return dict(zip(keys, list(info)[:7]))


def gdn_chunk_bwd(q, k, v, g, beta, dout, h0=None, dht=None, scale=1.0, *, workspace=None,
                  need_dh0=True):
    """Fused chunked backward.  Returns a dict with dq, dk, dv (I/O dtype), dg, dbeta
    (float32) and dh0 (float32, or None when need_dh0 is False)."""
    torch = _torch()
    lib = _lib.load()
    _dev(q, "q")
    dt = q.dtype
    _dev(k, "k", dt), _dev(v, "v", dt), _dev(dout, "dout", dt)
    _dev(g, "g", torch.float32), _dev(beta, "beta", torch.float32)
    _dev(h0, "h0", torch.float32), _dev(dht, "dht", torch.float32)
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, T, H, d]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    _shape(k, "k", (B, T, H, dk), dev)
    _shape(v, "v", (B, T, H, dv), dev)
    _shape(dout, "dout", (B, T, H, dv), dev)
    _shape(g, "g", (B, T, H), dev)
    _shape(beta, "beta", (B, T, H), dev)
    _shape(h0, "h0", (B, H, dk, dv), dev)
    _shape(dht, "dht", (B, H, dk, dv), dev)
    _workspace_arg(workspace, dev)
    dq = torch.empty_like(q)
    dkk = torch.empty_like(k)
    dvv = torch.empty_like(v)
    dg = torch.empty_like(g)
    db = torch.empty_like(beta)
    dh0 = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device) if need_dh0 else None
    code = _dtype_code(q)
    if workspace is None:
        n = lib.gdn_chunk_bwd_workspace_size(B, T, H, dk, dv, code)
        if n == ctypes.c_size_t(-1).value:
            raise _lib.GDNError(_lib.GDN_ERR_INVALID_ARG, _lib.last_error())
        workspace = _workspace(int(n), q.device)
    wsz = 0 if workspace is None else workspace.numel()
    _lib.check(lib.gdn_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0),
                                 _ptr(dout), _ptr(dht), _ptr(dq), _ptr(dkk), _ptr(dvv), _ptr(dg),
                                 _ptr(db), _ptr(dh0), B, T, H, dk, dv, code, float(scale),
                                 _ptr(workspace), wsz, _stream(q.device)))
    return {"dq": dq, "dk": dkk, "dv": dvv, "dg": dg, "dbeta": db, "dh0": dh0}


def gdn_chunk_bwd_varlen(q, k, v, g, beta, dout, cu_seqlens, h0=None, dht=None, scale=1.0, *,
                         workspace=None, need_dh0=True):
    """Backward of gdn_chunk_fwd_varlen (packed sequences, tensors [T, H, ..] or
    [1, T, H, ..], cu_seqlens int32 [S + 1] on the device).  Returns a dict with
    dq, dk, dv, dg, dbeta shaped like their inputs and dh0 [S, H, dk, dv] (None
    when need_dh0 is False).  Tokens outside every sequence are not written
    (their gradients are left as allocated)."""
    torch = _torch()
    lib = _lib.load()
    _dev(q, "q")
    dt = q.dtype
    _dev(k, "k", dt), _dev(v, "v", dt), _dev(dout, "dout", dt)
    _dev(g, "g", torch.float32), _dev(beta, "beta", torch.float32)
    _dev(cu_seqlens, "cu_seqlens", torch.int32)
    _dev(h0, "h0", torch.float32), _dev(dht, "dht", torch.float32)
    T, H, dk, dv, S = _varlen_shapes(q, k, v, g, beta, cu_seqlens)
    dev = q.device
    _shape(dout, "dout", v.shape, dev)
    _shape(h0, "h0", (S, H, dk, dv), dev)
    _shape(dht, "dht", (S, H, dk, dv), dev)
    _workspace_arg(workspace, dev)
    dq, dkk, dvv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dg, db = torch.empty_like(g), torch.empty_like(beta)
    dh0 = torch.empty((S, H, dk, dv), dtype=torch.float32, device=q.device) if need_dh0 else None
    code = _dtype_code(q)
    if workspace is None:
        n = lib.gdn_chunk_bwd_varlen_workspace_size(S, T, H, dk, dv, code)
        if n == ctypes.c_size_t(-1).value:
            raise _lib.GDNError(_lib.GDN_ERR_INVALID_ARG, _lib.last_error())
        workspace = _workspace(int(n), q.device)
    _lib.check(lib.gdn_chunk_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0),
                                        _ptr(dout), _ptr(dht), _ptr(dq), _ptr(dkk), _ptr(dvv), _ptr(dg),
                                        _ptr(db), _ptr(dh0), _ptr(cu_seqlens), S, T, H, dk, dv, code,
                                        float(scale), _ptr(workspace), workspace.numel(),
                                        _stream(q.device)))
    return {"dq": dq, "dk": dkk, "dv": dvv, "dg": dg, "dbeta": db, "dh0": dh0}


def gdn_gate_scan(g, window_chunks=8, log_eps=DEFAULT_LOG_EPS):
    """Gate scan over g [B,T,H] float32.  Returns (flags [B,H] int32, max window
    log-decay [B,H] float32)."""
    torch = _torch()
    lib = _lib.load()
    _dev(g, "g", torch.float32)
    if g.dim() != 3:
        raise ValueError("g must be [B, T, H]")
    B, T, H = g.shape
    flags = torch.empty((B, H), dtype=torch.int32, device=g.device)
    mx = torch.empty((B, H), dtype=torch.float32, device=g.device)
    n = lib.gdn_gate_scan_workspace_size(B, T, H)
    ws = _workspace(int(n), g.device)
    _lib.check(lib.gdn_gate_scan(_ptr(g), B, T, H, int(window_chunks), float(log_eps), _ptr(flags),
                                 _ptr(mx), _ptr(ws), int(n), _stream(g.device)))
    return flags, mx
