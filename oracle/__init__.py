"""fp64 CPU oracle for the Gated DeltaNet chunked-prefill operator.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this package.  The GPU library never
loads it and shares no code with it; the two meet only in the seeded input
generator, which holds none of the method's arithmetic.

The arithmetic lives in ``gdn_oracle.c`` (token-by-token gated delta rule,
back-propagation through time and a brute-force gate scan, all float64).  This
module compiles it with gcc (OpenMP over heads) and calls it through ctypes.

Parity pins for every function here are in ``tests/test_oracle_pins.py``,
``tests/test_oracle_backward.py`` and ``tests/test_oracle_kda.py``.  One part is
"parity unpinned": in :func:`kda_fwd` (a reading; the pages do not print KDA's
recurrence) the order of the per-channel decay and the delta correction matters only
for keys that mix channels, and no value independent of the reading fixes it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "libgdn_oracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int)


def build(force: bool = True) -> str:
    """Compile the oracle into oracle/libgdn_oracle.so (gcc, -O2, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        lib.gdn_oracle_fwd.argtypes = [_dp] * 6 + [_dp, _dp] + [ctypes.c_int] * 5 + [
            ctypes.c_double, _ip, ctypes.c_int, ctypes.c_int]
        lib.gdn_oracle_fwd.restype = None
        lib.gdn_oracle_bwd.argtypes = [_dp] * 8 + [_dp] * 6 + [ctypes.c_int] * 5 + [
            ctypes.c_double, _ip, ctypes.c_int, ctypes.c_int]
        lib.gdn_oracle_bwd.restype = None
        lib.gdn_oracle_gate_scan.argtypes = [_dp] + [ctypes.c_int] * 5 + [
            ctypes.c_double, _ip, _dp]
        lib.gdn_oracle_gate_scan.restype = None
        lib.gdn_oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(x):
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(x, typ=_dp):
    return None if x is None else x.ctypes.data_as(typ)


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _heads(heads, B, H):
    if heads is None:
        return None, B * H
    arr = np.ascontiguousarray(np.asarray(heads, dtype=np.int32).reshape(-1))
    if arr.size and (arr.min() < 0 or arr.max() >= B * H):
        raise ValueError("head index out of range")
    return arr, int(arr.size)


def fwd(q, k, v, g, beta, h0=None, scale=1.0, heads=None, nthreads=None):
    """Token-by-token forward.  Shapes: q,k [B,T,H,dk]; v [B,T,H,dv]; g,beta [B,T,H];
    h0 [B,H,dk,dv] or None.  Returns (o [B,T,H,dv], ht [B,H,dk,dv]) in float64.
    ``heads`` restricts the work to the listed flat head indices b*H+h (the other
    outputs stay zero)."""
    q, k, v, g, beta, h0 = map(_f64, (q, k, v, g, beta, h0))
    B, T, H, dk = q.shape
    dv = v.shape[3]
    assert k.shape == q.shape and v.shape[:3] == (B, T, H)
    assert g.shape == (B, T, H) and beta.shape == (B, T, H)
    if h0 is not None:
        assert h0.shape == (B, H, dk, dv)
    o = np.zeros((B, T, H, dv), np.float64)
    ht = np.zeros((B, H, dk, dv), np.float64)
    hl, n = _heads(heads, B, H)
    nt = nthreads or min(default_threads(), n if n > 0 else 1)
    _load().gdn_oracle_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(o),
                           _ptr(ht), B, T, H, dk, dv, float(scale), _ptr(hl, _ip), n, nt)
    return o, ht


def bwd(q, k, v, g, beta, dout, h0=None, dht=None, scale=1.0, heads=None, nthreads=None):
    """Back-propagation through time of :func:`fwd`.  Returns a dict with dq, dk, dv,
    dg, dbeta, dh0 (float64, same shapes as the corresponding inputs)."""
    q, k, v, g, beta, dout, h0, dht = map(_f64, (q, k, v, g, beta, dout, h0, dht))
    B, T, H, dk = q.shape
    dv = v.shape[3]
    assert dout.shape == v.shape
    out = {
        "dq": np.zeros_like(q), "dk": np.zeros_like(k), "dv": np.zeros_like(v),
        "dg": np.zeros_like(g), "dbeta": np.zeros_like(beta),
        "dh0": np.zeros((B, H, dk, dv), np.float64),
    }
    hl, n = _heads(heads, B, H)
    nt = nthreads or min(default_threads(), n if n > 0 else 1)
    _load().gdn_oracle_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(dout),
                           _ptr(dht), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                           _ptr(out["dg"]), _ptr(out["dbeta"]), _ptr(out["dh0"]), B, T, H, dk, dv,
                           float(scale), _ptr(hl, _ip), n, nt)
    return out


def gate_scan(g, chunk=64, window_chunks=8, log_eps=float(np.log(2.0 ** -24))):
    """Brute-force gate scan.  Returns (flags [B,H] int32, max window sum [B,H] float64)."""
    g = _f64(g)
    B, T, H = g.shape
    flags = np.zeros((B, H), np.int32)
    mx = np.zeros((B, H), np.float64)
    _load().gdn_oracle_gate_scan(_ptr(g), B, T, H, int(chunk), int(window_chunks), float(log_eps),
                                 _ptr(flags, _ip), _ptr(mx))
    return flags, mx


def kda_fwd(q, k, v, g, beta, h0=None, scale=1.0):
    """Token-by-token forward of the per-channel-decay variant (KDA), float64 numpy.

    Reading (the pages name KDA as the sibling operator of Kimi's hybrid stack but
    do not print its recurrence): the scalar decay of the gated delta rule becomes
    one decay per key channel, applied to the state before the delta correction,

        S_t = (I - beta_t k_t k_t^T) diag(exp(g_t)) S_{t-1} + beta_t k_t v_t^T,
        o_t = scale * S_t^T q_t,

    with S of shape [dk, dv] (rows = key channels), the layout of :func:`fwd`'s
    states.  With g_t equal in every channel it is :func:`fwd`.

    Shapes: q,k,g [B,T,H,dk]; v [B,T,H,dv]; beta [B,T,H]; h0 [B,H,dk,dv] or None.
    Returns (o [B,T,H,dv], ht [B,H,dk,dv]).  The loop over tokens runs in Python
    (vectorised over batch and heads): for small cases.  Pinned in
    ``tests/test_oracle_kda.py``."""
    q, k, v, g, beta, h0 = map(_f64, (q, k, v, g, beta, h0))
    B, T, H, dk = q.shape
    dv = v.shape[3]
    assert k.shape == q.shape and g.shape == q.shape and v.shape[:3] == (B, T, H)
    assert beta.shape == (B, T, H)
    S = np.zeros((B, H, dk, dv)) if h0 is None else h0.copy()
    o = np.zeros((B, T, H, dv))
    for t in range(T):
        kt, vt, bt = k[:, t], v[:, t], beta[:, t]          # [B,H,dk], [B,H,dv], [B,H]
        S = np.exp(g[:, t])[..., None] * S                  # per-channel decay of the rows
        kS = np.einsum("bhk,bhkv->bhv", kt, S)              # k_t^T S
        S = S - bt[..., None, None] * kt[..., :, None] * kS[..., None, :]
        S = S + bt[..., None, None] * kt[..., :, None] * vt[..., None, :]
        o[:, t] = scale * np.einsum("bhkv,bhk->bhv", S, q[:, t])
    return o, S
