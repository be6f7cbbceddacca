"""Shared test helpers: moving seeded inputs to the GPU and the parity metric."""
from __future__ import annotations

import sys

import numpy as np

from gated_deltanet_chunked_prefill_amd import inputs

TOL_BF16 = 2e-2   # max|X - X_ref| <= TOL * max|X_ref| for bf16 I/O, fp32 accumulation
TOL_F32 = 1e-4    # the same bound for float32 I/O


def say(*a):
    """Progress line, flushed, so a GPU run that dies still names its case."""
    print(*a, file=sys.stderr, flush=True)


def rel_err(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(x - ref)) / (den if den > 0 else 1.0))


def to_gpu(x: inputs.GDNInputs, device="cuda"):
    import torch
    dt = torch.bfloat16 if x.dtype == "bf16" else torch.float32

    def t(a, d):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(device).to(d)

    return dict(q=t(x.q, dt), k=t(x.k, dt), v=t(x.v, dt), g=t(x.g, torch.float32),
                beta=t(x.beta, torch.float32), h0=t(x.h0, torch.float32),
                dout=t(x.dout, dt))


def to_np(t):
    return t.float().cpu().numpy().astype(np.float64)
