"""Seeded synthetic inputs for the GDN chunked-prefill operator.

This module is shared by the tests, the benchmark and the smoke check.  It only
draws random numbers and rounds them to the I/O dtype; it contains none of the
operator's arithmetic, so the GPU path and the CPU oracle can both be fed from
it without sharing any computation.

Distributions follow the workloads the operator is specified on:
  * q, k: rows of N(0,1), L2-normalised per (b, t, h) token (the FlashQLA talk
    summary, paragraph 5, relies on L2-normalised keys; normalisation is done
    here, never inside the op), then rounded to the I/O dtype.
  * v ~ N(0,1), rounded to the I/O dtype.
  * beta = beta_max * sigmoid(N(0,1)), float32 (beta_max = 1 by default; up to 2,
    the range in which each per-token map I - beta k k^T is still a contraction).
  * g = log(alpha), float32, one of
      - "uniform":       U[lo, hi] per token,
      - "softplus_head": -softplus(x) * A_h with x ~ N(0,1) per (b,t,h) and a
                         per-head decay rate A_h = exp(U[-4,-1]),
      - "mixed":         70% of the heads (chosen by a seeded permutation)
                         strongly decaying U[-0.5,-0.05] per token, the rest
                         near 1, U[-1e-3,-1e-5] per token.
  * h0 ~ N(0, std^2) float32 when requested, dout ~ N(0,1) in the I/O dtype.
  * key_corr = rho > 0 (optional): the keys of each head share a direction; a
    key becomes the normalised sqrt(1 - rho) sqrt(dk) k + sqrt(rho) c_h, with
    c_h ~ N(0, I) drawn once per head, so that two keys of a head have cosine
    about rho (projected keys of trained models are far from orthogonal; the
    default rho = 0 keeps independent keys).
The draw order is fixed: q, k, v, beta, gate parts, h0, dout, then the shared
key directions (only when key_corr > 0, so other draws do not move).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

#: Named workloads (shapes and distributions), keyed by a descriptive name.
WORKLOADS = {
    # tiny fp32 case: 2 chunks of 64 tokens, one head
    "fp32_t128_h1": dict(B=1, T=128, H=1, dk=128, dv=128, dtype="f32", gate="uniform",
                         gate_lo=-0.2, gate_hi=-0.005, h0_std=None, dout=False, seed=0),
    # bf16 I/O with an initial state
    "bf16_t4096_h16": dict(B=1, T=4096, H=16, dk=128, dv=128, dtype="bf16", gate="softplus_head",
                           h0_std=0.02, dout=False, seed=1),
    # bf16, few heads against many CUs: the throughput workload
    "bf16_t32768_h32": dict(B=1, T=32768, H=32, dk=128, dv=128, dtype="bf16",
                            gate="softplus_head", h0_std=None, dout=False, seed=2),
    # long context with a 70/30 mix of fast-decaying and near-1 heads
    "bf16_t262144_h16_mixed": dict(B=1, T=262144, H=16, dk=128, dv=128, dtype="bf16",
                                   gate="mixed", h0_std=None, dout=False, seed=3),
    # training shape, forward + backward
    "bf16_b4_t8192_h32_train": dict(B=4, T=8192, H=32, dk=128, dv=128, dtype="bf16",
                                    gate="softplus_head", h0_std=0.02, dout=True, seed=4),
}


@dataclass
class GDNInputs:
    q: np.ndarray            # [B,T,H,dk] float32 holding values exact in the I/O dtype
    k: np.ndarray            # [B,T,H,dk]
    v: np.ndarray            # [B,T,H,dv]
    g: np.ndarray            # [B,T,H] float32, log alpha
    beta: np.ndarray         # [B,T,H] float32
    h0: Optional[np.ndarray]  # [B,H,dk,dv] float32 or None
    dout: Optional[np.ndarray]  # [B,T,H,dv] float32 (I/O-dtype exact) or None
    dtype: str               # "bf16" or "f32"
    meta: dict = field(default_factory=dict)

    @property
    def shape(self):
        B, T, H, dk = self.q.shape
        return B, T, H, dk, self.v.shape[3]


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), in place where
    possible, and return them as float32.  Inputs here are finite."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    flat = u.reshape(-1)
    step = 1 << 24
    for s in range(0, flat.size, step):
        blk = flat[s:s + step]
        lsb = (blk >> 16) & np.uint32(1)
        blk += np.uint32(0x7FFF) + lsb
        blk &= np.uint32(0xFFFF0000)
    return x


def _normal_rows(rng, shape, dtype_tag):
    x = rng.standard_normal(shape, dtype=np.float32)
    flat = x.reshape(-1, shape[-1])
    step = 1 << 18
    for s in range(0, flat.shape[0], step):
        blk = flat[s:s + step]
        nrm = np.sqrt(np.sum(blk.astype(np.float64) ** 2, axis=1, keepdims=True))
        blk[...] = (blk / nrm).astype(np.float32)
    return round_to_bf16(x) if dtype_tag == "bf16" else x


def _plain_normal(rng, shape, dtype_tag):
    x = rng.standard_normal(shape, dtype=np.float32)
    return round_to_bf16(x) if dtype_tag == "bf16" else x


def _correlate_keys(rng, k, rho, dtype_tag):
    B, T, H, dk = k.shape
    c = rng.standard_normal((H, dk))
    a, b = np.sqrt((1.0 - rho) * dk), np.sqrt(rho)
    out = np.empty_like(k)
    for t0 in range(0, T, 4096):
        x = a * k[:, t0:t0 + 4096].astype(np.float64) + b * c
        x /= np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
        out[:, t0:t0 + 4096] = x.astype(np.float32)
    return round_to_bf16(out) if dtype_tag == "bf16" else out


def generate(B, T, H, dk=128, dv=128, dtype="bf16", gate="softplus_head", gate_lo=-0.2,
             gate_hi=-0.005, h0_std=None, dout=False, seed=0, strong_frac=0.7,
             key_corr=0.0, beta_max=1.0) -> GDNInputs:
    """Draw one seeded input set.  See the module docstring for the distributions."""
    if dtype not in ("bf16", "f32"):
        raise ValueError("dtype must be 'bf16' or 'f32'")
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _normal_rows(rng, (B, T, H, dk), dtype)
    k = _normal_rows(rng, (B, T, H, dk), dtype)
    v = _plain_normal(rng, (B, T, H, dv), dtype)
    beta = (beta_max / (1.0 + np.exp(-rng.standard_normal((B, T, H))))).astype(np.float32)
    meta = {"gate": gate}
    if gate == "uniform":
        g = rng.uniform(gate_lo, gate_hi, (B, T, H)).astype(np.float32)
    elif gate == "softplus_head":
        rate = np.exp(rng.uniform(-4.0, -1.0, H))
        x = rng.standard_normal((B, T, H))
        g = (-np.logaddexp(0.0, x) * rate[None, None, :]).astype(np.float32)
        meta["rate"] = rate
    elif gate == "mixed":
        n_strong = int(round(strong_frac * H))
        perm = rng.permutation(H)
        strong = np.zeros(H, bool)
        strong[perm[:n_strong]] = True
        u = rng.random((B, T, H))
        lo = np.where(strong, -0.5, -1e-3)
        hi = np.where(strong, -0.05, -1e-5)
        g = (lo[None, None, :] + (hi - lo)[None, None, :] * u).astype(np.float32)
        meta["strong_heads"] = strong
    else:
        raise ValueError(f"unknown gate kind {gate!r}")
    h0 = None
    if h0_std is not None:
        h0 = (rng.standard_normal((B, H, dk, dv), dtype=np.float32) * np.float32(h0_std))
    do = _plain_normal(rng, (B, T, H, dv), dtype) if dout else None
    if key_corr > 0.0:
        k = _correlate_keys(rng, k, key_corr, dtype)
        meta["key_corr"] = key_corr
    return GDNInputs(q=q, k=k, v=v, g=g, beta=beta, h0=h0, dout=do, dtype=dtype, meta=meta)


#: Named workloads of the per-key-channel-decay variant (KDA): g is [B,T,H,dk]
KDA_WORKLOADS = {
    # bf16 with an initial state; per-(head, channel) decay rates
    "bf16_kda_t4096_h16": dict(B=1, T=4096, H=16, h0_std=0.02, seed=7),
    # the throughput shape of the GDN benchmark, for the KDA kernel
    "bf16_kda_t32768_h32": dict(B=1, T=32768, H=32, h0_std=None, seed=8),
}


def generate_kda(B, T, H, dk=128, dv=128, gate="softplus_channel", gate_lo=-0.3, gate_hi=-0.01,
                 h0_std=None, seed=0, key_corr=0.0, beta_max=1.0) -> GDNInputs:
    """Seeded bf16 inputs of the per-key-channel-decay variant: q, k, v, beta as
    :func:`generate` (key_corr and beta_max included); g [B,T,H,dk] float32, either
    -softplus(x) * A_{h,i} with x ~ N(0,1) per element and a decay rate A_{h,i} =
    exp(U[-4,-1]) drawn once per (head, key channel) ("softplus_channel"), or
    U[gate_lo, gate_hi] per element ("uniform").  Draw order: q, k, v, beta, gate
    parts, h0, then the shared key directions when key_corr > 0."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _normal_rows(rng, (B, T, H, dk), "bf16")
    k = _normal_rows(rng, (B, T, H, dk), "bf16")
    v = _plain_normal(rng, (B, T, H, dv), "bf16")
    beta = (beta_max / (1.0 + np.exp(-rng.standard_normal((B, T, H))))).astype(np.float32)
    meta = {"gate": gate}
    if gate == "softplus_channel":
        rate = np.exp(rng.uniform(-4.0, -1.0, (H, dk)))
        x = rng.standard_normal((B, T, H, dk))
        g = (-np.logaddexp(0.0, x) * rate[None, None]).astype(np.float32)
        meta["rate"] = rate
    elif gate == "uniform":
        g = rng.uniform(gate_lo, gate_hi, (B, T, H, dk)).astype(np.float32)
    else:
        raise ValueError(f"unknown gate kind {gate!r}")
    h0 = None
    if h0_std is not None:
        h0 = (rng.standard_normal((B, H, dk, dv), dtype=np.float32) * np.float32(h0_std))
    if key_corr > 0.0:
        k = _correlate_keys(rng, k, key_corr, "bf16")
        meta["key_corr"] = key_corr
    return GDNInputs(q=q, k=k, v=v, g=g, beta=beta, h0=h0, dout=None, dtype="bf16", meta=meta)


def kda_workload(name: str, **overrides) -> GDNInputs:
    cfg = dict(KDA_WORKLOADS[name])
    cfg.update(overrides)
    return generate_kda(**cfg)


def workload(name: str, **overrides) -> GDNInputs:
    """Inputs of a named workload; keyword overrides replace any of its fields
    (e.g. ``T=`` to draw a shorter sample with the same distributions)."""
    cfg = dict(WORKLOADS[name])
    cfg.update(overrides)
    return generate(**cfg)
