"""Host study of the 32x32 diagonal-block inverse the chunk step needs (step 1 of
the chunk algorithm in the FlashQLA talk summary, paragraph 3), in numpy with the
kernel's operand rounding: bf16 matrix-product operands, float32 accumulation.

The inverse T0 = (I + Nd)^-1, Nd = diag(beta) strict_lower(K K^T), has a plain
definition (np.linalg.inv in float64).  Two ways to build it from 32x32 products:
  * the power series (I - Nd)(I + Nd^2)(I + Nd^4)(I + Nd^8)(I + Nd^16), exact in
    exact arithmetic (Nd^32 = 0), but its partial products hold entries far larger
    than the inverse's once the chunk's keys are correlated, and cancel;
  * recursive block doubling Z <- Z - Z No Z (No: the entries joining block
    pairs), whose every product forms entries of the inverse itself.
The kernel uses the second; these tests show why, with the keys of the seeded
generator's key_corr option.  The doubling's error grows with the largest entry
of Nd; a block with an entry above 1 (beta up to 2) gets one Newton step with a
split-precision residual, which the last test pins.  No kernel code is involved: this pins the method,
the GPU parity tests pin the kernels.
"""
import numpy as np
import torch

from gated_deltanet_chunked_prefill_amd import inputs


def _bf(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).to(torch.float32).numpy().astype(np.float64)


def _f32(x):
    return np.asarray(x, np.float64).astype(np.float32).astype(np.float64)


def _mm(x, y):   # one MFMA product: bf16 operands, float32 accumulation
    return _f32(_bf(x) @ _bf(y))


def _series(nd):
    m = -nd
    z = np.eye(32) + m
    for _ in range(4):
        m = _mm(m, m)
        z = _f32(z + _mm(z, m))
    return z


def _doubling(nd):
    i, j = np.meshgrid(np.arange(32), np.arange(32), indexing="ij")
    pair = (i == j + 1) & (i % 2 == 1)
    z = _f32(np.eye(32) - np.where(pair, nd, 0.0))
    for lev in range(1, 5):
        join = ((i >> lev) == (j >> lev) + 1) & (((i >> lev) & 1) == 1)
        q = _mm(np.where(join, nd, 0.0), z)
        z = _f32(z - _mm(z, q))
    return z


def _blocks(rho, n=12, seed=0, beta_max=1.0):
    x = inputs.generate(B=1, T=32 * n, H=1, key_corr=rho, seed=seed, beta_max=beta_max)
    for c in range(n):
        k = x.k[0, 32 * c:32 * c + 32, 0].astype(np.float64)
        beta = x.beta[0, 32 * c:32 * c + 32, 0].astype(np.float64)
        nd = _f32(np.tril(beta[:, None] * _f32(k @ k.T), -1))
        yield nd, np.linalg.inv(np.eye(32) + nd)


def _rel(a, ref):
    return float(np.max(np.abs(a - ref)) / np.max(np.abs(ref)))


def test_doubling_is_exact_in_float64():
    for nd, ref in _blocks(0.9, n=4):
        i, j = np.meshgrid(np.arange(32), np.arange(32), indexing="ij")
        z = np.eye(32) - np.where((i == j + 1) & (i % 2 == 1), nd, 0.0)
        for lev in range(1, 5):
            join = ((i >> lev) == (j >> lev) + 1) & (((i >> lev) & 1) == 1)
            z = z - z @ np.where(join, nd, 0.0) @ z
        assert _rel(z, ref) < 1e-12


def test_doubling_stays_at_bf16_rounding_for_correlated_keys():
    for rho in (0.0, 0.5, 0.9, 0.99):
        worst = max(_rel(_doubling(nd), ref) for nd, ref in _blocks(rho))
        # storing T0 in bf16 alone costs up to 2^-9 = 2e-3 relative
        assert worst < 1e-2, (rho, worst)


def test_series_fails_for_correlated_keys():
    # independent keys: the series is as good as the doubling
    assert max(_rel(_series(nd), ref) for nd, ref in _blocks(0.0)) < 1e-2
    # keys with pairwise cosine 0.9: the series loses every digit
    assert max(_rel(_series(nd), ref) for nd, ref in _blocks(0.9)) > 1.0


def _split(x):
    hi = _bf(x)
    return hi, _bf(_f32(x - hi))


def _refined(nd):
    # the doubling through its last step, then Z <- Z + Z R with R = I - Z - Nd Z,
    # Nd Z from split bf16 operands (hi*hi + hi*lo + lo*hi, float32 accumulation)
    z = _doubling(nd)
    nh, nl = _split(nd)
    zh, zl = _split(z)
    ndz = _f32(_f32(_f32(nh @ zl) + nl @ zh) + nh @ zh)
    r = _f32(np.eye(32) - z - ndz)
    return _f32(z + _mm(z, r))


def test_refinement_for_beta_up_to_two():
    for rho in (0.9, 0.99):
        blocks = list(_blocks(rho, beta_max=2.0, seed=3))
        assert max(np.abs(nd).max() for nd, _ in blocks) > 1.0   # the refinement's trigger
        plain = max(_rel(_doubling(nd), ref) for nd, ref in blocks)
        refined = max(_rel(_refined(nd), ref) for nd, ref in blocks)
        assert plain > 5e-3 and refined < 3e-4 and refined < plain / 30, (rho, plain, refined)
