"""Pins of the oracle's per-channel-decay variant (KDA, ``oracle.kda_fwd``).

The pages do not print KDA's recurrence; the oracle states its reading (one decay
per key channel, applied to the state before the delta correction).  These tests pin
that function to results fixed independently of it: the scalar-gate oracle when all
channels decay alike, closed forms for beta = 0 (pure per-channel decay) and for
keys along one channel with beta = 1 (last write, then per-channel decay), the
single-channel update rule for aligned keys with any beta, and linearity in V."""
import numpy as np
import pytest

import oracle
from gated_deltanet_chunked_prefill_amd import inputs


def _case(B=2, T=37, H=3, dk=8, dv=6, seed=0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    g = -rng.uniform(0.0, 0.3, (B, T, H, dk))
    beta = rng.uniform(0.05, 0.95, (B, T, H))
    h0 = rng.standard_normal((B, H, dk, dv))
    return q, k, v, g, beta, h0


def test_equal_channels_is_the_scalar_gate_oracle():
    """Every channel with the same decay: the gated delta rule itself."""
    x = inputs.generate(B=2, T=64 + 29, H=2, h0_std=0.1, seed=61)
    g4 = np.repeat(x.g[..., None], x.q.shape[3], axis=3)
    o1, h1 = oracle.kda_fwd(x.q, x.k, x.v, g4, x.beta, x.h0, scale=0.3)
    o2, h2 = oracle.fwd(x.q, x.k, x.v, x.g, x.beta, x.h0, scale=0.3)
    assert np.abs(o1 - o2).max() <= 1e-12 * np.abs(o2).max()
    assert np.abs(h1 - h2).max() <= 1e-12 * np.abs(h2).max()


def test_beta_zero_is_pure_per_channel_decay():
    """beta = 0: S_t = diag(exp(g_1 + ... + g_t)) S_0, rows scaled by their own
    key channel's cumulative decay."""
    q, k, v, g, beta, h0 = _case(seed=1)
    beta[...] = 0.0
    o, ht = oracle.kda_fwd(q, k, v, g, beta, h0, scale=1.7)
    G = np.cumsum(g, axis=1)                                   # [B,T,H,dk]
    S_t = np.exp(G)[..., None] * h0[:, None]                   # [B,T,H,dk,dv]
    o_ref = 1.7 * np.einsum("bthkv,bthk->bthv", S_t, q)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ht, S_t[:, -1], rtol=1e-12, atol=1e-12)


def test_aligned_keys_beta_one_last_write_then_decay():
    """Keys along one channel (k_t = e_j) with beta = 1: row i of the state holds the
    value last written to channel i, decayed by that channel's gates since (or the
    initial row decayed from the start, if channel i was never written)."""
    B, T, H, dk, dv = 1, 40, 2, 5, 4
    q, _, v, g, beta, h0 = _case(B, T, H, dk, dv, seed=2)
    rng = np.random.default_rng(3)
    ch = rng.integers(0, dk, (B, T, H))
    k = np.eye(dk)[ch]                                         # one-hot keys
    beta[...] = 1.0
    o, ht = oracle.kda_fwd(q, k, v, g, beta, h0)
    for b in range(B):
        for h in range(H):
            for t in range(T):
                S = np.empty((dk, dv))
                for i in range(dk):
                    w = [s for s in range(t + 1) if ch[b, s, h] == i]
                    if w:
                        tau = w[-1]
                        S[i] = v[b, tau, h] * np.exp(g[b, tau + 1:t + 1, h, i].sum())
                    else:
                        S[i] = h0[b, h, i] * np.exp(g[b, :t + 1, h, i].sum())
                np.testing.assert_allclose(o[b, t, h], S.T @ q[b, t, h], rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(ht[b, h], S, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("seed", [4, 5])
def test_aligned_keys_any_beta_row_update(seed):
    """Keys along channel j with gate beta: row j becomes (1 - beta) alpha_j S_j +
    beta v, every other row i only decays by alpha_i (derived from the reading:
    diag(alpha) commutes with e_j e_j^T)."""
    B, T, H, dk, dv = 1, 25, 1, 6, 3
    q, _, v, g, beta, h0 = _case(B, T, H, dk, dv, seed=seed)
    ch = np.random.default_rng(seed + 10).integers(0, dk, (B, T, H))
    k = np.eye(dk)[ch]
    o, ht = oracle.kda_fwd(q, k, v, g, beta, h0)
    S = h0[0, 0].copy()
    for t in range(T):
        a = np.exp(g[0, t, 0])
        j, bt = ch[0, t, 0], beta[0, t, 0]
        new = a[:, None] * S
        new[j] = (1.0 - bt) * a[j] * S[j] + bt * v[0, t, 0]
        S = new
        np.testing.assert_allclose(o[0, t, 0], S.T @ q[0, t, 0], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(ht[0, 0], S, rtol=1e-11, atol=1e-12)


def test_linear_in_values_from_zero_state():
    """From a zero state the outputs and the final state are linear in V."""
    q, k, v, g, beta, _ = _case(seed=6)
    v2 = np.random.default_rng(7).standard_normal(v.shape)
    o1, h1 = oracle.kda_fwd(q, k, v, g, beta)
    o2, h2 = oracle.kda_fwd(q, k, v2, g, beta)
    o3, h3 = oracle.kda_fwd(q, k, 2.0 * v - 3.0 * v2, g, beta)
    np.testing.assert_allclose(o3, 2.0 * o1 - 3.0 * o2, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(h3, 2.0 * h1 - 3.0 * h2, rtol=1e-10, atol=1e-10)
