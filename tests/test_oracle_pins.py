"""Pins of the fp64 forward oracle against facts that do not come from the oracle.

Each test below would fail for a plausible slip in the oracle (a dropped decay,
a transposed state, the output read before instead of after the update, a
wrong sign in the delta correction, an off-by-one in the gate index):
  * hand-derived golden values (tests/golden/delta_rule_2x2_forward.json),
  * closed forms: beta = 0 (pure decay), alpha = 1 and beta = 0 (constant
    state), write-at-key (beta = 1, q = k gives o = v), orthonormal keys
    (associative-memory sum),
  * brute force over explicit per-token transition matrices,
  * the chunk-wise WY form (FlashQLA talk summary, paragraph 3) with the gate
    scaling pulled outside the inverse (paragraph 6), at C in {1,4,16,64},
  * the sequence split with an associative correction (paragraph 4) and the
    sliding-window shortcut within its error bound (paragraph 5),
  * linearity in (v, h0), causality and exact call-splitting.
"""
import json
import os

import numpy as np
import pytest

import oracle
import mirrors

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rand(T, dk, dv, seed, B=1, H=1, h0=True, glo=-0.3, ghi=-0.01):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    g = rng.uniform(glo, ghi, (B, T, H))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    H0 = rng.standard_normal((B, H, dk, dv)) * 0.5 if h0 else None
    return q, k, v, g, beta, H0


def _rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


def test_golden_2x2_forward():
    d = json.load(open(os.path.join(GOLDEN, "delta_rule_2x2_forward.json")))
    q = np.array(d["q"], float)[None, :, None, :]
    k = np.array(d["k"], float)[None, :, None, :]
    v = np.array(d["v"], float)[None, :, None, :]
    g = np.log(np.array(d["alpha"], float))[None, :, None]
    beta = np.array(d["beta"], float)[None, :, None]
    h0 = np.array(d["h0"], float)[None, None]
    o, ht = oracle.fwd(q, k, v, g, beta, h0, scale=d["scale"])
    np.testing.assert_allclose(o[0, :, 0, :], np.array(d["o"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(ht[0, 0], np.array(d["ht"]), rtol=0, atol=1e-14)


def test_beta_zero_is_pure_decay():
    q, k, v, g, beta, h0 = _rand(40, 8, 6, 1, B=2, H=3)
    beta[:] = 0.0
    o, ht = oracle.fwd(q, k, v, g, beta, h0)
    gam = np.cumsum(g, axis=1)                      # [B,T,H]
    exp_ht = np.exp(gam[:, -1, :])[:, :, None, None] * h0
    np.testing.assert_allclose(ht, exp_ht, rtol=1e-13, atol=1e-15)
    exp_o = np.exp(gam)[..., None] * np.einsum("bthi,bhij->bthj", q, h0)
    np.testing.assert_allclose(o, exp_o, rtol=1e-12, atol=1e-14)


def test_alpha_one_beta_zero_constant_state():
    q, k, v, g, beta, h0 = _rand(17, 5, 7, 2, B=1, H=2)
    g[:] = 0.0
    beta[:] = 0.0
    o, ht = oracle.fwd(q, k, v, g, beta, h0, scale=0.75)
    np.testing.assert_allclose(ht, h0, rtol=0, atol=0)
    np.testing.assert_allclose(o, 0.75 * np.einsum("bthi,bhij->bthj", q, h0), rtol=1e-13,
                               atol=1e-15)


@pytest.mark.parametrize("seed", [3, 4])
def test_write_at_key(seed):
    """beta = 1 and a unit key overwrite the value stored at that key: reading the
    state back with q = k returns v exactly, whatever the decay and prior state."""
    q, k, v, g, beta, h0 = _rand(33, 16, 9, seed, B=1, H=2)
    beta[:] = 1.0
    q = k.copy()
    o, _ = oracle.fwd(q, k, v, g, beta, h0)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-12)


def test_orthonormal_keys_associative_memory():
    rng = np.random.default_rng(5)
    dk, dv, T = 12, 5, 12
    Q, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Q.T[None, :, None, :].copy()            # T = dk orthonormal keys
    v = rng.standard_normal((1, T, 1, dv))
    q = rng.standard_normal((1, T, 1, dk))
    g = np.zeros((1, T, 1))
    beta = np.ones((1, T, 1))
    o, ht = oracle.fwd(q, k, v, g, beta, None)
    np.testing.assert_allclose(ht[0, 0], k[0, :, 0, :].T @ v[0, :, 0, :], atol=1e-13)


@pytest.mark.parametrize("dk,dv,T,seed", [(4, 4, 9, 6), (8, 5, 16, 7), (6, 8, 13, 8)])
def test_brute_force_transition_products(dk, dv, T, seed):
    q, k, v, g, beta, h0 = _rand(T, dk, dv, seed)
    o, ht = oracle.fwd(q, k, v, g, beta, h0, scale=0.5)
    ob, hb = mirrors.brute_force_head(q[0, :, 0], k[0, :, 0], v[0, :, 0], g[0, :, 0],
                                      beta[0, :, 0], h0[0, 0], scale=0.5)
    assert _rel(o[0, :, 0], ob) < 1e-12
    assert _rel(ht[0, 0], hb) < 1e-12


@pytest.mark.parametrize("C", [1, 4, 16, 64])
def test_chunked_wy_form(C):
    q, k, v, g, beta, h0 = _rand(200, 128, 128, 9, B=1, H=2, glo=-0.2, ghi=-0.005)
    o, ht = oracle.fwd(q, k, v, g, beta, h0)
    for h in range(2):
        oc, hc = mirrors.chunked_head(q[0, :, h], k[0, :, h], v[0, :, h], g[0, :, h],
                                      beta[0, :, h], h0[0, h], C=C)
        assert _rel(o[0, :, h], oc) < 1e-10
        assert _rel(ht[0, h], hc) < 1e-10


def test_factored_inverse_equals_direct():
    """Pulling the unit-diagonal gate scaling outside the inverse is exact."""
    rng = np.random.default_rng(10)
    C, dk = 64, 128
    kc = rng.standard_normal((C, dk))
    kc /= np.linalg.norm(kc, axis=1, keepdims=True)
    gc = rng.uniform(-0.4, -0.01, C)
    bc = rng.uniform(0, 1, C)
    gam, T0, T = mirrors.chunk_prep(kc, gc, bc)
    A = np.tril(bc[:, None] * np.exp(gam[:, None] - gam[None, :]) * (kc @ kc.T), -1)
    Tdirect = np.linalg.inv(np.eye(C) + A)
    assert _rel(T, Tdirect) < 1e-12


def test_sequence_split_matches():
    q, k, v, g, beta, h0 = _rand(640, 128, 128, 11, glo=-0.02, ghi=-0.0005)
    o, ht = oracle.fwd(q, k, v, g, beta, h0)
    for bounds in ([0, 128, 320, 448], [0, 64, 128, 192, 256, 320, 384, 448, 512, 576]):
        os_, hs = mirrors.split_head(q[0, :, 0], k[0, :, 0], v[0, :, 0], g[0, :, 0],
                                     beta[0, :, 0], h0[0, 0], bounds)
        assert _rel(o[0, :, 0], os_) < 1e-10
        assert _rel(ht[0, 0], hs) < 1e-10


def test_window_shortcut_within_bound():
    """With every w-chunk window summing to at most log(eps), the window result
    differs from the exact one by at most eps * ||H||_2 * ||q|| per output."""
    q, k, v, g, beta, h0 = _rand(1024, 128, 128, 12, glo=-0.5, ghi=-0.05)
    w = 2
    o, ht = oracle.fwd(q, k, v, g, beta, h0)
    bounds = [0, 256, 512, 768]
    ow, hw = mirrors.window_head(q[0, :, 0], k[0, :, 0], v[0, :, 0], g[0, :, 0], beta[0, :, 0],
                                 h0[0, 0], bounds, w)
    flags, mx = oracle.gate_scan(g, chunk=64, window_chunks=w, log_eps=np.log(2.0 ** -24))
    assert flags[0, 0] == 1
    # the dropped term is the exact state at each warm-up start, decayed by at least
    # exp(max window sum); ||q|| = 1, and each per-token map has spectral norm <= alpha
    hmax = 0.0
    for s in bounds[1:]:
        _, hs = oracle.fwd(q[:, :s - w * 64], k[:, :s - w * 64], v[:, :s - w * 64],
                           g[:, :s - w * 64], beta[:, :s - w * 64], h0)
        hmax = max(hmax, np.linalg.norm(hs[0, 0], 2))
    bound = np.exp(mx[0, 0]) * hmax
    assert bound < 1e-5
    assert np.max(np.abs(o[0, :, 0] - ow)) <= bound
    assert np.max(np.abs(ht[0, 0] - hw)) <= bound
    # and the shortcut is not trivially exact: a one-chunk window with weak decay
    # is visibly wrong, so the comparison above is not vacuous
    ow1, _ = mirrors.window_head(q[0, :, 0], k[0, :, 0], v[0, :, 0], g[0, :, 0] * 0.01,
                                 beta[0, :, 0], h0[0, 0], bounds, 0)
    o1, _ = oracle.fwd(q, k, v, g * 0.01, beta, h0)
    assert np.max(np.abs(o1[0, :, 0] - ow1)) > 1e-6


def test_linearity_in_values_and_state():
    q, k, v, g, beta, h0 = _rand(70, 16, 8, 13)
    _, _, v2, _, _, h02 = _rand(70, 16, 8, 14)
    a, b = 0.7, -1.3
    o1, h1 = oracle.fwd(q, k, v, g, beta, h0)
    o2, h2 = oracle.fwd(q, k, v2, g, beta, h02)
    o3, h3 = oracle.fwd(q, k, a * v + b * v2, g, beta, a * h0 + b * h02)
    np.testing.assert_allclose(o3, a * o1 + b * o2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(h3, a * h1 + b * h2, rtol=1e-11, atol=1e-12)


def test_causality():
    q, k, v, g, beta, h0 = _rand(50, 16, 8, 15)
    o1, _ = oracle.fwd(q, k, v, g, beta, h0)
    t = 31
    k2, v2, g2 = k.copy(), v.copy(), g.copy()
    k2[0, t:] = -k2[0, t:]
    v2[0, t:] += 3.0
    g2[0, t:] *= 2
    o2, _ = oracle.fwd(q, k2, v2, g2, beta, h0)
    np.testing.assert_array_equal(o1[0, :t], o2[0, :t])
    assert np.max(np.abs(o1[0, t:] - o2[0, t:])) > 1e-3


def test_call_splitting():
    q, k, v, g, beta, h0 = _rand(150, 32, 24, 16, B=2, H=2)
    o, ht = oracle.fwd(q, k, v, g, beta, h0)
    s = 77
    oa, ha = oracle.fwd(q[:, :s], k[:, :s], v[:, :s], g[:, :s], beta[:, :s], h0)
    ob, hb = oracle.fwd(q[:, s:], k[:, s:], v[:, s:], g[:, s:], beta[:, s:], ha)
    np.testing.assert_allclose(np.concatenate([oa, ob], 1), o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(hb, ht, rtol=1e-12, atol=1e-13)


def test_head_subset_and_threads_agree():
    q, k, v, g, beta, h0 = _rand(65, 32, 16, 17, B=2, H=3)
    o, ht = oracle.fwd(q, k, v, g, beta, h0, nthreads=1)
    o4, ht4 = oracle.fwd(q, k, v, g, beta, h0, nthreads=4)
    np.testing.assert_array_equal(o, o4)
    np.testing.assert_array_equal(ht, ht4)
    os_, hs = oracle.fwd(q, k, v, g, beta, h0, heads=[4, 1])
    for bh in (4, 1):
        b, h = divmod(bh, 3)
        np.testing.assert_array_equal(os_[b, :, h], o[b, :, h])
        np.testing.assert_array_equal(hs[b, h], ht[b, h])
    assert np.all(os_[0, :, 0] == 0)
