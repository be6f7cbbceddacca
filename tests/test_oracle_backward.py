"""Pins of the fp64 backward oracle (back-propagation through time).

  * hand-derived gradients of a one-token case (tests/golden/delta_rule_2x2_backward.json),
  * central finite differences of the forward oracle (itself pinned in
    test_oracle_pins.py) for every input, on tiny random cases,
  * fp64 torch autograd through an independent token loop (a library check),
  * closed forms: alpha = 1, beta = 0 gives dq_t = h0 dout_t and
    dh0 = sum_t q_t dout_t^T; beta = 0 gives dk = dv = 0.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import mirrors

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rand(T, dk, dv, seed, B=1, H=2):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    g = rng.uniform(-0.3, -0.01, (B, T, H))
    beta = rng.uniform(0.05, 0.95, (B, T, H))
    h0 = rng.standard_normal((B, H, dk, dv)) * 0.5
    dout = rng.standard_normal((B, T, H, dv))
    dht = rng.standard_normal((B, H, dk, dv))
    return dict(q=q, k=k, v=v, g=g, beta=beta, h0=h0), dout, dht


def test_golden_one_token():
    d = json.load(open(os.path.join(GOLDEN, "delta_rule_2x2_backward.json")))
    q = np.array(d["q"], float)[None, :, None, :]
    k = np.array(d["k"], float)[None, :, None, :]
    v = np.array(d["v"], float)[None, :, None, :]
    g = np.log(np.array(d["alpha"], float))[None, :, None]
    beta = np.array(d["beta"], float)[None, :, None]
    h0 = np.array(d["h0"], float)[None, None]
    dout = np.array(d["dout"], float)[None, :, None, :]
    gr = oracle.bwd(q, k, v, g, beta, dout, h0=h0)
    np.testing.assert_allclose(gr["dq"][0, :, 0], d["dq"], atol=1e-14)
    np.testing.assert_allclose(gr["dk"][0, :, 0], d["dk"], atol=1e-14)
    np.testing.assert_allclose(gr["dv"][0, :, 0], d["dv"], atol=1e-14)
    np.testing.assert_allclose(gr["dbeta"][0, :, 0], d["dbeta"], atol=1e-14)
    np.testing.assert_allclose(gr["dg"][0, :, 0], d["dg"], atol=1e-14)
    np.testing.assert_allclose(gr["dh0"][0, 0], d["dh0"], atol=1e-14)


def _loss(x, dout, dht, scale):
    o, ht = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], scale=scale)
    return float(np.sum(o * dout) + np.sum(ht * dht))


@pytest.mark.parametrize("T,dk,dv,seed,scale", [(10, 4, 3, 1, 1.0), (70, 3, 5, 2, 0.5)])
def test_finite_differences(T, dk, dv, seed, scale):
    x, dout, dht = _rand(T, dk, dv, seed)
    gr = oracle.bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], dout, h0=x["h0"], dht=dht,
                    scale=scale)
    names = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta", "h0": "dh0"}
    rng = np.random.default_rng(seed + 100)
    eps = 1e-6
    for name, gname in names.items():
        arr = x[name]
        idx = [tuple(rng.integers(0, s) for s in arr.shape) for _ in range(25)]
        for ix in idx:
            old = arr[ix]
            arr[ix] = old + eps
            lp = _loss(x, dout, dht, scale)
            arr[ix] = old - eps
            lm = _loss(x, dout, dht, scale)
            arr[ix] = old
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - gr[gname][ix]) <= 1e-7 * max(1.0, abs(fd)), (name, ix, fd,
                                                                          gr[gname][ix])


def _torch_loop(q, k, v, g, beta, h0, scale):
    B, T, H, dk = q.shape
    outs = []
    S = h0
    for t in range(T):
        a = torch.exp(g[:, t])[..., None, None]                       # [B,H,1,1]
        kt, vt, bt = k[:, t], v[:, t], beta[:, t][..., None]          # [B,H,dk] ...
        S = a * S
        p = torch.einsum("bhij,bhi->bhj", S, kt)
        u = bt * (vt - p)
        S = S + kt[..., :, None] * u[..., None, :]
        outs.append(scale * torch.einsum("bhij,bhi->bhj", S, q[:, t]))
    return torch.stack(outs, 1), S


def test_torch_autograd_agrees():
    x, dout, dht = _rand(37, 6, 5, 3, B=2, H=2)
    tx = {n: torch.tensor(a, dtype=torch.float64, requires_grad=True) for n, a in x.items()}
    o, ht = _torch_loop(tx["q"], tx["k"], tx["v"], tx["g"], tx["beta"], tx["h0"], 0.8)
    (o * torch.tensor(dout)).sum().add((ht * torch.tensor(dht)).sum()).backward()
    gr = oracle.bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], dout, h0=x["h0"], dht=dht,
                    scale=0.8)
    for n, gn in {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta",
                  "h0": "dh0"}.items():
        np.testing.assert_allclose(gr[gn], tx[n].grad.numpy(), rtol=1e-10, atol=1e-12)


def test_closed_form_constant_state():
    x, dout, _ = _rand(21, 5, 4, 4)
    x["g"][:] = 0.0
    x["beta"][:] = 0.0
    gr = oracle.bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], dout, h0=x["h0"])
    np.testing.assert_allclose(gr["dq"], np.einsum("bhij,bthj->bthi", x["h0"], dout),
                               rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(gr["dh0"], np.einsum("bthi,bthj->bhij", x["q"], dout),
                               rtol=1e-13, atol=1e-14)
    assert np.all(gr["dk"] == 0) and np.all(gr["dv"] == 0)


def test_beta_zero_no_key_value_gradient():
    x, dout, dht = _rand(30, 5, 4, 5)
    x["beta"][:] = 0.0
    gr = oracle.bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], dout, h0=x["h0"], dht=dht)
    assert np.all(gr["dk"] == 0) and np.all(gr["dv"] == 0)
    assert np.max(np.abs(gr["dbeta"])) > 1e-3


@pytest.mark.parametrize("C", [64, 16, 7])
def test_chunked_backward_mirror_matches_oracle(C):
    """The chunk-wise backward (entry states forward, state gradient backward over
    chunks, local gradients per chunk with the gate gradient as a reverse
    cumulative sum) reaches the token-by-token BPTT gradients (talk summary,
    paragraph 3: the four chunk steps; paragraph 6: the K K^T gradient bundled as
    (dA + dA^T) K)."""
    rng = np.random.default_rng(11)
    B, T, H, dk, dv = 1, 150, 2, 16, 12
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    g = -rng.uniform(0.01, 0.5, (B, T, H))
    beta = rng.uniform(0.0, 1.0, (B, T, H))
    h0 = rng.standard_normal((B, H, dk, dv))
    do = rng.standard_normal((B, T, H, dv))
    dht = rng.standard_normal((B, H, dk, dv))
    ref = oracle.bwd(q, k, v, g, beta, do, h0, dht, scale=0.7)
    for h in range(H):
        m = mirrors.chunked_backward_head(q[0, :, h], k[0, :, h], v[0, :, h], g[0, :, h],
                                          beta[0, :, h], h0[0, h], do[0, :, h], dht[0, h],
                                          C=C, scale=0.7)
        for name in ("dq", "dk", "dv", "dg", "dbeta"):
            r = ref[name][0, :, h]
            assert np.abs(m[name] - r).max() <= 1e-10 * np.abs(r).max(), name
        assert np.abs(m["dh0"] - ref["dh0"][0, h]).max() <= 1e-10 * np.abs(ref["dh0"][0, h]).max()
