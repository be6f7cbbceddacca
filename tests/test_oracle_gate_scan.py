"""Pins of the oracle's gate scan (FlashQLA talk summary, paragraph 5: one light
kernel scans the gate distribution and marks the heads whose alpha-powers decay
below a threshold within a window).

  * brute force: every window of w whole chunks summed token by token in Python,
  * closed form: a constant gate g gives window sum g * C * w exactly,
  * edge cases: fewer than w chunks never flags; a short last chunk only adds
    its own tokens; the comparison is "<=" at the threshold.
"""
import numpy as np
import pytest

import oracle


def _brute(g, C, w, log_eps):
    B, T, H = g.shape
    N = -(-T // C)
    flags = np.zeros((B, H), np.int32)
    mx = np.full((B, H), -np.inf)
    for b in range(B):
        for h in range(H):
            best = -np.inf
            for c in range(w - 1, N):
                tot = 0.0
                for t in range((c - w + 1) * C, min((c + 1) * C, T)):
                    tot += float(g[b, t, h])
                best = max(best, tot)
            mx[b, h] = best
            flags[b, h] = int(N >= w and best <= log_eps)
    return flags, mx


@pytest.mark.parametrize("T,C,w,seed", [(100, 8, 3, 0), (257, 16, 4, 1), (64, 64, 1, 2),
                                        (40, 8, 6, 3)])
def test_brute_force(T, C, w, seed):
    rng = np.random.default_rng(seed)
    g = -rng.exponential(0.4, (2, T, 3)) * rng.uniform(0.01, 3, (1, 1, 3))
    log_eps = float(np.quantile(g.sum(1), 0.5)) * w * C / T
    f, m = oracle.gate_scan(g, chunk=C, window_chunks=w, log_eps=log_eps)
    fb, mb = _brute(g, C, w, log_eps)
    np.testing.assert_allclose(m, mb, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(f, fb)


def test_constant_gate_closed_form():
    C, w = 64, 8
    g = np.full((1, 64 * 20, 2), -0.03)
    g[..., 1] = -0.04
    f, m = oracle.gate_scan(g, chunk=C, window_chunks=w, log_eps=-16.0)
    np.testing.assert_allclose(m[0], [-0.03 * C * w, -0.04 * C * w], rtol=1e-12)
    # -15.36 > -16 (not flagged); -20.48 <= -16 (flagged)
    np.testing.assert_array_equal(f[0], [0, 1])


def test_short_sequences_and_threshold():
    g = np.full((1, 64 * 7 + 5, 1), -1.0)
    f, m = oracle.gate_scan(g, chunk=64, window_chunks=8, log_eps=-1.0)
    assert f[0, 0] == 1 and m[0, 0] == -(64 * 7 + 5)      # 8 chunks, the last one short
    f, m = oracle.gate_scan(g[:, :64 * 7], chunk=64, window_chunks=8, log_eps=0.0)
    assert f[0, 0] == 0 and m[0, 0] == -np.inf             # fewer than w chunks
    g2 = np.full((1, 128, 1), -0.25)
    f, m = oracle.gate_scan(g2, chunk=64, window_chunks=2, log_eps=-32.0)
    assert m[0, 0] == -32.0 and f[0, 0] == 1                # equality flags
