"""GPU parity of the per-key-channel-decay forward (KDA, gdn_kda_fwd) against the
oracle's token-by-token KDA recurrence (oracle.kda_fwd, float64) on the same
seeded bf16 inputs: max|X - X_ref| <= 2e-2 * max|X_ref| for o and the final
state.  The oracle runs its token loop in Python, so these cases stay small."""
import numpy as np
import pytest

import oracle
from gated_deltanet_chunked_prefill_amd import inputs
from helpers import TOL_BF16, rel_err, say, to_gpu, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdn():
    import torch
    assert torch.cuda.is_available()
    import gated_deltanet_chunked_prefill_amd as m
    return m


def _run(gdn, x, scale=1.0):
    import torch
    t = to_gpu(x)
    g = torch.from_numpy(np.ascontiguousarray(x.g)).cuda()
    o, ht = gdn.gdn_kda_fwd(t["q"], t["k"], t["v"], g, t["beta"], t["h0"], scale=scale)
    torch.cuda.synchronize()
    oref, href = oracle.kda_fwd(x.q, x.k, x.v, x.g, x.beta, x.h0, scale=scale)
    return to_np(o), to_np(ht), oref, href


def _check(o, ht, oref, href, label):
    eo, eh = rel_err(o, oref), rel_err(ht, href)
    say(f"  {label}: o err {eo:.3e}  ht err {eh:.3e}  (tol {TOL_BF16})")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(ht))
    assert eo <= TOL_BF16 and eh <= TOL_BF16, (eo, eh)


@pytest.mark.parametrize("T", [1, 31, 63, 64, 65, 150])
def test_kda_ragged_lengths(gdn, T):
    say(f"case KDA T={T}")
    x = inputs.generate_kda(B=2, T=T, H=2, h0_std=0.05, seed=200 + T)
    _check(*_run(gdn, x, scale=0.7), f"T={T}")


def test_kda_no_initial_state_uniform_gates(gdn):
    say("case KDA uniform per-channel gates, no h0")
    x = inputs.generate_kda(B=1, T=64 * 5 + 9, H=3, gate="uniform", gate_lo=-0.5, gate_hi=-0.001, seed=211)
    _check(*_run(gdn, x), "uniform gates")


def test_kda_correlated_keys(gdn):
    """Keys sharing a direction (pairwise cosine about 0.9)."""
    say("case KDA correlated keys rho=0.9")
    x = inputs.generate_kda(B=1, T=64 * 4 + 7, H=2, h0_std=0.05, seed=213, key_corr=0.9)
    _check(*_run(gdn, x), "rho=0.9")


def test_kda_beta_up_to_two(gdn):
    """beta up to 2 with keys of cosine 0.9."""
    say("case KDA beta up to 2, key cosine 0.9")
    x = inputs.generate_kda(B=1, T=64 * 4 + 7, H=2, h0_std=0.05, seed=214, key_corr=0.9, beta_max=2.0)
    _check(*_run(gdn, x), "beta<=2 rho=0.9")


def test_kda_strong_channel_decay(gdn):
    """Channels that decay by up to e^-3 per token (e^-96 over a 32-token half):
    the re-centred tiles keep every factor finite and the result matches."""
    say("case KDA strong per-channel decay")
    x = inputs.generate_kda(B=1, T=64 * 4, H=2, gate="uniform", gate_lo=-3.0, gate_hi=-0.0, h0_std=0.05,
                            seed=212)
    _check(*_run(gdn, x), "strong decay")


def test_kda_equal_channels_match_gdn_forward(gdn):
    """Every key channel with the same gate: the KDA kernel computes the gated
    delta rule, so it agrees with the oracle's scalar-gate recurrence and with
    the GDN forward kernel."""
    import torch
    say("case KDA with equal channels vs the GDN forward")
    x = inputs.generate(B=1, T=64 * 6 + 21, H=3, h0_std=0.05, seed=213)
    g4 = np.ascontiguousarray(np.repeat(x.g[..., None], 128, axis=3))
    t = to_gpu(x)
    o1, h1 = gdn.gdn_kda_fwd(t["q"], t["k"], t["v"], torch.from_numpy(g4).cuda(), t["beta"], t["h0"])
    o2, h2 = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["h0"], split_mode=1)
    torch.cuda.synchronize()
    oref, href = oracle.fwd(x.q, x.k, x.v, x.g, x.beta, x.h0)
    _check(to_np(o1), to_np(h1), oref, href, "KDA kernel vs scalar-gate oracle")
    assert rel_err(to_np(o1), to_np(o2)) <= TOL_BF16 and rel_err(to_np(h1), to_np(h2)) <= TOL_BF16


@pytest.mark.slow
def test_kda_t4096_h16(gdn):
    say("case bf16_kda_t4096_h16 (every head)")
    x = inputs.kda_workload("bf16_kda_t4096_h16")
    _check(*_run(gdn, x), "t4096 h16")
