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


def _run(gdn, x, scale=1.0, n_segments=0):
    import torch
    t = to_gpu(x)
    g = torch.from_numpy(np.ascontiguousarray(x.g)).cuda()
    o, ht = gdn.gdn_kda_fwd(t["q"], t["k"], t["v"], g, t["beta"], t["h0"], scale=scale, n_segments=n_segments)
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


@pytest.mark.parametrize("nseg", [1, 2])
def test_kda_decay_at_range_limit(gdn, nseg):
    """Every channel decaying by 5.3 to 5.4 per token (up to 86 over 16 tokens,
    just inside the float32 range that the re-centred factors need): finite and
    equal to the oracle, unsplit and split."""
    say(f"case KDA decay at the range limit, n_segments={nseg}")
    x = inputs.generate_kda(B=1, T=64 * 3 + 5, H=2, gate="uniform", gate_lo=-5.4, gate_hi=-5.3, h0_std=0.05,
                            seed=215)
    _check(*_run(gdn, x, n_segments=nseg), f"decay 5.4 per token, n_segments={nseg}")


def test_kda_no_final_state_split(gdn):
    """Split into 3 segments without a final state (ht not written)."""
    import torch
    say("case KDA split 3 without ht")
    x = inputs.generate_kda(B=1, T=64 * 7 + 3, H=2, h0_std=0.05, seed=216)
    t = to_gpu(x)
    g = torch.from_numpy(np.ascontiguousarray(x.g)).cuda()
    o, ht = gdn.gdn_kda_fwd(t["q"], t["k"], t["v"], g, t["beta"], t["h0"], output_final_state=False, n_segments=3)
    torch.cuda.synchronize()
    assert ht is None
    oref, _ = oracle.kda_fwd(x.q, x.k, x.v, x.g, x.beta, x.h0)
    eo = rel_err(to_np(o), oref)
    say(f"  o err {eo:.3e}")
    assert eo <= TOL_BF16, eo


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


# Sequence split: segments 0 .. P-2 give their transition M and zero-start state
# b, the chain composes them, every segment then runs from its entering state.
@pytest.mark.parametrize("nseg", [2, 3, 4, 10])
def test_kda_split(gdn, nseg):
    """T = 9 chunks + 13 tokens (10 chunks, the last ragged): 2 (no chain), 3,
    4 and 10 segments (one chunk each) with h0, against the oracle and the
    unsplit call."""
    say(f"case KDA split n_segments={nseg}")
    x = inputs.generate_kda(B=2, T=64 * 9 + 13, H=2, h0_std=0.05, seed=220 + nseg)
    o, ht, oref, href = _run(gdn, x, scale=0.8, n_segments=nseg)
    _check(o, ht, oref, href, f"split {nseg}")
    o1, h1, _, _ = _run(gdn, x, scale=0.8, n_segments=1)
    d = max(rel_err(o, o1), rel_err(ht, h1))
    say(f"  split {nseg} vs unsplit: {d:.3e}")
    assert d <= 1e-2, d


def test_kda_split_no_h0_correlated_keys(gdn):
    """Split into 3 segments (4, 4, 3 chunks), no h0, keys of cosine 0.9, beta up to 2."""
    say("case KDA split 3, no h0, rho=0.9, beta<=2")
    x = inputs.generate_kda(B=1, T=64 * 11 - 5, H=3, seed=231, key_corr=0.9, beta_max=2.0)
    _check(*_run(gdn, x, n_segments=3), "split 3 rho=0.9 beta<=2")


def test_kda_split_strong_decay(gdn):
    """Split into 4 segments with channels decaying by up to e^-3 per token: the
    transitions are near zero in those rows, the composed states still match."""
    say("case KDA split 4, strong per-channel decay")
    x = inputs.generate_kda(B=1, T=64 * 8, H=2, gate="uniform", gate_lo=-3.0, gate_hi=-0.0, h0_std=0.05,
                            seed=232)
    _check(*_run(gdn, x, n_segments=4), "split 4 strong decay")


def test_kda_split_workspace_reuse(gdn):
    """One caller-owned workspace for two calls in a row, the second smaller and
    with other segment counts: stale slots from the first call change nothing."""
    import torch
    say("case KDA split workspace reuse")
    xa = inputs.generate_kda(B=1, T=64 * 12, H=3, h0_std=0.05, seed=233)
    xb = inputs.generate_kda(B=2, T=64 * 5 + 1, H=1, h0_std=0.05, seed=234)
    n = gdn.gdn_kda_fwd_workspace_size(1, 64 * 12, 3, n_segments=6)
    assert n == 3 * 5 * 2 * 128 * 128 * 4
    ws = torch.full((n,), 255, dtype=torch.uint8, device="cuda")   # NaN bit patterns
    for x, nseg in ((xa, 6), (xb, 3)):
        t = to_gpu(x)
        g = torch.from_numpy(np.ascontiguousarray(x.g)).cuda()
        o, ht = gdn.gdn_kda_fwd(t["q"], t["k"], t["v"], g, t["beta"], t["h0"], n_segments=nseg, workspace=ws)
        torch.cuda.synchronize()
        oref, href = oracle.kda_fwd(x.q, x.k, x.v, x.g, x.beta, x.h0)
        _check(to_np(o), to_np(ht), oref, href, f"reuse n_segments={nseg}")


@pytest.mark.slow
def test_kda_throughput_shape_split_sampled(gdn):
    """The throughput shape (T = 32768, H = 32) with the automatic split (9
    segments of 57 chunks on 256 CUs): heads 0 and 31 against the oracle over the
    whole sequence, every head against the unsplit call."""
    import torch
    say("case bf16_kda_t32768_h32 automatic split, heads 0 and 31 vs the oracle")
    x = inputs.kda_workload("bf16_kda_t32768_h32")
    t = to_gpu(x)
    g = torch.from_numpy(np.ascontiguousarray(x.g)).cuda()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    say(f"  {cus} CUs: {gdn.gdn_kda_plan_segments(1, 32768, 32, cus)} segments per head")
    o, ht = gdn.gdn_kda_fwd(t["q"], t["k"], t["v"], g, t["beta"], None)
    o1, h1 = gdn.gdn_kda_fwd(t["q"], t["k"], t["v"], g, t["beta"], None, n_segments=1)
    torch.cuda.synchronize()
    d = max(rel_err(to_np(o), to_np(o1)), rel_err(to_np(ht), to_np(h1)))
    say(f"  split vs unsplit, every head: {d:.3e}")
    assert d <= 1e-2, d
    for h in (0, 31):
        sl = slice(h, h + 1)
        oref, href = oracle.kda_fwd(x.q[:, :, sl], x.k[:, :, sl], x.v[:, :, sl], x.g[:, :, sl], x.beta[:, :, sl])
        _check(to_np(o[:, :, sl]), to_np(ht[:, sl]), oref, href, f"head {h}")


@pytest.mark.slow
def test_kda_t4096_h16(gdn):
    say("case bf16_kda_t4096_h16 (every head)")
    x = inputs.kda_workload("bf16_kda_t4096_h16")
    _check(*_run(gdn, x), "t4096 h16")
