"""GPU parity of the fused forward and the gate scan against the fp64 oracle.

Every case draws seeded inputs, runs the HIP path through the C ABI and the
oracle on the same values, and checks max|X - X_ref| <= tol * max|X_ref| for
the output o and the final state ht (tol = 2e-2 for bf16 I/O, 1e-4 for fp32).
"""
import numpy as np
import pytest

import oracle
from gated_deltanet_chunked_prefill_amd import inputs
from helpers import TOL_BF16, TOL_F32, rel_err, say, to_gpu, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdn():
    import torch
    assert torch.cuda.is_available()
    import gated_deltanet_chunked_prefill_amd as m
    return m


def _run(gdn, x, heads=None, scale=1.0, **opts):
    t = to_gpu(x)
    o, ht = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["h0"], scale=scale,
                              **opts)
    import torch
    torch.cuda.synchronize()
    oref, href = oracle.fwd(x.q, x.k, x.v, x.g, x.beta, x.h0, scale=scale, heads=heads)
    return to_np(o), to_np(ht), oref, href


def _check(o, ht, oref, href, tol, heads=None, H=None, label=""):
    if heads is not None:
        sel = [(bh // H, bh % H) for bh in heads]
        eo = max(rel_err(o[b, :, h], oref[b, :, h]) for b, h in sel)
        eh = max(rel_err(ht[b, h], href[b, h]) for b, h in sel)
    else:
        eo, eh = rel_err(o, oref), rel_err(ht, href)
    say(f"  {label}: o err {eo:.3e}  ht err {eh:.3e}  (tol {tol})")
    assert eo <= tol and eh <= tol, (eo, eh)


def test_fp32_tiny(gdn):
    say("case fp32_t128_h1")
    x = inputs.workload("fp32_t128_h1")
    _check(*_run(gdn, x), TOL_F32, label="fp32 tiny")


@pytest.mark.parametrize("T", [1, 63, 64, 65, 100, 200])
def test_bf16_ragged_lengths(gdn, T):
    say(f"case bf16 ragged T={T}")
    x = inputs.generate(B=2, T=T, H=3, h0_std=0.02, seed=100 + T)
    _check(*_run(gdn, x), TOL_BF16, label=f"T={T}")


def test_fp32_ragged_with_state(gdn):
    say("case fp32 ragged T=150 with h0, scale 0.5")
    x = inputs.generate(B=1, T=150, H=2, dtype="f32", gate="uniform", gate_lo=-0.3,
                        gate_hi=-0.01, h0_std=0.1, seed=7)
    _check(*_run(gdn, x, scale=0.5), TOL_F32, label="fp32 ragged")


@pytest.mark.parametrize("P,window", [(1, 0), (2, 0), (3, 0), (5, 1), (8, 1), (8, 0)])
def test_forced_split(gdn, P, window):
    """Any segment count gives the same result within tolerance; with the window
    shortcut on, fast-decaying heads take the window path."""
    say(f"case forced split P={P} window={window}")
    x = inputs.generate(B=1, T=64 * 24 + 17, H=4, h0_std=0.02, seed=11)
    _check(*_run(gdn, x, split_mode=2, n_segments=P, use_window=window), TOL_BF16,
           label=f"P={P} w={window}")


def test_forced_split_one_chunk_segments(gdn):
    """As many segments as chunks: every segment is one chunk, every window
    job warms up from the sequence start or over w earlier chunks."""
    say("case forced split, one chunk per segment")
    x = inputs.generate(B=1, T=64 * 9 + 3, H=3, gate="mixed", strong_frac=0.34, h0_std=0.02, seed=18)
    _check(*_run(gdn, x, split_mode=2, n_segments=10, window_chunks=2), TOL_BF16,
           label="P = N = 10")


def test_forced_split_more_jobs_than_workgroups(gdn):
    """More jobs than persistent workgroups: workgroups run several jobs and the
    waits between exact-head segments still resolve."""
    import torch
    say("case forced split, 64 heads x 12 segments")
    x = inputs.generate(B=2, T=64 * 24 + 5, H=32, gate="mixed", strong_frac=0.5, h0_std=0.02, seed=19)
    t = to_gpu(x)
    B, T, H = 2, 64 * 24 + 5, 32
    opts = dict(split_mode=2, n_segments=12, window_chunks=3)
    ws = torch.zeros(gdn.gdn_chunk_fwd_workspace_size(B, T, H, **opts), dtype=torch.uint8, device="cuda")
    o, ht = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["h0"], workspace=ws, **opts)
    info = gdn.gdn_chunk_fwd_plan_info(B, T, H, workspace=ws, **opts)
    say(f"  plan {info}")
    assert info["error"] == 0
    assert info["P_exact"] == 12 and info["P_window"] == 12
    assert info["n_exact"] + info["n_window"] == B * H
    # exact head: segment 0, 10 pass-1 runs, 4 chain jobs (one per 32 state
    # columns), 11 pass-3 runs; window head: 12 runs
    assert info["n_jobs"] == info["n_exact"] * 26 + info["n_window"] * 12 > 256
    assert info["handed_out"] >= info["n_jobs"]
    oref, href = oracle.fwd(x.q, x.k, x.v, x.g, x.beta, x.h0)
    _check(to_np(o), to_np(ht), oref, href, TOL_BF16, label="64 heads x 12 segments")


def test_split_mixed_heads_window(gdn):
    say("case mixed heads split with window, w=2")
    x = inputs.generate(B=2, T=64 * 40, H=4, gate="mixed", strong_frac=0.5, seed=12)
    flags, _ = oracle.gate_scan(x.g, window_chunks=2)
    assert flags.sum() >= 2 and flags.sum() < flags.size
    _check(*_run(gdn, x, split_mode=2, n_segments=10, window_chunks=2), TOL_BF16,
           label="mixed P=10 w=2")


@pytest.mark.parametrize("rho", [0.5, 0.9, 0.99])
def test_correlated_keys(gdn, rho):
    """Keys of a head sharing a direction (pairwise cosine about rho): the
    diagonal-block inverse keeps its accuracy (a power series in the strictly
    lower part loses every digit at rho = 0.9; see test_inverse_numerics)."""
    say(f"case correlated keys rho={rho}")
    x = inputs.generate(B=1, T=64 * 8 + 21, H=3, h0_std=0.02, seed=40, key_corr=rho)
    _check(*_run(gdn, x), TOL_BF16, label=f"rho={rho}")


@pytest.mark.parametrize("window", [0, 1])
def test_correlated_keys_split(gdn, window):
    """Correlated keys through the split forward: exact heads' gate-free
    transitions (pass 1), the chain and pass 3, and window heads."""
    say(f"case correlated keys rho=0.9, forced split window={window}")
    x = inputs.generate(B=1, T=64 * 16 + 5, H=4, gate="mixed", strong_frac=0.5, h0_std=0.02, seed=41,
                        key_corr=0.9)
    _check(*_run(gdn, x, split_mode=2, n_segments=4, use_window=window), TOL_BF16,
           label=f"rho=0.9 P=4 w={window}")


@pytest.mark.parametrize("opts", [dict(), dict(split_mode=2, n_segments=3, use_window=0)])
def test_beta_up_to_two(gdn, opts):
    """beta up to 2 (each map I - beta k k^T still a contraction) with keys of
    cosine 0.99: entries of Nd above 1, so the diagonal blocks take the Newton
    step after the doubling (pass 1 of the split keeps the plain doubling)."""
    say(f"case beta up to 2, key cosine 0.99 {opts}")
    x = inputs.generate(B=1, T=64 * 8 + 3, H=3, h0_std=0.02, seed=43, key_corr=0.99, beta_max=2.0)
    _check(*_run(gdn, x, **opts), TOL_BF16, label=f"beta<=2 rho=0.99 {opts}")


@pytest.mark.parametrize("opts", [dict(), dict(split_mode=2, n_segments=3)])
def test_correlated_keys_fp32(gdn, opts):
    say(f"case correlated keys rho=0.9 fp32 {opts}")
    x = inputs.generate(B=1, T=64 * 6 + 10, H=2, dtype="f32", gate="uniform", gate_lo=-0.2, gate_hi=-0.005,
                        h0_std=0.05, seed=42, key_corr=0.9)
    _check(*_run(gdn, x, **opts), TOL_F32, label=f"fp32 rho=0.9 {opts}")


@pytest.mark.parametrize("case", ["no_decay", "beta0", "beta1"])
@pytest.mark.parametrize("split", [1, 0, 2])
def test_degenerate_gates(gdn, case, split):
    """Degenerate gates of the recurrence, against the oracle: alpha = 1 (g = 0,
    no decay: no head may take the window shortcut, the split must be exact),
    beta = 0 (the state only decays, o = scale decayed h0^T q) and beta = 1 (each
    token overwrites the value stored at its key), unsplit (1), automatic (0) and
    forced into 5 segments (2)."""
    import torch
    say(f"case degenerate gates {case} split_mode={split}")
    B, T, H = 1, 64 * 12 + 9, 3
    x = inputs.generate(B=B, T=T, H=H, h0_std=0.05, seed=31)
    if case == "no_decay":
        x.g[...] = 0.0
    elif case == "beta0":
        x.beta[...] = 0.0
    else:
        x.beta[...] = 1.0
    opts = dict(split_mode=split, n_segments=5) if split == 2 else dict(split_mode=split)
    t = to_gpu(x)
    ws = torch.empty(max(1, gdn.gdn_chunk_fwd_workspace_size(B, T, H, **opts)), dtype=torch.uint8, device="cuda")
    o, ht = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["h0"], workspace=ws, **opts)
    torch.cuda.synchronize()
    if split == 2 and case == "no_decay":
        info = gdn.gdn_chunk_fwd_plan_info(B, T, H, workspace=ws, **opts)
        assert info["error"] == 0 and info["n_window"] == 0 and info["n_exact"] == B * H, info
    oref, href = oracle.fwd(x.q, x.k, x.v, x.g, x.beta, x.h0)
    _check(to_np(o), to_np(ht), oref, href, TOL_BF16, label=f"{case} split={split}")


def test_strong_decay_pairwise_fallback(gdn):
    """Chunks whose total decay exceeds the factored-exponential range use
    pairwise exponentials; results stay finite and correct."""
    say("case strong decay (|gamma_C| > 160)")
    x = inputs.generate(B=1, T=300, H=2, gate="uniform", gate_lo=-4.0, gate_hi=-2.0,
                        h0_std=0.02, seed=13)
    o, ht, oref, href = _run(gdn, x, split_mode=1)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(ht))
    _check(o, ht, oref, href, TOL_BF16, label="strong decay")


def test_bf16_t4096_h16(gdn):
    say("case bf16_t4096_h16 (auto split)")
    x = inputs.workload("bf16_t4096_h16")
    _check(*_run(gdn, x), TOL_BF16, label="t4096 h16")


def test_call_splitting(gdn):
    """Chunked prefill: running T1 then T2 from the carried state equals one call."""
    import torch
    say("case call splitting")
    x = inputs.generate(B=1, T=64 * 10 + 30, H=2, h0_std=0.02, seed=14)
    t = to_gpu(x)
    o, ht = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["h0"])
    s = 64 * 4 + 7
    sl = lambda a: a[:, :s].contiguous()
    sr = lambda a: a[:, s:].contiguous()
    oa, ha = gdn.gdn_chunk_fwd(sl(t["q"]), sl(t["k"]), sl(t["v"]), sl(t["g"]), sl(t["beta"]), t["h0"])
    ob, hb = gdn.gdn_chunk_fwd(sr(t["q"]), sr(t["k"]), sr(t["v"]), sr(t["g"]), sr(t["beta"]), ha)
    torch.cuda.synchronize()
    oc = torch.cat([oa, ob], 1)
    assert rel_err(to_np(oc), to_np(o)) < TOL_BF16
    assert rel_err(to_np(hb), to_np(ht)) < TOL_BF16


def test_causality_bitwise(gdn):
    """Changing keys and values at and after token t leaves every earlier output
    bit-identical (the split and window choices do not depend on k or v)."""
    import torch
    say("case causality")
    x = inputs.generate(B=1, T=64 * 20, H=2, seed=15)
    t = to_gpu(x)
    o1, _ = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], split_mode=2, n_segments=4)
    cut = 64 * 9 + 5
    k2, v2 = t["k"].clone(), t["v"].clone()
    k2[:, cut:] = -k2[:, cut:]
    v2[:, cut:] += 1.0
    o2, _ = gdn.gdn_chunk_fwd(t["q"], k2, v2, t["g"], t["beta"], split_mode=2, n_segments=4)
    torch.cuda.synchronize()
    assert torch.equal(o1[:, :cut], o2[:, :cut])
    assert not torch.equal(o1[:, cut:], o2[:, cut:])


def test_gate_scan_flags(gdn):
    import torch
    say("case gate scan")
    x = inputs.generate(B=2, T=64 * 50 + 9, H=16, gate="softplus_head", seed=16)
    g = torch.from_numpy(x.g).cuda()
    flags, mx = gdn.gdn_gate_scan(g, window_chunks=8)
    torch.cuda.synchronize()
    fref, mref = oracle.gate_scan(x.g, window_chunks=8)
    mx = mx.cpu().numpy()
    np.testing.assert_allclose(mx, mref, rtol=1e-4, atol=1e-3)
    margin = np.abs(mref - np.log(2.0 ** -24)) > 1e-3
    np.testing.assert_array_equal(flags.cpu().numpy()[margin], fref[margin])
    assert 0 < fref.sum() < fref.size
    # fewer chunks than the window: never flagged
    f2, m2 = gdn.gdn_gate_scan(g[:, :64 * 7].contiguous(), window_chunks=8)
    torch.cuda.synchronize()
    assert int(f2.sum()) == 0 and bool(torch.all(torch.isinf(m2)))


def test_workspace_too_small(gdn):
    import torch
    from gated_deltanet_chunked_prefill_amd import _lib
    x = inputs.generate(B=1, T=64 * 40, H=2, seed=17)
    t = to_gpu(x)
    ws = torch.empty(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(_lib.GDNError) as ei:
        gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], split_mode=2, n_segments=4,
                          workspace=ws)
    assert ei.value.status == _lib.GDN_ERR_WORKSPACE


def _window_levels(g, w=8, levels=4):
    """Per head the smallest m <= levels whose windows of m*w chunks all decay
    below the threshold (oracle gate scan), 0 when none does."""
    lev = np.zeros(g.shape[0] * g.shape[2], np.int64)
    for m in range(levels, 0, -1):
        f, _ = oracle.gate_scan(g, window_chunks=m * w)
        lev[f.reshape(-1) == 1] = m
    return lev


def _check_plan_levels(info, lev, nbh):
    """The device plan keeps the window heads of levels 1 .. Lc for some Lc (the
    rest are exact), so the window count is a prefix sum of the oracle's counts."""
    counts = [int(np.sum(lev == m)) for m in range(1, 9)]
    prefixes = [sum(counts[:lc]) for lc in range(0, 9)]
    assert info["error"] == 0
    assert info["n_exact"] + info["n_window"] == nbh
    assert info["n_window"] in prefixes, (info, counts)


def test_window_levels_mixed(gdn):
    """Heads with different window lengths (8, 16, 24, 32 chunks) in one call:
    the automatic plan and the plan with a single window length agree with the
    oracle, and the levels turn exact heads into window heads."""
    import torch
    say("case window levels, B=1 T=64*160+21 H=12")
    x = inputs.generate(B=1, T=64 * 160 + 21, H=12, gate="softplus_head", h0_std=0.02, seed=24)
    B, T, H = 1, 64 * 160 + 21, 12
    lev = _window_levels(x.g)
    say(f"  oracle levels {lev.tolist()}")
    assert len(set(lev.tolist())) >= 3
    t = to_gpu(x)
    oref, href = oracle.fwd(x.q, x.k, x.v, x.g, x.beta, x.h0)
    infos = {}
    for lv in (1, 4):
        ws = torch.empty(gdn.gdn_chunk_fwd_workspace_size(B, T, H), dtype=torch.uint8, device="cuda")
        o, ht = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["h0"], workspace=ws,
                                  window_levels=lv)
        infos[lv] = gdn.gdn_chunk_fwd_plan_info(B, T, H, workspace=ws, window_levels=lv)
        say(f"  levels={lv}: plan {infos[lv]}")
        _check_plan_levels(infos[lv], np.where(lev <= lv, lev, 0), B * H)
        _check(to_np(o), to_np(ht), oref, href, TOL_BF16, label=f"window_levels={lv}")
    assert infos[4]["n_window"] >= infos[1]["n_window"]


def test_planner_eight_levels(gdn):
    """Window heads of all eight levels (w = 8 chunks) and exact heads in one
    automatic call with window_levels = 8 and a ragged tail: the plan keeps the
    levels up to some cutoff, every job is handed out, and the output agrees with
    the oracle.  Exercises the planner's candidate and breakpoint tables and the
    spare-workgroup boost across many levels."""
    import torch
    say("case planner with eight window levels, B=1 T=64*72+13 H=12")
    B, T, H = 1, 64 * 72 + 13, 12
    x = inputs.generate(B=B, T=T, H=H, h0_std=0.02, seed=41)
    want = [1, 2, 3, 4, 5, 6, 7, 8, 0, 0, 1, 2]
    for h, m in enumerate(want):
        # constant gates with a total decay of 18.7 over m windows of 8 chunks:
        # beyond log(2^-24) = -16.64 over m*8 chunks (also for the windows that
        # end in the 13-token tail), not over (m-1)*8 chunks
        x.g[:, :, h] = -18.7 / (m * 8 * 64) if m else -1e-3
    lev = _window_levels(x.g, levels=8)
    assert lev.tolist() == want, lev.tolist()
    t = to_gpu(x)
    ws = torch.empty(gdn.gdn_chunk_fwd_workspace_size(B, T, H), dtype=torch.uint8, device="cuda")
    o, ht = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["h0"], workspace=ws,
                              window_levels=8)
    info = gdn.gdn_chunk_fwd_plan_info(B, T, H, workspace=ws, window_levels=8)
    say(f"  plan {info}")
    _check_plan_levels(info, lev, B * H)
    assert info["handed_out"] >= info["n_jobs"]
    oref, href = oracle.fwd(x.q, x.k, x.v, x.g, x.beta, x.h0)
    _check(to_np(o), to_np(ht), oref, href, TOL_BF16, label="eight levels")


def test_forced_split_600_heads(gdn):
    """More heads than the planner has threads (600 > 512): the ranking of the
    heads by class runs in two rounds.  Forced split into 3 segments, exact and
    window heads mixed, many jobs per workgroup."""
    import torch
    say("case forced split, 600 heads x 3 segments")
    B, T, H = 2, 64 * 4 + 7, 300
    x = inputs.generate(B=B, T=T, H=H, gate="mixed", strong_frac=0.5, h0_std=0.02, seed=43)
    opts = dict(split_mode=2, n_segments=3, window_chunks=2)
    t = to_gpu(x)
    ws = torch.empty(gdn.gdn_chunk_fwd_workspace_size(B, T, H, **opts), dtype=torch.uint8, device="cuda")
    o, ht = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["h0"], workspace=ws, **opts)
    info = gdn.gdn_chunk_fwd_plan_info(B, T, H, workspace=ws, **opts)
    say(f"  plan {info}")
    assert info["error"] == 0 and info["P_exact"] == 3
    assert info["n_exact"] + info["n_window"] == B * H and info["n_window"] > 0 and info["n_exact"] > 0
    # exact head: segment 0, one pass-1 run, 4 chain jobs, 2 pass-3 runs; window head: 3 runs
    assert info["n_jobs"] == info["n_exact"] * 8 + info["n_window"] * 3
    assert info["handed_out"] >= info["n_jobs"]
    oref, href = oracle.fwd(x.q, x.k, x.v, x.g, x.beta, x.h0)
    _check(to_np(o), to_np(ht), oref, href, TOL_BF16, label="600 heads x 3 segments")


def test_forced_split_4200_heads_global_tables(gdn):
    """More heads than the planner's LDS tables hold (4200 > 4096): one
    workgroup plans with its per-head tables in the workspace and the others
    wait for the job list; 8400 jobs, nearly all taken from the list."""
    import torch
    say("case forced split, 4200 heads x 2 segments (planner tables in the workspace)")
    B, T, H = 2, 64 * 2 + 48, 2100
    x = inputs.generate(B=B, T=T, H=H, h0_std=0.02, seed=47)
    # every other head decays by 25.6 per chunk (19.2 over the 48-token tail): a
    # window head at w = 1
    x.g[:, :, 0::2] = -0.4
    opts = dict(split_mode=2, n_segments=2, window_chunks=1)
    t = to_gpu(x)
    ws = torch.empty(gdn.gdn_chunk_fwd_workspace_size(B, T, H, **opts), dtype=torch.uint8, device="cuda")
    o, ht = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["h0"], workspace=ws, **opts)
    info = gdn.gdn_chunk_fwd_plan_info(B, T, H, workspace=ws, **opts)
    say(f"  plan {info}")
    assert info["error"] == 0 and info["P_exact"] == 2
    assert info["n_exact"] + info["n_window"] == B * H and info["n_window"] > 0 and info["n_exact"] > 0
    # exact head: segment 0 and one pass-3 run; window head: 2 runs
    assert info["n_jobs"] == 2 * B * H and info["handed_out"] >= info["n_jobs"]
    oref, href = oracle.fwd(x.q, x.k, x.v, x.g, x.beta, x.h0)
    _check(to_np(o), to_np(ht), oref, href, TOL_BF16, label="4200 heads x 2 segments")


@pytest.mark.parametrize("opts", [dict(), dict(split_mode=2, n_segments=5)])
def test_fp32_split(gdn, opts):
    """fp32 inputs through the split forward (the persistent kernel's fp32
    instantiation): exact and window heads, a ragged tail and an entering state,
    automatic plan and a forced split into 5 segments."""
    import torch
    say(f"case fp32 split {opts}, B=1 T=64*40+17 H=4")
    B, T, H = 1, 64 * 40 + 17, 4
    x = inputs.generate(B=B, T=T, H=H, dtype="f32", gate="mixed", strong_frac=0.5, h0_std=0.05, seed=53)
    t = to_gpu(x)
    ws = torch.empty(gdn.gdn_chunk_fwd_workspace_size(B, T, H, **opts), dtype=torch.uint8, device="cuda")
    o, ht = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["h0"], workspace=ws, scale=0.5,
                              **opts)
    info = gdn.gdn_chunk_fwd_plan_info(B, T, H, workspace=ws, **opts)
    say(f"  plan {info}")
    assert info["error"] == 0 and info["n_exact"] + info["n_window"] == B * H
    assert info["P_exact"] > 1 or info["P_window"] > 1
    oref, href = oracle.fwd(x.q, x.k, x.v, x.g, x.beta, x.h0, scale=0.5)
    _check(to_np(o), to_np(ht), oref, href, TOL_F32, label=f"fp32 split {opts}")


def _varlen_case(gdn, lens, H, dtype, seed, tol, **gen):
    import torch
    T = int(sum(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    S = len(lens)
    x = inputs.generate(B=1, T=T, H=H, dtype=dtype, seed=seed, **gen)
    h0 = inputs.generate(B=S, T=1, H=H, dtype=dtype, h0_std=0.05, seed=seed + 1).h0
    t = to_gpu(x)
    sq = lambda a: a[0]   # [1, T, ...] -> [T, ...]
    o, ht = gdn.gdn_chunk_fwd_varlen(sq(t["q"]), sq(t["k"]), sq(t["v"]), sq(t["g"]), sq(t["beta"]),
                                     torch.from_numpy(cu).cuda(), h0=torch.from_numpy(h0).cuda())
    torch.cuda.synchronize()
    o, ht = to_np(o), to_np(ht)
    for s_ in range(S):
        a, b = int(cu[s_]), int(cu[s_ + 1])
        if a == b:
            assert np.array_equal(ht[s_], h0[s_].astype(np.float64)), "empty sequence keeps its state"
            continue
        sl = lambda arr: arr[:, a:b]
        oref, href = oracle.fwd(sl(x.q), sl(x.k), sl(x.v), sl(x.g), sl(x.beta), h0[s_:s_ + 1])
        _check(o[None, a:b], ht[s_:s_ + 1], oref, href, tol, label=f"sequence {s_} ({b - a} tokens)")


def test_varlen_packed_bf16(gdn):
    """Packed sequences of ragged lengths (one empty) against the oracle run on
    each sequence alone."""
    say("case varlen bf16 lengths 1, 63, 64, 65, 200, 0, 130")
    _varlen_case(gdn, [1, 63, 64, 65, 200, 0, 130], H=2, dtype="bf16", seed=41, tol=TOL_BF16)


def test_varlen_packed_fp32(gdn):
    say("case varlen fp32 lengths 5, 64, 70")
    _varlen_case(gdn, [5, 64, 70], H=2, dtype="f32", seed=43, tol=TOL_F32)


def _varlen_segments(lens, H, cus):
    """Segments per sequence of the packed forward's cut: target chunks per segment
    = max(2 windows, ceil(total chunks * H / CUs)), at most 16 segments."""
    nch = -(-int(sum(lens)) // 64)
    target = max(16, -(-nch * H // cus))
    pmax = min(16, -(-nch // target))
    if pmax <= 1:
        return [1] * len(lens)
    return [min(pmax, max(1, -(-(-(-n // 64)) // target))) for n in lens]


def test_varlen_split_long_prompt(gdn):
    """A long prompt among short and empty ones is cut into segments, each later
    segment warming up over its own decay window or running from the sequence
    start; every sequence is checked against the oracle run on it alone."""
    import torch
    lens = [4096, 100, 300, 0, 2500]
    segs = _varlen_segments(lens, 2, torch.cuda.get_device_properties(0).multi_processor_count)
    say(f"case varlen split bf16 lengths {lens}, H=2, segments {segs}")
    assert max(segs) > 1
    _varlen_case(gdn, lens, H=2, dtype="bf16", seed=61, tol=TOL_BF16)


def test_varlen_split_mixed_decay(gdn):
    """Strongly decaying heads take the window; near-1 heads find no window whose
    decay reaches eps and run their later segments from the sequence start."""
    import torch
    lens = [3000, 64, 5000, 129]
    segs = _varlen_segments(lens, 4, torch.cuda.get_device_properties(0).multi_processor_count)
    say(f"case varlen split bf16 lengths {lens}, H=4, mixed gates, segments {segs}")
    assert max(segs) > 1
    _varlen_case(gdn, lens, H=4, dtype="bf16", seed=63, tol=TOL_BF16, gate="mixed", strong_frac=0.5)


def test_varlen_split_fp32(gdn):
    say("case varlen split fp32 lengths 2100, 70, 1500")
    _varlen_case(gdn, [2100, 70, 1500], H=2, dtype="f32", seed=65, tol=TOL_F32, gate="uniform",
                 gate_lo=-0.3, gate_hi=-0.05)


def test_varlen_equals_fixed_length(gdn):
    """Equal-length packed sequences give bit-identical results to the unsplit
    fixed-length forward on [B, T, H, d] (the same kernel with shifted pointers)."""
    import torch
    say("case varlen vs fixed length")
    B, T, H = 3, 64 * 5 + 7, 2
    x = inputs.generate(B=B, T=T, H=H, h0_std=0.05, seed=45)
    t = to_gpu(x)
    o1, h1 = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["h0"], split_mode=1)
    fl = lambda a: a.reshape((B * T,) + tuple(a.shape[2:])).contiguous()
    cu = torch.arange(0, B * T + 1, T, dtype=torch.int32, device="cuda")
    o2, h2 = gdn.gdn_chunk_fwd_varlen(fl(t["q"]), fl(t["k"]), fl(t["v"]), fl(t["g"]), fl(t["beta"]), cu,
                                      h0=t["h0"])
    torch.cuda.synchronize()
    assert torch.equal(o1.reshape(o2.shape), o2)
    assert torch.equal(h1, h2)


@pytest.mark.slow
def test_bf16_t32768_h32_all_heads(gdn):
    """The throughput workload (B=1, T=32768, H=32) at full size, in the launch
    configuration the benchmark times (automatic plan, workspace reused), against
    the oracle on every head; the device plan's window levels match the oracle's
    gate scan."""
    say("case bf16_t32768_h32 (full size, every head)")
    import torch
    x = inputs.workload("bf16_t32768_h32")
    B, T, H = 1, 32768, 32
    lev = _window_levels(x.g)
    say(f"  oracle levels {lev.tolist()}")
    t = to_gpu(x)
    ws = torch.empty(gdn.gdn_chunk_fwd_workspace_size(B, T, H), dtype=torch.uint8, device="cuda")
    o, ht = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], workspace=ws)
    info = gdn.gdn_chunk_fwd_plan_info(B, T, H, workspace=ws)
    say(f"  plan {info}")
    _check_plan_levels(info, lev, B * H)
    o, ht = to_np(o), to_np(ht)
    del t
    oref, href = oracle.fwd(x.q, x.k, x.v, x.g, x.beta, x.h0)
    _check(o, ht, oref, href, TOL_BF16, label="t32768 h32, all heads")


@pytest.mark.slow
def test_bf16_t262144_h16_all_heads(gdn):
    """Long context (B=1, T=262144, H=16; 11 strongly decaying heads and 5 near-1
    heads) at full size against the oracle on every head."""
    say("case bf16_t262144_h16_mixed (full size, every head)")
    import torch
    x = inputs.workload("bf16_t262144_h16_mixed")
    B, T, H = 1, 262144, 16
    t = to_gpu(x)
    ws = torch.empty(gdn.gdn_chunk_fwd_workspace_size(B, T, H), dtype=torch.uint8, device="cuda")
    o, ht = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], workspace=ws)
    info = gdn.gdn_chunk_fwd_plan_info(B, T, H, workspace=ws)
    say(f"  plan {info}")
    assert info["error"] == 0 and info["n_exact"] + info["n_window"] == B * H
    o, ht = to_np(o), to_np(ht)
    del t
    oref, href = oracle.fwd(x.q, x.k, x.v, x.g, x.beta, x.h0)
    strong = np.flatnonzero(x.meta["strong_heads"])
    weak = np.flatnonzero(~x.meta["strong_heads"])
    for name, hs in (("strongly decaying", strong), ("near-1", weak)):
        _check(o, ht, oref, href, TOL_BF16, heads=[int(h) for h in hs], H=H, label=f"t262144 h16, {name} heads")
    _check(o, ht, oref, href, TOL_BF16, label="t262144 h16, all heads")


@pytest.mark.slow
def test_bf16_b4_t8192_h32_forward_all_heads(gdn):
    """The training shape's forward (B=4, T=8192, H=32, h0 given) at full size
    against the oracle on every head of every batch entry: o and ht."""
    say("case bf16_b4_t8192_h32_train forward (full size, every head)")
    import torch
    x = inputs.workload("bf16_b4_t8192_h32_train")
    B, T, H = 4, 8192, 32
    t = to_gpu(x)
    ws = torch.empty(max(1, gdn.gdn_chunk_fwd_workspace_size(B, T, H)), dtype=torch.uint8, device="cuda")
    o, ht = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["h0"], workspace=ws)
    info = gdn.gdn_chunk_fwd_plan_info(B, T, H, workspace=ws)
    say(f"  plan {info}")
    assert info["error"] == 0
    # 128 heads on 256 compute units: the cost model splits them (every head is
    # a window head here), so the launch has more jobs than heads
    assert info["n_jobs"] > B * H and info["n_exact"] + info["n_window"] == B * H
    o, ht = to_np(o), to_np(ht)
    del t
    oref, href = oracle.fwd(x.q, x.k, x.v, x.g, x.beta, x.h0)
    for b in range(B):
        _check(o[b:b + 1], ht[b:b + 1], oref[b:b + 1], href[b:b + 1], TOL_BF16, label=f"b4 t8192 h32, batch {b}")
    _check(o, ht, oref, href, TOL_BF16, label="b4 t8192 h32, all heads")
