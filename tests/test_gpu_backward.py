"""GPU parity of the chunked backward against the fp64 BPTT oracle.

Each case runs gdn_chunk_bwd through the C ABI on seeded inputs and compares
every gradient (dq, dk, dv, dg, dbeta, dh0) with the oracle's on the same
values: max|X - X_ref| <= 2e-2 * max|X_ref| per tensor (bf16 I/O).
"""
import numpy as np
import pytest

import oracle
from gated_deltanet_chunked_prefill_amd import inputs
from helpers import TOL_BF16, rel_err, say, to_gpu, to_np

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dh0")


@pytest.fixture(scope="module")
def gdn():
    import torch
    assert torch.cuda.is_available()
    import gated_deltanet_chunked_prefill_amd as m
    return m


def _bwd(gdn, x, dht=None, scale=1.0, heads=None):
    import torch
    t = to_gpu(x)
    dht_t = None if dht is None else torch.from_numpy(dht).float().cuda()
    out = gdn.gdn_chunk_bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["dout"], h0=t["h0"],
                            dht=dht_t, scale=scale)
    torch.cuda.synchronize()
    got = {n: to_np(out[n]) for n in NAMES}
    ref = oracle.bwd(x.q, x.k, x.v, x.g, x.beta, x.dout, x.h0, dht, scale=scale, heads=heads)
    return got, ref


def _check(got, ref, label, heads=None, H=None):
    errs = {}
    for n in NAMES:
        if heads is None:
            errs[n] = rel_err(got[n], ref[n])
        elif n == "dh0":
            errs[n] = max(rel_err(got[n][bh // H, bh % H], ref[n][bh // H, bh % H]) for bh in heads)
        else:
            errs[n] = max(rel_err(got[n][bh // H, :, bh % H], ref[n][bh // H, :, bh % H])
                          for bh in heads)
    say(f"  {label}: " + "  ".join(f"{n} {e:.2e}" for n, e in errs.items()))
    bad = {n: e for n, e in errs.items() if not e <= TOL_BF16}
    assert not bad, bad


@pytest.mark.parametrize("T", [1, 63, 64, 65, 200])
def test_bwd_ragged_lengths(gdn, T):
    say(f"case bwd bf16 T={T}")
    x = inputs.generate(B=2, T=T, H=2, h0_std=0.02, dout=True, seed=300 + T)
    got, ref = _bwd(gdn, x)
    _check(got, ref, f"T={T}")


def test_bwd_final_state_gradient_and_scale(gdn):
    say("case bwd with dht and scale 0.5")
    x = inputs.generate(B=1, T=256, H=3, h0_std=0.05, dout=True, seed=7)
    dht = np.random.default_rng(8).standard_normal((1, 3, 128, 128)).astype(np.float32) * 0.1
    got, ref = _bwd(gdn, x, dht=dht, scale=0.5)
    _check(got, ref, "dht, scale 0.5")


def test_bwd_no_initial_state(gdn):
    say("case bwd without h0")
    x = inputs.generate(B=1, T=192, H=2, h0_std=None, dout=True, seed=9)
    got, ref = _bwd(gdn, x)
    _check(got, ref, "no h0")


def test_bwd_strong_decay(gdn):
    say("case bwd strong decay")
    x = inputs.generate(B=1, T=256, H=2, gate="uniform", gate_lo=-2.0, gate_hi=-0.5, h0_std=0.02,
                        dout=True, seed=10)
    got, ref = _bwd(gdn, x)
    _check(got, ref, "strong decay")


@pytest.mark.parametrize("rho", [0.5, 0.9])
def test_bwd_correlated_keys(gdn, rho):
    """Keys sharing a direction (pairwise cosine about rho) through every
    gradient: the inverse blocks of the state store, the sweep and the local
    gradients stay accurate."""
    say(f"case bwd correlated keys rho={rho}")
    x = inputs.generate(B=1, T=64 * 5 + 9, H=2, h0_std=0.02, dout=True, seed=320, key_corr=rho)
    got, ref = _bwd(gdn, x)
    _check(got, ref, f"rho={rho}")


def test_bwd_beta_up_to_two(gdn):
    """beta up to 2 with keys of cosine 0.99 (the inverse blocks' Newton step)."""
    say("case bwd beta up to 2, key cosine 0.99")
    x = inputs.generate(B=1, T=64 * 5 + 9, H=2, h0_std=0.02, dout=True, seed=321, key_corr=0.99, beta_max=2.0)
    got, ref = _bwd(gdn, x)
    _check(got, ref, "beta<=2 rho=0.99")


@pytest.mark.parametrize("case", ["no_decay", "beta0", "beta1"])
def test_bwd_degenerate_gates(gdn, case):
    """alpha = 1 (g = 0), beta = 0 (then dk = dv = 0 exactly: keys and values never
    reach the state) and beta = 1, against the BPTT oracle."""
    say(f"case bwd degenerate gates {case}")
    x = inputs.generate(B=1, T=64 * 3 + 17, H=2, h0_std=0.05, dout=True, seed=33)
    if case == "no_decay":
        x.g[...] = 0.0
    elif case == "beta0":
        x.beta[...] = 0.0
    else:
        x.beta[...] = 1.0
    got, ref = _bwd(gdn, x)
    if case == "beta0":
        assert np.max(np.abs(ref["dk"])) == 0.0 and np.max(np.abs(ref["dv"])) == 0.0
        assert np.max(np.abs(got["dk"])) < 1e-6 and np.max(np.abs(got["dv"])) < 1e-6
    _check(got, ref, case)


def _bwd_both(gdn, x, dht=None, scale=1.0):
    """The same call twice: with the library's workspace query (the few-heads
    path: split state store and split sweep) and with a workspace of the unsplit
    backward's size (the unsplit path)."""
    import torch
    from gated_deltanet_chunked_prefill_amd import _lib
    t = to_gpu(x)
    B, T, H = x.beta.shape
    dht_t = None if dht is None else torch.from_numpy(dht).float().cuda()
    SS = 128 * 128
    N = -(-T // 64)
    small = torch.empty(B * H * (2 * N + 1) * SS * 2 + 4096, dtype=torch.uint8, device="cuda")
    outs = []
    for ws in (None, small):
        out = gdn.gdn_chunk_bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["dout"], h0=t["h0"],
                                dht=dht_t, scale=scale, workspace=ws)
        torch.cuda.synchronize()
        outs.append({n: to_np(out[n]) for n in NAMES})
    ref = oracle.bwd(x.q, x.k, x.v, x.g, x.beta, x.dout, x.h0, dht, scale=scale)
    return outs[0], outs[1], ref


# Few heads (2 B H below the CU count) with enough chunks: the state store runs
# through the split forward and the state-gradient sweep in segments (segment
# P-1 from dht beside the other segments' maps, the chain, then segments 0..P-2).
@pytest.mark.parametrize("B,T,H", [(1, 64 * 40 + 17, 2), (1, 64 * 24, 3), (1, 64 * 97, 1),
                                   (2, 64 * 30 + 5, 3), (3, 64 * 150 + 40, 1)])
def test_bwd_few_heads_split(gdn, B, T, H):
    # (2, 1925, 3): three segments per head over two batch entries; (3, 9640, 1):
    # the largest segment count (17) with a ragged tail
    say(f"case bwd few heads split B={B} T={T} H={H}")
    x = inputs.generate(B=B, T=T, H=H, h0_std=0.05, dout=True, seed=400 + H + 10 * (B - 1))
    dht = np.random.default_rng(401).standard_normal((B, H, 128, 128)).astype(np.float32) * 0.05
    split, unsplit, ref = _bwd_both(gdn, x, dht=dht, scale=0.75)
    _check(split, ref, f"split B={B} T={T} H={H}")
    _check(unsplit, ref, f"unsplit B={B} T={T} H={H}")
    d = max(rel_err(split[n], unsplit[n]) for n in NAMES)
    say(f"  split vs unsplit: {d:.2e}")
    assert d <= 1e-2, d


def test_bwd_few_heads_split_correlated_keys(gdn):
    """Split path with keys of cosine 0.9, beta up to 2, no h0, window and
    exact heads mixed in the state store (one slowly decaying head)."""
    say("case bwd few heads split, correlated keys, beta<=2")
    x = inputs.generate(B=2, T=64 * 33 + 5, H=2, h0_std=None, dout=True, seed=410, key_corr=0.9, beta_max=2.0)
    split, _, ref = _bwd_both(gdn, x)
    _check(split, ref, "split rho=0.9 beta<=2")


@pytest.mark.slow
def test_bwd_train_workload_all_heads(gdn):
    """The training shape (B=4, T=8192, H=32, h0 given, dO ~ N(0,1)) at full size:
    every gradient of every head of every batch entry against the BPTT oracle."""
    say("case bf16_b4_t8192_h32_train backward (full size, every head)")
    x = inputs.workload("bf16_b4_t8192_h32_train")
    got, ref = _bwd(gdn, x)
    B, H = 4, 32
    for b in range(B):
        heads = list(range(b * H, (b + 1) * H))
        _check(got, ref, f"b4 t8192 h32, batch {b}", heads=heads, H=H)
    _check(got, ref, "b4 t8192 h32, all heads")


def test_bwd_varlen_packed(gdn):
    """Packed sequences of ragged lengths (one empty): every gradient against the
    BPTT oracle run on each sequence alone."""
    import torch
    say("case bwd varlen lengths 1, 63, 64, 65, 130, 0, 200")
    lens = [1, 63, 64, 65, 130, 0, 200]
    H, S, T = 2, len(lens), sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    x = inputs.generate(B=1, T=T, H=H, dout=True, seed=51)
    h0 = inputs.generate(B=S, T=1, H=H, h0_std=0.05, seed=52).h0
    dht = inputs.generate(B=S, T=1, H=H, h0_std=0.1, seed=53).h0
    t = to_gpu(x)
    sq = lambda a: a[0]
    out = gdn.gdn_chunk_bwd_varlen(sq(t["q"]), sq(t["k"]), sq(t["v"]), sq(t["g"]), sq(t["beta"]),
                                   sq(t["dout"]), torch.from_numpy(cu).cuda(), h0=torch.from_numpy(h0).cuda(),
                                   dht=torch.from_numpy(dht).cuda())
    torch.cuda.synchronize()
    got = {n: to_np(out[n]) for n in NAMES}
    for s_ in range(S):
        a, b = int(cu[s_]), int(cu[s_ + 1])
        if a == b:
            assert np.array_equal(got["dh0"][s_], dht[s_].astype(np.float64)), "empty sequence passes dht on"
            continue
        sl = lambda arr: arr[:, a:b]
        ref = oracle.bwd(sl(x.q), sl(x.k), sl(x.v), sl(x.g), sl(x.beta), sl(x.dout), h0[s_:s_ + 1],
                         dht[s_:s_ + 1])
        g1 = {n: (got[n][None, a:b] if n != "dh0" else got[n][s_:s_ + 1]) for n in NAMES}
        _check(g1, ref, f"sequence {s_} ({b - a} tokens)")


def test_bwd_varlen_equals_fixed_length(gdn):
    """Equal-length packed sequences give bit-identical gradients to the
    fixed-length backward on [B, T, H, d]."""
    import torch
    say("case bwd varlen vs fixed length")
    B, T, H = 3, 64 * 3 + 5, 2
    x = inputs.generate(B=B, T=T, H=H, h0_std=0.05, dout=True, seed=55)
    t = to_gpu(x)
    a = gdn.gdn_chunk_bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["dout"], h0=t["h0"])
    fl = lambda z: z.reshape((B * T,) + tuple(z.shape[2:])).contiguous()
    cu = torch.arange(0, B * T + 1, T, dtype=torch.int32, device="cuda")
    b = gdn.gdn_chunk_bwd_varlen(fl(t["q"]), fl(t["k"]), fl(t["v"]), fl(t["g"]), fl(t["beta"]),
                                 fl(t["dout"]), cu, h0=t["h0"])
    torch.cuda.synchronize()
    for n in ("dq", "dk", "dv", "dg", "dbeta"):
        assert torch.equal(a[n].reshape(b[n].shape), b[n]), n
    assert torch.equal(a["dh0"], b["dh0"])


def test_varlen_many_sequences(gdn):
    """300 short packed sequences (more than one 256-sequence round of the chunk
    prefix; lengths 0 to 70, empty ones included): forward outputs, final states
    and every gradient of each sequence against the oracle."""
    import torch
    say("case varlen 300 sequences, forward and backward")
    rng = np.random.default_rng(61)
    lens = rng.integers(0, 71, size=300)
    lens[[5, 17, 260]] = 0
    H, S, T = 1, len(lens), int(lens.sum())
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    x = inputs.generate(B=1, T=T, H=H, dout=True, seed=62)
    h0 = inputs.generate(B=S, T=1, H=H, h0_std=0.05, seed=63).h0
    t = to_gpu(x)
    sq = lambda a: a[0]
    cu_t, h0_t = torch.from_numpy(cu).cuda(), torch.from_numpy(h0).cuda()
    o, ht = gdn.gdn_chunk_fwd_varlen(sq(t["q"]), sq(t["k"]), sq(t["v"]), sq(t["g"]), sq(t["beta"]), cu_t,
                                     h0=h0_t)
    out = gdn.gdn_chunk_bwd_varlen(sq(t["q"]), sq(t["k"]), sq(t["v"]), sq(t["g"]), sq(t["beta"]),
                                   sq(t["dout"]), cu_t, h0=h0_t)
    torch.cuda.synchronize()
    o, ht = to_np(o), to_np(ht)
    got = {n: to_np(out[n]) for n in NAMES}
    worst = {}
    for s_ in range(S):
        a, b = int(cu[s_]), int(cu[s_ + 1])
        if a == b:
            assert np.array_equal(ht[s_], h0[s_].astype(np.float64))
            assert np.max(np.abs(got["dh0"][s_])) == 0.0
            continue
        sl = lambda arr: arr[:, a:b]
        oref, href = oracle.fwd(sl(x.q), sl(x.k), sl(x.v), sl(x.g), sl(x.beta), h0[s_:s_ + 1])
        ref = oracle.bwd(sl(x.q), sl(x.k), sl(x.v), sl(x.g), sl(x.beta), sl(x.dout), h0[s_:s_ + 1])
        errs = {"o": rel_err(o[None, a:b], oref), "ht": rel_err(ht[s_:s_ + 1], href)}
        for n in NAMES:
            errs[n] = rel_err(got[n][None, a:b] if n != "dh0" else got[n][s_:s_ + 1], ref[n])
        for n, e in errs.items():
            worst[n] = max(worst.get(n, 0.0), e)
    say("  worst over sequences: " + "  ".join(f"{n} {e:.2e}" for n, e in worst.items()))
    assert all(e <= TOL_BF16 for e in worst.values()), worst
