"""Run-to-run determinism of the shipped schedules.

The split forward hands segment states between workgroups through a work queue
whose job-to-workgroup assignment differs from call to call, the backward runs
its state store and state-gradient sweep on two streams (or, with few heads,
through the split forward, segment maps and a chain), and the KDA forward splits
each head into segments with a chain.  None of these orders may change a single
bit of the results: every case calls the same entry point three times on the same
device inputs and requires bitwise-equal outputs, and checks the first call
against the oracle once (so equal results are also right ones).
"""
import numpy as np
import pytest

import oracle
from gated_deltanet_chunked_prefill_amd import inputs
from helpers import TOL_BF16, rel_err, say, to_gpu, to_np

pytestmark = pytest.mark.gpu

CALLS = 3


@pytest.fixture(scope="module")
def gdn():
    import torch
    assert torch.cuda.is_available()
    import gated_deltanet_chunked_prefill_amd as m
    return m


def _same(outs, label):
    for i in range(1, len(outs)):
        for name in outs[0]:
            a, b = outs[0][name], outs[i][name]
            if a is None:
                assert b is None
                continue
            diff = int(np.count_nonzero(a.view(np.uint8) != b.view(np.uint8)))
            assert diff == 0, f"{label}: {name} differs between call 1 and call {i + 1} ({diff} bytes)"
    say(f"  {label}: {len(outs)} calls bitwise equal")


def _fwd_calls(gdn, x, **opts):
    import torch
    t = to_gpu(x)
    outs = []
    for _ in range(CALLS):
        o, ht = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["h0"], **opts)
        torch.cuda.synchronize()
        outs.append({"o": to_np(o), "ht": to_np(ht)})
    return outs


@pytest.mark.parametrize("case", ["auto_mixed", "forced_exact", "forced_window"])
def test_forward_split_deterministic(gdn, case):
    say(f"case determinism forward {case}")
    if case == "auto_mixed":
        # exact and window heads in one automatic plan, ragged tail, entering state
        x = inputs.generate(B=1, T=64 * 200 + 23, H=8, gate="mixed", h0_std=0.02, seed=900)
        outs = _fwd_calls(gdn, x)
    elif case == "forced_exact":
        x = inputs.generate(B=2, T=64 * 96 + 5, H=3, gate="mixed", strong_frac=0.0, seed=901)
        outs = _fwd_calls(gdn, x, split_mode=2, n_segments=7, use_window=0)
    else:
        x = inputs.generate(B=1, T=64 * 128, H=4, seed=902)
        outs = _fwd_calls(gdn, x, split_mode=2, n_segments=5, use_window=1)
    _same(outs, case)
    o_ref, ht_ref = oracle.fwd(x.q, x.k, x.v, x.g, x.beta, x.h0)
    e = max(rel_err(outs[0]["o"], o_ref), rel_err(outs[0]["ht"], ht_ref))
    say(f"  vs oracle {e:.2e}")
    assert e <= TOL_BF16


@pytest.mark.parametrize("path", ["split", "unsplit"])
def test_backward_deterministic(gdn, path):
    import torch
    say(f"case determinism backward {path}")
    x = inputs.generate(B=1, T=64 * 48 + 9, H=2, h0_std=0.05, dout=True, seed=910)
    dht = np.random.default_rng(911).standard_normal((1, 2, 128, 128)).astype(np.float32) * 0.05
    t = to_gpu(x)
    dht_t = torch.from_numpy(dht).cuda()
    B, T, H = x.beta.shape
    ws = None
    if path == "unsplit":
        # a workspace of the unsplit backward's size selects the unsplit path
        N = -(-T // 64)
        ws = torch.empty(B * H * (2 * N + 1) * 128 * 128 * 2 + 4096, dtype=torch.uint8, device="cuda")
    names = ("dq", "dk", "dv", "dg", "dbeta", "dh0")
    outs = []
    for _ in range(CALLS):
        out = gdn.gdn_chunk_bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["dout"], h0=t["h0"],
                                dht=dht_t, scale=0.5, workspace=ws)
        torch.cuda.synchronize()
        outs.append({n: to_np(out[n]) for n in names})
    _same(outs, path)
    ref = oracle.bwd(x.q, x.k, x.v, x.g, x.beta, x.dout, x.h0, dht, scale=0.5)
    e = max(rel_err(outs[0][n], ref[n]) for n in names)
    say(f"  vs oracle {e:.2e}")
    assert e <= TOL_BF16


def test_kda_split_deterministic(gdn):
    import torch
    say("case determinism KDA split")
    x = inputs.generate_kda(B=1, T=64 * 64 + 31, H=2, h0_std=0.02, seed=920)
    t = to_gpu(x)
    outs = []
    for _ in range(CALLS):
        o, ht = gdn.gdn_kda_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["h0"], n_segments=5)
        torch.cuda.synchronize()
        outs.append({"o": to_np(o), "ht": to_np(ht)})
    _same(outs, "KDA 5 segments")
    o_ref, ht_ref = oracle.kda_fwd(x.q, x.k, x.v, x.g, x.beta, x.h0)
    e = max(rel_err(outs[0]["o"], o_ref), rel_err(outs[0]["ht"], ht_ref))
    say(f"  vs oracle {e:.2e}")
    assert e <= TOL_BF16
