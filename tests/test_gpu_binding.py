"""The Python binding refuses tensors the library would index out of bounds
(wrong shape, wrong device, wrong dtype) with ValueError or TypeError before any
library call: no kernel is launched.  Launches are counted through the
library's profiling hook (gdn_profile_events)."""
import ctypes

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


class _Launches:
    """Counts the library's kernel launches between enter and exit."""

    def __enter__(self):
        from gated_deltanet_chunked_prefill_amd import _lib
        self.lib = _lib.load()
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.cap = 8
        self.ev = (ctypes.c_void_p * (2 * self.cap))()
        for i in range(2 * self.cap):
            e = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
            self.ev[i] = e
        self.labels = (ctypes.c_int * self.cap)()
        self.lib.gdn_profile_events(ctypes.cast(self.ev, ctypes.c_void_p),
                                    ctypes.cast(self.labels, ctypes.c_void_p), self.cap)
        return self

    def __exit__(self, *exc):
        import torch
        self.count = self.lib.gdn_profile_events(None, None, 0)
        torch.cuda.synchronize()
        for i in range(2 * self.cap):
            self.hip.hipEventDestroy(self.ev[i])
        return False


def _inputs(B=1, T=100, H=2):
    x = inputs.generate(B=B, T=T, H=H, h0_std=0.02, dout=True, seed=71)
    return x, to_gpu(x)


def test_forward_rejects_mismatched_tensors(gdn):
    import torch
    say("case binding: forward shape checks")
    x, t = _inputs()
    B, T, H = 1, 100, 2
    bad = {
        "k": dict(k=t["k"][:, :-1].contiguous()),
        "v": dict(v=torch.zeros(B, T + 1, H, 128, dtype=torch.bfloat16, device="cuda")),
        "g": dict(g=t["g"][:, :-1].contiguous()),
        "beta": dict(beta=torch.zeros(B, T, H + 1, device="cuda")),
        "h0": dict(h0=torch.zeros(B, H + 1, 128, 128, device="cuda")),
        "h0 on host": dict(h0=torch.zeros(B, H, 128, 128)),
        "out": dict(out=torch.empty(B, T - 1, H, 128, dtype=torch.bfloat16, device="cuda")),
        "out_ht": dict(out_ht=torch.empty(B, H, 128, 64, device="cuda")),
    }
    for name, over in bad.items():
        args = dict(q=t["q"], k=t["k"], v=t["v"], g=t["g"], beta=t["beta"], h0=t["h0"])
        kw = {}
        for key, val in over.items():
            (args if key in args else kw)[key] = val
        with _Launches() as n, pytest.raises((ValueError, TypeError)):
            gdn.gdn_chunk_fwd(**args, **kw)
        assert n.count == 0, name
    # the good call launches and matches the oracle
    with _Launches() as n:
        o, ht = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["h0"])
    assert n.count >= 1
    oref, href = oracle.fwd(x.q, x.k, x.v, x.g, x.beta, x.h0)
    assert rel_err(to_np(o), oref) <= TOL_BF16 and rel_err(to_np(ht), href) <= TOL_BF16


def test_backward_rejects_mismatched_tensors(gdn):
    import torch
    say("case binding: backward shape checks")
    x, t = _inputs()
    base = dict(q=t["q"], k=t["k"], v=t["v"], g=t["g"], beta=t["beta"], dout=t["dout"], h0=t["h0"])
    bad = {
        "dout": dict(dout=t["dout"][:, 1:].contiguous()),
        "dht": dict(dht=torch.zeros(1, 2, 128, 127, device="cuda")),
        "k": dict(k=torch.zeros(1, 100, 3, 128, dtype=torch.bfloat16, device="cuda")),
        "workspace dtype": dict(workspace=torch.zeros(1 << 20, dtype=torch.float32, device="cuda")),
    }
    for name, over in bad.items():
        args = dict(base)
        args.update(over)
        with _Launches() as n, pytest.raises((ValueError, TypeError)):
            gdn.gdn_chunk_bwd(**args)
        assert n.count == 0, name


def test_varlen_rejects_mismatched_tensors(gdn):
    import torch
    say("case binding: packed-sequence shape checks")
    x, t = _inputs(T=130)
    sq = lambda a: a[0]
    cu = torch.tensor([0, 60, 130], dtype=torch.int32, device="cuda")
    base = dict(q=sq(t["q"]), k=sq(t["k"]), v=sq(t["v"]), g=sq(t["g"]), beta=sq(t["beta"]), cu_seqlens=cu)
    bad = {
        "g": dict(g=sq(t["g"])[:-1].contiguous()),
        "cu on host": dict(cu_seqlens=cu.cpu()),
        "cu 2-D": dict(cu_seqlens=cu.reshape(1, 3)),
        "h0": dict(h0=torch.zeros(3, 2, 128, 128, device="cuda")),
        "q batch of 2": dict(q=torch.zeros(2, 130, 2, 128, dtype=torch.bfloat16, device="cuda")),
    }
    for name, over in bad.items():
        args = dict(base)
        args.update(over)
        with _Launches() as n, pytest.raises((ValueError, TypeError)):
            gdn.gdn_chunk_fwd_varlen(**args)
        assert n.count == 0, name
    with _Launches() as n, pytest.raises(ValueError):
        gdn.gdn_chunk_bwd_varlen(**base, dout=sq(t["dout"])[:, :1].contiguous())
    assert n.count == 0


def test_bwd_varlen_decreasing_cu_seqlens(gdn):
    """A decreasing cu_seqlens in the packed backward: the sequences are taken as
    [max(cu[0..s]), max(cu[0..s+1])) (here [0, 200), an empty one, and [200, 300)),
    every workspace slot stays in bounds, and the gradients of those sequences
    match the BPTT oracle run on each alone."""
    import torch
    say("case bwd varlen, cu_seqlens 0, 200, 100, 300")
    H, T = 2, 300
    x = inputs.generate(B=1, T=T, H=H, dout=True, seed=73)
    t = to_gpu(x)
    sq = lambda a: a[0]
    cu = torch.tensor([0, 200, 100, 300], dtype=torch.int32, device="cuda")
    out = gdn.gdn_chunk_bwd_varlen(sq(t["q"]), sq(t["k"]), sq(t["v"]), sq(t["g"]), sq(t["beta"]),
                                   sq(t["dout"]), cu)
    torch.cuda.synchronize()
    got = {n: to_np(out[n]) for n in ("dq", "dk", "dv", "dg", "dbeta", "dh0")}
    for s_, (a, b) in enumerate([(0, 200), (200, 200), (200, 300)]):
        if a == b:
            assert np.max(np.abs(got["dh0"][s_])) == 0.0
            continue
        sl = lambda arr: arr[:, a:b]
        ref = oracle.bwd(sl(x.q), sl(x.k), sl(x.v), sl(x.g), sl(x.beta), sl(x.dout))
        for n in ("dq", "dk", "dv", "dg", "dbeta"):
            e = rel_err(got[n][None, a:b], ref[n])
            assert e <= TOL_BF16, (s_, n, e)
        assert rel_err(got["dh0"][s_:s_ + 1], ref["dh0"]) <= TOL_BF16


def test_stream_probe_copies_v(gdn):
    """The memory-pattern probe writes each chunk's V tile to o, except the last
    chunk of every segment (a copy, bit-exact), and reads k and q in full."""
    import torch
    say("case stream probe T=64*12 H=3 segments=4")
    T, H, seg = 64 * 12, 3, 4
    gen = torch.Generator().manual_seed(5)
    k, q, v = (torch.randn((T, H, 128), generator=gen).to(torch.bfloat16).cuda() for _ in range(3))
    o = torch.zeros_like(v)
    gdn.gdn_stream_probe(k, q, v, o, seg)
    torch.cuda.synchronize()
    cpw = T // 64 // seg
    written = torch.ones(T, dtype=torch.bool)
    for p in range(seg):
        last = (p + 1) * cpw - 1
        written[last * 64:(last + 1) * 64] = False
    assert torch.equal(o.cpu()[written], v.cpu()[written])
    assert torch.count_nonzero(o.cpu()[~written]) == 0


def test_profile_kinds_mask_brackets_only_the_selected_launches(gdn):
    """With the mask set to the persistent forward launch, a split forward call
    records exactly that launch (its two preparation launches go unbracketed)."""
    import torch
    say("case profiling hook restricted to the persistent forward launch")
    x = inputs.generate(B=1, T=64 * 40, H=2, seed=72)
    t = to_gpu(x)
    kind_queue = 4   # GDN_LAUNCH_FWD_QUEUE
    with _Launches() as all_kinds:
        gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], None, split_mode=2, n_segments=4)
    assert all_kinds.count >= 2
    prev = all_kinds.lib.gdn_profile_kinds(1 << kind_queue)
    try:
        with _Launches() as only:
            o, ht = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], None, split_mode=2, n_segments=4)
    finally:
        all_kinds.lib.gdn_profile_kinds(prev)
    torch.cuda.synchronize()
    assert only.count == 1 and only.labels[0] == kind_queue, (only.count, list(only.labels)[:only.count])
    oref, href = oracle.fwd(x.q, x.k, x.v, x.g, x.beta, None)
    assert rel_err(to_np(o), oref) <= TOL_BF16 and rel_err(to_np(ht), href) <= TOL_BF16
