"""gdn_chunk_fwd_noalloc (the forward without a workspace, for callers that
cannot allocate) against gdn_chunk_fwd with its workspace, through the C ABI:
two calls in a row, the second on a smaller input (the fixed scratch keeps the
first call's contents), within the bf16 parity bound; a forced split gives
bit-identical results (same plan, same kernels); a forced split too large for
the scratch is refused before any launch."""
import numpy as np
import pytest

from gated_deltanet_chunked_prefill_amd import inputs
from helpers import TOL_BF16, rel_err, say, to_gpu, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdn():
    import torch
    assert torch.cuda.is_available()
    import gated_deltanet_chunked_prefill_amd as m
    return m


def _both(gdn, x, **opts):
    import torch
    t = to_gpu(x)
    B, T, H, dk, dv = x.shape
    o_ref, ht_ref = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["h0"], **opts)
    o = torch.full_like(o_ref, float("nan"))
    ht = torch.full_like(ht_ref, float("nan"))
    gdn.gdn_chunk_fwd_noalloc(t["q"], t["k"], t["v"], t["g"], t["beta"], t["h0"], out=o, out_ht=ht, **opts)
    torch.cuda.synchronize()
    return o, ht, o_ref, ht_ref


def test_noalloc_matches_workspace_forward(gdn):
    import torch
    cases = [
        # forced split, exact and window heads, ragged tail, entering state
        ("forced 5 segments, B=1 T=64*40+17 H=4",
         inputs.generate(B=1, T=64 * 40 + 17, H=4, gate="mixed", strong_frac=0.5, h0_std=0.05, seed=81),
         dict(split_mode=2, n_segments=5)),
        # a smaller input next: the scratch holds the previous call's data
        ("automatic plan, B=1 T=64*12+3 H=2",
         inputs.generate(B=1, T=64 * 12 + 3, H=2, h0_std=0.02, seed=82), dict()),
    ]
    for label, x, opts in cases:
        say(f"case noalloc {label}")
        o, ht, o_ref, ht_ref = _both(gdn, x, **opts)
        eo = rel_err(to_np(o), to_np(o_ref))
        eh = rel_err(to_np(ht), to_np(ht_ref))
        say(f"  o err {eo:.3e}  ht err {eh:.3e}")
        assert eo <= TOL_BF16 and eh <= TOL_BF16
        if opts.get("split_mode") == 2:
            assert torch.equal(o, o_ref) and torch.equal(ht, ht_ref)


def test_noalloc_benchmark_shape_fewer_slots(gdn):
    """At B=1, T=32768, H=32 the workspace forward's segment slots need more
    than the fixed scratch: the no-allocation forward plans with fewer slots and
    still agrees within the bf16 bound."""
    say("case noalloc B=1 T=32768 H=32 (segment slots capped by the scratch)")
    from gated_deltanet_chunked_prefill_amd import _lib
    B, T, H = 1, 32768, 32
    assert gdn.gdn_chunk_fwd_workspace_size(B, T, H) > _lib.NOALLOC_SCRATCH_BYTES
    x = inputs.workload("bf16_t32768_h32")
    o, ht, o_ref, ht_ref = _both(gdn, x)
    eo = rel_err(to_np(o), to_np(o_ref))
    eh = rel_err(to_np(ht), to_np(ht_ref))
    say(f"  o err {eo:.3e}  ht err {eh:.3e}")
    assert eo <= TOL_BF16 and eh <= TOL_BF16


def test_noalloc_forced_split_beyond_scratch(gdn):
    import torch
    from gated_deltanet_chunked_prefill_amd import _lib
    say("case noalloc forced split beyond the scratch")
    B, T, H = 1, 64 * 128, 64
    x = inputs.generate(B=B, T=T, H=H, seed=83)
    t = to_gpu(x)
    o = torch.empty_like(t["v"])
    with pytest.raises(_lib.GDNError) as ei:
        gdn.gdn_chunk_fwd_noalloc(t["q"], t["k"], t["v"], t["g"], t["beta"], out=o, split_mode=2, n_segments=64)
    assert ei.value.status == _lib.GDN_ERR_WORKSPACE
    assert "scratch" in str(ei.value)
