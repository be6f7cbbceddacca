"""Host-side checks of the C ABI (no GPU needed): every symbol include/gdn.h
declares is exported, the planner follows its rule, and invalid arguments are
rejected before anything touches the device."""
import ctypes
import math
import os
import re

import pytest

from gated_deltanet_chunked_prefill_amd import _lib
import gated_deltanet_chunked_prefill_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    txt = open(os.path.join(ROOT, "include", "gdn.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z0-9_]+)\s*\(", txt)))


def test_exports_match_header():
    lib = _lib.load()
    names = _declared()
    assert sorted(_lib.EXPORTS) == names
    for n in names:
        assert hasattr(lib, n), n


def test_default_options():
    o = _lib.Options()
    _lib.load().gdn_default_options(ctypes.byref(o))
    assert (o.split_mode, o.use_window, o.window_chunks, o.window_levels) == (0, 1, 8, 4)
    assert abs(o.log_eps - math.log(2.0 ** -24)) < 1e-5


@pytest.mark.parametrize("B,T,H,cus,expect", [
    (1, 32768, 32, 256, 22),    # 512 chunks: min(32, floor(sqrt(512)) = 22, 256)
    (1, 262144, 16, 256, 32),   # min(32, 64, 2048)
    (1, 4096, 16, 256, 8),      # min(32, 8, 32)
    (4, 8192, 32, 256, 11),     # 128 heads < 256 CUs: min(32, floor(sqrt(128)) = 11, 64)
    (8, 8192, 32, 256, 1),      # 256 heads >= 256 CUs: no split
    (1, 128, 1, 256, 1),        # 2 chunks < 2w
    (1, 1000, 1, 256, 4),       # 16 chunks: min(32, 4, 8)
    (1, 64 * 100, 2, 256, 10),  # min(32, 10, 50)
])
def test_planner_rule(B, T, H, cus, expect):
    assert gdn.gdn_plan_segments(B, T, H, cus) == expect


def test_planner_modes():
    assert gdn.gdn_plan_segments(1, 32768, 32, 256, split_mode=1) == 1
    assert gdn.gdn_plan_segments(1, 32768, 32, 256, split_mode=2, n_segments=5) == 5
    assert gdn.gdn_plan_segments(1, 32768, 32, 256, split_mode=2, n_segments=0) == 0
    assert gdn.gdn_plan_segments(1, 32768, 32, 256, split_mode=3) == 0
    assert gdn.gdn_plan_segments(0, 32768, 32, 256) == 0


def _fwd(lib, q=8, k=8, v=8, g=16, beta=16, o=16, B=1, T=64, H=1, dk=128, dv=128, dt=1,
         opt=None, ws=None, wsz=0):
    P = ctypes.c_void_p
    return lib.gdn_chunk_fwd(P(q) if q else None, P(k) if k else None, P(v) if v else None,
                             P(g) if g else None, P(beta) if beta else None, None,
                             P(o) if o else None, None, B, T, H, dk, dv, dt, 1.0,
                             ctypes.byref(opt) if opt else None, P(ws) if ws else None, wsz, None)


def test_validation_before_launch():
    lib = _lib.load()
    A = 1 << 20   # a fake, aligned address: validation must fail before any use
    assert _fwd(lib, q=0) == _lib.GDN_ERR_INVALID_ARG
    assert "required" in _lib.last_error()
    assert _fwd(lib, q=A, k=A, v=A, g=A, beta=A, o=A, dk=64) == _lib.GDN_ERR_UNSUPPORTED
    assert _fwd(lib, q=A, k=A, v=A, g=A, beta=A, o=A, dt=7) == _lib.GDN_ERR_UNSUPPORTED
    assert _fwd(lib, q=A, k=A, v=A, g=A, beta=A, o=A, T=0) == _lib.GDN_ERR_INVALID_ARG
    assert _fwd(lib, q=A + 2, k=A, v=A, g=A, beta=A, o=A) == _lib.GDN_ERR_INVALID_ARG
    assert "aligned" in _lib.last_error()
    assert _fwd(lib, q=A, k=A, v=A, g=A + 2, beta=A, o=A) == _lib.GDN_ERR_INVALID_ARG
    bad = gdn.options(split_mode=2, n_segments=5)   # T=64 has one chunk
    assert _fwd(lib, q=A, k=A, v=A, g=A, beta=A, o=A, opt=bad) == _lib.GDN_ERR_INVALID_ARG
    bad = gdn.options(window_chunks=0)
    assert _fwd(lib, q=A, k=A, v=A, g=A, beta=A, o=A, opt=bad) == _lib.GDN_ERR_INVALID_ARG
    for lv in (0, 9):
        bad = gdn.options(window_levels=lv)
        assert _fwd(lib, q=A, k=A, v=A, g=A, beta=A, o=A, opt=bad) == _lib.GDN_ERR_INVALID_ARG
        assert "window_levels" in _lib.last_error()


def test_gate_scan_and_bwd_validation():
    lib = _lib.load()
    A = ctypes.c_void_p(1 << 20)
    st = lib.gdn_gate_scan(None, 1, 64, 1, 8, -16.0, A, None, A, 1 << 20, None)
    assert st == _lib.GDN_ERR_INVALID_ARG
    st = lib.gdn_gate_scan(A, 1, 64 * 10, 4, 8, -16.0, A, None, A, 4, None)
    assert st == _lib.GDN_ERR_WORKSPACE
    assert lib.gdn_gate_scan_workspace_size(1, 64 * 10, 4) == 256
    assert lib.gdn_chunk_bwd_workspace_size(1, 64, 1, 64, 128, 1) == ctypes.c_size_t(-1).value


def _bwd(lib, ptrs, B=1, T=64, H=1, dt=1, ws=None, wsz=0):
    P = lambda a: ctypes.c_void_p(a) if a else None
    q, k, v, g, beta, dout, dq, dk, dv, dg, db = ptrs
    return lib.gdn_chunk_bwd(P(q), P(k), P(v), P(g), P(beta), None, P(dout), None, P(dq), P(dk),
                             P(dv), P(dg), P(db), None, B, T, H, 128, 128, dt, 1.0, P(ws), wsz,
                             None)


def test_bwd_validation_before_launch():
    lib = _lib.load()
    A = 1 << 20
    full = [A] * 11
    SS = 128 * 128 * 2   # bf16 states
    # two chunks: 3 entry/final states + 2 state gradients per head
    assert lib.gdn_chunk_bwd_workspace_size(1, 128, 1, 128, 128, 1) == 5 * SS
    assert lib.gdn_chunk_bwd_workspace_size(2, 100, 3, 128, 128, 1) == 6 * 5 * SS
    assert _bwd(lib, [0] + full[1:]) == _lib.GDN_ERR_INVALID_ARG
    assert _bwd(lib, full[:10] + [0]) == _lib.GDN_ERR_INVALID_ARG
    assert _bwd(lib, full, dt=0, ws=A, wsz=1 << 30) == _lib.GDN_ERR_UNSUPPORTED
    assert "bf16" in _lib.last_error()
    assert _bwd(lib, full) == _lib.GDN_ERR_WORKSPACE
    assert _bwd(lib, full, ws=A, wsz=3 * SS - 1) == _lib.GDN_ERR_WORKSPACE
    assert _bwd(lib, full, ws=A + 16, wsz=1 << 30) == _lib.GDN_ERR_INVALID_ARG
    assert _bwd(lib, [A + 2] + full[1:], ws=A, wsz=1 << 30) == _lib.GDN_ERR_INVALID_ARG


def test_varlen_validation_before_launch():
    """gdn_chunk_fwd_varlen rejects bad arguments before anything is launched."""
    lib = _lib.load()
    A = 1 << 20
    P = lambda a: ctypes.c_void_p(a) if a else None

    def call(q=A, cu=A, n_seqs=2, T=128, H=1, dk=128, dt=1):
        return lib.gdn_chunk_fwd_varlen(P(q), P(A), P(A), P(A), P(A), None, P(A), None, P(cu), n_seqs, T, H,
                                        dk, 128, dt, 1.0, None)
    assert call(cu=0) == _lib.GDN_ERR_INVALID_ARG
    assert "cu_seqlens" in _lib.last_error()
    assert call(n_seqs=0) == _lib.GDN_ERR_INVALID_ARG
    assert call(T=0) == _lib.GDN_ERR_INVALID_ARG
    assert call(dk=64) == _lib.GDN_ERR_UNSUPPORTED
    assert call(q=A + 8) == _lib.GDN_ERR_INVALID_ARG
    assert call(cu=A + 2) == _lib.GDN_ERR_INVALID_ARG


def test_stream_probe_validation_before_launch():
    """The memory-pattern probe rejects bad shapes before anything is launched."""
    lib = _lib.load()
    A = 1 << 20
    P = lambda a: ctypes.c_void_p(a) if a else None

    def call(k=A, o=A, T=1024, H=2, seg=4):
        return lib.gdn_stream_probe(P(k), P(A), P(A), P(o), T, H, seg, None)
    assert call(k=0) == _lib.GDN_ERR_INVALID_ARG
    assert call(o=0) == _lib.GDN_ERR_INVALID_ARG
    assert call(T=1000) == _lib.GDN_ERR_INVALID_ARG   # not a multiple of 64 * segments
    assert "multiple" in _lib.last_error()
    assert call(T=64 * 3) == _lib.GDN_ERR_INVALID_ARG
    assert call(seg=0) == _lib.GDN_ERR_INVALID_ARG
    assert call(H=0) == _lib.GDN_ERR_INVALID_ARG
    assert call(k=A + 8) == _lib.GDN_ERR_INVALID_ARG


def test_bwd_varlen_validation_before_launch():
    lib = _lib.load()
    A = 1 << 20
    SS = 128 * 128 * 2
    # 2 sequences, T = 128: cmax = 2 + 2 chunk slots; per head 6 states and 4 gradients
    assert lib.gdn_chunk_bwd_varlen_workspace_size(2, 128, 1, 128, 128, 1) == 256 + 6 * SS + 4 * SS
    assert lib.gdn_chunk_bwd_varlen_workspace_size(0, 128, 1, 128, 128, 1) == ctypes.c_size_t(-1).value
    P = lambda a: ctypes.c_void_p(a) if a else None

    def call(cu=A, dt=1, ws=A, wsz=1 << 30):
        # q, k, v, g, beta, h0 = NULL, dout, dht = NULL, five gradients, dh0 = NULL
        return lib.gdn_chunk_bwd_varlen(*([P(A)] * 5), None, P(A), None, *([P(A)] * 5), None, P(cu), 2, 128,
                                        1, 128, 128, dt, 1.0, P(ws), wsz, None)
    assert call(cu=0) == _lib.GDN_ERR_INVALID_ARG
    assert call(dt=0) == _lib.GDN_ERR_UNSUPPORTED
    assert call(ws=0) == _lib.GDN_ERR_WORKSPACE
    assert call(wsz=1024) == _lib.GDN_ERR_WORKSPACE
    assert call(ws=A + 16) == _lib.GDN_ERR_INVALID_ARG


def test_head_count_bound():
    """Head counts whose 64-row chunk span does not fit the tile loaders' 32-bit
    offsets (64 * H * 128 * element size >= 2^31) are rejected before anything
    touches the device, in every entry point that takes them."""
    lib = _lib.load()
    A = 1 << 20
    P = lambda a: ctypes.c_void_p(a) if a else None
    big = {0: 65536, 1: 131072}   # float32, bfloat16: the first rejected head count
    for dt, H in big.items():
        assert _fwd(lib, q=A, k=A, v=A, g=A, beta=A, o=A, H=H, dt=dt) == _lib.GDN_ERR_INVALID_ARG
        assert "too large" in _lib.last_error()
        # one head fewer passes validation (it then fails at the device query here)
        assert _fwd(lib, q=A, k=A, v=A, g=A, beta=A, o=A, H=H - 1, dt=dt) != _lib.GDN_ERR_INVALID_ARG
        assert lib.gdn_chunk_fwd_workspace_size(1, 64, H, 128, 128, dt, None) == ctypes.c_size_t(-1).value
        st = lib.gdn_chunk_fwd_varlen(*([P(A)] * 5), None, P(A), None, P(A), 1, 64, H, 128, 128, dt, 1.0, None)
        assert st == _lib.GDN_ERR_INVALID_ARG
    assert _bwd(lib, [A] * 11, H=big[1], ws=A, wsz=1 << 40) == _lib.GDN_ERR_INVALID_ARG
    assert lib.gdn_chunk_bwd_varlen_workspace_size(1, 64, big[1], 128, 128, 1) == ctypes.c_size_t(-1).value
    st = lib.gdn_chunk_bwd_varlen(*([P(A)] * 5), None, P(A), None, *([P(A)] * 5), None, P(A), 1, 64,
                                  big[1], 128, 128, 1, 1.0, P(A), 1 << 40, None)
    assert st == _lib.GDN_ERR_INVALID_ARG
    # the gate scan bounds B*H by the int range and B*T*H by 2^40
    st = lib.gdn_gate_scan(P(A), 1 << 16, 64, 1 << 16, 8, -16.0, P(A), None, P(A), 1 << 40, None)
    assert st == _lib.GDN_ERR_INVALID_ARG


def _prefix_model(cu, T):
    """The packed-sequence prefix launch as the kernel computes it: rounds of 256
    bound indices, a running prefix maximum of the clamped cu_seqlens and a
    running chunk count.  Returns (chunk prefix [S+1], bounds [S+1])."""
    S = len(cu) - 1
    clamp = lambda x, lo: lo if x < lo else (T if x > T else x)
    cstart, bnd_out = [0] * (S + 1), [0] * (S + 1)
    carry, lastb = 0, 0
    for s0 in range(0, S + 1, 256):
        part = [clamp(cu[s], 0) if s <= S else 0 for s in range(s0, s0 + 256)]
        for i in range(1, 256):
            part[i] = max(part[i], part[i - 1])
        b = [max(x, lastb) for x in part]
        bnd = [lastb] + b
        for i, s in enumerate(range(s0, s0 + 256)):
            if s <= S:
                bnd_out[s] = b[i]
        nch = [(bnd[i + 1] - bnd[i] + 63) // 64 if 1 <= s <= S else 0
               for i, s in enumerate(range(s0, s0 + 256))]
        run = 0
        for i, s in enumerate(range(s0, s0 + 256)):
            run += nch[i]
            if 1 <= s <= S:
                cstart[s - 1] = carry + run - nch[i]
        carry += run
        lastb = bnd[256]
    cstart[S] = carry
    return cstart, bnd_out


@pytest.mark.parametrize("case", ["valid", "decreasing", "repeat_full", "out_of_range", "many"])
def test_varlen_prefix_spans_stay_in_slots(case):
    """Packed-sequence backward: whatever cu_seqlens holds, the bounds the prefix
    launch derives are non-decreasing inside [0, T], every sequence's chunks fit
    the per-head slots the workspace provides (cmax = ceil(T/64) + S chunk slots,
    cmax + S state slots), and for a valid cu_seqlens the bounds are cu_seqlens
    itself."""
    rng = __import__("numpy").random.default_rng(5)
    T = 1024
    cu = {"valid": [0, 100, 100, 640, 1024],
          "decreasing": [0, 500, 100, 300, 1024],
          "repeat_full": [0, T, 0, T, 0, T],
          "out_of_range": [-50, 2000, -7, 5000, 30],
          "many": list(rng.integers(-100, T + 100, size=601))}[case]
    S = len(cu) - 1
    cstart, bnd = _prefix_model(cu, T)
    assert all(0 <= bnd[s] <= bnd[s + 1] <= T for s in range(S))
    assert bnd[0] >= 0 and bnd[S] <= T
    nch = [(bnd[s + 1] - bnd[s] + 63) // 64 for s in range(S)]
    assert cstart == [sum(nch[:s]) for s in range(S + 1)]
    cmax = (T + 63) // 64 + S
    assert cstart[S] <= cmax
    for s in range(S):
        # states: slot c0 + s + c for c = 0 .. nch (the last is the final state);
        # state gradients: slot c0 + c for c < nch
        assert cstart[s] + s + nch[s] < cmax + S
        assert nch[s] == 0 or cstart[s] + nch[s] - 1 < cmax
    if case == "valid":
        assert bnd == cu


def test_kda_validation_before_launch():
    """gdn_kda_fwd: bf16 only, the forward's argument checks, the segment count
    and the workspace, all checked before anything is launched."""
    lib = _lib.load()
    A = 1 << 20
    P = lambda a: ctypes.c_void_p(a) if a else None

    def call(q=A, g=A, dt=1, T=128, H=1, dk=128, nseg=1, ws=0, wsz=0):
        return lib.gdn_kda_fwd(P(q), P(A), P(A), P(g), P(A), None, P(A), None, 1, T, H, dk, 128, dt, 1.0,
                               nseg, P(ws), wsz, None)
    assert call(q=0) == _lib.GDN_ERR_INVALID_ARG
    assert call(g=0) == _lib.GDN_ERR_INVALID_ARG
    assert call(dt=0) == _lib.GDN_ERR_UNSUPPORTED
    assert "bf16" in _lib.last_error()
    assert call(dk=64) == _lib.GDN_ERR_UNSUPPORTED
    assert call(T=0) == _lib.GDN_ERR_INVALID_ARG
    assert call(g=A + 2) == _lib.GDN_ERR_INVALID_ARG
    assert call(H=65536) == _lib.GDN_ERR_INVALID_ARG   # 64 rows of 65536 * 512 bytes of gates: past 2^31
    assert "KDA gates" in _lib.last_error()
    assert call(nseg=-1) == _lib.GDN_ERR_INVALID_ARG
    assert call(nseg=1025) == _lib.GDN_ERR_INVALID_ARG
    # two segments of one chunk each need (P - 1) slots of 2 x 128 x 128 floats
    need = 2 * 128 * 128 * 4
    assert call(nseg=2) == _lib.GDN_ERR_WORKSPACE
    assert call(nseg=2, ws=A, wsz=need - 1) == _lib.GDN_ERR_WORKSPACE
    assert call(nseg=2, ws=A + 16, wsz=need) == _lib.GDN_ERR_INVALID_ARG


def test_kda_plan_and_workspace():
    """The KDA split's host planner and workspace size (no device needed for
    n_segments >= 1; the automatic count reads num_cus)."""
    lib = _lib.load()
    plan = lib.gdn_kda_plan_segments
    assert plan(1, 32768, 32, 256, 0) == 9           # 8 workgroups per head on 256 CUs, one segment more
    assert plan(1, 32768, 8, 256, 0) == 17           # capped at 16 + 1
    assert plan(1, 32768, 128, 256, 0) == 3          # two workgroups per head
    assert plan(1, 32768, 256, 256, 0) == 1          # one workgroup per head: unsplit
    assert plan(1, 32768, 64, 256, 0) == 5
    assert plan(1, 32768, 80, 256, 0) == 4
    assert plan(1, 1024, 4, 256, 0) == 1             # 16 chunks: a = 16/8 - 1 = 1
    assert plan(1, 3072, 4, 256, 0) == 6             # 48 chunks: a = 5, 6 segments of 8
    assert plan(1, 128, 1, 256, 1) == 1
    assert plan(1, 128, 1, 256, 5) == 2              # at most one segment per chunk
    assert plan(1, 64 * 10, 1, 0, 4) == 4            # 3, 3, 3, 1 chunks
    assert plan(1, 64 * 10, 1, 0, 6) == 5            # S = 2: 5 segments, none empty
    assert plan(1, 64 * 10, 1, 0, 0) == 0            # automatic needs the CU count
    assert plan(0, 128, 1, 256, 1) == 0
    assert plan(1, 128, 1, 256, -1) == 0
    wsz = lib.gdn_kda_fwd_workspace_size
    assert wsz(2, 64 * 10, 3, 128, 128, 1) == 0
    assert wsz(2, 64 * 10, 3, 128, 128, 4) == 2 * 3 * 3 * 2 * 128 * 128 * 4
    assert wsz(2, 64 * 10, 3, 128, 128, -2) == ctypes.c_size_t(-1).value
    assert wsz(2, 64 * 10, 3, 64, 128, 2) == ctypes.c_size_t(-1).value


def test_bwd_plan_segments():
    """The backward's host rule for splitting the state-gradient sweep (few heads:
    2 B H below the CU count), written out here from its documented form."""
    lib = _lib.load()
    plan = lib.gdn_chunk_bwd_plan_segments
    assert plan(1, 32768, 32, 256) == 9             # 8 workgroups per head, one segment more
    assert plan(4, 8192, 32, 256) == 1              # 2 B H = 256 CUs: unsplit
    assert plan(1, 32768, 127, 256) == 3            # 2 B H = 254: a = 2
    assert plan(1, 32768, 128, 256) == 1            # 2 B H = 256: unsplit
    assert plan(1, 64 * 97, 1, 256) == 11           # a = 97 // 8 - 1 = 11: 12 -> S = 9, P = 11
    assert plan(3, 64 * 150 + 40, 1, 256) == 17     # a capped at 16
    assert plan(2, 64 * 30 + 5, 3, 256) == 3        # 31 chunks: a = 2, S = 11
    assert plan(1, 64 * 23, 2, 256) == 1            # 23 chunks: a = 1
    assert plan(1, 64 * 24, 2, 256) == 3            # 24 chunks: a = 2
    assert plan(1, 32768, 32, 0) == 1               # no CU count: unsplit
    assert plan(0, 128, 1, 256) == 0
    assert plan(1, 0, 1, 256) == 0

    def rule(B, T, H, cus):
        N = -(-T // 64)
        if cus <= 0 or 2 * B * H >= cus:
            return 1
        a = min(16, cus // (B * H), N // 8 - 1)
        if a < 2:
            return 1
        S = -(-N // (a + 1))
        return -(-N // S)
    for B, T, H, cus in [(1, 4096, 1, 304), (2, 100000, 5, 256), (1, 640, 1, 80), (7, 65536, 3, 256),
                         (1, 262144, 16, 256), (1, 513, 1, 256)]:
        assert plan(B, T, H, cus) == rule(B, T, H, cus), (B, T, H, cus)


def test_profile_kinds_mask_is_thread_local_bookkeeping():
    """gdn_profile_kinds sets the launch kinds the profiling hook brackets and
    returns the previous mask (all kinds by default); host-only."""
    lib = _lib.load()
    prev = lib.gdn_profile_kinds(1 << 4)
    assert prev == 0xFFFFFFFF
    assert lib.gdn_profile_kinds(prev) == 1 << 4
    assert lib.gdn_profile_kinds(0xFFFFFFFF) == 0xFFFFFFFF
