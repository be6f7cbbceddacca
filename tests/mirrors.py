"""Independent float64 NumPy evaluations used to pin the oracle (test-only).

These compute the same operator as the oracle by different routes: explicit
per-token transition matrices, the chunk-wise WY form, the intra-sequence split
with an associative correction, and the sliding-window shortcut.  They share no
code with the oracle (which is C) or with the GPU library.

Sources (the FlashQLA pages):
  * talk summary (onedev.kr), paragraph 3: per chunk (usually 64 tokens),
    (1) K K^T inside the chunk and its triangular inverse, (2) W and U,
    (3) the state passed from chunk to chunk, (4) the output;
  * paragraph 4: the state difference between adjacent chunks is one dk x dk
    matrix product, so a sequence split can be corrected associatively, keeping
    only each segment's last correction and computing the state twice;
  * paragraph 5: with alpha in (0,1) and unit keys, old state decays like powers
    of alpha, so heads with enough decay only need to look back one window;
  * paragraph 6: the gamma outer-product matrix has unit diagonal, so the
    diagonal scaling can be pulled outside the inverse (the inverse itself is
    gate-free) and every exponential is taken once per position.
"""
from __future__ import annotations

import numpy as np


def brute_force_head(q, k, v, g, beta, h0, scale=1.0):
    """Explicit transition matrices for one head.  q,k [T,dk]; v [T,dv]; g,beta [T];
    h0 [dk,dv].  S_t = P_t S_{t-1} + beta_t k_t v_t^T with
    P_t = alpha_t (I - beta_t k_t k_t^T); o_t = scale S_t^T q_t.

    The final state is also assembled as the closed sum
    h_T = P_T...P_1 h0 + sum_t P_T...P_{t+1} beta_t k_t v_t^T."""
    T, dk = k.shape
    Ps = [np.exp(g[t]) * (np.eye(dk) - beta[t] * np.outer(k[t], k[t])) for t in range(T)]

    def prod(hi, lo):  # P_hi P_{hi-1} ... P_lo, identity when hi < lo
        M = np.eye(dk)
        for j in range(lo, hi + 1):
            M = Ps[j] @ M
        return M

    o = np.zeros((T, v.shape[1]))
    S = h0.copy()
    for t in range(T):
        S = prod(t, 0) @ h0
        for s in range(t + 1):
            S = S + prod(t, s + 1) @ (beta[s] * np.outer(k[s], v[s]))
        o[t] = scale * S.T @ q[t]
    return o, S


def chunk_prep(kc, gc, bc):
    """Chunk-independent part of one chunk (steps 1-2 of the WY form, with the
    diagonal gate scaling pulled outside the inverse).

    Returns gamma (in-chunk inclusive cumsum of g), T0 = (I + diag(beta) L)^-1 with
    L = strictly-lower(K K^T) (gate-free), and the gated inverse
    T = diag(Gamma) T0 diag(1/Gamma) formed from the 2C exponentials only."""
    C = kc.shape[0]
    gam = np.cumsum(gc)
    L = np.tril(kc @ kc.T, -1)
    T0 = np.linalg.inv(np.eye(C) + bc[:, None] * L)
    Gam = np.exp(gam)
    invGam = np.exp(-gam)
    T = Gam[:, None] * T0 * invGam[None, :]
    return gam, T0, T


def chunk_step(qc, kc, vc, gc, bc, H, scale=1.0):
    """One chunk of the WY form.  H is the dk x dv state entering the chunk.
    V' = T diag(beta) (V - diag(Gamma) K H)         (true new values)
    O  = diag(Gamma) Q H + (Mask o Q K^T) V'        Mask_rs = Gamma_r/Gamma_s, s <= r
    H' = Gamma_C H + K^T diag(Gamma_C / Gamma) V'
    Returns (O, H')."""
    gam, T0, T = chunk_prep(kc, gc, bc)
    Gam = np.exp(gam)
    Vp = (T * bc[None, :]) @ (vc - Gam[:, None] * (kc @ H))
    mask = np.tril(Gam[:, None] * np.exp(-gam)[None, :])
    O = scale * (Gam[:, None] * (qc @ H) + (mask * (qc @ kc.T)) @ Vp)
    GC = np.exp(gam[-1])
    Hn = GC * H + kc.T @ (np.exp(gam[-1] - gam)[:, None] * Vp)
    return O, Hn


def chunked_head(q, k, v, g, beta, h0, C=64, scale=1.0):
    """Whole head by the chunk-wise WY form; the last chunk may be short."""
    T = q.shape[0]
    H = h0.copy()
    o = np.zeros((T, v.shape[1]))
    for s in range(0, T, C):
        e = min(s + C, T)
        o[s:e], H = chunk_step(q[s:e], k[s:e], v[s:e], g[s:e], beta[s:e], H, scale)
    return o, H


def segment_map(k, v, g, beta, C=64):
    """Pass over one segment from the zero state (the split's first pass).
    The segment acts on its entering state as H -> e^G Mt H + b, where b is the
    zero-start final state, G = sum of g over the segment and
    Mt = prod_c (I - K_c^T T0_c diag(beta_c) K_c) is gate-free."""
    dk = k.shape[1]
    b = np.zeros((dk, v.shape[1]))
    Mt = np.eye(dk)
    for s in range(0, k.shape[0], C):
        e = min(s + C, k.shape[0])
        kc, bc = k[s:e], beta[s:e]
        _, T0, _ = chunk_prep(kc, g[s:e], bc)
        Mt = (np.eye(dk) - kc.T @ (T0 * bc[None, :]) @ kc) @ Mt
        _, b = chunk_step(np.zeros_like(kc), kc, v[s:e], g[s:e], bc, b)
    return float(np.sum(g)), Mt, b


def split_head(q, k, v, g, beta, h0, bounds, C=64, scale=1.0):
    """Intra-sequence split.  bounds are token offsets of the segment starts
    (bounds[0] == 0, multiples of C).  Segment 0 runs from h0; segments 1..P-2
    run from zero and keep only (G, Mt, b); a sequential combine gives every
    segment's true entering state; each segment is then re-run from it."""
    T = q.shape[0]
    ends = list(bounds[1:]) + [T]
    P = len(bounds)
    o = np.zeros((T, v.shape[1]))
    starts = [h0]
    o0, Hend = chunked_head(q[:ends[0]], k[:ends[0]], v[:ends[0]], g[:ends[0]], beta[:ends[0]],
                            h0, C, scale)
    o[:ends[0]] = o0
    starts.append(Hend)
    for p in range(1, P - 1):
        s, e = bounds[p], ends[p]
        G, Mt, b = segment_map(k[s:e], v[s:e], g[s:e], beta[s:e], C)
        starts.append(np.exp(G) * Mt @ starts[p] + b)
    H = Hend
    for p in range(1, P):
        s, e = bounds[p], ends[p]
        o[s:e], H = chunked_head(q[s:e], k[s:e], v[s:e], g[s:e], beta[s:e], starts[p], C, scale)
    return o, H


def window_head(q, k, v, g, beta, h0, bounds, w, C=64, scale=1.0):
    """Sliding-window shortcut: segment p warms up from the zero state over the
    w chunks before its start (from h0 when that reaches the sequence start) and
    then produces its outputs; no correction is applied."""
    T = q.shape[0]
    ends = list(bounds[1:]) + [T]
    o = np.zeros((T, v.shape[1]))
    H = None
    for p, s in enumerate(bounds):
        e = ends[p]
        ws = s - w * C
        if ws <= 0:
            ws, Hs = 0, h0
        else:
            Hs = np.zeros_like(h0)
        oo, H = chunked_head(q[ws:e], k[ws:e], v[ws:e], g[ws:e], beta[ws:e], Hs, C, scale)
        o[s:e] = oo[s - ws:]
    return o, H


def chunk_backward_local(qc, kc, vc, gc, bc, doc, H, dHn, Hn, scale=1.0):
    """Local gradients of one chunk given its entering state H, the gradient dHn
    that reaches the chunk's final state from the right, and that final state Hn.

    Forward in gated-matrix form (Sg_rs = Gamma_r / Gamma_s for s <= r):
      Pm = tril(Q K^T) o Sg (with diagonal), Mg = strict_lower(K K^T) o Sg,
      T = (I + diag(beta) Mg)^-1, Y = V - diag(Gamma) K H, V' = T diag(beta) Y,
      O = scale (diag(Gamma) Q H + Pm V'), Hn = Gamma_C H + K^T diag(E) V',
      E_r = Gamma_C / Gamma_r.
    Reverse mode of exactly these lines; the gate gradient arrives per position as
    d(gamma_r) and becomes d(g_t) by a reverse cumulative sum inside the chunk.
    Returns (dq, dk, dv, dg, dbeta, dH) where dH is the gradient reaching H."""
    C = kc.shape[0]
    gam = np.cumsum(gc)
    Gam = np.exp(gam)
    GC = Gam[-1]
    E = np.exp(gam[-1] - gam)
    Sg = np.tril(np.exp(gam[:, None] - gam[None, :]))
    Sqk = qc @ kc.T
    Skk = kc @ kc.T
    Pm = np.tril(Sqk) * Sg
    Mg = np.tril(Skk, -1) * Sg
    T = np.linalg.inv(np.eye(C) + bc[:, None] * Mg)
    Y = vc - Gam[:, None] * (kc @ H)
    Z = bc[:, None] * Y
    Vp = T @ Z
    # reverse
    dVp = scale * Pm.T @ doc + E[:, None] * (kc @ dHn)
    dZ = T.T @ dVp
    dY = bc[:, None] * dZ
    dA = -np.tril(dZ @ Vp.T, -1)
    dMg = bc[:, None] * dA
    dPm = scale * np.tril(doc @ Vp.T)
    dPg = dPm * Sg                      # gradient w.r.t. the raw entries of Q K^T
    dMgg = dMg * Sg                     # gradient w.r.t. the raw entries of K K^T (strict lower)
    dq2 = scale * Gam[:, None] * (doc @ H.T)
    dq = dPg @ kc + dq2
    dk3 = -Gam[:, None] * (dY @ H.T)
    dk4 = E[:, None] * (Vp @ dHn.T)
    dk = dPg.T @ qc + (dMgg + dMgg.T) @ kc + dk3 + dk4
    dv = dY
    dbeta = np.sum(Y * dZ, axis=1) + np.sum(dA * Mg, axis=1)
    X = dPm * Pm + dMg * Mg
    dgam = X.sum(axis=1) - X.sum(axis=0)
    dgam += np.sum(qc * dq2, axis=1) + np.sum(kc * dk3, axis=1) - np.sum(kc * dk4, axis=1)
    dgam[-1] += np.sum(dHn * Hn)
    dg = np.cumsum(dgam[::-1])[::-1]
    dH = scale * qc.T @ (Gam[:, None] * doc) + GC * dHn - kc.T @ (Gam[:, None] * dY)
    return dq, dk, dv, dg, dbeta, dH


def chunked_backward_head(q, k, v, g, beta, h0, dout, dht=None, C=64, scale=1.0):
    """Backward of one head in three sweeps: the chunk-entry states forward, the
    state gradient backward over chunks, then every chunk's local gradients from
    its entering state and the gradient reaching its end."""
    T = q.shape[0]
    starts = list(range(0, T, C))
    Hs = [h0.copy()]
    for s in starts:
        e = min(s + C, T)
        _, Hn = chunk_step(q[s:e], k[s:e], v[s:e], g[s:e], beta[s:e], Hs[-1], scale)
        Hs.append(Hn)
    dHs = [None] * (len(starts) + 1)
    dHs[-1] = np.zeros_like(h0) if dht is None else dht.copy()
    out = {n: np.zeros_like(a) for n, a in (("dq", q), ("dk", k), ("dv", v), ("dg", g),
                                            ("dbeta", beta))}
    for i in range(len(starts) - 1, -1, -1):
        s = starts[i]
        e = min(s + C, T)
        dq, dk, dv, dg, db, dH = chunk_backward_local(q[s:e], k[s:e], v[s:e], g[s:e], beta[s:e],
                                                      dout[s:e], Hs[i], dHs[i + 1], Hs[i + 1], scale)
        out["dq"][s:e], out["dk"][s:e], out["dv"][s:e] = dq, dk, dv
        out["dg"][s:e], out["dbeta"][s:e] = dg, db
        dHs[i] = dH
    out["dh0"] = dHs[0]
    return out
