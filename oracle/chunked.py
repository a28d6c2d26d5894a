"""TEST INFRASTRUCTURE ONLY: the chunk-parallel (WY / UT-transform) form of the
gated delta rule in NumPy fp64.

This is a second CPU implementation, independent of the token loop in
``gdn_oracle.c``: it splits each sequence into chunks of C tokens and computes
each chunk from its entering state with dense matrix algebra, the
decomposition behind the kernel family the XTuner / Ascend 910C article
describes in section 3.1.2 (Fig. 7: a per-chunk triangular solve, a forward
state pass, an output step; backward: a dv-local step, a reverse state-gradient
pass and a dq/dk/dw/dg step).  The article gives no equations; the ones below
are derived from the recurrence (see ``gdn_oracle.c``).  Agreement of the two
forms is one of the oracle's pins.

Per chunk (rows r, s = 0..L-1, entering state h = S^T, d_k x d_v):
  gamma_r = sum_{s<=r} g_s                        chunk-local log-decay prefix
  D_rs    = exp(gamma_r - gamma_s) for s <= r, else 0
  A       = strict_lower(diag(beta) (K K^T) * D)
  T       = (I + A)^-1                            unit lower triangular
  W       = T diag(beta * exp(gamma)) K,   U = T diag(beta) V
  V'      = U - W h
  O       = scale [diag(exp(gamma)) Q h + ((Q K^T) * D) V']
  h_next  = exp(gamma_L) h + Kt^T V',      Kt = diag(exp(gamma_L - gamma)) K
"""
from __future__ import annotations

import numpy as np


def _chunks(length, C):
    return [(c, min(c + C, length)) for c in range(0, length, C)]


def chunk_prep(Kc, Vc, gc, bc):
    """gamma, D, A, T, W, U for one chunk (fp64)."""
    L = Kc.shape[0]
    gamma = np.cumsum(gc)
    diff = gamma[:, None] - gamma[None, :]
    mask = np.tril(np.ones((L, L), dtype=bool))
    D = np.where(mask, np.exp(np.where(mask, diff, 0.0)), 0.0)
    G = Kc @ Kc.T
    A = np.tril(bc[:, None] * G * D, -1)
    T = np.linalg.inv(np.eye(L) + A)
    Gam = np.exp(gamma)
    W = T @ ((bc * Gam)[:, None] * Kc)
    U = T @ (bc[:, None] * Vc)
    return dict(gamma=gamma, D=D, G=G, A=A, T=T, W=W, U=U, Gam=Gam)


def _unit_fwd(Q, K, V, g, b, h, C, scale):
    """One (sequence, head): Q,K [len,dk], V [len,dv], h [dk,dv]."""
    n = Q.shape[0]
    O = np.zeros((n, V.shape[1]))
    states = []
    for c0, c1 in _chunks(n, C):
        Qc, Kc, Vc = Q[c0:c1] * scale, K[c0:c1], V[c0:c1]
        p = chunk_prep(Kc, Vc, g[c0:c1], b[c0:c1])
        states.append(h.copy())
        Vp = p["U"] - p["W"] @ h
        P = (Qc @ Kc.T) * p["D"]
        O[c0:c1] = p["Gam"][:, None] * (Qc @ h) + P @ Vp
        gL = p["gamma"][-1]
        Kt = np.exp(gL - p["gamma"])[:, None] * Kc
        h = np.exp(gL) * h + Kt.T @ Vp
    return O, h, states


def _unit_bwd(Q, K, V, g, b, h0, dO, dhT, C, scale):
    n, dk = Q.shape
    dv = V.shape[1]
    _, _, states = _unit_fwd(Q, K, V, g, b, h0, C, scale)
    dQ = np.zeros_like(Q); dK = np.zeros_like(K); dV = np.zeros_like(V)
    dg = np.zeros(n); db = np.zeros(n)
    Hp = dhT.copy()  # dL/dh_next of the current chunk
    for ci, (c0, c1) in reversed(list(enumerate(_chunks(n, C)))):
        h = states[ci]
        Qc, Kc, Vc, dOc = Q[c0:c1] * scale, K[c0:c1], V[c0:c1], dO[c0:c1]
        bc = b[c0:c1]
        p = chunk_prep(Kc, Vc, g[c0:c1], bc)
        gamma, D, A, T, W, Gam = p["gamma"], p["D"], p["A"], p["T"], p["W"], p["Gam"]
        L = c1 - c0
        gL = gamma[-1]
        sK = np.exp(gL - gamma)
        Kt = sK[:, None] * Kc
        Vp = p["U"] - W @ h
        P = (Qc @ Kc.T) * D
        # state-gradient side
        dVp = P.T @ dOc + Kt @ Hp
        Hprev = np.exp(gL) * Hp + (Gam[:, None] * Qc).T @ dOc - W.T @ dVp
        # output side
        dP = np.tril(dOc @ Vp.T)
        dQc = Gam[:, None] * (dOc @ h.T) + (dP * D) @ Kc
        dKc = (dP * D).T @ Qc + sK[:, None] * (Vp @ Hp.T)
        dgam = np.zeros(L)
        dgam += Gam * np.sum((Qc @ h) * dOc, axis=1)           # from diag(Gam) Q h
        MO = dP * P
        dgam += MO.sum(1) - MO.sum(0)                            # from D inside P
        cs = sK * np.sum(Kc * (Vp @ Hp.T), axis=1)               # from Kt in h_next
        dgam -= cs
        dgam[-1] += cs.sum() + np.exp(gL) * np.sum(h * Hp)       # from exp(gamma_L)
        # WY side: W = T Xw, U = T Xu
        dW = -dVp @ h.T
        dU = dVp
        Xw = (bc * Gam)[:, None] * Kc
        Xu = bc[:, None] * Vc
        dT = dW @ Xw.T + dU @ Xu.T
        dXw = T.T @ dW
        dXu = T.T @ dU
        dKc += (bc * Gam)[:, None] * dXw
        dVc = bc[:, None] * dXu
        dbc = Gam * np.sum(Kc * dXw, axis=1) + np.sum(Vc * dXu, axis=1)
        dgam += bc * Gam * np.sum(Kc * dXw, axis=1)
        dA = np.tril(-T.T @ dT @ T.T, -1)
        GD = np.tril(p["G"] * D, -1)
        E = dA * bc[:, None] * D
        dKc += (E + E.T) @ Kc
        dbc += np.sum(dA * GD, axis=1)
        MA = dA * A
        dgam += MA.sum(1) - MA.sum(0)
        dg[c0:c1] = np.cumsum(dgam[::-1])[::-1]
        dQ[c0:c1] = dQc * scale
        dK[c0:c1] = dKc
        dV[c0:c1] = dVc
        db[c0:c1] = dbc
        Hp = Hprev
    return dQ, dK, dV, dg, db, Hp


def _units(q, cu_seqlens):
    B, T = q.shape[:2]
    if cu_seqlens is None:
        return [(b, 0, T) for b in range(B)], B
    cu = [int(x) for x in cu_seqlens]
    return [(0, cu[n], cu[n + 1]) for n in range(len(cu) - 1)], len(cu) - 1


def fwd(q, k, v, g, beta, initial_state=None, cu_seqlens=None, scale=1.0, chunk=64):
    q, k, v, g, beta = (np.asarray(x, np.float64) for x in (q, k, v, g, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    units, N = _units(q, cu_seqlens)
    o = np.zeros((B, T, H, dv))
    ht = np.zeros((N, H, dk, dv))
    for n, (bb, t0, t1) in enumerate(units):
        for hh in range(H):
            h0 = np.zeros((dk, dv)) if initial_state is None else np.asarray(
                initial_state[n, hh], np.float64)
            O, h, _ = _unit_fwd(q[bb, t0:t1, hh], k[bb, t0:t1, hh], v[bb, t0:t1, hh],
                                g[bb, t0:t1, hh], beta[bb, t0:t1, hh], h0, chunk, scale)
            o[bb, t0:t1, hh] = O
            ht[n, hh] = h
    return o, ht


def bwd(q, k, v, g, beta, do, initial_state=None, dht=None, cu_seqlens=None, scale=1.0,
        chunk=64):
    q, k, v, g, beta, do = (np.asarray(x, np.float64) for x in (q, k, v, g, beta, do))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    units, N = _units(q, cu_seqlens)
    out = [np.zeros_like(q), np.zeros_like(k), np.zeros_like(v), np.zeros_like(g),
           np.zeros_like(beta), np.zeros((N, H, dk, dv))]
    for n, (bb, t0, t1) in enumerate(units):
        for hh in range(H):
            h0 = np.zeros((dk, dv)) if initial_state is None else np.asarray(
                initial_state[n, hh], np.float64)
            dhT = np.zeros((dk, dv)) if dht is None else np.asarray(dht[n, hh], np.float64)
            r = _unit_bwd(q[bb, t0:t1, hh], k[bb, t0:t1, hh], v[bb, t0:t1, hh],
                          g[bb, t0:t1, hh], beta[bb, t0:t1, hh], h0, do[bb, t0:t1, hh], dhT,
                          chunk, scale)
            for x, val in zip(out[:5], r[:5]):
                x[bb, t0:t1, hh] = val
            out[5][n, hh] = r[5]
    return tuple(out)
