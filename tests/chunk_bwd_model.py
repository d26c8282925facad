"""fp64 numpy model of a chunked backward of the gated delta rule (test
infrastructure: it documents and checks, on the CPU, the matrix form a
matrix-core backward would compute; no kernel implements it yet, the HIP
path does not import it, and it imports nothing from the HIP path).

One head, one fragment of L tokens from a start state S (K x V) with the
cotangent dS_end of its end state, processed in chunks of C tokens from the
last.  In a chunk with tokens i = 0 .. C-1 (rows of the C x K and C x V
matrices below) and per-channel log-decays g_i (natural units):
    G_i  = g_0 + ... + g_i,  Gamma_i = exp(G_i),  gC = exp(G_{C-1})
    Kd   = k o Gamma,  Qd = q o Gamma,  Ki = k o exp(-G),  Kh = k o exp(G_{C-1} - G)
    A    = diag(beta) strictly_lower(Kd Ki^T),  T = (I + A)^-1
    R    = V - Kd S,  X = diag(beta) R,  U = T X          (U's rows are the u_t)
    O    = Qd S + P U,  P = lower_incl(Qd Ki^T)
    S'   = diag(gC) S + Kh^T U
The loss is <O, dO> + <S', dS'> with dS' from the later chunks; reverse mode:
    dU   = P^T dO + Kh dS'
    dX   = T^T dU,  dR = diag(beta) dX,  dbeta += rowdot(dX, R),  dV = dR
    dT   = dU X^T,  dA = strictly_lower(-T^T dT T^T)
    dbeta += rowsum(dA o strictly_lower(Kd Ki^T)),  dA' = diag(beta) dA
    dP   = lower_incl(dO U^T)
    dQd  = dO S^T + dP Ki
    dKd  = -dR S^T + dA' Ki
    dKi  = dP^T Qd + dA'^T Kd
    dKh  = U dS'^T
    dS   = diag(gC) dS' + Qd^T dO - Kd^T dR
and through the exponentials (dG_i the gradient of G_i):
    dq   = dQd o Gamma
    dk   = dKd o Gamma + dKi o exp(-G) + dKh o exp(G_{C-1} - G)
    dG   = dQd o Qd + dKd o Kd - dKi o Ki - dKh o Kh,
    dG_{C-1} += colsum(dKh o Kh) + gC o rowsum(dS' o S)
    dg_t = dG_t + ... + dG_{C-1}                       (reverse prefix sum)
Every product is a dense C x K x V, C x C x (K or V) or K x C x V
contraction: the per-token reverse walk becomes matrix-core work.  The
exponentials exp(-G) bound the chunk's decay range in FP32 (about 88 nats
per channel), the same domain question the forward's anchored form answers.
"""
from __future__ import annotations

import numpy as np


def _chunk(S, dS_next, q, k, v, g, beta, do):
    """One chunk: the start state S, the cotangent dS_next of its end state;
    returns (dS at its start, dq, dk, dv, dg, dbeta)."""
    C = k.shape[0]
    G = np.cumsum(g, axis=0)
    Gam = np.exp(G)
    Einv = np.exp(-G)
    gC = Gam[-1]
    Kd, Qd, Ki = k * Gam, q * Gam, k * Einv
    Eh = np.exp(G[-1][None, :] - G)
    Kh = k * Eh
    lower = np.tril(np.ones((C, C)), -1)
    lower_incl = np.tril(np.ones((C, C)))
    Ap = (Kd @ Ki.T) * lower                    # A' (without beta)
    A = beta[:, None] * Ap
    T = np.linalg.inv(np.eye(C) + A)
    R = v - Kd @ S
    X = beta[:, None] * R
    U = T @ X
    P = (Qd @ Ki.T) * lower_incl

    dU = P.T @ do + Kh @ dS_next
    dX = T.T @ dU
    dR = beta[:, None] * dX
    dbeta = np.sum(dX * R, axis=1)
    dv = dR
    dT = dU @ X.T
    dA = (-(T.T @ dT @ T.T)) * lower
    dbeta = dbeta + np.sum(dA * Ap, axis=1)
    dAp = beta[:, None] * dA
    dP = (do @ U.T) * lower_incl
    dQd = do @ S.T + dP @ Ki
    dKd = -dR @ S.T + dAp @ Ki
    dKi = dP.T @ Qd + dAp.T @ Kd
    dKh = U @ dS_next.T
    dS = gC[:, None] * dS_next + Qd.T @ do - Kd.T @ dR

    dq = dQd * Gam
    dk = dKd * Gam + dKi * Einv + dKh * Eh
    dG = dQd * Qd + dKd * Kd - dKi * Ki - dKh * Kh
    dG[-1] += np.sum(dKh * Kh, axis=0) + gC * np.sum(dS_next * S, axis=1)
    dg = np.cumsum(dG[::-1], axis=0)[::-1]
    return dS, dq, dk, dv, dg, dbeta


def _forward_chunk(S, k, v, g, beta):
    """The state at the chunk's end (the same chunk form, forward only)."""
    C = k.shape[0]
    G = np.cumsum(g, axis=0)
    Gam = np.exp(G)
    Kd, Ki = k * Gam, k * np.exp(-G)
    Kh = k * np.exp(G[-1][None, :] - G)
    A = beta[:, None] * ((Kd @ Ki.T) * np.tril(np.ones((C, C)), -1))
    U = np.linalg.solve(np.eye(C) + A, beta[:, None] * (v - Kd @ S))
    return Gam[-1][:, None] * S + Kh.T @ U


def chunk_backward(q, k, v, g, beta, do, S0, dS_end, C=32):
    """Gradients of one head's fragment: q, k, g [L, K]; v, do [L, V];
    beta [L]; S0 and dS_end [K, V].  Returns (dq, dk, dv, dg, dbeta, dS0)."""
    L = k.shape[0]
    bounds = list(range(0, L, C)) + [L]
    states = [np.array(S0, dtype=np.float64)]
    for a, b in zip(bounds[:-1], bounds[1:-1]):
        states.append(_forward_chunk(states[-1], k[a:b], v[a:b], g[a:b], beta[a:b]))
    dq, dk, dg = (np.zeros_like(k, dtype=np.float64) for _ in range(3))
    dv = np.zeros_like(v, dtype=np.float64)
    dbeta = np.zeros(L)
    dS = np.array(dS_end, dtype=np.float64)
    for c in range(len(bounds) - 2, -1, -1):
        a, b = bounds[c], bounds[c + 1]
        dS, dq[a:b], dk[a:b], dv[a:b], dg[a:b], dbeta[a:b] = _chunk(
            states[c], dS, q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], do[a:b])
    return dq, dk, dv, dg, dbeta, dS
