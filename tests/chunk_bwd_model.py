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


# ---------------------------------------------------------------------------
# The same backward in the anchored three-pass form the matrix-core kernels
# take.  Per chunk of C tokens (a ragged last chunk padded with zero tokens,
# g = 0: G is flat past the end), with a = G_15 the chunk's anchor and
# Gc = G_{C-1}:
#     Kr = k e^{G-a},  Kc = k e^{a-G},  Qr = q e^{G-a}
#     A' = strict_lower(Kr Kc^T),  T = (I + diag(beta) A')^-1,  Tb = T diag(beta)
#     P  = lower_incl(Qr Kc^T)
# pass 1 (forward): R_c = e^{a_c} o S_c (the state entering chunk c, rows
#     scaled by its anchor), R_{c+1} = fac_c o (R_c + Kc^T Tb (V - Kr R_c)),
#     fac_c = e^{a_{c+1} + Gc_c - a_c};
# pass 2 (reverse): D_c = fac_c o Delta_{c+1} (the cotangent of the state
#     leaving chunk c, rows scaled by e^{Gc - a}; Delta_n is the fragment
#     end's cotangent and fac_{n-1} = e^{Gc - a} there),
#     dU = P^T dO + Kc D_c,  dR = Tb^T dU,
#     Delta_c = D_c + Qr^T dO - Kr^T dR,  dS_start = e^{a_0} o Delta_0;
# pass 3 (every chunk on its own, from R_c and D_c):
#     W = Kr R,  X = diag(beta)(V - W),  U = T X,  dU = P^T dO + Kc D
#     dX = T^T dU,  dR = diag(beta) dX = dv,  dA = strict_lower(-dX U^T)
#     dbeta = rowsum(dX o (V - W)) + rowsum(dA o A'),  dA' = diag(beta) dA
#     dP = lower_incl(dO U^T)
#     dq   = (dO R^T + dP Kc) o e^{G-a}
#     dk_d = (-dR R^T + dA' Kc) o e^{G-a}
#     dk_i = (dP^T Qr + dA'^T Kr) o e^{a-G}
#     dk_h = (U D^T) o e^{a-G}
#     dk = dk_d + dk_i + dk_h,  dG = q o dq + k o (dk_d - dk_i - dk_h)
#     dG_{C-1} += colsum(k o dk_h) + rowsum(D o R),  dg = reverse cumsum of dG
# ---------------------------------------------------------------------------
def _anchored_operands(q, k, g, C):
    G = np.cumsum(g, axis=0)
    a = G[min(15, C - 1)]
    Gc = G[-1]
    Kr, Kc, Qr = k * np.exp(G - a), k * np.exp(a - G), q * np.exp(G - a)
    Ap = (Kr @ Kc.T) * np.tril(np.ones((C, C)), -1)
    P = (Qr @ Kc.T) * np.tril(np.ones((C, C)))
    return G, a, Gc, Kr, Kc, Qr, Ap, P


def _pad(x, C):
    out = np.zeros((C,) + x.shape[1:])
    out[:x.shape[0]] = x
    return out


def anchored_backward(q, k, v, g, beta, do, S0, dS_end, C=32):
    """Gradients of one head's fragment by the three passes above; returns
    (dq, dk, dv, dg, dbeta, dS0) and the per-chunk R_c and D_c."""
    L, K = k.shape
    nc = (L + C - 1) // C
    ch = []
    for c in range(nc):
        s = slice(c * C, min(L, (c + 1) * C))
        ch.append(dict(q=_pad(q[s], C), k=_pad(k[s], C), v=_pad(v[s], C), g=_pad(g[s], C),
                       beta=_pad(beta[s], C), do=_pad(do[s], C), n=s.stop - s.start))
    for x in ch:
        x["G"], x["a"], x["Gc"], x["Kr"], x["Kc"], x["Qr"], x["Ap"], x["P"] = _anchored_operands(x["q"], x["k"], x["g"], C)
        x["T"] = np.linalg.inv(np.eye(C) + x["beta"][:, None] * x["Ap"])
        x["Tb"] = x["T"] * x["beta"][None, :]
    fac = [np.exp(ch[c + 1]["a"] + ch[c]["Gc"] - ch[c]["a"]) for c in range(nc - 1)]
    fac.append(np.exp(ch[-1]["Gc"] - ch[-1]["a"]))
    # pass 1
    R = [np.exp(ch[0]["a"])[:, None] * S0]
    for c in range(nc - 1):
        x = ch[c]
        U = x["Tb"] @ (x["v"] - x["Kr"] @ R[c])
        R.append(fac[c][:, None] * (R[c] + x["Kc"].T @ U))
    # pass 2
    D = [None] * nc
    delta = np.array(dS_end, dtype=np.float64)
    for c in range(nc - 1, -1, -1):
        x = ch[c]
        D[c] = fac[c][:, None] * delta
        dU = x["P"].T @ x["do"] + x["Kc"] @ D[c]
        dR = x["Tb"].T @ dU
        delta = D[c] + x["Qr"].T @ x["do"] - x["Kr"].T @ dR
    dS0 = np.exp(ch[0]["a"])[:, None] * delta
    # pass 3
    outs = {n: [] for n in ("dq", "dk", "dv", "dg", "dbeta")}
    for c in range(nc):
        x = ch[c]
        Rc, Dc = R[c], D[c]
        eGa, eaG = np.exp(x["G"] - x["a"]), np.exp(x["a"] - x["G"])
        Rv = x["v"] - x["Kr"] @ Rc
        U = x["T"] @ (x["beta"][:, None] * Rv)
        dU = x["P"].T @ x["do"] + x["Kc"] @ Dc
        dX = x["T"].T @ dU
        dR = x["beta"][:, None] * dX
        dA = -(dX @ U.T) * np.tril(np.ones((C, C)), -1)
        dbeta = np.sum(dX * Rv, axis=1) + np.sum(dA * x["Ap"], axis=1)
        dAp = x["beta"][:, None] * dA
        dP = (x["do"] @ U.T) * np.tril(np.ones((C, C)))
        dq = (x["do"] @ Rc.T + dP @ x["Kc"]) * eGa
        dk_d = (-dR @ Rc.T + dAp @ x["Kc"]) * eGa
        dk_i = (dP.T @ x["Qr"] + dAp.T @ x["Kr"]) * eaG
        dk_h = (U @ Dc.T) * eaG
        dG = x["q"] * dq + x["k"] * (dk_d - dk_i - dk_h)
        dG[-1] += np.sum(x["k"] * dk_h, axis=0) + np.sum(Dc * Rc, axis=1)
        dg = np.cumsum(dG[::-1], axis=0)[::-1]
        n = x["n"]
        for name, val in (("dq", dq), ("dk", dk_d + dk_i + dk_h), ("dv", dR), ("dg", dg), ("dbeta", dbeta)):
            outs[name].append(val[:n])
    res = tuple(np.concatenate(outs[nm], axis=0) for nm in ("dq", "dk", "dv", "dg", "dbeta"))
    return res + (dS0,), R, D
