"""float32 numpy model of the chunked factorisation the HIP chunk kernels use
(test infrastructure: it documents and checks the algorithm on the CPU; the
HIP path does not import it, and it imports nothing from the HIP path).

Per head, state S (K x V), one fragment of tokens processed in 32-token
chunks.  All exponent arithmetic is in log2 units.

In a chunk with per-channel log-decays l_0 .. l_31:
    G_i = l_0 + ... + l_i                in-chunk prefix
    a   = G_15                           the anchor's decay from the chunk start
    x_i = G_i - a                        factor exponents around the anchor
    d   = x_31                           decay from the anchor to the chunk end
The anchored form holds the state as R = 2^a o S and uses
    Kr = k 2^x,  Kc = k 2^-x,  Qr = q 2^x,
    A  = beta o (Kr Kc^T) strictly lower,  T = (I + A)^-1,  P = Qr Kc^T (j <= i)
    Y  = Kr R,  U = T diag(beta) (V - Y),  O = Qr R + P U,  R <- R + Kc^T U
and re-anchors with R <- 2^(a_next + d) o R.  With g <= 0 its factors stay
inside 2^[-XF, XF] when a >= -XF and d >= -XF on every channel (|x_0| <= -a).
A chunk beyond that is "extreme"; a fragment with any extreme chunk is run
again from its starting state with every token one by one in FP32 (its
anchored results discarded), the log2 decay floored at -300 (2^-300 times
any FP32 value is below the smallest FP32 denormal):
    R <- 2^l o R;  u = beta (v - R^T k);  R <- R + k u^T;  o = R^T q.
"""
from __future__ import annotations

import numpy as np

CH = 32
XF = 96.0            # largest in-chunk factor exponent of the anchored form (log2 units)
GFLOOR = -300.0      # floor of the per-token log2 decay
LOG2E = 1.4426950408889634

f32 = np.float32


def bf16_round(x):
    """Round float32 values to bfloat16 (nearest, ties to even), as float32."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32)


def split(x):
    """x as hi + lo bf16 parts, returned as their float32 sum (about 16
    significant bits), the precision of the split operands on the matrix cores."""
    x = np.asarray(x, dtype=np.float32)
    hi = bf16_round(x)
    lo = bf16_round(x - hi)
    return hi, lo


def smm(a, b):
    """a @ b with split operands, hi*hi + hi*lo + lo*hi, FP32 accumulation."""
    ah, al = split(a)
    bh, bl = split(b)
    return (ah @ bh + ah @ bl + al @ bh).astype(np.float32)


def exp2(x):
    return np.exp2(np.asarray(x, dtype=np.float32)).astype(np.float32)


def chunk_factors(l):
    """Per-chunk exponents from the log2 decays l [32, K]."""
    l = l.astype(np.float32)
    G = np.cumsum(l, 0, dtype=np.float32)
    a = G[15]
    x = (G - a).astype(np.float32)
    d = x[31]
    extreme = not bool(np.all(np.minimum(a, d) >= -XF))
    return x, a, d, extreme


def rescale(R, t):
    """R <- 2^t o R (rows), applied as a normal factor and a power of two where
    one FP32 factor would underflow."""
    t = t.astype(np.float32)
    e = np.where(t < -120.0, np.floor(t) + 60.0, 0.0).astype(np.int32)
    fv = exp2(t - e.astype(np.float32))
    return np.ldexp((R * fv[:, None]).astype(np.float32), e[:, None]).astype(np.float32)


def run_fragment(k, v, q, g, beta, S0, robust=True, want_o=True):
    """One fragment (tokens of one sequence inside one segment) from S0.

    k, q, g: [L, K]; v: [L, V]; beta: [L] (float32 values of the BF16 inputs);
    S0: [K, V].  ``robust=False`` keeps the anchored form's results even with
    extreme chunks (to show what it does beyond its range).  Returns
    (o [L, V], S_end, number of extreme chunks)."""
    L, K = k.shape
    V = v.shape[1]
    nc = (L + CH - 1) // CH
    pad = nc * CH - L

    def padded(a):
        return np.concatenate([a, np.zeros((pad,) + a.shape[1:], a.dtype)], 0).astype(np.float32)

    k, v, q, beta = padded(k), padded(v), padded(q), padded(beta)
    lg = (padded(g) * f32(LOG2E)).astype(np.float32)
    with np.errstate(invalid="ignore"):
        facts = [chunk_factors(lg[m * CH:(m + 1) * CH]) for m in range(nc)]
    n_ext = sum(f[3] for f in facts)
    o = np.zeros((nc * CH, V), np.float32)
    if robust and n_ext:
        R = S0.astype(np.float32).copy()
        for t in range(L):
            R = (R * exp2(np.maximum(lg[t], f32(GFLOOR)))[:, None]).astype(np.float32)
            u = (beta[t] * (v[t] - k[t] @ R)).astype(np.float32)
            R = (R + np.outer(k[t], u)).astype(np.float32)
            o[t] = q[t] @ R
        return o[:L], R, n_ext

    A_ = [f[1] for f in facts]
    D_ = [f[2] for f in facts]
    R = rescale(S0.astype(np.float32), A_[0])
    tri_s = np.tril(np.ones((CH, CH), bool), -1)
    tri_i = np.tril(np.ones((CH, CH), bool), 0)
    for m in range(nc):
        sl = slice(m * CH, (m + 1) * CH)
        km, vm, qm, bm = k[sl], v[sl], q[sl], beta[sl]
        x = facts[m][0]
        Kr = (km * exp2(x)).astype(np.float32)
        Kc = (km * exp2(-x)).astype(np.float32)
        Qr = (qm * exp2(x)).astype(np.float32)
        Amat = np.where(tri_s, bm[:, None] * smm(Kr, Kc.T), 0).astype(np.float32)
        T = np.linalg.inv((np.eye(CH) + Amat).astype(np.float64)).astype(np.float32)
        Tb = (T * bm[None, :]).astype(np.float32)
        Y = smm(Kr, R)
        U = smm(Tb, (vm - Y).astype(np.float32))
        if want_o:
            P = np.where(tri_i, smm(Qr, Kc.T), 0).astype(np.float32)
            o[sl] = smm(Qr, R) + smm(P, U)
        R = (R + smm(Kc.T, U)).astype(np.float32)
        nxt = A_[m + 1] if m + 1 < nc else np.zeros_like(A_[0])
        R = rescale(R, (nxt + D_[m]).astype(np.float32))
    return o[:L], R, n_ext
