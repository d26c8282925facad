"""fp64 reference for the segmented KDA forward pass (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this module.  It is deliberately slow and literal: one token at
a time, no chunking, no blocking, no reordering beyond what the definitions
below state.  See ``oracle/__init__.py`` for the page citations.

Arrays (numpy, float64 after decoding):
    q, k, g : [T, H, K]      packed-THD, tokens of all sequences back to back
    v       : [T, H, V]
    beta    : [T, H]
    cu_seqlens : [N+1] int   sequence n owns tokens cu_seqlens[n] .. cu_seqlens[n+1]-1
State matrices are [H, K, V] (K-major, "non-transposed").
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "decode_bf16",
    "kda_step",
    "recurrence",
    "segment_updates",
    "segment_transitions",
    "compose",
    "compose_pair",
    "segmented_forward",
    "safe_gate",
    "backward",
    "backward_summaries",
    "compose_backward",
    "segmented_backward",
]


def decode_bf16(bits) -> np.ndarray:
    """BF16 bit patterns (uint16 / int16 array) -> exact float64 values.

    The device receives the same bytes ([cuLA#110] Supported configuration:
    BF16 KDA inputs), so the oracle decodes them bit for bit: a bfloat16 is the
    top half of an IEEE binary32, which float64 holds exactly.
    """
    b = np.ascontiguousarray(np.asarray(bits).view(np.uint16)).astype(np.uint32)
    return (b << np.uint32(16)).view(np.float32).astype(np.float64)


def safe_gate(g, lower_bound=None):
    """The optional safe gate: the log-decays the recurrence runs on.

    [cuLA#136] Summary by CodeRabbit names "optional safe-gate parameters" and
    defines nothing more.  The reading taken here is a lower bound on each
    per-step, per-channel log-decay: g <- max(g, lower_bound) elementwise
    (a decay factor exp(g) never below exp(lower_bound)); ``None`` leaves g
    as given.
    """
    if lower_bound is None:
        return g
    return np.maximum(g, float(lower_bound))


def kda_step(S, q_t, k_t, v_t, g_t, beta_t):
    """One token of the gated delta rule for all heads at once.

    S: [H, K, V]; q_t, k_t, g_t: [H, K]; v_t: [H, V]; beta_t: [H].
    Order of operations (the reading of the recurrence's factor order):
      1. decay      S <- Diag(exp g_t) S                (per key channel)
      2. erase      S <- S - beta_t k_t (k_t^T S)
      3. write      S <- S + beta_t k_t v_t^T
      4. read       o_t = S^T q_t                       (post-update state)
    Returns (S_new, o_t [H, V]).
    """
    S = np.exp(g_t)[:, :, None] * S
    kS = np.einsum("hk,hkv->hv", k_t, S)
    bk = beta_t[:, None] * k_t
    S = S - bk[:, :, None] * kS[:, None, :]
    S = S + bk[:, :, None] * v_t[:, None, :]
    o_t = np.einsum("hk,hkv->hv", q_t, S)
    return S, o_t


def _seq_starts(cu_seqlens, T):
    starts = np.zeros(T + 1, dtype=bool)
    for n in range(len(cu_seqlens) - 1):
        starts[int(cu_seqlens[n])] = True
    return starts


def _start_state(cu_seqlens, t, h0, shape):
    """The state a sequence starting at token t begins from: zero, or h0[n]."""
    if h0 is None:
        return np.zeros(shape)
    n = [int(c) for c in cu_seqlens].index(t)
    return np.array(h0[n], dtype=np.float64)


def recurrence(q, k, v, g, beta, cu_seqlens, h0=None):
    """Monolithic recurrence over every packed sequence.

    Each sequence starts from a zero state (the configurations state no initial
    state), or from ``h0[n]`` ([N, H, K, V]) when given.  Returns
    ``(o [T, H, V], final [N, H, K, V])`` where ``final[n]`` is the state after
    the sequence's last token.
    """
    T, H, K = k.shape
    V = v.shape[2]
    N = len(cu_seqlens) - 1
    o = np.zeros((T, H, V))
    final = np.zeros((N, H, K, V))
    for n in range(N):
        bos, eos = int(cu_seqlens[n]), int(cu_seqlens[n + 1])
        S = np.zeros((H, K, V)) if h0 is None else np.array(h0[n], dtype=np.float64)
        for t in range(bos, eos):
            S, o[t] = kda_step(S, q[t], k[t], v[t], g[t], beta[t])
        final[n] = S
    return o, final


def segment_updates(k, v, g, beta, cu_seqlens, bounds, h0=None):
    """B_r: the state at the end of segment r when the segment starts from zero.

    [cuLA#136] Summary names the pair preceding_state_update /
    preceding_transition; the update is the affine map's constant term, i.e.
    the segment run from a zero state, with the state reset at every sequence
    start inside the segment to that sequence's initial state (zero, or
    ``h0[n]`` when given: the reset is an affine map whose constant term is the
    initial state).  Returns [R, H, K, V].
    """
    T, H, K = k.shape
    V = v.shape[2]
    starts = _seq_starts(cu_seqlens, T)
    R = len(bounds) - 1
    B = np.zeros((R, H, K, V))
    zeros_q = np.zeros((H, K))
    for r in range(R):
        S = np.zeros((H, K, V))
        for t in range(int(bounds[r]), int(bounds[r + 1])):
            if starts[t]:
                S = _start_state(cu_seqlens, t, h0, (H, K, V))
            S, _ = kda_step(S, zeros_q, k[t], v[t], g[t], beta[t])
        B[r] = S
    return B


def segment_transitions(k, g, beta, cu_seqlens, bounds):
    """A_r: the K x K linear part of segment r's affine map.

    The product of the per-token maps M_t = (I - beta_t k_t k_t^T) Diag(exp g_t),
    latest on the left, so that S_out = A_r S_in + B_r.  A sequence start inside
    the segment (or at its first token) resets the state, whose linear part is
    the zero map, so the running product becomes 0 there.
    Returns [R, H, K, K].
    """
    T, H, K = k.shape
    starts = _seq_starts(cu_seqlens, T)
    R = len(bounds) - 1
    A = np.zeros((R, H, K, K))
    for r in range(R):
        Phi = np.broadcast_to(np.eye(K), (H, K, K)).copy()
        for t in range(int(bounds[r]), int(bounds[r + 1])):
            if starts[t]:
                Phi = np.zeros((H, K, K))
            Phi = np.exp(g[t])[:, :, None] * Phi
            kPhi = np.einsum("hk,hkj->hj", k[t], Phi)
            Phi = Phi - (beta[t][:, None] * k[t])[:, :, None] * kPhi[:, None, :]
        A[r] = Phi
    return A


def compose_pair(second, first):
    """Affine composition (A2, B2) o (A1, B1) = (A2 A1, A2 B1 + B2).

    Applying ``first`` and then ``second`` to a state S gives
    A2 (A1 S + B1) + B2.  [cuLA#136] Summary: affine summary composition.
    """
    A2, B2 = second
    A1, B1 = first
    return A2 @ A1, A2 @ B1 + B2


def compose(A, B):
    """Ordered scan of the segment summaries into carry-in states.

    C_0 = 0 and C_{r+1} = A_r C_r + B_r; C_r is the state entering segment r
    ([cuLA#136] Summary: preceding_state_update / preceding_transition and
    their composition; [cuLA#110] Motivation: assembling the state from every
    predecessor).  Returns C [R, H, K, V]; also returns the state after the last
    segment as the second value.
    """
    R = A.shape[0]
    C = np.zeros_like(B)
    cur = np.zeros_like(B[0])
    for r in range(R):
        C[r] = cur
        cur = A[r] @ cur + B[r]
    return C, cur


def segmented_forward(q, k, v, g, beta, cu_seqlens, bounds, C, h0=None):
    """Re-run each segment from its carry-in C_r (reset at sequence starts to
    zero, or to ``h0[n]`` when given).

    This is the segmented execution the pages' context-parallel forward
    performs once every rank has its predecessors' summaries ([cuLA#136]
    Sequence Diagram).  Returns (o, final) like :func:`recurrence`.
    """
    T, H, K = k.shape
    V = v.shape[2]
    N = len(cu_seqlens) - 1
    starts = _seq_starts(cu_seqlens, T)
    ends = {int(cu_seqlens[n + 1]) - 1: n for n in range(N)}
    o = np.zeros((T, H, V))
    final = np.zeros((N, H, K, V))
    for r in range(len(bounds) - 1):
        S = np.array(C[r], dtype=np.float64)
        for t in range(int(bounds[r]), int(bounds[r + 1])):
            if starts[t]:
                S = _start_state(cu_seqlens, t, h0, (H, K, V))
            S, o[t] = kda_step(S, q[t], k[t], v[t], g[t], beta[t])
            if t in ends:
                final[ends[t]] = S
    return o, final


# ----------------------------------------------------------------- backward
#
# The pages validate the forward and the gradients of q, k, v, g and beta
# together ([cuLA#110] Correctness; [cuLA#136] Sequence Diagram: the backward
# gathers the following ranks' summaries).  The loss is the pairing of the
# forward's outputs with given cotangents,
#     L = sum_t <o_t, do_t> + sum_n <final_n, dfinal_n>,
# and the gradients are those of the recurrence as the forward defines it
# (one token: decay, erase, write, read).


def _step_parts(S_prev, k_t, v_t, g_t, beta_t):
    """The intermediate values of one token (all heads): decayed state
    S~ = Diag(exp g) S_prev, p = S~^T k, u = beta (v - p), S = S~ + k u^T."""
    St = np.exp(g_t)[:, :, None] * S_prev
    p = np.einsum("hk,hkv->hv", k_t, St)
    u = beta_t[:, None] * (v_t - p)
    S = St + k_t[:, :, None] * u[:, None, :]
    return St, p, u, S


def _token_backward(dS, S_prev, q_t, k_t, v_t, g_t, beta_t, do_t):
    """Reverse one token.  dS is dL/dS_t from the later tokens; returns
    (dL/dS_{t-1}, dq_t, dk_t, dv_t, dg_t, dbeta_t), each the chain rule through
    o_t = S_t^T q_t, S_t = S~ + k u^T, u = beta (v - S~^T k), S~ = e^g o S_prev."""
    St, p, u, S = _step_parts(S_prev, k_t, v_t, g_t, beta_t)
    dS = dS + q_t[:, :, None] * do_t[:, None, :]                  # o_t = S_t^T q_t
    dq = np.einsum("hkv,hv->hk", S, do_t)
    du = np.einsum("hkv,hk->hv", dS, k_t)                          # S_t = S~ + k u^T
    dk = np.einsum("hkv,hv->hk", dS, u)
    dbeta = np.sum(du * (v_t - p), axis=-1)                        # u = beta (v - p)
    dv = beta_t[:, None] * du
    dp = -beta_t[:, None] * du
    dSt = dS + k_t[:, :, None] * dp[:, None, :]                    # p = S~^T k
    dk = dk + np.einsum("hkv,hv->hk", St, dp)
    dg = np.sum(dSt * St, axis=-1)                                 # S~ = e^g o S_prev
    dS_prev = np.exp(g_t)[:, :, None] * dSt
    return dS_prev, dq, dk, dv, dg, dbeta


def backward(q, k, v, g, beta, cu_seqlens, do, dfinal=None, h0=None):
    """Gradients of L = sum <o, do> + sum <final, dfinal> for the monolithic
    recurrence: one reverse pass per sequence over its forward states.

    do: [T, H, V]; dfinal: [N, H, K, V] or None (zero); h0 as in recurrence.
    Returns (dq, dk, dv, dg, dbeta, dh0) with the shapes of q, k, v, g, beta
    and [N, H, K, V]."""
    T, H, K = k.shape
    V = v.shape[2]
    N = len(cu_seqlens) - 1
    dq, dk, dg = (np.zeros((T, H, K)) for _ in range(3))
    dv = np.zeros((T, H, V))
    dbeta = np.zeros((T, H))
    dh0 = np.zeros((N, H, K, V))
    for n in range(N):
        bos, eos = int(cu_seqlens[n]), int(cu_seqlens[n + 1])
        S = np.zeros((H, K, V)) if h0 is None else np.array(h0[n], dtype=np.float64)
        prev = []
        for t in range(bos, eos):
            prev.append(S)
            S = _step_parts(S, k[t], v[t], g[t], beta[t])[3]
        dS = np.zeros((H, K, V)) if dfinal is None else np.array(dfinal[n], dtype=np.float64)
        for t in range(eos - 1, bos - 1, -1):
            dS, dq[t], dk[t], dv[t], dg[t], dbeta[t] = _token_backward(
                dS, prev[t - bos], q[t], k[t], v[t], g[t], beta[t], do[t])
        dh0[n] = dS
    return dq, dk, dv, dg, dbeta, dh0


def backward_summaries(q, k, v, g, beta, cu_seqlens, bounds, do, dfinal=None, h0=None, C=None):
    """The following summaries of the backward ([cuLA#136] Sequence Diagram:
    the backward gathers the following ranks' summaries).  A segment maps the
    gradient at its end, D (dL/dS at its last token, from the later tokens),
    to the gradient at its start affinely: dL/dS_in = A_r^T D + E_r, with A_r
    the segment's transition (forward) and E_r the gradient at its start from
    its own outputs alone (D = 0).  E_r is taken over the segment's first
    fragment, which starts from the carry-in C_r (the forward's state there;
    zero for C=None); a sequence start inside the segment resets the state,
    so gradients there do not reach S_in.  Returns E [R, H, K, V]."""
    T, H, K = k.shape
    V = v.shape[2]
    starts = _seq_starts(cu_seqlens, T)
    ends = {int(cu_seqlens[n + 1]) - 1: n for n in range(len(cu_seqlens) - 1)}
    R = len(bounds) - 1
    E = np.zeros((R, H, K, V))
    for r in range(R):
        b0, b1 = int(bounds[r]), int(bounds[r + 1])
        if starts[b0]:
            continue
        # the first fragment: tokens b0 .. up to (not incl.) the next sequence start
        f1 = b0 + 1
        while f1 < b1 and not starts[f1]:
            f1 += 1
        S = np.zeros((H, K, V)) if C is None else np.array(C[r], dtype=np.float64)
        prev = []
        for t in range(b0, f1):
            prev.append(S)
            S = _step_parts(S, k[t], v[t], g[t], beta[t])[3]
        dS = np.zeros((H, K, V))
        if f1 - 1 in ends and dfinal is not None:
            dS = np.array(dfinal[ends[f1 - 1]], dtype=np.float64)
        for t in range(f1 - 1, b0 - 1, -1):
            dS = _token_backward(dS, prev[t - b0], q[t], k[t], v[t], g[t], beta[t], do[t])[0]
        E[r] = dS
    return E


def compose_backward(A, E):
    """Reverse ordered scan of the backward summaries: D_{R-1} = 0 and
    D_{r-1} = A_r^T D_r + E_r, the gradient at the end of segment r-1 from
    every later token.  Returns D [R, H, K, V]."""
    R = A.shape[0]
    D = np.zeros_like(E)
    for r in range(R - 1, 0, -1):
        D[r - 1] = np.swapaxes(A[r], -1, -2) @ D[r] + E[r]
    return D


def segmented_backward(q, k, v, g, beta, cu_seqlens, bounds, do, D, C, dfinal=None, h0=None):
    """Each segment's backward from D_r at its end and its forward from the
    carry-in C_r (sequence starts reset to zero or h0[n]); the gradients that
    reach a sequence's start go to dh0.  Returns what backward() returns."""
    T, H, K = k.shape
    V = v.shape[2]
    N = len(cu_seqlens) - 1
    starts = _seq_starts(cu_seqlens, T)
    ends = {int(cu_seqlens[n + 1]) - 1: n for n in range(N)}
    first = {int(cu_seqlens[n]): n for n in range(N)}
    dq, dk, dg = (np.zeros((T, H, K)) for _ in range(3))
    dv = np.zeros((T, H, V))
    dbeta = np.zeros((T, H))
    dh0 = np.zeros((N, H, K, V))
    for r in range(len(bounds) - 1):
        b0, b1 = int(bounds[r]), int(bounds[r + 1])
        S = np.array(C[r], dtype=np.float64)
        prev = []
        for t in range(b0, b1):
            if starts[t]:
                S = _start_state(cu_seqlens, t, h0, (H, K, V))
            prev.append(S)
            S = _step_parts(S, k[t], v[t], g[t], beta[t])[3]
        dS = np.array(D[r], dtype=np.float64)
        for t in range(b1 - 1, b0 - 1, -1):
            if t in ends and dfinal is not None:
                dS = dS + dfinal[ends[t]]
            dS, dq[t], dk[t], dv[t], dg[t], dbeta[t] = _token_backward(
                dS, prev[t - b0], q[t], k[t], v[t], g[t], beta[t], do[t])
            if starts[t]:
                dh0[first[t]] = dS
                dS = np.zeros((H, K, V))
    return dq, dk, dv, dg, dbeta, dh0
