"""Pins of the fp64 backward oracle (CPU only), none of which reuses its
reverse recurrence:

* central finite differences of the loss L = sum <o, do> + sum <final, dfinal>
  (computed by the forward oracle) for every gradient: q, k, v, g, beta, h0;
* an independent dense-map form of dv, dq and dh0: with the per-token maps
  M_t = (I - beta_t k_t k_t^T) Diag(exp g_t) multiplied out densely, the state
  is linear in each v_s and in h0;
* the following-summary structure of the pages' backward: the segmented
  reverse pass from the composed summaries D_r gives the monolithic gradients,
  and the summaries E_r do not depend on the forward state.
"""
import numpy as np
import pytest

from oracle import kda_oracle as ko


def _inputs(rng, T, H, K, V, gscale=1.0):
    q, k = (rng.standard_normal((T, H, K)) for _ in range(2))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, V))
    g = -gscale * np.log1p(np.exp(rng.standard_normal((T, H, K))))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    return q, k, v, g, beta


def _loss(q, k, v, g, beta, cu, do, dfinal, h0):
    o, fin = ko.recurrence(q, k, v, g, beta, cu, h0=h0)
    return float(np.sum(o * do) + np.sum(fin * dfinal))


@pytest.mark.parametrize("seed", [0, 1])
def test_backward_matches_central_differences(seed):
    rng = np.random.default_rng(100 + seed)
    T, H, K, V = 7, 1, 3, 3
    cu = [0, 3, 7]
    q, k, v, g, beta = _inputs(rng, T, H, K, V)
    h0 = rng.standard_normal((2, H, K, V))
    do = rng.standard_normal((T, H, V))
    dfinal = rng.standard_normal((2, H, K, V))
    grads = ko.backward(q, k, v, g, beta, cu, do, dfinal=dfinal, h0=h0)
    args = dict(q=q, k=k, v=v, g=g, beta=beta, h0=h0)
    eps = 1e-6
    for name, grad in zip(("q", "k", "v", "g", "beta", "h0"), grads):
        x = args[name]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            saved = x[idx]
            x[idx] = saved + eps
            lp = _loss(q, k, v, g, beta, cu, do, dfinal, h0)
            x[idx] = saved - eps
            lm = _loss(q, k, v, g, beta, cu, do, dfinal, h0)
            x[idx] = saved
            fd[idx] = (lp - lm) / (2 * eps)
        err = np.abs(fd - grad).max()
        assert err <= 1e-7 * max(1.0, np.abs(fd).max()), (name, err)


def _maps(k, g, beta):
    """Dense per-token maps M_t = (I - beta_t k_t k_t^T) Diag(exp g_t), [T, H, K, K]."""
    T, H, K = k.shape
    eye = np.eye(K)
    M = np.zeros((T, H, K, K))
    for t in range(T):
        for h in range(H):
            M[t, h] = (eye - beta[t, h] * np.outer(k[t, h], k[t, h])) @ np.diag(np.exp(g[t, h]))
    return M


def test_backward_dense_map_form():
    """dv_s = beta_s [ sum_{t>=s} (q_t^T Phi(t,s) k_s) do_t + (Phi(end,s) k_s)^T dfinal ],
    dh0 = sum_t Phi(t,start)^T q_t do_t^T + Phi(end,start)^T dfinal and
    dq_t = S_t do_t, with Phi(t,s) = M_t ... M_{s+1} multiplied out densely."""
    rng = np.random.default_rng(7)
    T, H, K, V = 9, 2, 4, 5
    cu = [0, 9]
    q, k, v, g, beta = _inputs(rng, T, H, K, V)
    h0 = rng.standard_normal((1, H, K, V))
    do = rng.standard_normal((T, H, V))
    dfinal = rng.standard_normal((1, H, K, V))
    dq, dk, dv, dg, dbeta, dh0 = ko.backward(q, k, v, g, beta, cu, do, dfinal=dfinal, h0=h0)
    M = _maps(k, g, beta)
    o, fin = ko.recurrence(q, k, v, g, beta, cu, h0=h0)
    for h in range(H):
        def phi(t, s):
            P = np.eye(K)
            for j in range(s + 1, t + 1):
                P = M[j, h] @ P
            return P
        want_dh0 = phi(T - 1, -1).T @ dfinal[0, h]
        for t in range(T):
            want_dh0 += np.outer(phi(t, -1).T @ q[t, h], do[t, h])
        np.testing.assert_allclose(dh0[0, h], want_dh0, rtol=1e-11, atol=1e-12)
        for s in range(T):
            want = (phi(T - 1, s) @ k[s, h]) @ dfinal[0, h]
            for t in range(s, T):
                want = want + (q[t, h] @ phi(t, s) @ k[s, h]) * do[t, h]
            np.testing.assert_allclose(dv[s, h], beta[s, h] * want, rtol=1e-11, atol=1e-12)
        # S_t from the dense maps, then dq_t = S_t do_t
        S = h0[0, h].copy()
        for t in range(T):
            S = M[t, h] @ S + beta[t, h] * np.outer(k[t, h], v[t, h])
            np.testing.assert_allclose(dq[t, h], S @ do[t, h], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(S, fin[0, h], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("case", [
    ([0, 40], [0, 10, 25, 40]),
    ([0, 7, 19, 20, 40], [0, 12, 20, 33, 40]),
    ([0, 5, 40], [0, 5, 6, 39, 40]),
])
def test_segmented_backward_equals_monolithic(case):
    """The pages' backward structure: per-segment following summaries E_r,
    the reverse compose D_{r-1} = A_r^T D_r + E_r and each segment's backward
    from D_r give the monolithic gradients."""
    cu, bounds = case
    rng = np.random.default_rng(len(bounds) * 13 + cu[1])
    T, H, K, V = cu[-1], 2, 4, 4
    q, k, v, g, beta = _inputs(rng, T, H, K, V, gscale=0.3)
    N = len(cu) - 1
    h0 = rng.standard_normal((N, H, K, V))
    do = rng.standard_normal((T, H, V))
    dfinal = rng.standard_normal((N, H, K, V))
    want = ko.backward(q, k, v, g, beta, cu, do, dfinal=dfinal, h0=h0)
    A = ko.segment_transitions(k, g, beta, cu, bounds)
    B = ko.segment_updates(k, v, g, beta, cu, bounds, h0=h0)
    C, _ = ko.compose(A, B)
    E = ko.backward_summaries(q, k, v, g, beta, cu, bounds, do, dfinal=dfinal)
    # the summaries depend on the cotangents only, not on the forward state
    E_c = ko.backward_summaries(q, k, v, g, beta, cu, bounds, do, dfinal=dfinal, C=C)
    np.testing.assert_allclose(E_c, E, rtol=1e-12, atol=1e-12)
    D = ko.compose_backward(A, E)
    assert not D[-1].any()
    got = ko.segmented_backward(q, k, v, g, beta, cu, bounds, do, D, C, dfinal=dfinal, h0=h0)
    for name, a, b in zip(("dq", "dk", "dv", "dg", "dbeta", "dh0"), got, want):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-11, err_msg=name)


def test_backward_linearity_and_zero_cotangents():
    """Zero cotangents give zero gradients; every gradient is linear in
    (do, dfinal) jointly."""
    rng = np.random.default_rng(11)
    T, H, K, V = 12, 1, 4, 4
    cu = [0, 5, 12]
    q, k, v, g, beta = _inputs(rng, T, H, K, V)
    zero = ko.backward(q, k, v, g, beta, cu, np.zeros((T, H, V)))
    assert all(not z.any() for z in zero)
    do = rng.standard_normal((T, H, V))
    df = rng.standard_normal((2, H, K, V))
    one = ko.backward(q, k, v, g, beta, cu, do, dfinal=df)
    two = ko.backward(q, k, v, g, beta, cu, 2 * do, dfinal=2 * df)
    for a, b in zip(one, two):
        np.testing.assert_allclose(b, 2 * a, rtol=1e-12, atol=1e-14)
