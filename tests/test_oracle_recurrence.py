"""Pins for the fp64 oracle, independent of the oracle's own formulas.

Each test checks the oracle against something other than itself: dense
brute-force products of the per-token maps, closed forms, exact invariants of
the recurrence, and library routines.  A plausible slip in the oracle (a dropped
term, the wrong sign, decay and erase swapped, o read before the update, a
transposed state, the composition in the wrong order, a missing reset) fails at
least one of them.
"""
import numpy as np
import pytest
import torch

from oracle import kda_oracle as ko


def _rand_inputs(rng, T, H, K, V, unit_k=True, g_scale=1.0):
    q = rng.standard_normal((T, H, K))
    k = rng.standard_normal((T, H, K))
    if unit_k:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, V))
    g = -np.log1p(np.exp(rng.standard_normal((T, H, K)))) * g_scale
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    return q, k, v, g, beta


def _dense_map(k_t, g_t, b_t):
    """M_t = (I - beta k k^T) Diag(exp g) formed as a dense K x K matrix."""
    K = k_t.shape[0]
    return (np.eye(K) - b_t * np.outer(k_t, k_t)) @ np.diag(np.exp(g_t))


# ---------------------------------------------------------------- decoding

def test_decode_bf16_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x0001, 0x7F7F, 0x0000, 0x8000, 0x3E80], dtype=np.uint16)
    want = [1.0, -2.0, 2.0 ** -133, float.fromhex("0x1.fep127"), 0.0, -0.0, 0.25]
    got = ko.decode_bf16(bits)
    assert list(got) == want


def test_decode_bf16_matches_torch_widening():
    x = torch.randn(4096, dtype=torch.float32).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ko.decode_bf16(bits), x.to(torch.float64).numpy())


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("K,V", [(4, 3), (3, 5), (8, 8)])
def test_recurrence_matches_dense_maps(K, V):
    rng = np.random.default_rng(K * 10 + V)
    T, H = 11, 2
    q, k, v, g, beta = _rand_inputs(rng, T, H, K, V, unit_k=False)
    cu = np.array([0, 4, T])
    o, final = ko.recurrence(q, k, v, g, beta, cu)
    for h in range(H):
        for n in range(2):
            S = np.zeros((K, V))
            for t in range(cu[n], cu[n + 1]):
                S = _dense_map(k[t, h], g[t, h], beta[t, h]) @ S + beta[t, h] * np.outer(k[t, h], v[t, h])
                np.testing.assert_allclose(o[t, h], S.T @ q[t, h], rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(final[n, h], S, rtol=1e-12, atol=1e-13)


def test_transition_matches_dense_product():
    rng = np.random.default_rng(7)
    T, H, K, V = 10, 2, 5, 3
    q, k, v, g, beta = _rand_inputs(rng, T, H, K, V, g_scale=0.3)
    cu = np.array([0, T])
    bounds = [0, 3, 10]
    A = ko.segment_transitions(k, g, beta, cu, bounds)
    for h in range(H):
        np.testing.assert_array_equal(A[0, h], 0.0)  # segment 0 starts a sequence
        P = np.eye(K)
        for t in range(3, 10):
            P = _dense_map(k[t, h], g[t, h], beta[t, h]) @ P  # latest on the left
        np.testing.assert_allclose(A[1, h], P, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- closed forms

def test_scalar_closed_form():
    """K = V = 1: S_t = c S_{t-1} + beta v with c = (1 - beta k^2) e^g."""
    T = 9
    g0, b0 = -0.3, 0.25
    ones = np.ones((T, 1, 1))
    o, final = ko.recurrence(ones, ones, 2 * ones, g0 * ones, b0 * np.ones((T, 1)), [0, T])
    c = (1 - b0) * np.exp(g0)
    for t in range(T):
        want = b0 * 2 * (1 - c ** (t + 1)) / (1 - c)  # o_t reads the post-update state
        assert abs(o[t, 0, 0] - want) < 1e-14
    assert abs(final[0, 0, 0, 0] - b0 * 2 * (1 - c ** T) / (1 - c)) < 1e-14


def test_beta_zero_is_pure_decay():
    rng = np.random.default_rng(3)
    T, H, K, V = 12, 3, 6, 4
    q, k, v, g, _ = _rand_inputs(rng, T, H, K, V, g_scale=0.2)
    beta = np.zeros((T, H))
    h0 = rng.standard_normal((1, H, K, V))
    o, final = ko.recurrence(q, k, v, g, beta, [0, T], h0=h0)
    np.testing.assert_allclose(final[0], np.exp(g.sum(0))[:, :, None] * h0[0], rtol=1e-13)
    o0, f0 = ko.recurrence(q, k, v, g, beta, [0, T])
    assert not o0.any() and not f0.any()
    bounds = [0, 5, 12]
    A = ko.segment_transitions(k, g, beta, [0, T], bounds)
    B = ko.segment_updates(k, v, g, beta, [0, T], bounds)
    assert not B.any()
    for h in range(H):
        np.testing.assert_allclose(A[1, h], np.diag(np.exp(g[5:12, h].sum(0))), rtol=1e-13, atol=0)


def test_projection_with_basis_keys():
    """g = 0, beta = 1, k = e_i: step t overwrites row i of S with v_t."""
    T, K, V = 10, 5, 3
    rng = np.random.default_rng(11)
    idx = rng.integers(0, K, size=T)
    k = np.zeros((T, 1, K))
    k[np.arange(T), 0, idx] = 1.0
    v = rng.standard_normal((T, 1, V))
    g = np.zeros((T, 1, K))
    beta = np.ones((T, 1))
    qj = 2
    q = np.zeros((T, 1, K))
    q[:, 0, qj] = 1.0
    o, final = ko.recurrence(q, k, v, g, beta, [0, T])
    S = np.zeros((K, V))
    for t in range(T):
        S[idx[t]] = v[t, 0]
        np.testing.assert_array_equal(o[t, 0], S[qj])
    np.testing.assert_array_equal(final[0, 0], S)
    A = ko.segment_transitions(k, g, beta, [0, T], [0, 3, T])
    want = np.ones(K)
    want[np.unique(idx[3:])] = 0.0
    np.testing.assert_array_equal(A[1, 0], np.diag(want))


def test_projection_invariant_unit_keys():
    """g = 0, beta = 1, |k| = 1: the new state maps k_t to v_t exactly."""
    rng = np.random.default_rng(5)
    T, H, K, V = 8, 2, 6, 4
    q, k, v, _, _ = _rand_inputs(rng, T, H, K, V)
    g = np.zeros((T, H, K))
    beta = np.ones((T, H))
    S = np.zeros((H, K, V))
    for t in range(T):
        S, _ = ko.kda_step(S, q[t], k[t], v[t], g[t], beta[t])
        np.testing.assert_allclose(np.einsum("hk,hkv->hv", k[t], S), v[t], atol=1e-14)


# ---------------------------------------------------------------- invariants

def _random_case(seed, T=40, H=2, K=5, V=4, g_scale=0.1):
    rng = np.random.default_rng(seed)
    q, k, v, g, beta = _rand_inputs(rng, T, H, K, V, g_scale=g_scale)
    cuts = np.sort(rng.choice(np.arange(1, T), size=3, replace=False))
    cu = np.concatenate([[0], cuts, [T]])
    bcuts = np.sort(rng.choice(np.arange(1, T), size=4, replace=False))
    bounds = np.concatenate([[0], bcuts, [T]])
    return q, k, v, g, beta, cu, bounds


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_segmented_plus_composed_equals_monolithic(seed):
    q, k, v, g, beta, cu, bounds = _random_case(seed)
    o, final = ko.recurrence(q, k, v, g, beta, cu)
    A = ko.segment_transitions(k, g, beta, cu, bounds)
    B = ko.segment_updates(k, v, g, beta, cu, bounds)
    C, last = ko.compose(A, B)
    o2, final2 = ko.segmented_forward(q, k, v, g, beta, cu, bounds, C)
    np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(final2, final, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(last, final[-1], rtol=1e-12, atol=1e-13)
    # every carry-in equals the monolithic state just before the segment starts
    starts = set(int(x) for x in cu[:-1])
    for r in range(1, len(bounds) - 1):
        b = int(bounds[r])
        if b in starts:
            continue
        cu_prefix = np.array([int(x) for x in cu if x < b] + [b])  # truncate at token b
        _, state = ko.recurrence(q[:b], k[:b], v[:b], g[:b], beta[:b], cu_prefix)
        np.testing.assert_allclose(C[r], state[-1], rtol=1e-12, atol=1e-13)


def test_composition_is_associative():
    rng = np.random.default_rng(9)
    K, V = 6, 4
    s = [(rng.standard_normal((K, K)) * 0.5, rng.standard_normal((K, V))) for _ in range(3)]
    left = ko.compose_pair(ko.compose_pair(s[2], s[1]), s[0])
    right = ko.compose_pair(s[2], ko.compose_pair(s[1], s[0]))
    for a, b in zip(left, right):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)
    # and acting on a state equals applying the maps one after another
    S0 = rng.standard_normal((K, V))
    seq = S0
    for A, B in s:
        seq = A @ seq + B
    np.testing.assert_allclose(left[0] @ S0 + left[1], seq, rtol=1e-12, atol=1e-13)


def test_linearity_in_v():
    q, k, v, g, beta, cu, bounds = _random_case(4)
    o, f = ko.recurrence(q, k, v, g, beta, cu)
    o2, f2 = ko.recurrence(q, k, 2 * v, g, beta, cu)
    np.testing.assert_array_equal(o2, 2 * o)
    np.testing.assert_array_equal(f2, 2 * f)
    B = ko.segment_updates(k, v, g, beta, cu, bounds)
    B2 = ko.segment_updates(k, 2 * v, g, beta, cu, bounds)
    np.testing.assert_array_equal(B2, 2 * B)


def test_single_segment_update_is_monolithic_final():
    q, k, v, g, beta, cu, _ = _random_case(5)
    T = k.shape[0]
    _, final = ko.recurrence(q, k, v, g, beta, cu)
    B = ko.segment_updates(k, v, g, beta, cu, [0, T])
    np.testing.assert_allclose(B[0], final[-1], rtol=1e-13, atol=1e-14)
    A = ko.segment_transitions(k, g, beta, cu, [0, T])
    assert not A.any()


def test_transition_contracts():
    """g <= 0, beta in [0, 1], |k| = 1 make every per-token map a contraction."""
    rng = np.random.default_rng(12)
    T, H, K, V = 30, 2, 6, 3
    q, k, v, g, beta = _rand_inputs(rng, T, H, K, V, g_scale=0.05)
    A = ko.segment_transitions(k, g, beta, [0, T], [0, 1, T])
    for h in range(H):
        assert np.linalg.norm(A[1, h], 2) <= 1.0 + 1e-12


# ------------------------------------------------------ initial states h0

def test_h0_enters_through_the_dense_maps():
    """With h0, each sequence's o_t and final state gain exactly the image of
    h0[n] under the product of the dense per-token maps since the sequence
    start (the recurrence is affine in the state)."""
    rng = np.random.default_rng(21)
    T, H, K, V = 14, 2, 5, 3
    q, k, v, g, beta = _rand_inputs(rng, T, H, K, V, g_scale=0.3)
    cu = [0, 6, T]
    h0 = rng.standard_normal((2, H, K, V))
    o1, f1 = ko.recurrence(q, k, v, g, beta, cu, h0=h0)
    o0, f0 = ko.recurrence(q, k, v, g, beta, cu)
    for n in range(2):
        for h in range(H):
            M = np.eye(K)
            for t in range(cu[n], cu[n + 1]):
                M = _dense_map(k[t, h], g[t, h], beta[t, h]) @ M
                np.testing.assert_allclose(o1[t, h] - o0[t, h], (M @ h0[n, h]).T @ q[t, h],
                                           rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(f1[n, h] - f0[n, h], M @ h0[n, h], rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_segmented_plus_composed_equals_monolithic_with_h0(seed):
    q, k, v, g, beta, cu, bounds = _random_case(seed)
    N, H, K, V = len(cu) - 1, k.shape[1], k.shape[2], v.shape[2]
    h0 = np.random.default_rng(100 + seed).standard_normal((N, H, K, V))
    o, final = ko.recurrence(q, k, v, g, beta, cu, h0=h0)
    A = ko.segment_transitions(k, g, beta, cu, bounds)
    B = ko.segment_updates(k, v, g, beta, cu, bounds, h0=h0)
    C, last = ko.compose(A, B)
    o2, final2 = ko.segmented_forward(q, k, v, g, beta, cu, bounds, C, h0=h0)
    np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(final2, final, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(last, final[-1], rtol=1e-12, atol=1e-12)
    starts = set(int(x) for x in cu[:-1])
    for r in range(1, len(bounds) - 1):
        b = int(bounds[r])
        if b in starts:
            continue
        cu_prefix = np.array([int(x) for x in cu if x < b] + [b])
        _, state = ko.recurrence(q[:b], k[:b], v[:b], g[:b], beta[:b], cu_prefix, h0=h0)
        np.testing.assert_allclose(C[r], state[-1], rtol=1e-12, atol=1e-12)


def test_h0_pure_decay_update_closed_form():
    """beta = 0: a segment that holds a sequence start ends at that sequence's
    h0 decayed by the gates since the start; one without is zero."""
    rng = np.random.default_rng(22)
    T, H, K, V = 16, 2, 4, 3
    _, k, v, g, _ = _rand_inputs(rng, T, H, K, V, g_scale=0.2)
    beta = np.zeros((T, H))
    cu = [0, 7, T]
    h0 = rng.standard_normal((2, H, K, V))
    B = ko.segment_updates(k, v, g, beta, cu, [0, 5, 10, T], h0=h0)
    np.testing.assert_allclose(B[0], np.exp(g[0:5].sum(0))[:, :, None] * h0[0], rtol=1e-13)
    np.testing.assert_allclose(B[1], np.exp(g[7:10].sum(0))[:, :, None] * h0[1], rtol=1e-13)
    assert not B[2].any()


def test_linearity_in_v_and_h0():
    q, k, v, g, beta, cu, bounds = _random_case(6)
    N, H, K, V = len(cu) - 1, k.shape[1], k.shape[2], v.shape[2]
    h0 = np.random.default_rng(23).standard_normal((N, H, K, V))
    o, f = ko.recurrence(q, k, v, g, beta, cu, h0=h0)
    o2, f2 = ko.recurrence(q, k, 2 * v, g, beta, cu, h0=2 * h0)
    np.testing.assert_array_equal(o2, 2 * o)
    np.testing.assert_array_equal(f2, 2 * f)
    B = ko.segment_updates(k, v, g, beta, cu, bounds, h0=h0)
    B2 = ko.segment_updates(k, 2 * v, g, beta, cu, bounds, h0=2 * h0)
    np.testing.assert_array_equal(B2, 2 * B)


def test_safe_gate_pins():
    """The safe gate (a lower bound on g): a bound at or below every g changes
    nothing, a bound of 0 is exactly the recurrence with g = 0, and a bound in
    between replaces exactly the elements below it."""
    rng = np.random.default_rng(77)
    T, H, K, V = 20, 2, 8, 8
    q, k, v = (rng.standard_normal((T, H, d)) for d in (K, K, V))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    g = -rng.exponential(1.0, (T, H, K))
    beta = rng.uniform(0, 1, (T, H))
    cu = [0, 7, T]
    base = ko.recurrence(q, k, v, g, beta, cu)
    low = ko.safe_gate(g, g.min() - 1.0)
    np.testing.assert_array_equal(low, g)
    for got, want in zip(ko.recurrence(q, k, v, low, beta, cu), base):
        np.testing.assert_array_equal(got, want)
    zero = ko.safe_gate(g, 0.0)
    np.testing.assert_array_equal(zero, np.zeros_like(g))
    for got, want in zip(ko.recurrence(q, k, v, zero, beta, cu), ko.recurrence(q, k, v, np.zeros_like(g), beta, cu)):
        np.testing.assert_array_equal(got, want)
    mid = ko.safe_gate(g, -0.5)
    below = g < -0.5
    assert below.any() and (~below).any()
    np.testing.assert_array_equal(mid[below], -0.5)
    np.testing.assert_array_equal(mid[~below], g[~below])
    assert ko.safe_gate(g, None) is g
