"""CPU checks of the chunked backward model (``chunk_bwd_model``) against the
fp64 oracle's per-token backward: every gradient (q, k, v, g, beta and the
start state) agrees to rounding for chunk lengths 1 to 32, ragged last
chunks, a start state and an end cotangent, beta = 0 tokens and a stretch of
strong decay."""
import numpy as np
import pytest

import chunk_bwd_model as cbm
from oracle import kda_oracle as ko


def _inputs(T, K, V, seed, gate_scale=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, K))
    k = rng.standard_normal((T, K))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, V))
    g = -gate_scale * np.log1p(np.exp(rng.standard_normal((T, K))))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(T)))
    do = rng.standard_normal((T, V))
    S0 = 0.5 * rng.standard_normal((K, V))
    dS = 0.5 * rng.standard_normal((K, V))
    return q, k, v, g, beta, do, S0, dS


def _oracle(q, k, v, g, beta, do, S0, dS):
    T = k.shape[0]
    out = ko.backward(q[:, None], k[:, None], v[:, None], g[:, None], beta[:, None], [0, T], do[:, None],
                      dfinal=dS[None, None], h0=S0[None, None])
    dq, dk, dv, dg, dbeta, dh0 = out
    return dq[:, 0], dk[:, 0], dv[:, 0], dg[:, 0], dbeta[:, 0], dh0[0, 0]


NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dS0")


def _check(got, ref, rtol=1e-9):
    for name, a, b in zip(NAMES, got, ref):
        scale = max(float(np.abs(b).max()), 1e-300)
        err = float(np.abs(a - b).max())
        assert err <= rtol * scale, (name, err, scale)


@pytest.mark.parametrize("T,C", [(1, 32), (7, 1), (37, 5), (64, 16), (70, 32), (33, 32)])
def test_chunk_backward_matches_oracle(T, C):
    x = _inputs(T, 16, 12, seed=T * 100 + C)
    _check(cbm.chunk_backward(*x, C=C), _oracle(*x))


def test_chunk_backward_beta_zero_tokens():
    """beta = 0 makes a token pure decay: its u is zero but dbeta is not."""
    q, k, v, g, beta, do, S0, dS = _inputs(40, 16, 16, seed=5)
    beta[[0, 7, 8, 31, 39]] = 0.0
    got = cbm.chunk_backward(q, k, v, g, beta, do, S0, dS, C=16)
    ref = _oracle(q, k, v, g, beta, do, S0, dS)
    _check(got, ref)
    assert np.abs(ref[4][[0, 7, 8, 31, 39]]).max() > 1e-3   # the pin is not vacuous


def test_chunk_backward_strong_decay_in_fp64_range():
    """Gates four times the pages' scale: exp(-G) stays inside fp64 here (a
    32-token chunk decays by up to ~250 nats per channel), so the model is
    exact; in FP32 these chunks would leave the exponent range."""
    x = _inputs(64, 16, 16, seed=11, gate_scale=4.0)
    _check(cbm.chunk_backward(*x, C=32), _oracle(*x), rtol=1e-7)


def test_chunk_backward_chunking_invariance():
    """The same gradients whatever the chunk length (the chunk form is exact)."""
    x = _inputs(48, 8, 8, seed=3)
    a = cbm.chunk_backward(*x, C=48)
    b = cbm.chunk_backward(*x, C=3)
    _check(a, b)


@pytest.mark.parametrize("T", [1, 15, 16, 32, 33, 70, 96, 131])
def test_anchored_three_pass_matches_oracle(T):
    """The anchored three-pass form (forward anchored states R_c, reverse
    anchored cotangents D_c, then every chunk's gradients on their own) gives
    the oracle's gradients, ragged last chunks and one-token fragments
    included."""
    x = _inputs(T, 16, 12, seed=700 + T)
    got, R, D = cbm.anchored_backward(*x, C=32)
    _check(got, _oracle(*x))


def test_anchored_three_pass_beta_zero_and_strong_gates():
    """beta = 0 tokens and gates three times the pages' scale (in-chunk decay
    well inside the anchored range in fp64)."""
    q, k, v, g, beta, do, S0, dS = _inputs(80, 16, 16, seed=21, gate_scale=3.0)
    beta[[0, 5, 31, 32, 79]] = 0.0
    got, _, _ = cbm.anchored_backward(q, k, v, g, beta, do, S0, dS, C=32)
    _check(got, _oracle(q, k, v, g, beta, do, S0, dS), rtol=1e-8)


def test_anchored_three_pass_zero_start_and_end():
    """No start state and no end cotangent (a fragment that starts its
    sequence and ends where nothing follows): dS0 still picks up every
    output's cotangent."""
    q, k, v, g, beta, do, S0, dS = _inputs(64, 8, 8, seed=4)
    S0[:] = 0.0
    dS[:] = 0.0
    got, _, _ = cbm.anchored_backward(q, k, v, g, beta, do, S0, dS, C=32)
    ref = _oracle(q, k, v, g, beta, do, S0, dS)
    _check(got, ref)
    assert np.abs(ref[5]).max() > 1e-3
