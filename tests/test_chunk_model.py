"""CPU checks of the chunked factorisation (``chunk_model``) against the fp64
oracle: the anchored chunk form with the exact per-token form for chunks whose
in-chunk decay leaves its range gives the recurrence's results, finite and
within the parity tolerances, for every finite g <= 0 (and g = -inf), while
the anchored form alone overflows on strong decay."""
import numpy as np
import pytest
import torch

import chunk_model as cm
import parity_utils as pu
from gated_delta_rule_37_amd import synth
from oracle import kda_oracle as ko

T_DEFAULT = 160


def _inputs(T, seed, gate_scale=1.0, edit=None):
    x = synth.make_inputs(T, 1, 128, 128, seed=seed, cu_seqlens=[0, T], gate_scale=gate_scale)
    if edit is not None:
        edit(x)
    return x


def _both(x, h0_scale=0.5, seed=0, robust=True):
    """(model, oracle) results for one sequence from a random initial state:
    o, final state and the transition from the identity."""
    T = x["k"].shape[0]
    f = pu.oracle_inputs(x)
    f32 = {n: f[n][:, 0].astype(np.float32) for n in f}
    h0 = (h0_scale * np.random.default_rng(seed).standard_normal((128, 128))).astype(np.float32)
    o, S, n_ext = cm.run_fragment(f32["k"], f32["v"], f32["q"], f32["g"], f32["beta"], h0, robust=robust)
    _, Phi, _ = cm.run_fragment(f32["k"], np.zeros_like(f32["v"]), f32["q"], f32["g"], f32["beta"],
                                np.eye(128, dtype=np.float32), robust=robust, want_o=False)
    o_ref, fin_ref = ko.recurrence(f["q"], f["k"], f["v"], f["g"], f["beta"], [0, T],
                                   h0=h0.astype(np.float64)[None, None])
    return dict(o=o, S=S, A=Phi, n_ext=n_ext), dict(o=o_ref[:, 0], S=fin_ref[0, 0], A=_transition(f))


def _transition(f):
    """The oracle's product of the per-token maps of the whole input, with no
    reset: the input is the second segment of a sequence whose first token is
    the identity map (g = 0, beta = 0)."""
    T = f["k"].shape[0]
    pad = {n: np.concatenate([np.zeros_like(f[n][:1]), f[n]], 0) for n in f}
    return ko.segment_transitions(pad["k"], pad["g"], pad["beta"], [0, T + 1], [0, 1, T + 1])[1, 0]


def _check(got, ref, label):
    assert np.isfinite(got["o"]).all() and np.isfinite(got["S"]).all() and np.isfinite(got["A"]).all(), label
    o_err = float(np.abs(got["o"] - ref["o"]).max())
    s_scale = float(np.abs(ref["S"]).max())
    s_err = float(np.abs(got["S"] - ref["S"]).max())
    a_err = float(np.abs(got["A"] - ref["A"]).max())
    print(f"[{label}] extreme chunks {got['n_ext']}, o {o_err:.2e}, S {s_err / max(s_scale, 1e-300):.2e} rel, "
          f"A {a_err:.2e} abs", flush=True)
    assert o_err <= pu.O_ATOL, label
    assert s_err <= pu.STATE_RTOL * s_scale or (s_scale == 0.0 and s_err == 0.0), label
    assert a_err <= pu.A_ATOL, label
    a_scale = float(np.abs(ref["A"]).max())
    if a_scale >= 1e-3:
        assert a_err <= pu.STATE_RTOL * a_scale, label


@pytest.mark.parametrize("gs", [1.0, 2.5, 4.0, 8.0, 30.0])
def test_gate_scales(gs):
    x = _inputs(T_DEFAULT, seed=int(gs * 10), gate_scale=gs)
    got, ref = _both(x)
    _check(got, ref, f"gate x{gs}")
    if gs >= 8.0:
        assert got["n_ext"] > 0


def test_anchored_form_alone_overflows_on_strong_decay():
    """Without the per-token form the anchored factors overflow: non-finite
    results (what the extreme-chunk path is for)."""
    x = _inputs(T_DEFAULT, seed=80, gate_scale=8.0)
    f = pu.oracle_inputs(x)
    f32 = {n: f[n][:, 0].astype(np.float32) for n in f}
    with np.errstate(all="ignore"):
        o, S, _ = cm.run_fragment(f32["k"], f32["v"], f32["q"], f32["g"], f32["beta"],
                                  np.eye(128, dtype=np.float32), robust=False)
    assert not (np.isfinite(o).all() and np.isfinite(S).all())


def _channels(vals):
    def edit(x):
        g = x["g"].float()
        for c, val in vals:
            g[:, :, c] = val
        x["g"] = g.to(torch.bfloat16)
    return edit


@pytest.mark.parametrize("vals", [[(3, -20.0)], [(3, -20.0), (77, -60.0)], [(5, -60.0), (6, -1e4)]],
                         ids=["one_channel_-20", "channels_-20_-60", "channels_-60_-1e4"])
def test_strong_channels(vals):
    x = _inputs(T_DEFAULT, seed=3, edit=_channels(vals))
    got, ref = _both(x)
    _check(got, ref, str(vals))


@pytest.mark.parametrize("val", [-200.0, float("-inf")])
def test_whole_chunks_forget(val):
    """Tokens 40..100 forget everything on every channel (exp(g) is 0 in
    FP32, or exactly 0 for -inf)."""
    def edit(x):
        g = x["g"].float()
        g[40:101] = val
        x["g"] = g.to(torch.bfloat16)
    x = _inputs(T_DEFAULT, seed=4, edit=edit)
    got, ref = _both(x)
    _check(got, ref, f"forget {val}")
    assert got["n_ext"] > 0


def test_pure_forgetting_beta_zero():
    """beta = 0 and strong decay: the state only decays; the final state is
    Diag(exp sum g) h0 and o = S^T q, both against the oracle, including an
    FP32-representable tiny state."""
    def edit(x):
        x["beta"] = torch.zeros_like(x["beta"])
        g = x["g"].float() * 0.0
        g[10:12, :, :64] = -30.0      # 60 nats on half the channels
        x["g"] = g.to(torch.bfloat16)
    x = _inputs(96, seed=5, edit=edit)
    got, ref = _both(x, h0_scale=1.0)
    _check(got, ref, "pure forgetting")
    want = np.zeros(128)
    want[64:] = 1.0
    want[:64] = np.exp(-60.0)
    assert np.allclose(ref["A"], np.diag(want), rtol=1e-12, atol=0)
