"""Helpers shared by the GPU parity tests: run the HIP path through the C-ABI
binding, run the fp64 oracle on the same bytes, and compare with the stated
tolerances.

Tolerances (written here, used by every parity test):
  * o: max |o_gpu - o_ref| <= 2e-3 over every compared element;
  * final states, segment updates B_r, carry-ins C_r: per (index, head) matrix
    max |X_gpu - X_ref| <= 1e-4 * max |X_ref|;
  * transitions A_r: max |A_gpu - A_ref| <= 1e-4 (scale 1: every per-token map
    is a contraction, so |A_ref| <= 1, and at fast decay A_ref underflows FP32);
    in addition, every A_r matrix with max |A_ref| >= 1e-3 must meet the state
    tolerance relative to its own scale (a stricter check where A is O(1)).
"""
from __future__ import annotations

import numpy as np
import torch

from gated_delta_rule_37_amd import kda, synth
from oracle import kda_oracle as ko

O_ATOL = 2e-3
STATE_RTOL = 1e-4
A_ATOL = 1e-4

NAMES = ("q", "k", "v", "g", "beta")


def to_device(x, dev="cuda:0"):
    return {n: x[n].to(dev) for n in NAMES}


def run_gpu(x, cu, S, bounds=None, dev="cuda:0", h0=None, gate_lower_bound=None, piece_tokens=0, groups=1):
    plan = kda.Plan(cu, S, bounds, piece_tokens)
    d = to_device(x, dev)
    init = None if h0 is None else h0.to(dev)
    out = kda.forward(plan, d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=init,
                      gate_lower_bound=gate_lower_bound, groups=groups)
    torch.cuda.synchronize()
    out.pop("workspace")   # an internal cache between the two passes, not an output
    return plan, out


def oracle_inputs(x, heads=None):
    """fp64 decode of the bf16 bytes, optionally restricted to some heads."""
    res = {}
    for n in NAMES:
        b = synth.bits(x[n])
        if heads is not None:
            b = b[:, heads]
        res[n] = ko.decode_bf16(b)
    return res


def run_oracle(x, cu, plan, heads=None, want_o=True, h0=None, gate_lower_bound=None):
    """fp64 reference; ``h0`` is the FP32 initial-state tensor the GPU got (or
    None); ``gate_lower_bound`` the safe gate's bound (or None)."""
    f = oracle_inputs(x, heads)
    f["g"] = ko.safe_gate(f["g"], gate_lower_bound)
    bounds = plan.bounds.tolist()
    init = None
    if h0 is not None:
        init = h0.double().numpy()
        if heads is not None:
            init = init[:, heads]
    ref = {}
    if want_o:
        ref["o"], ref["final"] = ko.recurrence(f["q"], f["k"], f["v"], f["g"], f["beta"], cu, h0=init)
    ref["A"] = ko.segment_transitions(f["k"], f["g"], f["beta"], cu, bounds)
    ref["B"] = ko.segment_updates(f["k"], f["v"], f["g"], f["beta"], cu, bounds, h0=init)
    ref["C"], _ = ko.compose(ref["A"], ref["B"])
    return ref


def gpu_numpy(out, heads=None):
    sel = slice(None) if heads is None else heads
    return dict(
        o=out["o"][:, sel].double().cpu().numpy(),
        final=out["final_state"][:, sel].double().cpu().numpy(),
        A=out["transitions"][:, sel].double().cpu().numpy(),
        B=out["updates"][:, sel].double().cpu().numpy(),
        C=out["carry_in"][:, sel].double().cpu().numpy(),
    )


def state_errors(got, ref, min_scale=0.0):
    """Worst per-matrix ratio max|err| / max|ref| over [idx, head] matrices
    (matrices whose scale is below ``min_scale`` are skipped)."""
    worst = 0.0
    for idx in range(ref.shape[0]):
        for h in range(ref.shape[1]):
            scale = float(np.abs(ref[idx, h]).max())
            err = float(np.abs(got[idx, h] - ref[idx, h]).max())
            if not np.isfinite(err):
                return float("inf")   # a NaN must not vanish in max()
            if min_scale > 0.0 and scale < min_scale:
                continue
            if scale == 0.0:
                if err != 0.0:
                    return float("inf")
                continue
            worst = max(worst, err / scale)
    return worst


def compare(got, ref, label=""):
    """Assert every tolerance; return the measured errors for reporting."""
    for key in ("o", "final", "A", "B", "C"):
        if key in got and (key != "o" or "o" in ref):
            assert np.isfinite(got[key]).all(), f"[{label}] non-finite values in {key}"
    errs = {}
    if "o" in ref:
        errs["o_abs"] = float(np.abs(got["o"] - ref["o"]).max())
        errs["final_rel"] = state_errors(got["final"], ref["final"])
    errs["A_abs"] = float(np.abs(got["A"] - ref["A"]).max())
    errs["A_rel"] = state_errors(got["A"], ref["A"], min_scale=1e-3)
    errs["A_max"] = float(np.abs(ref["A"]).max())
    errs["B_rel"] = state_errors(got["B"], ref["B"])
    errs["C_rel"] = state_errors(got["C"], ref["C"])
    print(f"[{label}] " + ", ".join(f"{k}={v:.3e}" for k, v in errs.items()), flush=True)
    if "o" in ref:
        assert errs["o_abs"] <= O_ATOL, errs
        assert errs["final_rel"] <= STATE_RTOL, errs
    assert errs["A_abs"] <= A_ATOL, errs
    assert errs["A_rel"] <= STATE_RTOL, errs
    assert errs["B_rel"] <= STATE_RTOL, errs
    assert errs["C_rel"] <= STATE_RTOL, errs
    return errs
