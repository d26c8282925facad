"""GPU parity at the measured workloads' full sizes, in the launch configuration
bench.py times.  The GPU runs every head; the fp64 oracle recomputes sampled
heads over every token (o, final states, transitions, updates, carry-ins).
"""
import numpy as np
import pytest
import torch

from gated_delta_rule_37_amd import kda, synth
import parity_utils as pu

pytestmark = pytest.mark.gpu

CASES = [
    ("t1024_h4_s2", [0, 1, 2, 3]),
    ("t4096_h8_s4", [0, 3, 7]),
    ("t8192_h16_s4", [0, 11, 15]),
    ("varlen32k_h32_s8", [5, 31]),
    ("t65536_h32_s64", [0, 31]),
    ("t4096_h8_s4_slow", [2]),
    ("t65536_h32_s64_slow", [30]),
    ("t65536_h32_s64_longmem", [12]),
]


@pytest.mark.parametrize("name,heads", CASES, ids=[c[0] for c in CASES])
def test_workload_sampled_heads(name, heads):
    w = synth.WORKLOADS.get(name) or synth.STRESS[name]
    print(f"workload {name}: T={w.T} H={w.H} S={w.segments} heads={heads}", flush=True)
    x = synth.workload_inputs(w)
    cu = x["cu_seqlens"].tolist()
    # the largest decay over any 16 consecutive tokens (log2 units) bounds the
    # anchored chunk form's factor exponents whatever the chunk alignment: far
    # below its 96, so no fragment of the workload is re-run token by token
    c = torch.cumsum(x["g"].float() * 1.4426950408889634, 0)
    win = float((c[15:] - torch.cat([torch.zeros_like(c[:1]), c[:-16]], 0)).min())
    print(f"  largest 16-token decay {-win:.1f} log2 units", flush=True)
    assert -win < 60.0
    del c
    plan, out = pu.run_gpu(x, cu, w.segments)
    got = pu.gpu_numpy(out, heads)
    del out
    torch.cuda.empty_cache()
    ref = pu.run_oracle(x, cu, plan, heads)
    errs = pu.compare(got, ref, name)
    if w.gate_scale < 1.0:
        # slow decay: the transitions stay representable in FP32 (the delta-rule
        # erasure alone shrinks a 1024-token product to about 1e-5) and the
        # carries are large, so the composition is exercised for real
        assert np.abs(ref["A"][1:]).max() > 1e-7
        assert np.abs(ref["C"][1:]).max() > 1e-2
    if w.beta_scale < 1.0:
        # long memory: every transition is O(1), so each of the 63 compose
        # steps moves the carry by a full product (checked to the relative
        # tolerance on every A_r by compare())
        assert min(np.abs(ref["A"][r]).max() for r in range(1, w.segments)) > 0.1
    assert errs["o_abs"] <= pu.O_ATOL


def test_workload_with_initial_states():
    """The varlen workload at full size with an initial state for every
    sequence (sampled heads, every token)."""
    name, heads = "varlen32k_h32_s8", [9]
    w = synth.WORKLOADS[name]
    x = synth.workload_inputs(w)
    cu = x["cu_seqlens"].tolist()
    h0 = synth.initial_states(len(cu) - 1, w.H, 128, 128, seed=31)
    print(f"workload {name} with initial states: N={len(cu) - 1} heads={heads}", flush=True)
    plan, out = pu.run_gpu(x, cu, w.segments, h0=h0)
    got = pu.gpu_numpy(out, heads)
    del out
    torch.cuda.empty_cache()
    pu.compare(got, pu.run_oracle(x, cu, plan, heads, h0=h0), name + "+h0")


def test_bench_workload_bf16_output():
    """At the bench workload's full size, the BF16 o is the FP32 run's o
    rounded to nearest even, bit for bit (every element)."""
    w = synth.WORKLOADS["t65536_h32_s64"]
    x = synth.workload_inputs(w)
    cu = x["cu_seqlens"].tolist()
    print(f"workload {w.name} bf16 o", flush=True)
    plan = kda.Plan(cu, w.segments)
    d = pu.to_device(x)
    o32 = kda.forward(plan, d["q"], d["k"], d["v"], d["g"], d["beta"])["o"]
    o16 = kda.forward(plan, d["q"], d["k"], d["v"], d["g"], d["beta"], o_dtype=torch.bfloat16)["o"]
    torch.cuda.synchronize()
    assert torch.equal(o16, o32.to(torch.bfloat16))


@pytest.mark.parametrize("name,pieces", [("t65536_h32_s64", False), ("t8192_h16_s4", True)])
def test_full_size_forward_bitwise_deterministic(name, pieces):
    """Three launches of the whole forward at full size, in bench.py's
    configuration, give bitwise the same outputs (every MFMA result that a
    later instruction reads must have landed: a missing hazard wait shows up
    here as launch-to-launch differences)."""
    w = synth.WORKLOADS[name]
    x = synth.workload_inputs(w)
    cu = x["cu_seqlens"].tolist()
    L = kda.auto_piece_tokens(cu, w.segments, w.H) if pieces else 0
    plan = kda.Plan(cu, w.segments, None, L)
    d = pu.to_device(x)
    first = kda.forward(plan, d["q"], d["k"], d["v"], d["g"], d["beta"])
    for _ in range(2):
        again = kda.forward(plan, d["q"], d["k"], d["v"], d["g"], d["beta"])
        torch.cuda.synchronize()
        for key in ("o", "final_state", "transitions", "updates", "carry_in"):
            assert torch.equal(again[key], first[key]), key
        del again


def test_full_size_backward_bitwise_deterministic():
    """Two backward calls on the bench workload give bitwise the same
    gradients."""
    w = synth.WORKLOADS["t65536_h32_s64"]
    x = synth.workload_inputs(w)
    plan = kda.Plan([0, w.T], w.segments)
    d = pu.to_device(x)
    d_o = torch.randn(w.T, w.H, w.V, generator=torch.Generator().manual_seed(7)).cuda()
    a = kda.backward(plan, d["q"], d["k"], d["v"], d["g"], d["beta"], d_o)
    b = kda.backward(plan, d["q"], d["k"], d["v"], d["g"], d["beta"], d_o)
    torch.cuda.synchronize()
    for key in ("dq", "dk", "dv", "dg", "dbeta"):
        assert torch.equal(a[key], b[key]), key
