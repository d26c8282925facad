"""GPU parity of plans with pieces (each segment cut into pieces that run in
parallel; the device calls fold the pieces' summaries into the segment's and
scan the pieces' carry-ins from the segment's): against the fp64 oracle at
the segment level, exactly as plain plans are checked, so the results must
not depend on the pieces.  Also the backward over pieces, head groups, and the
three small workloads at full size with the piece length bench.py uses.
"""
import numpy as np
import pytest
import torch

from gated_delta_rule_37_amd import kda, synth
import parity_utils as pu
from oracle import kda_oracle as ko

pytestmark = pytest.mark.gpu

CASES = [
    # name, T, H, cu_seqlens, segments, custom bounds, gate scale, piece tokens, initial states
    ("one_sequence_pieces_128", 1000, 2, [0, 1000], 2, None, 0.3, 128, False),
    ("one_sequence_pieces_32", 500, 2, [0, 500], 2, None, 0.05, 32, False),
    ("varlen_pieces_64", 555, 2, [0, 37, 150, 151, 300, 555], 3, None, 0.1, 64, False),
    ("varlen_pieces_64_h0", 555, 2, [0, 37, 150, 151, 300, 555], 3, None, 0.1, 64, True),
    ("custom_bounds_pieces", 700, 3, [0, 90, 700], 3, [0, 45, 400, 700], 0.05, 96, True),
    ("fast_decay_pieces", 640, 2, [0, 640], 2, None, 2.5, 128, False),
    ("slow_long_scans", 2048, 1, [0, 2048], 4, None, 0.005, 64, True),
    ("pieces_longer_than_segments", 300, 2, [0, 300], 3, None, 0.5, 512, False),
    ("short_sequences_pieces", 200, 2, [0, 3, 10, 11, 40, 64, 65, 98, 200], 2, None, 1.0, 32, True),
]


@pytest.mark.parametrize("name,T,H,cu,S,bounds,gs,L,with_h0", CASES, ids=[c[0] for c in CASES])
def test_pieces_parity(name, T, H, cu, S, bounds, gs, L, with_h0):
    print(f"case {name}: T={T} H={H} S={S} pieces of {L} cu={cu}", flush=True)
    x = synth.make_inputs(T, H, 128, 128, seed=len(name) + T, cu_seqlens=cu, gate_scale=gs)
    h0 = synth.initial_states(len(cu) - 1, H, 128, 128, seed=T + 7) if with_h0 else None
    plan, out = pu.run_gpu(x, cu, S, bounds, h0=h0, piece_tokens=L)
    print(f"  S={plan.S} P={plan.P} F={plan.F}", flush=True)
    ref = pu.run_oracle(x, cu, plan, h0=h0)
    pu.compare(pu.gpu_numpy(out), ref, name)


def test_pieces_head_groups_match_single_launch():
    """Head groups over a plan with pieces give bitwise the one-launch results."""
    T, H, cu = 900, 4, [0, 400, 900]
    x = synth.make_inputs(T, H, 128, 128, seed=77, cu_seqlens=cu, gate_scale=0.2)
    _, one = pu.run_gpu(x, cu, 3, piece_tokens=96)
    _, grp = pu.run_gpu(x, cu, 3, piece_tokens=96, groups=2)
    for key in ("o", "final_state", "transitions", "updates", "carry_in"):
        assert torch.equal(one[key], grp[key]), key


def test_pieces_backward_parity():
    """The backward over a plan with pieces (the pieces are its segments)."""
    T, H, cu = 700, 2, [0, 300, 301, 700]
    x = synth.make_inputs(T, H, 128, 128, seed=91, cu_seqlens=cu, gate_scale=0.2)
    N = len(cu) - 1
    gen = torch.Generator().manual_seed(92)
    d_o = torch.randn(T, H, 128, generator=gen)
    d_final = torch.randn(N, H, 128, 128, generator=gen)
    h0 = synth.initial_states(N, H, 128, 128, seed=93)
    plan = kda.Plan(cu, 2, None, 64)
    assert plan.P > plan.S
    d = pu.to_device(x)
    got = kda.backward(plan, d["q"], d["k"], d["v"], d["g"], d["beta"], d_o.cuda(), d_final=d_final.cuda(),
                       initial_state=h0.cuda(), want_dh0=True)
    torch.cuda.synchronize()
    f = pu.oracle_inputs(x)
    ref = ko.backward(f["q"], f["k"], f["v"], f["g"], f["beta"], cu, d_o.double().numpy(),
                      dfinal=d_final.double().numpy(), h0=h0.double().numpy())
    for key, want in zip(("dq", "dk", "dv", "dg", "dbeta", "dh0"), ref):
        have = got[key].double().cpu().numpy()
        assert np.isfinite(have).all(), key
        for h in range(H):
            scale = np.abs(want[:, h]).max()
            err = np.abs(have[:, h] - want[:, h]).max()
            assert err <= 1e-4 * scale, (key, h, err, scale)


SMALL_WORKLOADS = [("t1024_h4_s2", [0, 3]), ("t4096_h8_s4", [5]), ("t8192_h16_s4", [9])]


@pytest.mark.parametrize("name,heads", SMALL_WORKLOADS, ids=[c[0] for c in SMALL_WORKLOADS])
def test_small_workloads_with_bench_pieces(name, heads):
    w = synth.WORKLOADS[name]
    x = synth.workload_inputs(w)
    cu = x["cu_seqlens"].tolist()
    L = kda.auto_piece_tokens(cu, w.segments, w.H)
    print(f"workload {name}: pieces of {L} tokens, heads {heads}", flush=True)
    assert L > 0
    plan, out = pu.run_gpu(x, cu, w.segments, piece_tokens=L)
    got = pu.gpu_numpy(out, heads)
    del out
    ref = pu.run_oracle(x, cu, plan, heads)
    pu.compare(got, ref, name)
