"""GPU parity of the backward (kda_backward through the C-ABI) against the
fp64 oracle's backward on the same bytes: gradients of q, k, v, g, beta and
the initial states for L = sum <o, d_o> + sum <final, d_final>, with one
segment and with several (segments run in parallel through the backward
summaries and their reverse compose; the result must not depend on S).

Tolerance (written here): every gradient tensor, per head,
max |grad_gpu - grad_ref| <= 1e-4 * max |grad_ref| -- the relative bound the
forward's states meet, for FP32 arithmetic on inputs of O(1).
"""
import numpy as np
import pytest
import torch

from gated_delta_rule_37_amd import kda, synth
import parity_utils as pu
from oracle import kda_oracle as ko

pytestmark = pytest.mark.gpu

GRAD_RTOL = 1e-4

CASES = [
    # name, T, H, cu_seqlens, segments, gate scale, initial states + d_final
    ("one_sequence_ragged", 70, 2, [0, 70], 1, 1.0, False),
    ("varlen_h0_dfinal", 300, 2, [0, 37, 150, 151, 300], 1, 0.3, True),
    ("chunk_aligned", 64, 1, [0, 32, 64], 1, 1.0, True),
    ("short_sequences", 40, 2, [0, 1, 2, 9, 40], 1, 0.5, True),
    ("fast_gates", 96, 1, [0, 96], 1, 4.0, True),
    # several segments: carried segments, the backward summaries E_r and
    # their reverse compose D_r (the pages' following summaries)
    ("one_sequence_5_segments", 300, 2, [0, 300], 5, 0.3, True),
    ("varlen_4_segments", 300, 2, [0, 37, 150, 151, 300], 4, 0.3, True),
    ("one_sequence_16_segments", 1000, 1, [0, 1000], 16, 0.1, False),
    ("varlen_7_segments_h0", 777, 3, [0, 5, 300, 301, 640, 777], 7, 0.2, True),
    ("segments_longer_than_sequences", 200, 1, [0, 10, 20, 30, 200], 3, 1.0, True),
    ("fast_gates_segments", 256, 2, [0, 256], 4, 4.0, True),
    # fragments of 33 and 67 tokens: a last 16-token checkpoint chunk of one
    # and of three tokens (its u and p reach the reverse from level 1 through
    # LDS)
    ("chunk_plus_one_fragments", 100, 2, [0, 33, 100], 1, 0.5, True),
    # fragments of 17, 48 (three whole chunks), 16 and 4 tokens
    ("checkpoint_chunk_edges", 85, 2, [0, 17, 65, 81, 85], 1, 0.5, True),
]


@pytest.mark.parametrize("name,T,H,cu,S,gs,with_h0", CASES, ids=[c[0] for c in CASES])
def test_backward_parity(name, T, H, cu, S, gs, with_h0):
    print(f"case {name}: T={T} H={H} cu={cu} S={S}", flush=True)
    x = synth.make_inputs(T, H, 128, 128, seed=len(name) + T, cu_seqlens=cu, gate_scale=gs)
    N = len(cu) - 1
    gen = torch.Generator().manual_seed(T + 3)
    d_o = torch.randn(T, H, 128, generator=gen)
    d_final = torch.randn(N, H, 128, 128, generator=gen) if with_h0 else None
    h0 = synth.initial_states(N, H, 128, 128, seed=T + 5) if with_h0 else None
    plan = kda.Plan(cu, S)
    d = pu.to_device(x)
    got = kda.backward(plan, d["q"], d["k"], d["v"], d["g"], d["beta"], d_o.cuda(),
                       d_final=None if d_final is None else d_final.cuda(),
                       initial_state=None if h0 is None else h0.cuda(), want_dh0=with_h0)
    torch.cuda.synchronize()
    f = pu.oracle_inputs(x)
    ref = ko.backward(f["q"], f["k"], f["v"], f["g"], f["beta"], cu, d_o.double().numpy(),
                      dfinal=None if d_final is None else d_final.double().numpy(),
                      h0=None if h0 is None else h0.double().numpy())
    names = ("dq", "dk", "dv", "dg", "dbeta", "dh0")
    errs = {}
    for key, want in zip(names, ref):
        if key == "dh0" and not with_h0:
            continue
        have = got[key].double().cpu().numpy()
        assert np.isfinite(have).all(), key
        worst = 0.0
        for h in range(H):
            a, b = have[:, h], want[:, h]
            scale = np.abs(b).max()
            err = np.abs(a - b).max()
            worst = max(worst, err / scale if scale > 0 else err)
        errs[key] = worst
    print(f"[{name}] " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    for key, e in errs.items():
        assert e <= GRAD_RTOL, (key, e)


def test_backward_mixed_paths():
    """One call in which some (fragment, head) items leave the anchored chunk
    form's range and take the token-by-token kernels while the others take
    the chunked ones: head 1's gates over sequence 1 (tokens 100..229) are
    eight times the pages' scale, so its two fragments there (one starting
    its sequence, one carried into the next segment, whose backward summary
    E_r then comes from the token-by-token launch) are flagged, while head 0
    and every other fragment stay chunked.  Both heads are checked against
    the oracle, with initial states and d_final."""
    T, H, cu, S = 300, 2, [0, 100, 230, 300], 3
    x = synth.make_inputs(T, H, 128, 128, seed=71, cu_seqlens=cu, gate_scale=1.0)
    strong = synth.make_inputs(T, H, 128, 128, seed=72, cu_seqlens=cu, gate_scale=8.0)
    x["g"][100:230, 1] = strong["g"][100:230, 1]
    N = len(cu) - 1
    gen = torch.Generator().manual_seed(73)
    d_o = torch.randn(T, H, 128, generator=gen)
    d_final = torch.randn(N, H, 128, 128, generator=gen)
    h0 = synth.initial_states(N, H, 128, 128, seed=74)
    plan = kda.Plan(cu, S)
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
            print(f"[mixed paths] {key} head {h}: {err / scale:.2e}", flush=True)
            assert err <= GRAD_RTOL * scale, (key, h, err / scale)


def test_backward_deterministic():
    T, H, cu = 150, 2, [0, 60, 150]
    x = synth.make_inputs(T, H, 128, 128, seed=31, cu_seqlens=cu)
    d_o = torch.randn(T, H, 128, generator=torch.Generator().manual_seed(32)).cuda()
    plan = kda.Plan(cu, 3)
    d = pu.to_device(x)
    outs = [kda.backward(plan, d["q"], d["k"], d["v"], d["g"], d["beta"], d_o) for _ in range(3)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        for key in ("dq", "dk", "dv", "dg", "dbeta"):
            assert torch.equal(o[key], outs[0][key]), key


def test_backward_from_forward_matches_backward():
    """kda_backward_from_forward with the forward's own transitions and
    carry-ins (kda_forward's outputs, no gate bound) gives kda_backward's
    gradients bit for bit (the same launches on the same values), over all
    heads and over a head range, with initial states and a final cotangent."""
    T, H, cu = 300, 4, [0, 100, 300]
    x = synth.make_inputs(T, H, 128, 128, seed=81, cu_seqlens=cu)
    N = len(cu) - 1
    gen = torch.Generator().manual_seed(82)
    d_o = torch.randn(T, H, 128, generator=gen).cuda()
    d_final = torch.randn(N, H, 128, 128, generator=gen).cuda()
    h0 = synth.initial_states(N, H, 128, 128, seed=83).cuda()
    plan = kda.Plan(cu, 5)
    d = pu.to_device(x)
    fwd = kda.forward(plan, d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=h0)
    saved = (fwd["transitions"], fwd["carry_in"])
    args = (plan, d["q"], d["k"], d["v"], d["g"], d["beta"], d_o)
    kw = dict(d_final=d_final, initial_state=h0, want_dh0=True)
    full = kda.backward(*args, **kw)
    kept = kda.backward(*args, **kw, saved=saved)
    part = kda.backward(*args, **kw, saved=saved, heads=(1, 2), sentinel=-5.0)
    torch.cuda.synchronize()
    print(f"[from_forward] T={T} H={H} segments=5", flush=True)
    for key in ("dq", "dk", "dv", "dg", "dbeta", "dh0"):
        assert torch.equal(full[key], kept[key]), key
        hs = (slice(None), slice(1, 3))
        assert torch.equal(full[key][hs], part[key][hs]), key
        assert (part[key][:, 0] == -5.0).all() and (part[key][:, 3] == -5.0).all(), key


def test_bench_workload_last_segments_sampled_head():
    """The backward at the bench workload's full size (65536 tokens x 32
    heads, 64 segments) as bench.py runs it.  One head's gradients over the
    last two segments (2048 tokens) depend on the forward state at their start
    and on nothing after them, so the oracle's backward of those tokens from
    that state (its forward over the first 63488 tokens) gives them exactly;
    segment 62's gradients include the cotangent D_62 = E_63 that the GPU
    forms through the backward summaries and the reverse compose."""
    w = synth.WORKLOADS["t65536_h32_s64"]
    x = synth.workload_inputs(w)
    cu = x["cu_seqlens"].tolist()
    assert cu == [0, w.T]
    plan = kda.Plan(cu, w.segments)
    d = pu.to_device(x)
    d_o = torch.randn(w.T, w.H, w.V, generator=torch.Generator().manual_seed(w.seed + 2000))
    got = kda.backward(plan, d["q"], d["k"], d["v"], d["g"], d["beta"], d_o.cuda())
    torch.cuda.synchronize()
    h = 9
    b = int(plan.bounds[w.segments - 2])
    f = pu.oracle_inputs(x, [h])
    _, c_in = ko.recurrence(f["q"][:b], f["k"][:b], f["v"][:b], f["g"][:b], f["beta"][:b], [0, b])
    win = slice(b, w.T)
    ref = ko.backward(f["q"][win], f["k"][win], f["v"][win], f["g"][win], f["beta"][win], [0, w.T - b],
                      d_o[win, h:h + 1].double().numpy(), h0=c_in)
    errs = {}
    for key, want in zip(("dq", "dk", "dv", "dg", "dbeta"), ref):
        have = got[key][win, h:h + 1].double().cpu().numpy()
        assert np.isfinite(have).all(), key
        scale = np.abs(want).max()
        errs[key] = np.abs(have - want).max() / scale
    print("[bench workload, head 9, last 2048 tokens] " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()),
          flush=True)
    for key, e in errs.items():
        assert e <= GRAD_RTOL, (key, e)


def test_backward_head_range_touches_only_its_heads():
    """kda_backward over heads [1, 3) of 4: those heads' gradients equal the
    all-heads call's bit for bit, and the other heads' gradient buffers keep
    a sentinel."""
    T, H, cu = 260, 4, [0, 100, 260]
    x = synth.make_inputs(T, H, 128, 128, seed=61, cu_seqlens=cu, gate_scale=0.3)
    N = len(cu) - 1
    gen = torch.Generator().manual_seed(62)
    d_o = torch.randn(T, H, 128, generator=gen).cuda()
    d_final = torch.randn(N, H, 128, 128, generator=gen).cuda()
    h0 = synth.initial_states(N, H, 128, 128, seed=63).cuda()
    plan = kda.Plan(cu, 3)
    d = pu.to_device(x)
    full = kda.backward(plan, d["q"], d["k"], d["v"], d["g"], d["beta"], d_o, d_final=d_final,
                        initial_state=h0, want_dh0=True)
    part = kda.backward(plan, d["q"], d["k"], d["v"], d["g"], d["beta"], d_o, d_final=d_final,
                        initial_state=h0, want_dh0=True, heads=(1, 2), sentinel=-5.0)
    torch.cuda.synchronize()
    for key in ("dq", "dk", "dv", "dg", "dbeta", "dh0"):
        a, b = full[key], part[key]
        hs = (slice(None), slice(1, 3))
        assert torch.equal(a[hs], b[hs]), key
        assert (b[:, 0] == -5.0).all() and (b[:, 3] == -5.0).all(), key
