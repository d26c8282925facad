"""The allocation-free entry point kda_forward_noalloc against kda_forward:
bitwise the same results (hence the same parity with the oracle), on two
calls in a row whose second input is smaller, and a clear error for a
workspace beyond the fixed array."""
import pytest
import torch

from gated_delta_rule_37_amd import kda, synth
import parity_utils as pu

pytestmark = pytest.mark.gpu

KEYS = ("o", "final_state", "transitions", "updates", "carry_in")


def _run_both(T, H, cu, S, seed, gs, with_h0, piece_tokens=0):
    print(f"case noalloc: T={T} H={H} S={S} cu={cu} h0={with_h0} pieces={piece_tokens}", flush=True)
    x = synth.make_inputs(T, H, 128, 128, seed=seed, cu_seqlens=cu, gate_scale=gs)
    plan = kda.Plan(cu, S, None, piece_tokens)
    d = pu.to_device(x)
    pd = plan.device_blob("cuda:0")
    h0 = synth.initial_states(len(cu) - 1, H, 128, 128, seed=seed + 1) if with_h0 else None
    init = None if h0 is None else h0.to("cuda:0")
    ref = kda.alloc_outputs(plan, H, 128, 128, "cuda:0")
    kda.forward_call(plan, pd, d["q"], d["k"], d["v"], d["g"], d["beta"], ref, initial_state=init)
    out = kda.alloc_outputs(plan, H, 128, 128, "cuda:0")
    out.pop("workspace")
    for key in KEYS:
        out[key].fill_(-7.0)
    kda.forward_noalloc(plan, pd, d["q"], d["k"], d["v"], d["g"], d["beta"], out, initial_state=init)
    torch.cuda.synchronize()
    for key in KEYS:
        assert torch.equal(out[key], ref[key]), key
    out.pop("workspace", None)
    pu.compare(pu.gpu_numpy(out), pu.run_oracle(x, cu, plan, h0=h0), "noalloc")


def test_noalloc_matches_forward_two_calls_second_smaller():
    _run_both(600, 4, [0, 37, 600], 6, seed=41, gs=0.3, with_h0=False)
    _run_both(200, 2, [0, 90, 200], 3, seed=42, gs=0.05, with_h0=True)


def test_noalloc_with_pieces_matches_forward():
    """A plan with pieces: the pieces' summaries and carry-ins live in the
    fixed array too, behind the chunk cache."""
    _run_both(700, 2, [0, 300, 700], 2, seed=43, gs=0.2, with_h0=True, piece_tokens=128)


def test_noalloc_refuses_workspace_beyond_fixed_array():
    cap = kda.noalloc_max_workspace_bytes()
    assert cap == 64 << 20
    # 65536 tokens x 32 heads need (2048 + 64) * 32 * 4096 bytes > 64 MiB;
    # the size is refused before any buffer is looked at
    plan = kda.Plan([0, 65536], 64)
    assert plan.workspace_bytes(32) > cap
    L = kda.lib()
    args = ([plan.handle, 16, 0] + [16, 0] * 5 + [float("-inf")] + [16, 0] + [32, 128, 128, 0, 32]
            + [16, 0] * 4 + [0] + [16, 0] + [None])
    assert L.kda_forward_noalloc(*args) == -8
