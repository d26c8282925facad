"""Host-side checks of the C-ABI library (no GPU needed).

The library loads, exports every function ``include/kda.h`` declares, builds
plans bit-identical to the reference plan, and rejects bad arguments with the
documented status before anything reaches the device.
"""
import ctypes
import json
import os
import re

import numpy as np
import pytest

from gated_delta_rule_37_amd import kda
from oracle import plan_oracle as po

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")
GOLDEN = os.path.join(ROOT, "tests", "golden", "plan_cases.json")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = kda.lib()
    declared = _declared_functions()
    assert set(declared) == set(kda.SYMBOLS)
    for name in declared:
        assert hasattr(L, name), name


def test_status_strings():
    L = kda.lib()
    for code, name in kda.STATUS.items():
        assert L.kda_status_string(code).decode() == name


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_plan_blob_matches_golden(case):
    plan = kda.Plan(case["cu_seqlens"], case["segments"], case["custom_bounds"])
    assert plan.blob.tolist() == case["blob"] + case["frag_order"]


@pytest.mark.parametrize("seed", range(40))
def test_plan_blob_matches_oracle_random(seed):
    rng = np.random.default_rng(1000 + seed)
    N = int(rng.integers(1, 30))
    lens = rng.integers(1, 300, size=N)
    cu = [0] + np.cumsum(lens).astype(int).tolist()
    T = cu[-1]
    S = int(rng.integers(1, min(T, 70) + 1))
    bounds = None
    if seed % 3 == 0 and S > 1:
        cuts = sorted(rng.choice(np.arange(1, T), size=S - 1, replace=False).tolist())
        bounds = [0] + cuts + [T]
    want = po.build_plan(cu, S, bounds)["blob"]
    got = kda.Plan(cu, S, bounds).blob
    np.testing.assert_array_equal(got, want)


def test_plan_blob_matches_oracle_workloads():
    from gated_delta_rule_37_amd import synth
    import torch
    for w in synth.WORKLOADS.values():
        if w.varlen:
            gen = torch.Generator("cpu").manual_seed(w.seed)
            lens = synth.draw_lengths(gen, w.T, w.min_len, w.max_len)
            cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
        else:
            cu = [0, w.T]
        np.testing.assert_array_equal(kda.Plan(cu, w.segments).blob,
                                      po.build_plan(cu, w.segments)["blob"])


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["invalid"])
def test_plan_rejects_invalid(case):
    with pytest.raises(kda.KdaError) as e:
        kda.Plan(case["cu_seqlens"], case["segments"], case["custom_bounds"])
    assert e.value.name == "KDA_ERR_" + case["kind"]


def test_summary_workspace_64_segments_32_heads_is_256_mib():
    # 64 shards, H = 32, K = V = 128: the prepared summary workspace of
    # cuLA PR #136, Latest cuDNN compatibility, is 256 MiB.
    plan = kda.Plan([0, 65536], 64)
    assert plan.summary_bytes(32, 128, 128) == 256 * 1024 * 1024


def test_workspace_bytes():
    # (ceil(T / 32) + S) slots of 4096 bytes per head
    assert kda.Plan([0, 65536], 64).workspace_bytes(32) == (2048 + 64) * 32 * 4096
    assert kda.Plan([0, 100], 3).workspace_bytes(2) == (4 + 3) * 2 * 4096
    assert kda.Plan([0, 1], 1).workspace_bytes(1) == 2 * 4096
    L = kda.lib()
    assert L.kda_workspace_bytes(None, 4, 128, 128) == 0
    assert kda.Plan([0, 100], 3).workspace_bytes(0) == 0
    assert kda.Plan([0, 100], 3).workspace_bytes(2, 64, 128) == 0


# ------------------------------------------------ device entry points: host checks
# No call below ever has every argument valid: each one fails a host check,
# so nothing is launched (the fake addresses are never dereferenced).

_FAKE = 1 << 20   # a 16-byte-aligned non-null address
_BIG = 1 << 40    # a size larger than any buffer a call needs


class Call:
    """One device call with fake buffers of ample size; keyword overrides
    replace a buffer's address (``<name>``), its size (``<name>_bytes``) or a
    scalar argument."""

    SUMMARIES = ("plan_dev", "k", "v", "g", "beta", "gate", "init", "dims", "transitions", "updates",
                 "workspace")
    COMPOSE = ("plan_dev", "transitions", "updates", "dims", "carry")
    CARRY = ("plan_dev", "q", "k", "v", "g", "beta", "gate", "init", "dims", "carry", "o", "fmt", "final",
             "workspace")
    FORWARD = ("plan_dev", "q", "k", "v", "g", "beta", "gate", "init", "dims", "transitions", "updates",
               "carry", "o", "fmt", "final", "workspace")
    NOALLOC = ("plan_dev", "q", "k", "v", "g", "beta", "gate", "init", "dims", "transitions", "updates",
               "carry", "o", "fmt", "final")

    def __init__(self, fn, order):
        self.fn, self.order = fn, order

    def __call__(self, plan, H=2, K=128, V=128, h0=0, hn=None, fmt=0, gate=float("-inf"), **kw):
        args = [None if plan is None else plan.handle]
        for name in self.order:
            if name == "dims":
                args += [H, K, V, h0, H if hn is None else hn]
            elif name == "fmt":
                args.append(fmt)
            elif name == "gate":
                args.append(gate)
            else:
                default = None if name == "init" else _FAKE
                args += [kw.get(name, default), kw.get(name + "_bytes", _BIG)]
        args.append(None)   # stream
        return self.fn(*args)


def _calls():
    L = kda.lib()
    return dict(summaries=Call(L.kda_segment_summaries, Call.SUMMARIES),
                compose=Call(L.kda_compose_summaries, Call.COMPOSE),
                carry=Call(L.kda_apply_carry, Call.CARRY),
                forward=Call(L.kda_forward, Call.FORWARD))


def _first_output(call):
    return "carry" if "transitions" not in call.order else "transitions"


def test_head_ranges_validate_before_launch():
    plan = kda.Plan([0, 100], 2)
    # every call below also has a misaligned pointer (checked after the head
    # range), so a range check that let one through returns -5 and still
    # launches nothing
    bad = _FAKE + 4
    for name, call in _calls().items():
        out = _first_output(call)
        for h0, hn in ((0, 0), (-1, 2), (1, 2), (0, 3), (2, 1), (0, -1)):
            assert call(plan, h0=h0, hn=hn, **{out: bad}) == -1, (name, h0, hn)
        # a valid range reaches the pointer checks
        assert call(plan, h0=1, hn=1, **{out: bad}) == -5, name


def test_head_groups_cover_every_head_once():
    for H in (1, 3, 4, 7, 32, 33):
        for groups in (1, 2, 4, 5, 64):
            runs = kda.head_groups(H, groups)
            assert len(runs) == min(groups, H)
            heads = [h for b, n in runs for h in range(b, b + n)]
            assert heads == list(range(H))
            assert max(n for _, n in runs) - min(n for _, n in runs) <= 1


def test_device_calls_validate_before_launch():
    plan = kda.Plan([0, 100], 2)
    c = _calls()
    for name, call in c.items():
        # each of these fails one check, before any size check
        assert call(plan, K=64) == -4, name
        assert call(plan, V=256) == -4, name
        assert call(plan, H=0) == -1, name
        assert call(plan, H=70000) == -4, name
        assert call(plan, plan_dev=0) == -1, name
        assert call(plan, plan_dev=_FAKE + 4) == -5, name
        assert call(None) == -1, name
    for name in ("summaries", "carry", "forward"):
        assert c[name](plan, k=0) == -1, name
        assert c[name](plan, k=_FAKE + 2) == -5, name
        assert c[name](plan, workspace=0) == -1, name
        assert c[name](plan, workspace=_FAKE + 8) == -5, name
        # the optional initial states: misaligned is refused (NULL is valid and
        # means zero)
        assert c[name](plan, init=_FAKE + 4) == -5, name
    for name in ("summaries", "compose", "forward"):
        assert c[name](plan, updates=_FAKE + 8) == -5, name
        assert c[name](plan, transitions=0) == -1, name
    for name in ("compose", "carry", "forward"):
        assert c[name](plan, carry=_FAKE + 4) == -5, name
        assert c[name](plan, carry=0) == -1, name
    for name in ("carry", "forward"):
        assert c[name](plan, o=0) == -1, name
        assert c[name](plan, final=0) == -1, name
        # an unknown o format is refused before launch
        for fmt in (-1, 2, 7):
            assert c[name](plan, fmt=fmt) == -1, (name, fmt)
    # the safe gate's bound: NaN or > 0 is refused (checked before the
    # buffers: a misaligned buffer would otherwise give -5)
    for name in ("summaries", "carry", "forward"):
        for bad in (float("nan"), 0.5, float("inf")):
            assert c[name](plan, gate=bad, k=_FAKE + 4) == -1, (name, bad)
        for ok in (float("-inf"), 0.0, -3.0):
            assert c[name](plan, gate=ok, k=_FAKE + 4) == -5, (name, ok)
    assert kda.lib().kda_last_hip_error() == 0


def _needs(plan, H):
    """Bytes each buffer of a call needs (K = V = 128), by argument name."""
    T, N, S = plan.T, plan.N, plan.S
    return dict(plan_dev=4 * len(plan.blob), q=T * H * 256, k=T * H * 256, v=T * H * 256,
                g=T * H * 256, beta=T * H * 2, init=N * H * 65536, transitions=S * H * 65536,
                updates=S * H * 65536, carry=S * H * 65536, o=T * H * 512, final=N * H * 65536,
                workspace=plan.workspace_bytes(H))


@pytest.mark.parametrize("cu,S,H", [([0, 100], 2, 2), ([0, 37, 150, 151, 300], 4, 3), ([0, 1], 1, 1)])
def test_undersized_buffers_are_refused(cu, S, H):
    """Every buffer of every call at exactly the bytes its shape needs except
    one, which is one byte short: the call returns KDA_ERR_WORKSPACE_TOO_SMALL
    for the workspace and KDA_ERR_BUFFER_TOO_SMALL for any other buffer, and
    launches nothing.  A given initial state is checked like the others."""
    plan = kda.Plan(cu, S)
    need = _needs(plan, H)
    for name, call in _calls().items():
        exact = {b + "_bytes": need[b] for b in call.order if b in need}
        for buf in call.order:
            if buf not in need:
                continue
            args = dict(exact, init=_FAKE)
            args[buf + "_bytes"] = need[buf] - 1
            want = -8 if buf == "workspace" else -9
            assert call(plan, H=H, **args) == want, (name, buf)
        if "o" in call.order:
            # BF16 o needs half the FP32 bytes
            args = dict(exact, o_bytes=need["o"] // 2 - 1)
            assert call(plan, H=H, fmt=1, **args) == -9, name
    assert kda.lib().kda_last_hip_error() == 0


def test_unsupported_token_count_boundary():
    """2^30 tokens is the largest plan accepted; one more is KDA_ERR_UNSUPPORTED."""
    L = kda.lib()
    out = ctypes.c_void_p()
    over = (ctypes.c_int32 * 2)(0, (1 << 30) + 1)
    assert L.kda_plan_segments(over, 1, 1, None, ctypes.byref(out)) == -4
    at = (ctypes.c_int32 * 2)(0, 1 << 30)
    assert L.kda_plan_segments(at, 1, 1, None, ctypes.byref(out)) == 0
    L.kda_plan_destroy(out)


def test_plan_info_and_null_handling():
    L = kda.lib()
    plan = kda.Plan([0, 5, 9], 3)
    T, N, S, F = (ctypes.c_int32() for _ in range(4))
    assert L.kda_plan_info(plan.handle, ctypes.byref(T), ctypes.byref(N), ctypes.byref(S),
                           ctypes.byref(F)) == 0
    assert (T.value, N.value, S.value, F.value) == (9, 2, 3, plan.F)
    assert L.kda_plan_info(None, None, None, None, None) == -1
    assert L.kda_summary_bytes(None, 1, 128, 128) == 0
    out = ctypes.c_void_p()
    assert L.kda_plan_segments(None, 1, 1, None, ctypes.byref(out)) == -1
    L.kda_plan_destroy(None)


def test_backward_validates_before_launch():
    """kda_backward refuses bad arguments with the documented codes (fake,
    never dereferenced buffers; every call below fails a check)."""
    L = kda.lib()
    plan = kda.Plan([0, 70, 100], 2)
    H = 2
    T, N = 100, 2
    need = dict(plan_dev=4 * len(plan.blob), q=T * H * 256, k=T * H * 256, v=T * H * 256, g=T * H * 256,
                beta=T * H * 2, init=N * H * 65536, do=T * H * 512, dfinal=N * H * 65536, dq=T * H * 512,
                dk=T * H * 512, dv=T * H * 512, dg=T * H * 512, dbeta=T * H * 4, dh0=N * H * 65536,
                ws=L.kda_backward_workspace_bytes(plan.handle, H, 128, 128))
    # the forward's chunk cache (256-byte aligned), five S x H state arrays
    # (transitions, updates, carry-ins, backward summaries and their compose),
    # (floor(T/16) + F) x H checkpoints and every token's u and p (1 KiB per
    # token and head) for the token-by-token path; for the chunked path, per
    # chunk slot (ceil(T/32) + F of them) and head an anchored state, an
    # anchored cotangent, a 4 KiB T diag(beta) and the chunk's V - Kr R and dU
    # (16 KiB each), then F x H path flags and the slot map (int32, each
    # 256-byte aligned)
    S, F = 2, plan.F
    cache = ((T + 31) // 32 + S) * H * 4096
    cache = (cache + 255) // 256 * 256
    slots = (T + 31) // 32 + F
    al = lambda x: (x + 255) // 256 * 256
    assert need["ws"] == (cache + 5 * S * H * 65536 + (T // 16 + F) * H * 65536 + T * H * 1024
                          + 2 * slots * H * 65536 + slots * H * 4096 + 2 * slots * H * 16384 + al(F * H * 4)
                          + al(slots * 4))
    order = ("plan_dev", "q", "k", "v", "g", "beta", "init", "do", "dfinal", "dq", "dk", "dv", "dg", "dbeta",
             "dh0", "ws")

    def call(H=H, K=128, **over):
        args = [plan.handle]
        for name in order:
            if name == "dq":
                args += [H, K, 128, 0, H]
            args += [over.get(name, _FAKE), over.get(name + "_bytes", need[name])]
        args.append(None)
        return L.kda_backward(*args)

    assert call(K=64) == -4
    assert call(do=0) == -1
    assert call(dq=_FAKE + 4) == -5
    assert call(ws=0) == -1
    for name in order:
        short = {name + "_bytes": need[name] - 1, "q": _FAKE + 4} if name == "q" else {name + "_bytes": need[name] - 1}
        if name == "q":
            continue
        want = -8 if name == "ws" else -9
        assert call(**short) == want, name
    assert L.kda_last_hip_error() == 0


def test_backward_from_forward_validates_before_launch():
    """kda_backward_from_forward checks the saved transitions and carry-ins
    (shape [S, H, K, V] fp32 each) beside kda_backward's arguments, and
    refuses a plan with pieces (fake, never dereferenced buffers)."""
    L = kda.lib()
    H, T, N = 2, 100, 2

    def sizes(plan):
        S = plan.S
        return dict(plan_dev=4 * len(plan.blob), q=T * H * 256, k=T * H * 256, v=T * H * 256, g=T * H * 256,
                    beta=T * H * 2, init=N * H * 65536, do=T * H * 512, dfinal=N * H * 65536,
                    trans=S * H * 65536, carry=S * H * 65536, dq=T * H * 512, dk=T * H * 512, dv=T * H * 512,
                    dg=T * H * 512, dbeta=T * H * 4, dh0=N * H * 65536,
                    ws=L.kda_backward_workspace_bytes(plan.handle, H, 128, 128))

    def call(plan, K=128, **over):
        need = sizes(plan)
        order = ("plan_dev", "q", "k", "v", "g", "beta", "init", "do", "dfinal", "trans", "carry", "dq", "dk",
                 "dv", "dg", "dbeta", "dh0", "ws")
        args = [plan.handle]
        for name in order:
            if name == "trans":
                args += [H, K, 128, 0, H]
            args += [over.get(name, _FAKE), over.get(name + "_bytes", need[name])]
        args.append(None)
        return L.kda_backward_from_forward(*args)

    plan = kda.Plan([0, 70, 100], 2)
    need = sizes(plan)
    assert call(plan, K=64) == -4
    assert call(plan, trans=0) == -1
    assert call(plan, carry=0) == -1
    assert call(plan, trans_bytes=need["trans"] - 1) == -9
    assert call(plan, carry_bytes=need["carry"] - 1) == -9
    assert call(plan, carry=_FAKE + 4) == -5
    assert call(plan, ws_bytes=need["ws"] - 1) == -8
    pieces = kda.Plan([0, 100], 1, None, 32)
    assert pieces.pieces
    assert call(pieces) == -4
    assert L.kda_last_hip_error() == 0


PIECES_GOLDEN = os.path.join(ROOT, "tests", "golden", "plan_pieces_cases.json")


@pytest.mark.parametrize("case", json.load(open(PIECES_GOLDEN))["cases"], ids=lambda c: c["name"])
def test_pieces_plan_blob_matches_golden(case):
    plan = kda.Plan(case["cu_seqlens"], case["segments"], case["custom_bounds"], case["piece_tokens"])
    assert plan.blob.tolist() == case["blob"]
    assert plan.S == case["segments"] and plan.P > plan.S and plan.pieces


@pytest.mark.parametrize("seed", range(30))
def test_pieces_plan_blob_matches_oracle_random(seed):
    rng = np.random.default_rng(3000 + seed)
    N = int(rng.integers(1, 20))
    lens = rng.integers(1, 400, size=N)
    cu = [0] + np.cumsum(lens).astype(int).tolist()
    T = cu[-1]
    S = int(rng.integers(1, min(T, 12) + 1))
    bounds = None
    if seed % 3 == 0 and S > 1:
        cuts = sorted(rng.choice(np.arange(1, T), size=S - 1, replace=False).tolist())
        bounds = [0] + cuts + [T]
    L = 32 * int(rng.integers(1, 8))
    want = po.build_plan(cu, S, bounds, L)["blob"]
    plan = kda.Plan(cu, S, bounds, L)
    np.testing.assert_array_equal(plan.blob, want)
    P = ctypes.c_int32()
    assert kda.lib().kda_plan_pieces(plan.handle, ctypes.byref(P)) == 0
    assert P.value == plan.P == int(want[2])
    assert plan.bounds.tolist() == (bounds if bounds is not None else [(r * T) // S for r in range(S + 1)])


def test_pieces_plan_refuses_bad_piece_length():
    L = kda.lib()
    out = ctypes.c_void_p()
    cu = (ctypes.c_int32 * 2)(0, 100)
    for bad in (-32, 16, 33):
        assert L.kda_plan_segments_pieces(cu, 1, 2, None, bad, ctypes.byref(out)) == -3
    assert L.kda_plan_pieces(None, None) == -1


def test_pieces_plan_workspace_grows_by_piece_states():
    """kda_workspace_bytes: the chunk cache over pieces, then 3 P H states."""
    plain = kda.Plan([0, 1000], 2)
    cut = kda.Plan([0, 1000], 2, None, 128)
    H = 3
    cache = lambda P: (((1000 + 31) // 32 + P) * H * 4096 + 255) // 256 * 256
    assert plain.workspace_bytes(H) == ((1000 + 31) // 32 + 2) * H * 4096
    assert cut.P == 8
    assert cut.workspace_bytes(H) == cache(8) + 3 * 8 * H * 65536
    assert cut.summary_bytes(H) == plain.summary_bytes(H)   # results stay per segment
