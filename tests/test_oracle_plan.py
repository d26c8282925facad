"""Pins for the reference segment plan: hand-derived fixtures and invariants."""
import json
import os

import numpy as np
import pytest

from oracle import plan_oracle as po

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "plan_cases.json")


def _cases():
    with open(GOLDEN) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _cases()["cases"], ids=lambda c: c["name"])
def test_plan_matches_hand_derived_blob(case):
    plan = po.build_plan(case["cu_seqlens"], case["segments"], case["custom_bounds"])
    assert plan["blob"].tolist() == case["blob"] + case["frag_order"]


@pytest.mark.parametrize("case", _cases()["invalid"])
def test_plan_rejects_invalid(case):
    with pytest.raises(po.PlanError) as e:
        po.build_plan(case["cu_seqlens"], case["segments"], case["custom_bounds"])
    assert e.value.kind == case["kind"]


def _check_invariants(cu, plan):
    T, S = plan["T"], plan["S"]
    b = plan["seg_bounds"]
    starts = set(cu[:-1])
    covered = np.zeros(T, dtype=int)
    for f in range(plan["F"]):
        n, lo, hi, r = (plan["frag_seq"][f], plan["frag_begin"][f], plan["frag_end"][f],
                        plan["frag_seg"][f])
        assert cu[n] <= lo < hi <= cu[n + 1]           # inside one sequence
        assert b[r] <= lo and hi <= b[r + 1]           # inside one segment
        assert plan["seg_frag_ptr"][r] <= f < plan["seg_frag_ptr"][r + 1]
        covered[lo:hi] += 1
        fl = plan["frag_flags"][f]
        assert bool(fl & po.FRAG_CARRIED) == (lo == b[r] and lo not in starts and r > 0)
        assert bool(fl & po.FRAG_SEG_LAST) == (hi == b[r + 1])
        assert bool(fl & po.FRAG_SEQ_END) == (hi == cu[n + 1])
    assert (covered == 1).all()                         # fragments partition the tokens
    for r in range(S):
        assert plan["seg_transition_live"][r] == int(
            plan["seg_carry_in"][r] == 1 and not any(b[r] < s < b[r + 1] for s in starts))
    for n in range(plan["N"]):
        r = plan["seq_end_seg"][n]
        assert b[r] <= cu[n + 1] - 1 < b[r + 1]
        owners = [f for f in range(plan["F"]) if plan["frag_seq"][f] == n
                  and plan["frag_flags"][f] & po.FRAG_SEQ_END]
        assert len(owners) == 1 and plan["frag_seg"][owners[0]] == r


@pytest.mark.parametrize("seed", range(25))
def test_plan_invariants_random(seed):
    rng = np.random.default_rng(seed)
    N = int(rng.integers(1, 9))
    lens = rng.integers(1, 40, size=N)
    cu = [0] + list(np.cumsum(lens).astype(int))
    T = cu[-1]
    S = int(rng.integers(1, min(T, 12) + 1))
    if seed % 2:
        cuts = sorted(rng.choice(np.arange(1, T), size=S - 1, replace=False).tolist()) if S > 1 else []
        plan = po.build_plan(cu, S, [0] + cuts + [T])
    else:
        plan = po.build_plan(cu, S)
    _check_invariants(cu, plan)


PIECES_GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "plan_pieces_cases.json")


@pytest.mark.parametrize("case", json.load(open(PIECES_GOLDEN))["cases"], ids=lambda c: c["name"])
def test_pieces_plan_matches_hand_derived_blob(case):
    plan = po.build_plan(case["cu_seqlens"], case["segments"], case["custom_bounds"], case["piece_tokens"])
    assert plan["blob"].tolist() == case["blob"]


@pytest.mark.parametrize("seed", range(20))
def test_pieces_plan_invariants_random(seed):
    """Pieces partition every segment at multiples of piece_tokens from its
    start; the per-piece arrays obey the segment invariants; piece_ptr maps
    segments to their pieces; larger pieces than any segment give the plain
    plan's blob."""
    rng = np.random.default_rng(500 + seed)
    N = int(rng.integers(1, 6))
    lens = rng.integers(1, 120, size=N)
    cu = [0] + list(np.cumsum(lens).astype(int))
    T = cu[-1]
    S = int(rng.integers(1, min(T, 6) + 1))
    L = 32 * int(rng.integers(1, 4))
    plan = po.build_plan(cu, S, None, L)
    _check_invariants(cu, plan)
    segb, ptr = plan["segment_bounds"], plan["piece_ptr"]
    pb = plan["seg_bounds"]
    assert ptr[0] == 0 and ptr[-1] == plan["S"]
    for r in range(S):
        want = list(range(segb[r], segb[r + 1], L))
        assert pb[ptr[r]:ptr[r + 1]] == want
    plain = po.build_plan(cu, S)
    if plan["S"] == S:
        assert plan["blob"].tolist() == plain["blob"].tolist()
    else:
        assert len(plan["blob"]) > len(plain["blob"])
    big = po.build_plan(cu, S, None, 32 * ((T + 31) // 32))
    assert big["blob"].tolist() == plain["blob"].tolist()


@pytest.mark.parametrize("bad", [-32, 16, 33])
def test_pieces_plan_rejects_bad_piece_length(bad):
    with pytest.raises(po.PlanError) as e:
        po.build_plan([0, 100], 2, None, bad)
    assert e.value.kind == "BAD_SEGMENTS"
