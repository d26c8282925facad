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


def test_chunk_cache_bytes():
    # (ceil(T / 32) + S) slots of 4096 bytes per head
    assert kda.Plan([0, 65536], 64).chunk_cache_bytes(32) == (2048 + 64) * 32 * 4096
    assert kda.Plan([0, 100], 3).chunk_cache_bytes(2) == (4 + 3) * 2 * 4096
    assert kda.Plan([0, 1], 1).chunk_cache_bytes(1) == 2 * 4096
    L = kda.lib()
    assert L.kda_chunk_cache_bytes(None, 4) == 0
    assert kda.Plan([0, 100], 3).chunk_cache_bytes(0) == 0


# ------------------------------------------------ device entry points: host checks

_FAKE = 1 << 20   # a 16-byte-aligned non-null address that is never dereferenced


def _call_summaries(plan, plan_dev=_FAKE, H=2, K=128, V=128, k=_FAKE, upd=_FAKE, cache=_FAKE,
                    h0=0, hn=None, init=None):
    L = kda.lib()
    return L.kda_segment_summaries(plan.handle, plan_dev, k, _FAKE, _FAKE, _FAKE, init,
                                   H, K, V, h0, H if hn is None else hn, _FAKE, upd, cache, None)


def test_head_ranges_validate_before_launch():
    plan = kda.Plan([0, 100], 2)
    L = kda.lib()
    # every call below also has a misaligned pointer (checked after the head
    # range), so a range check that let one through returns -5 and still
    # launches nothing
    bad = _FAKE + 4
    for h0, hn in ((0, 0), (-1, 2), (1, 2), (0, 3), (2, 1), (0, -1)):
        assert _call_summaries(plan, k=bad, h0=h0, hn=hn) == -1, (h0, hn)
        assert L.kda_compose_summaries(plan.handle, _FAKE, _FAKE, _FAKE, 2, 128, 128, h0, hn,
                                       bad, None) == -1, (h0, hn)
        assert L.kda_apply_carry(plan.handle, _FAKE, _FAKE, _FAKE, _FAKE, _FAKE, _FAKE, None, 2, 128, 128,
                                 h0, hn, bad, _FAKE, 0, _FAKE, _FAKE, None) == -1, (h0, hn)
    # a valid range reaches the pointer checks
    assert _call_summaries(plan, k=bad, h0=1, hn=1) == -5


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
    assert _call_summaries(plan, K=64) == -4
    assert _call_summaries(plan, V=256) == -4
    assert _call_summaries(plan, H=0) == -1
    assert _call_summaries(plan, H=70000) == -4
    assert _call_summaries(plan, plan_dev=0) == -1
    assert _call_summaries(plan, k=0) == -1
    assert _call_summaries(plan, k=_FAKE + 2) == -5
    assert _call_summaries(plan, upd=_FAKE + 8) == -5
    assert _call_summaries(plan, plan_dev=_FAKE + 4) == -5
    assert _call_summaries(plan, cache=0) == -1
    assert _call_summaries(plan, cache=_FAKE + 8) == -5
    L = kda.lib()
    assert L.kda_segment_summaries(None, _FAKE, _FAKE, _FAKE, _FAKE, _FAKE, None, 2, 128, 128, 0, 2,
                                   _FAKE, _FAKE, _FAKE, None) == -1
    # the optional initial states: misaligned is refused (NULL is valid and
    # means zero, so it is not tried here with fake buffers)
    assert _call_summaries(plan, init=_FAKE + 4) == -5
    assert L.kda_apply_carry(plan.handle, _FAKE, _FAKE, _FAKE, _FAKE, _FAKE, _FAKE, _FAKE + 8, 2, 128,
                             128, 0, 2, _FAKE, _FAKE, 0, _FAKE, _FAKE, None) == -5
    assert L.kda_compose_summaries(plan.handle, _FAKE, _FAKE, _FAKE, 2, 96, 128, 0, 2, _FAKE,
                                   None) == -4
    assert L.kda_compose_summaries(plan.handle, _FAKE, 0, _FAKE, 2, 128, 128, 0, 2, _FAKE,
                                   None) == -1
    assert L.kda_apply_carry(plan.handle, _FAKE, _FAKE, _FAKE, _FAKE, _FAKE, _FAKE, None, 2, 128, 128,
                             0, 2, _FAKE + 4, _FAKE, 0, _FAKE, _FAKE, None) == -5
    assert L.kda_apply_carry(plan.handle, _FAKE, _FAKE, _FAKE, _FAKE, _FAKE, _FAKE, None, 2, 128, 128,
                             0, 2, _FAKE, 0, 0, _FAKE, _FAKE, None) == -1
    assert L.kda_apply_carry(plan.handle, _FAKE, _FAKE, _FAKE, _FAKE, _FAKE, _FAKE, None, 2, 128, 128,
                             0, 2, _FAKE, _FAKE, 0, _FAKE, 0, None) == -1
    # an unknown o format is refused before launch
    for fmt in (-1, 2, 7):
        assert L.kda_apply_carry(plan.handle, _FAKE, _FAKE, _FAKE, _FAKE, _FAKE, _FAKE, None, 2, 128,
                                 128, 0, 2, _FAKE, _FAKE, fmt, _FAKE, _FAKE, None) == -1, fmt
    assert L.kda_last_hip_error() == 0


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
