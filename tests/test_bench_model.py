"""The algorithmic work model behind bench.py's roofline (CPU only), checked
against counts written out by hand from the plan's structure.

Per token-head, FP32-grade multiply-adds at C = 32, K = V = 128: forward
59,584; zero-start segment update 38,976; transition 36,864.  HBM bytes per
token-head: forward 1538 (q, k, v, g 256 each, beta 2, o 512), segment update
770 (k, v, g, beta); one 128 x 128 FP32 state is 65,536 bytes.
"""
import bench
from gated_delta_rule_37_amd import kda

FWD, SUM_S, SUM_PHI = 59_584, 38_976, 36_864
STATE = 128 * 128 * 4


def test_per_token_head_figures():
    assert bench.MACS["fwd"] == FWD
    assert bench.MACS["sum_s"] == SUM_S
    assert bench.MACS["sum_phi"] == SUM_PHI
    assert bench.BYTES["fwd"] == 1538
    assert bench.BYTES["sum_s"] == 770


def test_bench_workload_counts():
    """One sequence of 65536 tokens in 64 segments, 32 heads: every fragment
    ends its segment, the first starts the sequence, the other 63 carry in
    with a live transition."""
    T, H, S = 65536, 32, 64
    w = bench.chunk_kernel_work(kda.Plan([0, T], S).blob, H)
    assert w["summaries"]["macs"] == T * H * SUM_S + (T - T // S) * H * SUM_PHI
    assert w["summaries"]["bytes"] == T * H * 770 + S * 2 * STATE * H == 1_883_242_496
    # every fragment's T diag(beta) comes from the cache: no A, no T products
    cached = bench.MACS["fwd"] - bench.TRI_STRICT - bench.TRI_INCL
    assert w["carry"]["macs"] == T * H * cached
    assert w["carry"]["bytes"] == T * H * 1538 + STATE * H * (63 + 1) == 3_359_637_504
    w16 = bench.chunk_kernel_work(kda.Plan([0, T], S).blob, H, o_bytes=2)
    assert w16["carry"]["bytes"] == w["carry"]["bytes"] - T * H * 128 * 2


def test_varlen_counts():
    """Sequences [0, 100) and [100, 300) in segments [0, 150) and [150, 300):
    fragments [0,100) (ends sequence 0, not segment-ending), [100,150)
    (starts sequence 1, ends segment 0), [150,300) (carries in, live, ends
    segment 1 and sequence 1)."""
    H = 3
    w = bench.chunk_kernel_work(kda.Plan([0, 100, 300], 2).blob, H)
    assert w["summaries"]["macs"] == (50 + 150) * H * SUM_S + 150 * H * SUM_PHI
    assert w["summaries"]["bytes"] == (50 + 150) * H * 770 + 2 * 2 * STATE * H
    cached = bench.MACS["fwd"] - bench.TRI_STRICT - bench.TRI_INCL
    assert w["carry"]["macs"] == 100 * H * FWD + 200 * H * cached
    # states: C_1 read by [150,300); final states of sequences 0 and 1 written
    assert w["carry"]["bytes"] == 300 * H * 1538 + 3 * STATE * H
