"""Plain fp64 CPU oracle for the segmented KDA forward pass.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import anything from this package.  It shares no code, header, table or helper
with the HIP path in ``gated_delta_rule_37_amd/`` and imports nothing from it.

Sources (the three pages; only two are on topic):

* [cuLA#110] inclusionAI/cuLA pull request #110, "feat(cp): add opt-in NVSHMEM
  CP state handoff" -- sections Summary, Motivation, Supported configuration,
  Correctness, Performance.
* [cuLA#136] inclusionAI/cuLA pull request #136, "feat(kda): add cuDNN
  concatenated-summary Kimi CP" -- sections Summary, Latest cuDNN
  compatibility, Summary by CodeRabbit, Walkthrough (change table), Sequence
  Diagram.

The pages never print the recurrence.  The oracle takes the standard KDA
(Kimi Delta Attention) gated delta rule as the reading of "KDA" and "affine
recurrence state" ([cuLA#110] Motivation):

    S_t = (I - beta_t k_t k_t^T) Diag(exp g_t) S_{t-1} + beta_t k_t v_t^T
    o_t = S_t^T q_t

with S_t a K x V matrix per head, stored K-major ("non-transposed state
layout", [cuLA#110] Supported configuration), BF16 inputs and an FP32 state on
the device side ([cuLA#110] Supported configuration); the oracle itself is
fp64 throughout.

Modules
-------
``kda_oracle``  recurrence, segment summaries, ordered composition, segmented
                reconstruction, the optional safe gate; the backward:
                gradients of q, k, v, g, beta and the initial states by a
                reverse pass, the following summaries of each segment, their
                reverse composition and the segmented reverse pass.
``plan_oracle`` the contiguous segment plan over packed sequences.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, brute force, invariants and hand-derived fixtures; none
is "parity unpinned".
"""
