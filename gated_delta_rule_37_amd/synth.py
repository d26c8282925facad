"""Seeded synthetic inputs for the segmented KDA forward pass.

This module only draws random numbers and shapes them into the inputs'
distributions; it holds none of the recurrence's arithmetic, so both the HIP
path's tests and the fp64 oracle can be fed from it.

Distributions (the five workloads the pages' measurements stand for: BF16 KDA
inputs with an FP32 state, cuLA PR #110 "feat(cp): add opt-in NVSHMEM CP state
handoff", Supported configuration; H=32, K=V=128 and 64 shards, cuLA PR #136
"feat(kda): add cuDNN concatenated-summary Kimi CP", Latest cuDNN
compatibility):

* q, k ~ N(0, 1), then L2-normalised over the key dimension in fp32;
* v ~ N(0, 1);
* g = -softplus(N(0, 1)) per key channel (a log-decay, always <= 0);
* beta = sigmoid(N(0, 1)) per (token, head);
* all cast to bfloat16 (round to nearest even).

Draw order with ``torch.Generator('cpu').manual_seed(seed)``: the sequence
lengths (varlen workloads only), then q, k, v, x_g, x_beta.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: packed tokens, heads, dims, segment count."""

    name: str
    T: int
    H: int
    K: int
    V: int
    segments: int
    seed: int
    varlen: bool = False
    min_len: int = 512
    max_len: int = 8192
    gate_scale: float = 1.0
    beta_scale: float = 1.0
    notes: str = field(default="", compare=False)


# The five measured workloads.  seed = the workload's index.
WORKLOADS = {
    "t1024_h4_s2": Workload("t1024_h4_s2", 1024, 4, 128, 128, 2, seed=0),
    "t4096_h8_s4": Workload("t4096_h8_s4", 4096, 8, 128, 128, 4, seed=1),
    "t8192_h16_s4": Workload("t8192_h16_s4", 8192, 16, 128, 128, 4, seed=2),
    "varlen32k_h32_s8": Workload("varlen32k_h32_s8", 32768, 32, 128, 128, 8, seed=3,
                                 varlen=True),
    "t65536_h32_s64": Workload("t65536_h32_s64", 65536, 32, 128, 128, 64, seed=4),
}

# Slow-decay stress variants (g scaled by 0.01) so that transitions and carries
# stay far from FP32 underflow and the composition is exercised for real.
STRESS = {
    "t4096_h8_s4_slow": Workload("t4096_h8_s4_slow", 4096, 8, 128, 128, 4, seed=101,
                                 gate_scale=0.01),
    "t65536_h32_s64_slow": Workload("t65536_h32_s64_slow", 65536, 32, 128, 128, 64,
                                    seed=104, gate_scale=0.01),
    # long memory: slow gates and weak writes (beta x 0.01), so every 1024-token
    # transition stays O(1) and the 63-step composition carries real products
    "t65536_h32_s64_longmem": Workload("t65536_h32_s64_longmem", 65536, 32, 128, 128, 64,
                                       seed=105, gate_scale=0.001, beta_scale=0.01),
}


def draw_lengths(gen: torch.Generator, total: int, lo: int, hi: int) -> list[int]:
    """Sequence lengths in [lo, hi] summing to ``total``; the last absorbs the rest."""
    lengths = []
    rem = total
    while rem > 0:
        if rem <= hi:
            L = rem
        else:
            L = int(torch.randint(lo, min(hi, rem - lo) + 1, (1,), generator=gen).item())
        lengths.append(L)
        rem -= L
    return lengths


def make_inputs(T: int, H: int, K: int, V: int, seed: int, *, cu_seqlens=None,
                varlen: bool = False, min_len: int = 512, max_len: int = 8192,
                gate_scale: float = 1.0, beta_scale: float = 1.0):
    """Return a dict of CPU tensors: q, k, g [T,H,K], v [T,H,V], beta [T,H] (bf16)
    and cu_seqlens (int32, [N+1])."""
    gen = torch.Generator("cpu").manual_seed(int(seed))
    if cu_seqlens is None:
        if varlen:
            lengths = draw_lengths(gen, T, min_len, max_len)
        else:
            lengths = [T]
        cu = [0]
        for L in lengths:
            cu.append(cu[-1] + L)
        cu_seqlens = torch.tensor(cu, dtype=torch.int32)
    else:
        cu_seqlens = torch.as_tensor(cu_seqlens, dtype=torch.int32)
    xq = torch.randn(T, H, K, generator=gen, dtype=torch.float32)
    xk = torch.randn(T, H, K, generator=gen, dtype=torch.float32)
    xv = torch.randn(T, H, V, generator=gen, dtype=torch.float32)
    xg = torch.randn(T, H, K, generator=gen, dtype=torch.float32)
    xb = torch.randn(T, H, generator=gen, dtype=torch.float32)
    q = xq / xq.norm(dim=-1, keepdim=True)
    k = xk / xk.norm(dim=-1, keepdim=True)
    g = -torch.nn.functional.softplus(xg) * gate_scale
    beta = torch.sigmoid(xb) * beta_scale
    return dict(
        q=q.to(torch.bfloat16), k=k.to(torch.bfloat16), v=xv.to(torch.bfloat16),
        g=g.to(torch.bfloat16), beta=beta.to(torch.bfloat16), cu_seqlens=cu_seqlens,
    )


def workload_inputs(w: Workload):
    """Inputs of a named workload (see ``WORKLOADS``)."""
    return make_inputs(w.T, w.H, w.K, w.V, w.seed, varlen=w.varlen, min_len=w.min_len,
                       max_len=w.max_len, gate_scale=w.gate_scale, beta_scale=w.beta_scale)


def initial_states(N: int, H: int, K: int, V: int, seed: int, scale: float = 0.5) -> torch.Tensor:
    """Per-sequence initial states [N, H, K, V], FP32, scale * N(0, 1) drawn from
    ``torch.Generator('cpu').manual_seed(seed)`` (no workload specifies one;
    these exercise the optional initial-state input)."""
    gen = torch.Generator("cpu").manual_seed(seed)
    return (scale * torch.randn(N, H, K, V, generator=gen, dtype=torch.float32)).contiguous()


def bits(t: torch.Tensor):
    """The raw 16-bit patterns of a bf16 tensor as a numpy uint16 array."""
    return t.contiguous().view(torch.int16).numpy().view("uint16")


def sha256(t: torch.Tensor) -> str:
    """SHA-256 of a tensor's bytes (for reproducibility reports)."""
    return hashlib.sha256(t.contiguous().view(torch.uint8).numpy().tobytes()).hexdigest()
