"""Reference segment plan over packed sequences (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this module.

[cuLA#136] Walkthrough (change table, "Packed-shard planning"): a CPU-only plan
of balanced or custom contiguous shards over the global sequence boundaries,
validated, and tested on sequence boundaries, rank spans and invalid inputs;
Summary by CodeRabbit: reusable shard plans for packed sequences.  Segments are
the one-GPU stand-in for those shards.

Readings (the pages leave these open):
  * balanced bounds are b_r = floor(r * T / S);
  * custom bounds must satisfy 0 = b_0 < b_1 < ... < b_S = T;
  * every sequence is non-empty (cu_seqlens strictly increasing from 0);
  * a segment "carries in" when r > 0 and b_r is not a sequence start;
  * its transition is "live" when it carries in and no sequence starts inside it.

The plan is serialised as one int32 vector (the "blob"):
  header  [T, N, S, F]
  seg_bounds[S+1], seg_first_seq[S], seg_last_seq[S], seg_carry_in[S],
  seg_transition_live[S], seg_frag_ptr[S+1],
  frag_seq[F], frag_begin[F], frag_end[F], frag_seg[F], frag_flags[F],
  seq_end_seg[N], frag_order[F]
frag_flags bits: 1 = first fragment of a carrying segment, 2 = ends at its
segment's end, 4 = ends at its sequence's end.  frag_order lists the fragments
longest first (ties by index): the order in which they are worth starting, so
that the long sequential ones do not start last (a scheduling choice, not part
of the method).

Pieces (a one-GPU scheduling choice, not on the pages): with piece_tokens > 0
(a multiple of 32) every segment is cut every piece_tokens tokens from its
start, the last piece shorter.  The arrays above then describe the P pieces
(header [T, N, P, F]), and when P > S the blob ends with the segments' own
block: S, seg_bounds[S+1], seg_carry_in[S], seg_transition_live[S],
piece_ptr[S+1] (segment r owns pieces [piece_ptr[r], piece_ptr[r+1])).
Without pieces (or when no segment is longer than piece_tokens) the blob is
exactly the plain one.
"""
from __future__ import annotations

import numpy as np

FRAG_CARRIED = 1
FRAG_SEG_LAST = 2
FRAG_SEQ_END = 4


class PlanError(ValueError):
    """Raised for inputs the plan rejects; ``kind`` names the class of error."""

    def __init__(self, kind: str, msg: str):
        super().__init__(f"{kind}: {msg}")
        self.kind = kind


def _seq_of_token(cu, t):
    """Index n with cu[n] <= t < cu[n+1] (linear scan; the oracle is slow on purpose)."""
    for n in range(len(cu) - 1):
        if cu[n] <= t < cu[n + 1]:
            return n
    raise AssertionError("token outside every sequence")


def _flags(cu, bounds):
    """Per span of ``bounds``: first and last sequence, carry-in, live."""
    starts = set(cu[:-1])
    R = len(bounds) - 1
    first = [_seq_of_token(cu, bounds[r]) for r in range(R)]
    last = [_seq_of_token(cu, bounds[r + 1] - 1) for r in range(R)]
    carry = [1 if (r > 0 and bounds[r] not in starts) else 0 for r in range(R)]
    live = [1 if (carry[r] and first[r] == last[r]) else 0 for r in range(R)]
    return first, last, carry, live


def build_plan(cu_seqlens, num_segments, custom_bounds=None, piece_tokens=0):
    """Return the plan as a dict of python lists plus the int32 blob."""
    cu = [int(x) for x in cu_seqlens]
    if len(cu) < 2:
        raise PlanError("BAD_CU_SEQLENS", "need at least one sequence")
    if cu[0] != 0:
        raise PlanError("BAD_CU_SEQLENS", "cu_seqlens[0] must be 0")
    for n in range(len(cu) - 1):
        if cu[n + 1] <= cu[n]:
            raise PlanError("BAD_CU_SEQLENS", "sequence lengths must be positive")
    T = cu[-1]
    N = len(cu) - 1
    S = int(num_segments)
    if S < 1 or S > T:
        raise PlanError("BAD_SEGMENTS", "need 1 <= num_segments <= T")
    if custom_bounds is None:
        bounds = [(r * T) // S for r in range(S + 1)]
    else:
        bounds = [int(x) for x in custom_bounds]
        if len(bounds) != S + 1 or bounds[0] != 0 or bounds[-1] != T:
            raise PlanError("BAD_SEGMENTS", "custom bounds must run from 0 to T")
        for r in range(S):
            if bounds[r + 1] <= bounds[r]:
                raise PlanError("BAD_SEGMENTS", "custom bounds must be strictly increasing")

    piece_tokens = int(piece_tokens)
    if piece_tokens < 0 or piece_tokens % 32:
        raise PlanError("BAD_SEGMENTS", "piece_tokens must be a non-negative multiple of 32")
    seg_bounds = bounds
    pbounds, piece_ptr = [], []
    for r in range(S):
        piece_ptr.append(len(pbounds))
        x = seg_bounds[r]
        while x < seg_bounds[r + 1]:
            pbounds.append(x)
            if piece_tokens == 0:
                break
            x += piece_tokens
    piece_ptr.append(len(pbounds))
    pbounds.append(T)
    P = len(pbounds) - 1
    pieces = P > S
    bounds = pbounds           # everything below is per piece
    seg_first, seg_last, carry, live = _flags(cu, bounds)

    frag_ptr = [0]
    f_seq, f_beg, f_end, f_seg, f_flags = [], [], [], [], []
    for r in range(P):
        for n in range(seg_first[r], seg_last[r] + 1):
            b = max(bounds[r], cu[n])
            e = min(bounds[r + 1], cu[n + 1])
            flags = 0
            if b == bounds[r] and carry[r]:
                flags |= FRAG_CARRIED
            if e == bounds[r + 1]:
                flags |= FRAG_SEG_LAST
            if e == cu[n + 1]:
                flags |= FRAG_SEQ_END
            f_seq.append(n)
            f_beg.append(b)
            f_end.append(e)
            f_seg.append(r)
            f_flags.append(flags)
        frag_ptr.append(len(f_seq))
    F = len(f_seq)
    # the segment holding the sequence's last token (bounds partition [0, T) like cu_seqlens)
    seq_end_seg = [_seq_of_token(bounds, cu[n + 1] - 1) for n in range(N)]
    frag_order = sorted(range(F), key=lambda f: (-(f_end[f] - f_beg[f]), f))

    plan = dict(
        T=T, N=N, S=P, F=F,
        seg_bounds=bounds, seg_first_seq=seg_first, seg_last_seq=seg_last,
        seg_carry_in=carry, seg_transition_live=live, seg_frag_ptr=frag_ptr,
        frag_seq=f_seq, frag_begin=f_beg, frag_end=f_end, frag_seg=f_seg,
        frag_flags=f_flags, seq_end_seg=seq_end_seg, frag_order=frag_order,
    )
    blob = [T, N, P, F]
    for key in ("seg_bounds", "seg_first_seq", "seg_last_seq", "seg_carry_in",
                "seg_transition_live", "seg_frag_ptr", "frag_seq", "frag_begin",
                "frag_end", "frag_seg", "frag_flags", "seq_end_seg", "frag_order"):
        blob.extend(plan[key])
    plan["segments"] = S
    plan["segment_bounds"] = seg_bounds
    plan["piece_ptr"] = piece_ptr
    if pieces:
        _, _, ucarry, ulive = _flags(cu, seg_bounds)
        blob.append(S)
        blob.extend(seg_bounds)
        blob.extend(ucarry)
        blob.extend(ulive)
        blob.extend(piece_ptr)
    plan["blob"] = np.asarray(blob, dtype=np.int32)
    return plan
