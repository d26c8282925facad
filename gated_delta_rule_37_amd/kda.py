"""Thin Python binding of the segmented KDA C-ABI library (``libkda.so``).

Argument marshalling only: every step of the forward pass runs in the HIP
kernels behind ``include/kda.h``.  PyTorch provides device memory and the
stream.  If the compiled library is missing, importing the entry points fails
loudly; there is no CPU fallback.

Entry points mirror the C names:

* :class:`Plan` (``kda_plan_segments`` / ``kda_plan_blob`` / ``kda_plan_destroy``)
* :func:`segment_summaries` (``kda_segment_summaries``)
* :func:`compose_summaries` (``kda_compose_summaries``)
* :func:`apply_carry` (``kda_apply_carry``)
* :func:`forward_call` (``kda_forward``): the three device calls in one C call
* :func:`forward_noalloc` (``kda_forward_noalloc``): the same without a
  caller workspace (the library's fixed per-GPU array instead)
* :func:`backward` (``kda_backward``): gradients of q, k, v, g, beta, h0
* :func:`forward` runs the three device calls in order (optionally per head
  group, with the compose launches on a second stream) on fresh output buffers.

Every device tensor is passed as its address and its size in bytes, so the
library can refuse an undersized buffer before it launches anything.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")

STATUS = {
    0: "KDA_OK",
    -1: "KDA_ERR_INVALID_ARG",
    -2: "KDA_ERR_BAD_CU_SEQLENS",
    -3: "KDA_ERR_BAD_SEGMENTS",
    -4: "KDA_ERR_UNSUPPORTED",
    -5: "KDA_ERR_MISALIGNED",
    -6: "KDA_ERR_HIP",
    -7: "KDA_ERR_NO_MEMORY",
    -8: "KDA_ERR_WORKSPACE_TOO_SMALL",
    -9: "KDA_ERR_BUFFER_TOO_SMALL",
}

# Every symbol include/kda.h declares.
SYMBOLS = (
    "kda_plan_segments", "kda_plan_segments_pieces", "kda_plan_pieces", "kda_plan_blob", "kda_plan_info",
    "kda_plan_destroy",
    "kda_summary_bytes", "kda_workspace_bytes", "kda_segment_summaries", "kda_compose_summaries",
    "kda_apply_carry", "kda_forward", "kda_forward_noalloc", "kda_noalloc_max_workspace_bytes",
    "kda_backward", "kda_backward_from_forward", "kda_backward_workspace_bytes", "kda_status_string", "kda_last_hip_error",
)


class KdaError(RuntimeError):
    """A negative status returned by the C library."""

    def __init__(self, status: int, where: str):
        name = STATUS.get(status, f"status {status}")
        extra = ""
        if status == -6:
            extra = f" (hipError_t {lib().kda_last_hip_error()})"
        super().__init__(f"{where}: {name}{extra}")
        self.status = status
        self.name = name


_lib = None


def lib() -> ctypes.CDLL:
    """Load ``libkda.so`` (built by ``__graft_entry__.build()``) once."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python -c 'import __graft_entry__ as g; g.build()')")
    L = ctypes.CDLL(LIB_PATH)
    i32, p, sz = ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
    L.kda_plan_segments.argtypes = [p, i32, i32, p, ctypes.POINTER(p)]
    L.kda_plan_segments.restype = ctypes.c_int
    L.kda_plan_segments_pieces.argtypes = [p, i32, i32, p, i32, ctypes.POINTER(p)]
    L.kda_plan_segments_pieces.restype = ctypes.c_int
    L.kda_plan_pieces.argtypes = [p, p]
    L.kda_plan_pieces.restype = ctypes.c_int
    L.kda_plan_blob.argtypes = [p, ctypes.POINTER(p), ctypes.POINTER(sz)]
    L.kda_plan_blob.restype = ctypes.c_int
    L.kda_plan_info.argtypes = [p, p, p, p, p]
    L.kda_plan_info.restype = ctypes.c_int
    L.kda_plan_destroy.argtypes = [p]
    L.kda_plan_destroy.restype = None
    L.kda_summary_bytes.argtypes = [p, i32, i32, i32]
    L.kda_summary_bytes.restype = sz
    L.kda_workspace_bytes.argtypes = [p, i32, i32, i32]
    L.kda_workspace_bytes.restype = sz
    buf = [p, sz]            # a device pointer and its size in bytes
    dims = [i32] * 5         # H, K, V, head_begin, head_count
    f32 = ctypes.c_float     # the safe gate's lower bound
    L.kda_segment_summaries.argtypes = [p, *buf, *buf * 4, f32, *buf, *dims, *buf, *buf, *buf, p]
    L.kda_segment_summaries.restype = ctypes.c_int
    L.kda_compose_summaries.argtypes = [p, *buf, *buf, *buf, *dims, *buf, p]
    L.kda_compose_summaries.restype = ctypes.c_int
    L.kda_apply_carry.argtypes = [p, *buf, *buf * 5, f32, *buf, *dims, *buf, *buf, i32, *buf, *buf, p]
    L.kda_apply_carry.restype = ctypes.c_int
    L.kda_forward.argtypes = [p, *buf, *buf * 5, f32, *buf, *dims, *buf, *buf, *buf, *buf, i32, *buf, *buf, p]
    L.kda_forward.restype = ctypes.c_int
    L.kda_forward_noalloc.argtypes = [p, *buf, *buf * 5, f32, *buf, *dims, *buf, *buf, *buf, *buf, i32, *buf, p]
    L.kda_forward_noalloc.restype = ctypes.c_int
    L.kda_backward.argtypes = [p, *buf, *buf * 5, *buf, *buf, *buf, *dims, *buf * 6, *buf, p]
    L.kda_backward.restype = ctypes.c_int
    L.kda_backward_from_forward.argtypes = [p, *buf, *buf * 5, *buf, *buf, *buf, *dims, *buf * 2, *buf * 6, *buf,
                                            p]
    L.kda_backward_from_forward.restype = ctypes.c_int
    L.kda_backward_workspace_bytes.argtypes = [p, i32, i32, i32]
    L.kda_backward_workspace_bytes.restype = sz
    L.kda_noalloc_max_workspace_bytes.argtypes = []
    L.kda_noalloc_max_workspace_bytes.restype = sz
    L.kda_status_string.argtypes = [ctypes.c_int]
    L.kda_status_string.restype = ctypes.c_char_p
    L.kda_last_hip_error.argtypes = []
    L.kda_last_hip_error.restype = ctypes.c_int
    _lib = L
    return L


def _check(status: int, where: str):
    if status != 0:
        raise KdaError(status, where)


class Plan:
    """Host-side segment plan (``kda_plan_segments_pieces``); reusable across
    calls.  ``piece_tokens`` > 0 (a multiple of 32) cuts every segment into
    pieces of that many tokens that run in parallel; the calls' results stay
    per segment.  ``S`` is the segment count, ``P`` the piece count (= S
    without pieces), ``bounds`` the segment bounds."""

    def __init__(self, cu_seqlens, num_segments: int, custom_bounds=None, piece_tokens: int = 0):
        L = lib()
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
        self._cu = cu
        bounds = None
        if custom_bounds is not None:
            bounds = np.ascontiguousarray(np.asarray(custom_bounds, dtype=np.int32))
        self._bounds = bounds
        handle = ctypes.c_void_p()
        st = L.kda_plan_segments_pieces(
            cu.ctypes.data, int(len(cu) - 1), int(num_segments),
            None if bounds is None else bounds.ctypes.data, int(piece_tokens), ctypes.byref(handle))
        _check(st, "kda_plan_segments_pieces")
        self._h = handle
        ptr = ctypes.c_void_p()
        n = ctypes.c_size_t()
        _check(L.kda_plan_blob(self._h, ctypes.byref(ptr), ctypes.byref(n)), "kda_plan_blob")
        arr = (ctypes.c_int32 * n.value).from_address(ptr.value)
        self.blob = np.array(arr, dtype=np.int32, copy=True)
        self.T, self.N, self.P, self.F = (int(x) for x in self.blob[:4])
        S = ctypes.c_int32()
        _check(L.kda_plan_info(self._h, None, None, ctypes.byref(S), None), "kda_plan_info")
        self.S = S.value
        self.pieces = self.P > self.S
        if self.pieces:
            # the segment-level block after the piece-level arrays: [S, bounds[S+1], ...]
            o = 4 + 6 * self.P + 2 + 6 * self.F + self.N
            assert int(self.blob[o]) == self.S
            self.bounds = self.blob[o + 1:o + 2 + self.S].copy()
            self.segment_live = self.blob[o + 2 + 2 * self.S:o + 2 + 3 * self.S].copy()
        else:
            self.bounds = self.blob[4:4 + self.S + 1].copy()
            self.segment_live = self.blob[4 + self.S + 1 + 3 * self.S:4 + self.S + 1 + 4 * self.S].copy()
        self._dev = {}

    @property
    def handle(self):
        return self._h

    def device_blob(self, device) -> torch.Tensor:
        """The caller-owned device copy of the blob (cached per device)."""
        device = torch.device(device)
        t = self._dev.get(device)
        if t is None:
            t = torch.from_numpy(self.blob.copy()).to(device)
            self._dev[device] = t
        return t

    def summary_bytes(self, H: int, K: int = 128, V: int = 128) -> int:
        return int(lib().kda_summary_bytes(self._h, H, K, V))

    def workspace_bytes(self, H: int, K: int = 128, V: int = 128) -> int:
        return int(lib().kda_workspace_bytes(self._h, H, K, V))

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().kda_plan_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _buf(t: torch.Tensor, dtype, shape, name: str):
    """(address, size in bytes) of a device tensor, after checking its dtype,
    shape and layout; None stands for an absent optional tensor."""
    if t is None:
        return (None, 0)
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a device tensor")
    return (t.data_ptr(), t.numel() * t.element_size())


def _stream(t: torch.Tensor, stream):
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(stream.cuda_stream)


def _inputs(plan: Plan, q, k, v, g, beta, initial_state, gate_lower_bound=None):
    """H, K, V and the flat argument list of (q,) k, v, g, beta (pointer, bytes
    each), the safe gate's lower bound and the initial states (q and
    initial_state may be None; no bound is -inf)."""
    T, H, K = k.shape
    V = v.shape[2]
    if T != plan.T:
        raise ValueError(f"inputs hold {T} tokens, the plan {plan.T}")
    bufs = [] if q is None else [_buf(q, torch.bfloat16, (T, H, K), "q")]
    bufs += [
        _buf(k, torch.bfloat16, (T, H, K), "k"), _buf(v, torch.bfloat16, (T, H, V), "v"),
        _buf(g, torch.bfloat16, (T, H, K), "g"), _buf(beta, torch.bfloat16, (T, H), "beta"),
    ]
    bound = float("-inf") if gate_lower_bound is None else float(gate_lower_bound)
    init = _buf(initial_state, torch.float32, (plan.N, H, K, V), "initial_state")
    return H, K, V, _flat(bufs) + [bound] + list(init)


def _flat(bufs):
    return [x for b in bufs for x in b]


def _heads(H: int, heads):
    """(head_begin, head_count) of a call: all heads when ``heads`` is None."""
    return (0, H) if heads is None else (int(heads[0]), int(heads[1]))


def _workspace(plan: Plan, H: int, workspace):
    return _buf(workspace, torch.uint8, (plan.workspace_bytes(H),), "workspace")


def _plan_dev(plan: Plan, plan_dev):
    return _buf(plan_dev, torch.int32, (len(plan.blob),), "plan_dev")


def segment_summaries(plan: Plan, plan_dev: torch.Tensor, k, v, g, beta, transitions, updates,
                      workspace, stream=None, heads=None, initial_state=None, gate_lower_bound=None):
    """``kda_segment_summaries``: the affine summary (A_r, B_r) of every segment,
    for the heads ``heads = (begin, count)`` (default: all).  Sequences start
    from ``initial_state`` [N, H, K, V] when given, else from zero."""
    H, K, V, ins = _inputs(plan, None, k, v, g, beta, initial_state, gate_lower_bound)
    outs = _flat([
        _buf(transitions, torch.float32, (plan.S, H, K, K), "transitions"),
        _buf(updates, torch.float32, (plan.S, H, K, V), "updates"),
        _workspace(plan, H, workspace),
    ])
    st = lib().kda_segment_summaries(plan.handle, *_plan_dev(plan, plan_dev), *ins, H, K, V,
                                     *_heads(H, heads), *outs, _stream(k, stream))
    _check(st, "kda_segment_summaries")


def compose_summaries(plan: Plan, plan_dev: torch.Tensor, transitions, updates, carry_in,
                      stream=None, heads=None):
    """``kda_compose_summaries``: ordered FP32 scan of the summaries."""
    S, H, K, _ = transitions.shape
    V = updates.shape[3]
    bufs = _flat([
        _buf(transitions, torch.float32, (plan.S, H, K, K), "transitions"),
        _buf(updates, torch.float32, (plan.S, H, K, V), "updates"),
    ])
    c = _buf(carry_in, torch.float32, (plan.S, H, K, V), "carry_in")
    st = lib().kda_compose_summaries(plan.handle, *_plan_dev(plan, plan_dev), *bufs, H, K, V,
                                     *_heads(H, heads), *c, _stream(transitions, stream))
    _check(st, "kda_compose_summaries")


def _o_buf(plan: Plan, o, H, V):
    if o.dtype not in O_FORMATS:
        raise TypeError(f"o: expected one of {list(O_FORMATS)}, got {o.dtype}")
    return _buf(o, o.dtype, (plan.T, H, V), "o"), O_FORMATS[o.dtype]


def apply_carry(plan: Plan, plan_dev: torch.Tensor, q, k, v, g, beta, carry_in, o, final_state,
                workspace, stream=None, heads=None, initial_state=None, gate_lower_bound=None):
    """``kda_apply_carry``: o and the final states, each segment from its carry-in C_r
    (a fragment that starts a sequence from ``initial_state``, else zero)."""
    H, K, V, ins = _inputs(plan, q, k, v, g, beta, initial_state, gate_lower_bound)
    c = _buf(carry_in, torch.float32, (plan.S, H, K, V), "carry_in")
    ob, fmt = _o_buf(plan, o, H, V)
    ff = _buf(final_state, torch.float32, (plan.N, H, K, V), "final_state")
    ws = _workspace(plan, H, workspace)
    st = lib().kda_apply_carry(plan.handle, *_plan_dev(plan, plan_dev), *ins, H, K, V, *_heads(H, heads),
                               *c, *ob, fmt, *ff, *ws, _stream(q, stream))
    _check(st, "kda_apply_carry")


def forward_call(plan: Plan, plan_dev: torch.Tensor, q, k, v, g, beta, out, stream=None, heads=None,
                 initial_state=None, gate_lower_bound=None):
    """``kda_forward``: summaries, compose and carry in one C call, into the
    buffers of ``out`` (as :func:`alloc_outputs` makes them)."""
    H, K, V, ins = _inputs(plan, q, k, v, g, beta, initial_state, gate_lower_bound)
    summ = _flat([
        _buf(out["transitions"], torch.float32, (plan.S, H, K, K), "transitions"),
        _buf(out["updates"], torch.float32, (plan.S, H, K, V), "updates"),
        _buf(out["carry_in"], torch.float32, (plan.S, H, K, V), "carry_in"),
    ])
    ob, fmt = _o_buf(plan, out["o"], H, V)
    ff = _buf(out["final_state"], torch.float32, (plan.N, H, K, V), "final_state")
    ws = _workspace(plan, H, out["workspace"])
    st = lib().kda_forward(plan.handle, *_plan_dev(plan, plan_dev), *ins, H, K, V, *_heads(H, heads),
                           *summ, *ob, fmt, *ff, *ws, _stream(q, stream))
    _check(st, "kda_forward")


def forward_noalloc(plan: Plan, plan_dev: torch.Tensor, q, k, v, g, beta, out, stream=None, heads=None,
                    initial_state=None, gate_lower_bound=None):
    """``kda_forward_noalloc``: :func:`forward_call` with the library's fixed
    workspace array (``out`` needs no "workspace" entry)."""
    H, K, V, ins = _inputs(plan, q, k, v, g, beta, initial_state, gate_lower_bound)
    summ = _flat([
        _buf(out["transitions"], torch.float32, (plan.S, H, K, K), "transitions"),
        _buf(out["updates"], torch.float32, (plan.S, H, K, V), "updates"),
        _buf(out["carry_in"], torch.float32, (plan.S, H, K, V), "carry_in"),
    ])
    ob, fmt = _o_buf(plan, out["o"], H, V)
    ff = _buf(out["final_state"], torch.float32, (plan.N, H, K, V), "final_state")
    st = lib().kda_forward_noalloc(plan.handle, *_plan_dev(plan, plan_dev), *ins, H, K, V, *_heads(H, heads),
                                   *summ, *ob, fmt, *ff, _stream(q, stream))
    _check(st, "kda_forward_noalloc")


def backward(plan: Plan, q, k, v, g, beta, d_o, d_final=None, initial_state=None, want_dh0=False,
             stream=None, heads=None, sentinel=None, saved=None):
    """``kda_backward``: gradients of L = sum <o, d_o> + sum <final, d_final>.
    Returns dict(dq, dk, dv, dg, dbeta, dh0) (fp32; dh0 None unless wanted).
    ``heads`` = (begin, count) restricts the call to those heads; the output
    buffers are filled with ``sentinel`` first when it is given.  ``saved`` =
    (transitions, carry_in) as the forward wrote them (no gate lower bound)
    calls ``kda_backward_from_forward``, which reads them instead of
    recomputing them."""
    T, H, K = k.shape
    V = v.shape[2]
    dev = q.device
    f32 = dict(dtype=torch.float32, device=dev)
    make = (lambda *shape: torch.empty(*shape, **f32)) if sentinel is None else (
        lambda *shape: torch.full(shape, float(sentinel), **f32))
    out = dict(dq=make(T, H, K), dk=make(T, H, K), dv=make(T, H, V), dg=make(T, H, K), dbeta=make(T, H),
               dh0=make(plan.N, H, K, V) if want_dh0 else None)
    ins = _flat([
        _buf(q, torch.bfloat16, (T, H, K), "q"), _buf(k, torch.bfloat16, (T, H, K), "k"),
        _buf(v, torch.bfloat16, (T, H, V), "v"), _buf(g, torch.bfloat16, (T, H, K), "g"),
        _buf(beta, torch.bfloat16, (T, H), "beta"),
        _buf(initial_state, torch.float32, (plan.N, H, K, V), "initial_state"),
        _buf(d_o, torch.float32, (T, H, V), "d_o"),
        _buf(d_final, torch.float32, (plan.N, H, K, V), "d_final"),
    ])
    grads = _flat([
        _buf(out["dq"], torch.float32, None, "dq"), _buf(out["dk"], torch.float32, None, "dk"),
        _buf(out["dv"], torch.float32, None, "dv"), _buf(out["dg"], torch.float32, None, "dg"),
        _buf(out["dbeta"], torch.float32, None, "dbeta"), _buf(out["dh0"], torch.float32, None, "dh0"),
    ])
    ws_bytes = int(lib().kda_backward_workspace_bytes(plan.handle, H, K, V))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    if saved is None:
        st = lib().kda_backward(plan.handle, *_plan_dev(plan, plan.device_blob(dev)), *ins, H, K, V,
                                *_heads(H, heads), *grads, *_buf(ws, torch.uint8, None, "workspace"),
                                _stream(q, stream))
        _check(st, "kda_backward")
        return out
    kept = _flat([_buf(saved[0], torch.float32, (plan.S, H, K, V), "transitions"),
                  _buf(saved[1], torch.float32, (plan.S, H, K, V), "carry_in")])
    st = lib().kda_backward_from_forward(plan.handle, *_plan_dev(plan, plan.device_blob(dev)), *ins, H, K, V,
                                         *_heads(H, heads), *kept, *grads,
                                         *_buf(ws, torch.uint8, None, "workspace"), _stream(q, stream))
    _check(st, "kda_backward_from_forward")
    return out


def noalloc_max_workspace_bytes() -> int:
    return int(lib().kda_noalloc_max_workspace_bytes())


# storage formats of o accepted by kda_apply_carry (kda_o_format)
O_FORMATS = {torch.float32: 0, torch.bfloat16: 1}


def auto_piece_tokens(cu_seqlens, num_segments: int, H: int, custom_bounds=None, target_items: int = 256,
                      min_piece: int = 128) -> int:
    """A piece length for ``Plan(..., piece_tokens=...)``: 0 (no pieces) when the
    plain plan already gives the GPU's 256 compute units a (fragment, head)
    item each; else the multiple of 32, at least ``min_piece``, that makes
    about ``target_items`` pieces times heads (0 if no segment is longer).
    Measured on the three small workloads (65536 tokens and more need none):
    about one item per compute unit, with pieces of at least 128 tokens, is
    where the shorter chunk chains stop paying for the longer scans."""
    plain = Plan(cu_seqlens, num_segments, custom_bounds)
    if plain.F * H >= 256:
        return 0
    b = plain.bounds
    longest = int(np.max(b[1:] - b[:-1]))
    L = max(int(min_piece), 32 * -(-(plain.T * H) // (int(target_items) * 32)))
    return L if L < longest else 0


def alloc_outputs(plan: Plan, H: int, K: int, V: int, device, o_dtype=torch.float32):
    """Fresh output buffers (o, final_state, transitions, updates, carry_in) and
    the workspace shared by the summaries and carry passes.  ``o_dtype`` is
    float32, or bfloat16 for the rounded BF16 output."""
    f32 = dict(dtype=torch.float32, device=device)
    return dict(
        o=torch.empty(plan.T, H, V, dtype=o_dtype, device=device),
        final_state=torch.empty(plan.N, H, K, V, **f32),
        transitions=torch.empty(plan.S, H, K, K, **f32),
        updates=torch.empty(plan.S, H, K, V, **f32),
        carry_in=torch.empty(plan.S, H, K, V, **f32),
        workspace=torch.empty(plan.workspace_bytes(H, K, V), dtype=torch.uint8, device=device),
    )


def head_groups(H: int, groups: int):
    """Split heads 0..H-1 into at most ``groups`` contiguous (begin, count) runs."""
    groups = max(1, min(int(groups), H))
    base, extra = divmod(H, groups)
    runs, h = [], 0
    for i in range(groups):
        n = base + (1 if i < extra else 0)
        runs.append((h, n))
        h += n
    return runs


_side_streams = {}


def _side_stream(device) -> torch.cuda.Stream:
    """A second stream per device (default priority) for the compose launches."""
    device = torch.device(device)
    s = _side_streams.get(device)
    if s is None:
        s = torch.cuda.Stream(device=device)
        _side_streams[device] = s
    return s


def forward(plan: Plan, q, k, v, g, beta, out=None, stream=None, groups=1, events=None,
            initial_state=None, o_dtype=torch.float32, gate_lower_bound=None):
    """The whole segmented forward: summaries, compose, carry.  Returns ``out``.
    Sequence n starts from ``initial_state[n]`` ([N, H, K, V] FP32) when given,
    else from zero.  ``o_dtype`` (used when ``out`` is None) is float32 or
    bfloat16.

    With ``groups`` > 1 the heads are cut into that many groups.  Summaries and
    carry launches of every group run in order on ``stream``; each group's
    compose runs on a second stream as soon as its summaries are done, so it
    overlaps the next groups' summaries and the earlier groups' carry.  Heads
    are independent, so the results do not depend on ``groups``.

    ``events``, if given, is a dict that receives per-launch (start, end) HIP
    event pairs under "summaries", "compose" and "carry", each recorded on the
    stream of its launch (for timing)."""
    T, H, K = q.shape
    V = v.shape[2]
    if out is None:
        out = alloc_outputs(plan, H, K, V, q.device, o_dtype)
    pd = plan.device_blob(q.device)
    main = torch.cuda.current_stream(q.device) if stream is None else stream
    runs = head_groups(H, groups)

    def timed(kind, st, fn):
        if events is None:
            fn()
            return
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(st)
        fn()
        e1.record(st)
        events.setdefault(kind, []).append((e0, e1))

    if len(runs) == 1:
        timed("summaries", main, lambda: segment_summaries(
            plan, pd, k, v, g, beta, out["transitions"], out["updates"], out["workspace"], main,
            initial_state=initial_state, gate_lower_bound=gate_lower_bound))
        timed("compose", main, lambda: compose_summaries(
            plan, pd, out["transitions"], out["updates"], out["carry_in"], main))
        timed("carry", main, lambda: apply_carry(
            plan, pd, q, k, v, g, beta, out["carry_in"], out["o"], out["final_state"],
            out["workspace"], main, initial_state=initial_state, gate_lower_bound=gate_lower_bound))
        return out

    side = _side_stream(q.device)
    done_s, done_c = [], []
    for hr in runs:
        timed("summaries", main, lambda hr=hr: segment_summaries(
            plan, pd, k, v, g, beta, out["transitions"], out["updates"], out["workspace"], main,
            heads=hr, initial_state=initial_state, gate_lower_bound=gate_lower_bound))
        ev = torch.cuda.Event()
        ev.record(main)
        done_s.append(ev)
    for hr, ev in zip(runs, done_s):
        side.wait_event(ev)
        timed("compose", side, lambda hr=hr: compose_summaries(
            plan, pd, out["transitions"], out["updates"], out["carry_in"], side, heads=hr))
        evc = torch.cuda.Event()
        evc.record(side)
        done_c.append(evc)
    for hr, evc in zip(runs, done_c):
        main.wait_event(evc)
        timed("carry", main, lambda hr=hr: apply_carry(
            plan, pd, q, k, v, g, beta, out["carry_in"], out["o"], out["final_state"],
            out["workspace"], main, heads=hr, initial_state=initial_state,
            gate_lower_bound=gate_lower_bound))
    # every launch on the side stream precedes the last carry launch on main,
    # so work issued later on main is ordered after all of it
    return out
