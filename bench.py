"""Benchmark of the segmented KDA forward pass on one MI355X.

One step = one whole forward over one batch of resident synthetic input:
kda_segment_summaries + kda_compose_summaries + kda_apply_carry over all
heads (the plan is built once and reused, as the pages' reusable shard plans
are).  The heads are cut into --groups groups: summaries and carry launches run
on the main stream, each group's compose on a second stream once that group's
summaries are done.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--groups G]

Workload default: 65536 packed tokens of one sequence, H = 32, K = V = 128, 64
equal segments (the 64-shard, 32-head configuration whose FP32 summary
workspace is 256 MiB).  Inputs follow gated_delta_rule_37_amd/synth.py.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published peaks
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP32_TFLOPS = 157.3      # dense FP32 matrix cores
HOST_CORE_SHARE = 16          # host cores one GPU's share of the box gives a job

# Algorithmic multiply-adds per token-head of the chunked method at chunk C=32,
# K = V = 128 (triangular products counted exactly, FP32-grade):
C, K, V = 32, 128, 128
TRI_STRICT = (C - 1) / 2 * K      # A = beta (K K^T) strictly lower
TRI_INCL = (C + 1) / 2 * K        # P, W = T(...), U~ = T V, P U (lower incl. diagonal)
STATE = K * V                     # one K x V product per token (W S, Q S, K^T U)
MACS = {
    "fwd": TRI_STRICT + 4 * TRI_INCL + 3 * STATE,
    # forward over chunks whose T diag(beta) the summaries launch left in the
    # chunk cache: no A, no T
    "fwd_cached": 3 * TRI_INCL + 3 * STATE,
    "sum_s": TRI_STRICT + 2 * TRI_INCL + 2 * STATE,
    "sum_phi": TRI_STRICT + TRI_INCL + 2 * K * K,
}
# bf16 MFMA work as executed: split operands cost three products, raw BF16 V
# against a split operand two.
MFMA_MACS = {
    "fwd": 3 * MACS["fwd"] - TRI_INCL,
    "fwd_cached": 3 * MACS["fwd_cached"] - TRI_INCL,
    "sum_s": 3 * MACS["sum_s"] - TRI_INCL,
    "sum_phi": 3 * MACS["sum_phi"],
}
# HBM bytes per token-head: bf16 inputs read, fp32 o written.
BYTES = {
    "fwd": 4 * 2 * K + 2 + 4 * V,   # q, k, v, g, beta in; o out
    "sum_s": 3 * 2 * K + 2,         # k, v, g, beta
    "sum_phi": 2 * 2 * K + 2,       # k, g, beta
}
STATE_BYTES = K * V * 4


def chunk_kernel_work(blob, H, o_bytes=4):
    """Algorithmic MACs, executed bf16 MFMA MACs and HBM bytes of the two chunk
    launches, from the plan blob: {"summaries": ..., "carry": ...}
    (kda_chunk_kernel, then kda_carry_kernel).  ``o_bytes`` is the size of one
    element of o (4 for FP32, 2 for the BF16 output)."""
    T, N, S, F = (int(x) for x in blob[:4])
    o = 4
    o += S + 1          # seg_bounds
    o += 2 * S          # first, last
    o += S              # carry
    seg_live = blob[o:o + S]; o += S
    o += S + 1          # frag_ptr
    f_seq = blob[o:o + F]; o += F
    f_beg = blob[o:o + F]; o += F
    f_end = blob[o:o + F]; o += F
    f_seg = blob[o:o + F]; o += F
    f_flags = blob[o:o + F]
    work = {k: {"macs": 0.0, "mfma_macs": 0.0, "bytes": 0.0} for k in ("summaries", "carry")}

    def add(launch, mode, L):
        work[launch]["macs"] += MACS[mode] * L * H
        work[launch]["mfma_macs"] += MFMA_MACS[mode] * L * H
        work[launch]["bytes"] += BYTES[mode] * L * H

    for f in range(F):
        L = int(f_end[f] - f_beg[f])
        fl = int(f_flags[f])
        carried, seg_last, seq_end = (fl & 1) > 0, (fl & 2) > 0, (fl & 4) > 0
        if seg_last:                     # summaries: B_r from zero, A_r from identity
            add("summaries", "sum_s", L)
            if carried and int(seg_live[int(f_seg[f])]) != 0:
                # one workgroup builds both: inputs read once
                work["summaries"]["macs"] += MACS["sum_phi"] * L * H
                work["summaries"]["mfma_macs"] += MFMA_MACS["sum_phi"] * L * H
            work["summaries"]["bytes"] += 2 * STATE_BYTES * H
        # carry: o and the final state of every fragment, from C_r or zero
        work["carry"]["macs"] += MACS["fwd_cached" if seg_last else "fwd"] * L * H
        work["carry"]["mfma_macs"] += MFMA_MACS["fwd_cached" if seg_last else "fwd"] * L * H
        work["carry"]["bytes"] += (BYTES["fwd"] - (4 - o_bytes) * V) * L * H + STATE_BYTES * H * (carried + seq_end)
    return work


def compose_work(S, H, live_count):
    """The ordered scan: one K x K by K x V product per live transition, on
    FP32 matrix cores; reads A_r (live ones) and B_r, writes every C_r."""
    macs = live_count * H * K * K * V
    bytes_ = (S - 1) * H * (K * V * 4) + live_count * H * K * K * 4 + S * H * K * V * 4
    return {"macs": macs, "bytes": bytes_}


_CPU_SAMPLE = {}


def _oracle_head(h):
    """The fp64 oracle over one head of the CPU sample (a pool worker)."""
    from threadpoolctl import threadpool_limits

    from oracle import kda_oracle as ko

    f, cu, bounds = _CPU_SAMPLE["f"], _CPU_SAMPLE["cu"], _CPU_SAMPLE["bounds"]
    one = {n: a[:, h:h + 1] for n, a in f.items()}
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        ko.recurrence(one["q"], one["k"], one["v"], one["g"], one["beta"], cu)
        A = ko.segment_transitions(one["k"], one["g"], one["beta"], cu, bounds)
        B = ko.segment_updates(one["k"], one["v"], one["g"], one["beta"], cu, bounds)
        ko.compose(A, B)
        return time.perf_counter() - t0


def cpu_baseline(x, w, tokens=65536):
    """The fp64 oracle timed on the host's cores: one process per core (at most
    the one-GPU share of the box), each running the whole method (monolithic o
    and final state, transitions, updates, composition) on one head of a
    bounded sample, the first ``tokens`` tokens with the workload's segment
    length; scaled to tokens/s over all H heads.  Must run before the process
    touches the GPU (the pool forks)."""
    import multiprocessing as mp

    from gated_delta_rule_37_amd import synth
    from oracle import kda_oracle as ko

    cores = min(len(os.sched_getaffinity(0)), HOST_CORE_SHARE)
    heads = min(cores, w.H)
    tokens = min(tokens, w.T)
    seg_len = w.T // w.segments
    cu_full = x["cu_seqlens"].tolist()
    cu = [c for c in cu_full if c < tokens] + [tokens]
    _CPU_SAMPLE["f"] = {n: ko.decode_bf16(synth.bits(x[n][:tokens, :heads]))
                        for n in ("q", "k", "v", "g", "beta")}
    _CPU_SAMPLE["cu"] = cu
    _CPU_SAMPLE["bounds"] = list(range(0, tokens, seg_len)) + [tokens]
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(heads) as pool:
        per_head = pool.map(_oracle_head, range(heads))
    wall = time.perf_counter() - t0
    return {
        "value": round(tokens * heads / w.H / wall, 3),
        "unit": "tokens/s",
        "cores": heads,
        "kind": "oracle",
        "sample": f"heads 0..{heads - 1} of {w.H} (one per process, BLAS 1 thread), tokens [0, {tokens}) "
                  f"of {w.name}, {len(_CPU_SAMPLE['bounds']) - 1} segments of {seg_len}; monolithic o + "
                  f"final, transitions, updates, composition; fp64 numpy; wall {wall:.1f} s "
                  f"(per head {min(per_head):.1f}-{max(per_head):.1f} s); scaled to all {w.H} heads",
    }


def traffic_from_profile(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed PMC summary, if it was
    taken on the current kernel source and this workload (default options);
    else None."""
    path = TRAFFIC_JSON
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("workload") != workload:
        return None
    digest = hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()
    if rec.get("kernel_source_sha256") != digest:
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_launch")


TRAFFIC_JSON = os.path.join(ROOT, "profiles", "chunk_kernel_t65536_h32_s64_traffic.json")
KERNEL_SRC = os.path.join(ROOT, "gated_delta_rule_37_amd", "csrc", "kda_kernels.hip")


def _pmc_per_dispatch(csv_path, counter, name_part):
    """Per-dispatch values of one counter for kernels whose name contains name_part."""
    import csv
    vals = {}
    for r in csv.DictReader(open(csv_path)):
        if r["Counter_Name"] != counter or name_part not in r["Kernel_Name"]:
            continue
        vals[r["Dispatch_Id"]] = vals.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return [vals[k] for k in sorted(vals, key=int)]


def summarize_traffic(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, copy_bytes):
    """HBM bytes per launch of each chunk kernel from rocprofv3 --pmc FETCH_SIZE /
    WRITE_SIZE runs (KiB per dispatch), each scaled by what the same counter reads
    for a plain device copy of copy_bytes (FETCH reads and WRITE writes copy_bytes
    once)."""
    cf = _pmc_per_dispatch(copy_fetch_csv, "FETCH_SIZE", "copy")
    cw = _pmc_per_dispatch(copy_write_csv, "WRITE_SIZE", "copy")
    big_f = max(cf)
    big_w = max(cw)
    f_scale = copy_bytes / (big_f * 1024.0)
    w_scale = copy_bytes / (big_w * 1024.0)
    kernels = {}
    for name in ("kda_chunk_kernel", "kda_carry_kernel"):
        kf = _pmc_per_dispatch(fetch_csv, "FETCH_SIZE", name)
        kw = _pmc_per_dispatch(write_csv, "WRITE_SIZE", name)
        if not kf or not kw:
            continue
        fetch_b = sum(kf) / len(kf) * 1024.0 * f_scale
        write_b = sum(kw) / len(kw) * 1024.0 * w_scale
        kernels[name] = {"bytes_per_launch": round(fetch_b + write_b),
                         "fetch_bytes_per_launch": round(fetch_b),
                         "write_bytes_per_launch": round(write_b),
                         "launches_averaged": len(kf)}
    rec = {
        "workload": "t65536_h32_s64",
        "kernels": kernels,
        "copy_calibration": {"bytes": copy_bytes, "fetch_kib": big_f, "write_kib": big_w,
                             "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4)},
        "kernel_source_sha256": hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest(),
    }
    with open(TRAFFIC_JSON, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec))


def copy_calibration(nbytes):
    """A plain device-to-device copy of nbytes, run three times (PMC calibration)."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="t65536_h32_s64")
    ap.add_argument("--groups", type=int, default=1,
                    help="head groups per step; each group's compose overlaps other groups' work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--initial-state", action="store_true",
                    help="give every sequence a (seeded, random) initial state")
    ap.add_argument("--o-bf16", action="store_true", help="store o as BF16 (rounded FP32 result)")
    ap.add_argument("--cpu-tokens", type=int, default=65536,
                    help="tokens of the CPU oracle's sample (one head per host core)")
    ap.add_argument("--no-pages-timing", action="store_true",
                    help="skip the pages' timing method (20 warmups, 60 iterations, 5 repeats)")
    ap.add_argument("--all-workloads", action="store_true",
                    help="one JSON line per workload (pages' timing method; no CPU leg)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device copy of this many bytes (PMC calibration)")
    ap.add_argument("--summarize-traffic", nargs=4, metavar="CSV",
                    help="fetch.csv write.csv copy_fetch.csv copy_write.csv from rocprofv3 --pmc runs")
    ap.add_argument("--copy-bytes-used", type=int, default=1 << 30)
    ap.add_argument("--pieces", default="auto",
                    help="piece length in tokens (a multiple of 32), 0 for none, or 'auto': pieces only "
                         "where segments x heads leave compute units idle (kda.auto_piece_tokens)")
    ap.add_argument("--backward-steps", type=int, default=3,
                    help="timed calls of the backward (kda_backward) on the same workload; 0: none")
    args = ap.parse_args()
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic, args.copy_bytes_used)
        return
    if args.copy_bytes:
        copy_calibration(args.copy_bytes)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build runs on one GPU only; the segments stand in for the "
              "context-parallel ranks on that GPU (no collectives). Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from gated_delta_rule_37_amd import kda, synth

    if args.all_workloads:
        # one line per workload, the pages' timing method only (no CPU leg)
        for name in list(synth.WORKLOADS) + list(synth.STRESS):
            w = synth.WORKLOADS.get(name) or synth.STRESS[name]
            x = synth.workload_inputs(w)
            res = measure(args, w, x, torch, kda, synth)
            if args.backward_steps > 0:
                res["backward"] = measure_backward(args, w, x, torch, kda)
            print(json.dumps(res), flush=True)
            del x, res
            torch.cuda.empty_cache()
        return

    w = synth.WORKLOADS.get(args.workload) or synth.STRESS[args.workload]
    x = synth.workload_inputs(w)
    # the CPU leg runs first: its process pool forks, which must happen before
    # this process touches the GPU
    cpu = None if args.no_cpu_baseline else cpu_baseline(x, w, args.cpu_tokens)
    res = measure(args, w, x, torch, kda, synth)
    res["cpu_baseline"] = cpu
    if args.backward_steps > 0:
        res["backward"] = measure_backward(args, w, x, torch, kda)
    print(json.dumps(res), flush=True)


def _median(v):
    v = sorted(v)
    n = len(v)
    return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


def pages_timing(step, torch, repeats=5, warmup=20, iters=60):
    """The pages' GPU timing method: 20 warmups and 60 timed iterations per
    repeat, 5 repeats, the median of each repeat's per-launch medians (HIP
    events on each launch's stream).  Returns ms per launch kind and their sum
    per step."""
    meds = {}
    for _ in range(repeats):
        for _ in range(warmup):
            step()
        ev = {}
        for _ in range(iters):
            step(ev)
        torch.cuda.synchronize()
        per = {kind: [a.elapsed_time(b) for a, b in pairs] for kind, pairs in ev.items()}
        n = len(per["summaries"]) // iters   # launches of a kind per step (head groups)
        for kind, times in per.items():
            # sum the launches of one step, then the median over steps
            step_sums = [sum(times[i * n:(i + 1) * n]) for i in range(iters)]
            meds.setdefault(kind, []).append(_median(step_sums))
    out = {kind: round(_median(v), 4) for kind, v in meds.items()}
    out["step_launch_sum"] = round(sum(out[k] for k in ("summaries", "compose", "carry")), 4)
    out["method"] = f"{repeats} repeats x ({warmup} warmups + {iters} timed), median of per-repeat medians"
    return out


def piece_tokens(args, kda, cu, w):
    """The plan's piece length: --pieces, or the binding's rule for 'auto'."""
    if args.pieces == "auto":
        return kda.auto_piece_tokens(cu, w.segments, w.H)
    return int(args.pieces)


def measure(args, w, x, torch, kda, synth):
    """Time the whole forward on one workload (inputs resident on the GPU):
    the driver's K timed steps, then the pages' method; return the JSON line."""
    dev = torch.device("cuda:0")
    d = {n: x[n].to(dev) for n in ("q", "k", "v", "g", "beta")}
    cu = x["cu_seqlens"].tolist()
    pieces = piece_tokens(args, kda, cu, w)
    plan = kda.Plan(cu, w.segments, None, pieces)
    out = kda.alloc_outputs(plan, w.H, w.K, w.V, dev, torch.bfloat16 if args.o_bf16 else torch.float32)
    h0 = None
    if args.initial_state:
        h0 = synth.initial_states(plan.N, w.H, w.K, w.V, seed=w.seed + 1000).to(dev)

    def step(ev=None):
        kda.forward(plan, d["q"], d["k"], d["v"], d["g"], d["beta"], out=out, groups=args.groups,
                    events=ev, initial_state=h0)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = {}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    pages = pages_timing(step, torch) if not args.no_pages_timing else None

    # per launch: each kind has steps * groups launches, each over one head group
    n_launch = {kind: len(pairs) for kind, pairs in events.items()}
    launch_ms = {kind: sum(a.elapsed_time(b) for a, b in pairs) / len(pairs)
                 for kind, pairs in events.items()}
    per_step = {kind: launch_ms[kind] * n_launch[kind] / args.steps for kind in launch_ms}
    groups = n_launch["summaries"] // args.steps
    pass1_ms, compose_ms, pass2_ms = per_step["summaries"], per_step["compose"], per_step["carry"]

    blob = plan.blob
    cw = chunk_kernel_work(blob, w.H, 2 if args.o_bf16 else 4)
    # one launch covers 1/groups of the heads: its work is the step's / groups
    # (groups of equal size; the bench workload's 32 heads split evenly)
    launches = {"kda_chunk_kernel": (cw["summaries"], launch_ms["summaries"]),
                "kda_carry_kernel": (cw["carry"], launch_ms["carry"])}

    def roofline(name):
        wk, ms = launches[name]
        wk = {key: val / groups for key, val in wk.items()}
        t_mfma = wk["mfma_macs"] * 2 / (PEAK_BF16_TFLOPS * 1e12) * 1e3
        t_hbm = wk["bytes"] / (PEAK_HBM_GBS * 1e9) * 1e3
        if t_mfma >= t_hbm:
            achieved = wk["mfma_macs"] * 2 / (ms * 1e-3) / 1e12
            r = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                 "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4)}
        else:
            achieved = wk["bytes"] / (ms * 1e-3) / 1e9
            r = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                 "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}
        # the committed counters were taken with one launch per step, FP32 o
        # and no initial states
        default_opts = groups == 1 and not args.o_bf16 and not args.initial_state
        r["traffic"] = traffic_from_profile(name, w.name) if default_opts else None
        r["kernel"] = name
        r["launch_ms_avg"] = round(ms, 4)
        r["launches_per_step"] = groups
        r["bounds_ms"] = {"mfma": round(t_mfma, 4), "hbm": round(t_hbm, 4)}
        # the method's own FP32-grade multiply-adds (each split-bf16 product
        # above executes about three bf16 ones) against the FP32 matrix peak
        fp32 = wk["macs"] * 2 / (ms * 1e-3) / 1e12
        r["fp32grade"] = {"achieved": round(fp32, 2), "unit": "TFLOP/s",
                          "fp32_mfma_peak": PEAK_FP32_TFLOPS,
                          "ratio_to_fp32_mfma_peak": round(fp32 / PEAK_FP32_TFLOPS, 4)}
        return r

    # the dominant kernel of the step is the longer of the two chunk launches
    dominant = "kda_chunk_kernel" if launch_ms["summaries"] >= launch_ms["carry"] else "kda_carry_kernel"
    roof = roofline(dominant)
    other = roofline("kda_carry_kernel" if dominant == "kda_chunk_kernel" else "kda_chunk_kernel")

    S = plan.S
    live = int(plan.segment_live.sum())
    comp = compose_work(S, w.H, live)
    t_c_mfma = comp["macs"] * 2 / (PEAK_FP32_TFLOPS * 1e12) * 1e3
    t_c_hbm = comp["bytes"] / (PEAK_HBM_GBS * 1e9) * 1e3

    return {
        "metric": "KDA fwd tokens/s at H=32,K=V=128 (segmented+compose)",
        "value": round(w.T / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 in, fp32 state (split-bf16 MFMA chunks, fp32 MFMA compose)",
        "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "H": w.H, "K": w.K, "V": w.V,
                   "segments": w.segments, "sequences": plan.N, "seed": w.seed,
                   "gate_scale": w.gate_scale, "beta_scale": w.beta_scale,
                   "piece_tokens": pieces, "pieces": plan.P,
                   "head_groups": groups, "initial_state": bool(args.initial_state),
                   "o": "bf16" if args.o_bf16 else "fp32"},
        "roofline": roof,
        # summed launch durations per step; with head groups the compose
        # launches overlap the other two on a second stream
        "kernels_ms": {"segment_summaries": round(pass1_ms, 4),
                       "compose_summaries": round(compose_ms, 4),
                       "apply_carry": round(pass2_ms, 4)},
        "pages_method_ms": pages,
        "compose_roofline": {
            "bound": "mfma" if t_c_mfma >= t_c_hbm else "hbm",
            "bound_ms_fp32_mfma": round(t_c_mfma, 4),
            "bound_ms_hbm": round(t_c_hbm, 4),
            "achieved_tflops_fp32": round(comp["macs"] * 2 / (compose_ms * 1e-3) / 1e12, 2),
            "achieved_gbs": round(comp["bytes"] / (compose_ms * 1e-3) / 1e9, 1),
            "frac": round(max(t_c_mfma, t_c_hbm) / compose_ms, 4),
        },
        "other_chunk_roofline": other,
    }


# Algorithmic FP32-grade flops of the backward per (token, head): the forward
# quantities it needs (p = S~^T k: 2KV, S_t = S~ + k u^T: 3KV) and the
# reverse step (dS += q do^T: 2KV, du: 2KV, dq: 2KV, dk: 4KV, dS~: 2KV,
# dg: 2KV, dS_{t-1}: KV) -- 20 K V; recomputation is not counted.  The
# chunked backward runs them as split-bf16 products on the matrix cores,
# charged three times against the bf16 peak as the forward's chunk kernels
# are.
BWD_FLOPS_PER_TOKEN_HEAD = 20 * 128 * 128
# Algorithmic HBM bytes of the backward per (token, head): q, k, v, g (bf16),
# beta (bf16) and d_o (FP32) in; dq, dk, dv, dg (FP32) and dbeta (FP32) out.
BWD_BYTES_PER_TOKEN_HEAD = 4 * 2 * 128 + 2 + 4 * 128 + 4 * 4 * 128 + 4


def measure_backward(args, w, x, torch, kda):
    """Time kda_backward (the gradients of q, k, v, g, beta for a seeded
    d_o) on the same workload: one untimed call, then args.backward_steps
    calls between events on the calling stream.  The roofline covers the
    whole call (every launch; the gradient launch dominates, its own
    duration is in the committed kernel trace): the larger of the
    algorithmic HBM bytes at 8 TB/s and the algorithmic multiply-adds as
    split bf16 at 2.5 PFLOP/s."""
    dev = torch.device("cuda:0")
    d = {n: x[n].to(dev) for n in ("q", "k", "v", "g", "beta")}
    cu = x["cu_seqlens"].tolist()
    plan = kda.Plan(cu, w.segments, None, piece_tokens(args, kda, cu, w))
    gen = torch.Generator().manual_seed(w.seed + 2000)
    d_o = torch.randn(w.T, w.H, w.V, generator=gen).to(dev)

    def call():
        return kda.backward(plan, d["q"], d["k"], d["v"], d["g"], d["beta"], d_o)

    call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.backward_steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.backward_steps
    th = w.T * w.H
    flops = BWD_FLOPS_PER_TOKEN_HEAD * th          # FP32-grade
    split = 3 * flops                              # as executed on bf16 matrix cores
    nbytes = BWD_BYTES_PER_TOKEN_HEAD * th
    bound_mfma = split / (PEAK_BF16_TFLOPS * 1e12) * 1e3
    bound_hbm = nbytes / (PEAK_HBM_GBS * 1e9) * 1e3
    if bound_hbm >= bound_mfma:
        roof = {"bound": "hbm", "achieved": round(nbytes / (ms * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(bound_hbm / ms, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(split / (ms * 1e-3) / 1e12, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(bound_mfma / ms, 4)}
    roof.update({
        "scope": "whole call (every launch of kda_backward)",
        "bounds_ms": {"mfma": round(bound_mfma, 4), "hbm": round(bound_hbm, 4)},
        "flops_per_token_head": BWD_FLOPS_PER_TOKEN_HEAD, "bytes_per_token_head": BWD_BYTES_PER_TOKEN_HEAD,
        "fp32grade": {"achieved": round(flops / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
                      "fp32_mfma_peak": PEAK_FP32_TFLOPS,
                      "ratio_to_fp32_mfma_peak": round(flops / (ms * 1e-3) / 1e12 / PEAK_FP32_TFLOPS, 4)},
    })
    res = {
        "ms_per_call": round(ms, 3),
        "tokens_per_s": round(w.T / (ms * 1e-3), 1),
        "calls": args.backward_steps,
        "roofline": roof,
    }
    if not plan.pieces:
        # kda_backward_from_forward: the same gradients from the forward's own
        # transitions and carry-ins (a training step keeps them), timed alike
        fwd = kda.forward(plan, d["q"], d["k"], d["v"], d["g"], d["beta"])
        saved = (fwd["transitions"], fwd["carry_in"])

        def call_saved():
            return kda.backward(plan, d["q"], d["k"], d["v"], d["g"], d["beta"], d_o, saved=saved)

        call_saved()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.backward_steps):
            call_saved()
        e1.record()
        torch.cuda.synchronize()
        ms2 = e0.elapsed_time(e1) / args.backward_steps
        res["from_forward"] = {"ms_per_call": round(ms2, 3), "tokens_per_s": round(w.T / (ms2 * 1e-3), 1),
                               "scope": "kda_backward_from_forward: the forward's transitions and carry-ins "
                                        "read, not recomputed"}
    return res


if __name__ == "__main__":
    main()
