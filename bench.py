#!/usr/bin/env python3
"""Throughput of the MoE token dispatch / unpermute-combine hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input, inputs already
resident in HBM: route_topk + build_index (one call, route_topk_index) -> permute (x into expert-major rows) ->
unpermute_combine (expert outputs back to token order, weighted). In group mode the permute is
the two-stage dedup dispatch and the combine is the per-group pre-combine plus the final sum.

Prints ONE JSON line. `value` is the whole step's algorithmic bytes (each stage's minimal HBM
traffic, computed from the actual routing) divided by the measured step time: the mean of K
steps, each timed by HIP events on its stream and preceded (outside the events) by a cache
flush -- 512 MiB written, then another 512 MiB read, which leaves the 256 MB MALL and every
XCD's L2 holding only clean lines of neither the step's inputs nor its outputs -- so that no
workload, however small, is served from a cache. The step is launched eagerly (its calls
enqueued behind the flush); the same step captured once in a HIP graph and replayed is timed
the same way (`ms_per_step_by_launch`; `--graph` reports the replays as `value`): on this
runtime a replay starts later after the flush than eager launches queued behind it. The graph
replays back to back without flushes give `ms_per_step_warm`; K eager steps back to back give
`ms_per_step_eager`. Per-kernel times (`kernel_us`: mean, with `kernel_us_median` and
`kernel_us_min`) come from K eager steps, each flushed before like the timed ones, with an event
between consecutive calls, so that each call is timed where the step runs it; `stage_us` sums
them per stage; `roofline` describes the dominant HBM-bound kernel with its own mean event time;
`cpu_baseline` is the CPU oracle on the same workload on this host, all usable cores (up to 16
threads) and one thread.
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

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E peak, 8 TB/s
METRIC = "permute+combine effective HBM GB/s (% of peak) and routed tokens/s"
_PERMUTE_SRC = ["unpermute_combine_amd/csrc/permute.hip", "unpermute_combine_amd/csrc/moe_common.h"]
_COMBINE_SRC = ["unpermute_combine_amd/csrc/combine.hip", "unpermute_combine_amd/csrc/moe_common.h"]
_FP8_SRC = ["unpermute_combine_amd/csrc/fp8.hip", "unpermute_combine_amd/csrc/moe_common.h"]
_BWD_SRC = ["unpermute_combine_amd/csrc/combine.hip", "unpermute_combine_amd/csrc/permute.hip",
            "unpermute_combine_amd/csrc/moe_common.h"]
# HBM-bound kernel calls of a step: sources (for the PMC summaries' digest) and kernel symbol.
# Standard and drop-and-pad steps run `permute` and `combine`; group-mode steps run the two
# dispatch stages (send: one copy per token and group; receive: group slots to expert-major
# rows), the per-group pre-combine and the final sum over groups.
# With --backward the step is the backward of the path on one saved forward index: the combine's
# backward (expert-row gradient and weight gradient), the dispatch's backward (the unit-weight
# combine of the expert-row gradient; in group mode the unit-weight pre-combine, then the final
# sum) and the router softmax's backward. With bf16 rows the combine's backward is two kernels, the
# weighted scatter of dout (dy) and a read-only pass of dots (dw): its PMC summary and roofline are
# those of the call (both kernels together).
KERNEL_SOURCES = {"permute": _PERMUTE_SRC, "combine": _COMBINE_SRC, "dispatch_send": _PERMUTE_SRC,
                  "dispatch_recv": _PERMUTE_SRC, "precombine": _COMBINE_SRC, "final_sum": _COMBINE_SRC,
                  "combine_bwd": _BWD_SRC, "dispatch_bwd": _COMBINE_SRC, "dispatch_bwd_recv": _COMBINE_SRC,
                  "dispatch_bwd_send": _COMBINE_SRC, "permute_fp8": _FP8_SRC, "dispatch_send_fp8": _FP8_SRC}
KERNEL_SYMBOLS = {"permute": "permute_scatter_vec16_kernel", "combine": "combine_kernel",
                  "dispatch_send": "permute_scatter_vec16_kernel", "dispatch_recv": "permute_grouped_vec16_kernel",
                  "precombine": "precombine_kernel", "final_sum": "combine_kernel",
                  "combine_bwd": "combine_backward_kernel", "dispatch_bwd": "combine_kernel",
                  "dispatch_bwd_recv": "precombine_kernel", "dispatch_bwd_send": "combine_kernel",
                  "permute_fp8": "permute_scatter_fp8_kernel", "dispatch_send_fp8": "permute_scatter_fp8_kernel"}


def combine_symbol(y_bf16: bool, out_bf16: bool, K: int, H: int, T: int) -> str:
    """Kernel the library launches for a combine call: bf16 rows with 5..8 slots per token, at
    most 128 KB of staged rows (8 * H * 2 bytes) and at least 2048 workgroups of 8 tokens take
    the batched combine, everything else the per-token one."""
    if y_bf16 and out_bf16 and H % 8 == 0 and 4 < K <= 8 and 16 * H <= 128 * 1024 and -(-T // 8) >= 2048:
        return "combine_batched_kernel"
    return "combine_kernel"


METRIC_BACKWARD = "backward of permute+combine (and router softmax) effective HBM GB/s (% of peak)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", type=int, default=3, help="named workload id (see workloads.py)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--seed", type=int, default=None,
                   help="draw the workload's inputs from another seed (same shapes and distributions); by "
                        "default each named workload has its one fixed draw")
    p.add_argument("--alignment", type=int, default=0,
                   help="round every expert segment up to a multiple of this many rows (padding rows)")
    p.add_argument("--route-groups", type=int, default=0,
                   help="group-limited routing: each token keeps this many of the workload's expert groups")
    p.add_argument("--bf16-partials", action="store_true",
                   help="group workloads: the per-group partial sums are rounded once to bf16 (the BF16 "
                        "exchange) instead of stored as float32")
    p.add_argument("--fp8", action="store_true",
                   help="FP8 dispatch: the permute quantizes x to E4M3 codes with one float32 scale per 128 "
                        "elements and moves codes and scales (the combine stays bf16)")
    p.add_argument("--graph", action="store_true",
                   help="report the step replayed from a HIP graph (captured once) as value / ms_per_step; by "
                        "default both launch modes are timed and value comes from the eager launches, which are "
                        "faster on this runtime (ms_per_step_by_launch gives both)")
    p.add_argument("--no-graph", action="store_true", help="skip the HIP graph capture and its timing")
    p.add_argument("--backward", action="store_true",
                   help="time the backward of the path (on one saved forward index) instead of the forward")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device copy (for scaling PMC byte counters)")
    p.add_argument("--stream-ceiling", action="store_true",
                   help="only time plain device streams (torch's 1 GiB device copy, a 2 GiB fill, a 2 GiB "
                        "reduction read) under the same flush protocol, as the chip's practical ceilings")
    p.add_argument("--no-warm", action="store_true",
                   help="skip the back-to-back (unflushed) passes, so that every step after the warmup "
                        "is preceded by a flush (for profiling runs whose per-kernel averages should match "
                        "kernel_us)")
    p.add_argument("--no-flush", action="store_true",
                   help="no cache flush before the timed steps and kernel calls (they still run one by one "
                        "between events)")
    return p.parse_args()


FLUSH_BYTES = 512 << 20  # twice the MI355X MALL (256 MB)


class CacheFlush:
    """Evicts the step's data from the caches: 512 MiB written by a fill kernel, then a different
    512 MiB read by a reduction. The read also pushes the fill's dirty lines out to HBM, so the
    caches end up holding only clean lines of the second buffer, which a timed kernel can evict
    without writing anything back."""

    def __init__(self, torch):
        self.torch = torch
        self.a = torch.empty(FLUSH_BYTES // 8, dtype=torch.int64, device="cuda")
        self.b = torch.zeros(FLUSH_BYTES // 8, dtype=torch.int64, device="cuda")
        self.n = 0

    def __call__(self):
        self.n += 1
        self.a.fill_(self.n)
        self.b.sum()


def _stats(xs):
    import numpy as np
    a = np.asarray(xs, dtype=np.float64)
    return float(a.mean()), float(np.median(a)), float(a.min())


def source_digest(kernel: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def profile_tag(workload: int, backward: bool = False, fp8: bool = False, bf16_partials: bool = False,
                alignment: int = 0, route_groups: int = 0) -> str:
    """The workload-and-mode part of a profiles/ file name, e.g. workload3_align128, workload4_bwd."""
    return (f"workload{workload}" + (f"_align{alignment}" if alignment else "")
            + (f"_groups{route_groups}" if route_groups else "") + ("_bwd" if backward else "")
            + ("_fp8" if fp8 else "") + ("_bf16p" if bf16_partials else ""))


def read_traffic(kernel: str, tag: str, symbol: str = None):
    """HBM bytes per launch from the committed PMC summary of this workload and mode; None if
    absent or stale."""
    path = os.path.join(ROOT, "profiles", f"{symbol or KERNEL_SYMBOLS[kernel]}__{tag}__pmc.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.strip().split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha") != source_digest(kernel):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration(torch):
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 5}), flush=True)


def stream_ceiling(torch, steps: int):
    """Plain streams timed like the path's kernels (each after a cache flush, HIP events around
    it): the rates a kernel that only copies, only writes or only reads reaches on this chip."""
    flush = CacheFlush(torch)
    a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    c = torch.empty(2 << 30, dtype=torch.uint8, device="cuda")
    d = torch.ones((2 << 30) // 4, dtype=torch.float32, device="cuda")
    streams = [("copy_1GiB", 2 << 30, lambda: b.copy_(a)), ("fill_2GiB", 2 << 30, lambda: c.fill_(3)),
               ("sum_read_2GiB", 2 << 30, lambda: d.sum())]
    out = {}
    for name, nbytes, fn in streams:
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(steps):
            flush()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        mean, med, mn = _stats(ts)
        out[name] = {"bytes": nbytes, "us_median": round(med, 1), "us_min": round(mn, 1),
                     "gbs_median": round(nbytes / (med * 1e-6) / 1e9, 1),
                     "pct_of_peak": round(100 * nbytes / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 1)}
    print(json.dumps({"stream_ceiling": out, "steps": steps,
                      "timing": "each stream after a 512 MiB write + 512 MiB read flush, HIP events around it"}),
          flush=True)


def to_dev(torch, a):
    import numpy as np
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to("cuda")
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def main():
    args = parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr, flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU (no CPU path)", file=sys.stderr, flush=True)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration(torch)
        return
    if args.stream_ceiling:
        stream_ceiling(torch, args.steps)
        return

    import unpermute_combine_amd as m
    import workloads as wl

    m.lib()  # fails loudly if the HIP library was not built
    cid = args.workload
    c = wl.WORKLOADS[cid]
    T, H, E, K, dt = c["T"], c["H"], c["E"], c["K"], c["dtype"]
    gs = c["group_size"]
    cap = m.expert_capacity(T, K, E, *c["cf"]) if c["cf"] else 0
    b = 2 if dt == "bf16" else 4
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    key = wl.workload_key(cid, args.seed)

    t0 = time.time()
    logits_np = wl.router_logits(key, T, E, zipf_s=c["zipf_s"])
    x_np = wl.hidden_states(key, T, H, dt)
    align = args.alignment if args.alignment > 1 else 0
    rows = m.index_rows(T, K, E, cap, align)
    y_np = None if c["identity_experts"] else wl.expert_outputs(key, rows, H, dt)
    logits = to_dev(torch, logits_np)
    x = to_dev(torch, x_np)
    y = None if y_np is None else to_dev(torch, y_np)
    log(f"[bench] workload {cid} ({c['name']}): inputs ready in {time.time() - t0:.1f}s")

    # preallocated outputs: nothing is allocated inside the timed region
    gi = torch.empty((T, K), dtype=torch.int32, device="cuda")
    gw = torch.empty((T, K), dtype=torch.float32, device="cuda")
    ix = m.alloc_index(T, K, E, cap, gs, alignment=align)
    xp = torch.empty((rows, H), dtype=tdt, device="cuda")
    fp8_block = 128
    nb = H // fp8_block
    if args.fp8:
        if args.backward or c["identity_experts"]:
            print("--fp8 times the forward dispatch of a workload with expert outputs (not 1, not --backward)",
                  file=sys.stderr, flush=True)
            sys.exit(2)
        xq = torch.empty((rows, H), dtype=torch.uint8, device="cuda")
        xs = torch.empty((rows, nb), dtype=torch.float32, device="cuda")
    out = torch.empty((T, H), dtype=tdt, device="cuda")
    G = E // gs if gs else 0
    gbuf = torch.empty((T * min(K, G), H), dtype=tdt, device="cuda") if gs and not args.fp8 else None
    if gs and args.fp8:
        gq = torch.empty((T * min(K, G), H), dtype=torch.uint8, device="cuda")
        gsc = torch.empty((T * min(K, G), nb), dtype=torch.float32, device="cuda")
    if args.bf16_partials and not gs:
        print("--bf16-partials needs a workload with expert groups (workload 4)", file=sys.stderr, flush=True)
        sys.exit(2)
    pb = 2 if args.bf16_partials else 4  # bytes per partial element
    part = torch.empty((T * min(K, G), H), dtype=torch.bfloat16 if args.bf16_partials else torch.float32,
                       device="cuda") if gs else None

    # the step's calls in order: (kernel name, stage, call)
    rg = args.route_groups
    if rg and not gs:
        print("--route-groups needs a workload with expert groups (workload 4)", file=sys.stderr, flush=True)
        sys.exit(2)
    # routing and index build in one call: for large inputs the workgroups that route a tile also
    # count its slots, one launch fewer than route_topk followed by build_index (same arrays)
    calls = [("route_index", "route_index",
              lambda: m.route_topk_index(logits, K, capacity=cap, group_size=gs, alignment=align,
                                         route_group_size=gs if rg else 0, topk_groups=rg, out=(gi, gw),
                                         index=ix))]
    src = xp if y is None else y
    if args.backward:
        # one forward pass (not timed) leaves the saved state the backward consumes
        for _, _, call in calls:
            call()
        if y is None:
            m.permute_scatter(x, ix.row_of, rows, src_row=ix.sorted_indices, out=xp)
        dout = to_dev(torch, wl.expert_outputs((*key, 7), T, H, dt))
        dxp = to_dev(torch, wl.expert_outputs((*key, 8), rows, H, dt))
        dy = torch.empty((rows, H), dtype=tdt, device="cuda")
        dw = torch.empty((T, K), dtype=torch.float32, device="cuda")
        dx = torch.empty((T, H), dtype=tdt, device="cuda")
        dlog = torch.empty((T, E), dtype=torch.float32, device="cuda")
        calls = [("combine_bwd", "combine_bwd",
                  lambda: m.unpermute_combine_backward(dout, src, ix.row_of, gw, src_row=ix.sorted_indices,
                                                       out=(dy, dw)))]
        if gs:
            calls += [("dispatch_bwd_recv", "dispatch_bwd",
                       lambda: m.group_precombine(dxp, ix.row_of, None, gi, E, gs, ix.slot_of, out=part)),
                      ("dispatch_bwd_send", "dispatch_bwd", lambda: m.unpermute_combine(part, ix.slot_of, None, out=dx))]
        else:
            calls += [("dispatch_bwd", "dispatch_bwd", lambda: m.unpermute_combine(dxp, ix.row_of, None, out=dx))]
        calls += [("route_bwd", "route_bwd", lambda: m.route_topk_backward(gi, gw, dw, E, out=dlog))]
    elif args.fp8 and gs:
        calls += [("dispatch_send_fp8", "permute",
                   lambda: m.permute_scatter_fp8(x, ix.slot_of, gq.shape[0], fp8_block, out=(gq, gsc))),
                  ("dispatch_recv", "permute", lambda: m.permute_grouped_fp8(gq, gsc, ix.esrc, ix.row_of,
                                                                             out=(xq, xs), src_of=ix.slot_src)),
                  ("precombine", "combine",
                   lambda: m.group_precombine(src, ix.row_of, gw, gi, E, gs, ix.slot_of, out=part)),
                  ("final_sum", "combine", lambda: m.unpermute_combine(part, ix.slot_of, None, out=out))]
    elif args.fp8:
        calls += [("permute_fp8", "permute",
                   lambda: m.permute_scatter_fp8(x, ix.row_of, rows, fp8_block, src_row=ix.sorted_indices,
                                                 out=(xq, xs))),
                  ("combine", "combine", lambda: m.unpermute_combine(src, ix.row_of, gw, out=out))]
    elif gs:
        # the number of group slots is only known on the device; every call is bounded by its
        # upper bound T*min(K,G) instead, so the step never waits for the host
        calls += [("dispatch_send", "permute", lambda: m.permute_scatter(x, ix.slot_of, gbuf.shape[0], out=gbuf)),
                  ("dispatch_recv", "permute", lambda: m.permute_grouped(gbuf, ix.esrc, ix.row_of, out=xp,
                                                                         src_of=ix.slot_src)),
                  ("precombine", "combine",
                   lambda: m.group_precombine(src, ix.row_of, gw, gi, E, gs, ix.slot_of, out=part)),
                  ("final_sum", "combine", lambda: m.unpermute_combine(part, ix.slot_of, None, out=out))]
    else:
        calls += [("permute", "permute",
                   lambda: m.permute_scatter(x, ix.row_of, rows, src_row=ix.sorted_indices, out=xp)),
                  ("combine", "combine", lambda: m.unpermute_combine(src, ix.row_of, gw, out=out))]

    def step():
        for _, _, call in calls:
            call()

    flush = None if args.no_flush else CacheFlush(torch)

    for _ in range(args.warmup):
        if flush is not None:
            flush()
        step()
    torch.cuda.synchronize()

    # eager steps back to back (launch gaps included)
    ms_per_step_eager = None
    if not args.no_warm:
        t_start = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        ms_per_step_eager = (time.perf_counter() - t_start) * 1e3 / args.steps

    # per-call times: K eager steps, each after one flush (as in the timed steps), the calls back to
    # back with an event between consecutive calls, so that every call runs where the step runs it:
    # after the previous call, not after a flush of its own (a flush between calls would absorb the
    # write-back that one call leaves to the next, e.g. the pre-combine's partials before the final
    # sum: 134 us flushed against 149 us in the step)
    sev_in = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s_ in range(args.steps):
        if flush is not None:
            flush()
        sev_in[s_][0].record()
        for i, (_, _, call) in enumerate(calls):
            call()
            sev_in[s_][i + 1].record()
    torch.cuda.synchronize()

    def timed_steps(run_step):
        """K steps, each flushed before (outside its events) unless --no-flush; per-step ms."""
        sev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        torch.cuda.synchronize()
        for a, b in sev:
            if flush is not None:
                flush()
            a.record()
            run_step()
            b.record()
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in sev]

    # the step launched eagerly: every call enqueued on the current stream behind the flush
    eager_ms = timed_steps(step)
    graph_ms = None
    graph_note = "not timed (--no-graph)"
    ms_per_step_warm = ms_per_step_eager
    if not args.no_graph:
        # the same calls captured once; no call allocates, waits on the host or records a memset
        try:
            graph = torch.cuda.CUDAGraph()
            cap_stream = torch.cuda.Stream()
            cap_stream.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(cap_stream):
                with torch.cuda.graph(graph, stream=cap_stream):
                    step()
            torch.cuda.current_stream().wait_stream(cap_stream)
            torch.cuda.synchronize()
        except RuntimeError as e:  # report the eager timing rather than nothing
            log(f"[bench] HIP graph capture failed, timing eager steps only: {e}")
            torch.cuda.synchronize()
            graph_note = f"graph capture failed: {type(e).__name__}"
        else:
            for _ in range(max(3, args.warmup)):
                if flush is not None:
                    flush()
                graph.replay()
            torch.cuda.synchronize()
            if not args.no_warm:
                t_start = time.perf_counter()
                for _ in range(args.steps):
                    graph.replay()
                torch.cuda.synchronize()
                ms_per_step_warm = (time.perf_counter() - t_start) * 1e3 / args.steps
            graph_ms = timed_steps(graph.replay)
            graph_note = None
    if args.graph and graph_ms is not None:
        step_ms, launch = graph_ms, "hip graph replay"
    else:
        step_ms = eager_ms
        launch = "eager" if graph_note is None or not args.graph else f"eager ({graph_note})"
    ms_per_step, ms_per_step_median, ms_per_step_min = _stats(step_ms)
    kernel_us, kernel_us_median, kernel_us_min = {}, {}, {}
    for i, (name, _, _) in enumerate(calls):
        kernel_us[name], kernel_us_median[name], kernel_us_min[name] = _stats(
            [sev_in[s_][i].elapsed_time(sev_in[s_][i + 1]) * 1e3 for s_ in range(args.steps)])
    stage_us = {}
    for name, stage, _ in calls:
        stage_us[stage] = stage_us.get(stage, 0.0) + kernel_us[name]

    # ---- algorithmic bytes from the actual routing
    row_of = ix.row_of.cpu().numpy()
    counts = ix.counts.cpu().numpy()
    valid = int((row_of >= 0).sum())  # rows the combine reads
    used = int((ix.sorted_indices != -2).sum().item())  # rows written (the slack after the last segment is not)
    routed = int((row_of >= 0).any(axis=1).sum()) if K else 0  # distinct source rows the permute reads
    kbytes = {"route_index": T * E * 4 + T * K * 8 + T * K * 8 + rows * 8 + T * K * 4 + E * 4 * 3}
    if args.backward:
        kbytes = {"combine_bwd": T * H * b + valid * H * b + used * H * b + T * K * 8 + rows * 4 + T * K * 4,
                  "route_bwd": T * K * 12 + T * E * 4}
        if gs:
            n = int(ix.n_slots.item())
            kbytes.update(dispatch_bwd_recv=valid * H * b + 2 * T * K * 4 + n * H * pb,
                          dispatch_bwd_send=n * H * pb + T * G * 4 + T * H * b)
        else:
            kbytes.update(dispatch_bwd=valid * H * b + T * K * 4 + T * H * b)
    elif args.fp8 and gs:
        n = int(ix.n_slots.item())
        kbytes.update(dispatch_send_fp8=routed * H * b + n * 4 + n * (H + nb * 4),
                      dispatch_recv=n * (H + nb * 4) + rows * 4 + used * (H + nb * 4),
                      precombine=valid * H * b + 2 * T * K * 4 + n * H * pb,
                      final_sum=n * H * pb + T * G * 4 + T * H * b)
    elif args.fp8:
        kbytes.update(permute_fp8=routed * H * b + rows * 4 + used * (H + nb * 4),
                      combine=valid * H * b + 2 * T * K * 4 + T * H * b)
    elif gs:
        n = int(ix.n_slots.item())
        kbytes.update(dispatch_send=routed * H * b + n * 4 + n * H * b,
                      dispatch_recv=n * H * b + rows * 4 + used * H * b,
                      precombine=valid * H * b + 2 * T * K * 4 + n * H * pb,
                      final_sum=n * H * pb + T * G * 4 + T * H * b)
    else:
        kbytes.update(permute=routed * H * b + rows * 4 + used * H * b,
                      combine=valid * H * b + 2 * T * K * 4 + T * H * b)
    stage_bytes = {}
    for name, stage, _ in calls:
        stage_bytes[stage] = stage_bytes.get(stage, 0) + kbytes[name]
    step_bytes = sum(kbytes.values())
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    routed_per_s = T * K / (ms_per_step * 1e-3)

    def gbs(nbytes, us):
        return round(nbytes / (us * 1e-6) / 1e9, 1)

    hbm_stages = ("permute", "combine", "combine_bwd", "dispatch_bwd")
    hbm_kernels = [name for name, stage, _ in calls if stage in hbm_stages]
    dom = max(hbm_kernels, key=lambda k: kernel_us[k])
    achieved = kbytes[dom] / (kernel_us[dom] * 1e-6) / 1e9
    symbol = KERNEL_SYMBOLS[dom]
    kernel_name = symbol
    if dom == "combine":
        symbol = kernel_name = combine_symbol(dt == "bf16", dt == "bf16", K, H, T)
    if dom == "combine_bwd" and dt == "bf16":
        symbol = "combine_backward_call"
        kernel_name = "permute_scatter_vec16_kernel<true> (dy) + combine_backward_kernel (dw dots)"
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": read_traffic(dom, profile_tag(cid, args.backward, args.fp8, args.bf16_partials, align, rg),
                                        symbol),
                "kernel": kernel_name, "call": dom, "algorithmic_bytes_per_launch": kbytes[dom],
                "avg_launch_us": round(kernel_us[dom], 2)}

    result = {
        "metric": METRIC_BACKWARD if args.backward else METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": dt, "accum_dtype": "f32", "data": "synthetic",
        "config": {"workload": c["name"] + (f" align{align}" if align else "") + (f" groups{rg}" if rg else "")
                   + (" fp8-dispatch" if args.fp8 else "") + (" bf16-partials" if args.bf16_partials else ""),
                   "fp8_dispatch": bool(args.fp8), "bf16_partials": bool(args.bf16_partials),
                   "T": T, "H": H, "E": E, "K": K, "capacity": cap, "alignment": align, "route_groups": rg,
                   "group_size": gs, "zipf_s": c["zipf_s"], "seed_key": list(key)},
        "pct_of_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "routed_tokens_per_s": round(routed_per_s, 1),
        "stage_us": {k: round(v, 2) for k, v in stage_us.items()},
        "stage_gbs": {k: gbs(stage_bytes[k], stage_us[k]) for k in stage_us if k in hbm_stages},
        "kernel_us": {k: round(v, 2) for k, v in kernel_us.items()},
        "kernel_us_median": {k: round(v, 2) for k, v in kernel_us_median.items()},
        "kernel_us_min": {k: round(v, 2) for k, v in kernel_us_min.items()},
        "kernel_gbs": {k: gbs(kbytes[k], kernel_us[k]) for k in hbm_kernels},
        "kernel_gbs_median": {k: gbs(kbytes[k], kernel_us_median[k]) for k in hbm_kernels},
        "kernel_bytes": kbytes,
        "max_expert_count": int(counts.max()), "empty_experts": int((counts == 0).sum()),
        "roofline": roofline,
    }
    if args.backward:
        result["pass"] = "backward"
    result["launch"] = launch
    result["ms_per_step_by_launch"] = {
        "eager": round(_stats(eager_ms)[0], 4),
        "hip graph replay": None if graph_ms is None else round(_stats(graph_ms)[0], 4)}
    result["timing"] = (("each step preceded by a 512 MiB write + 512 MiB read cache flush outside its events"
                         if flush is not None else "no cache flush") +
                        "; ms_per_step = mean of the per-step event times; kernel_us = per-call event times "
                        "inside such steps (eager launches, an event between consecutive calls)")
    result["ms_per_step_median"] = round(ms_per_step_median, 4)
    result["ms_per_step_min"] = round(ms_per_step_min, 4)
    result["ms_per_step_warm"] = None if ms_per_step_warm is None else round(ms_per_step_warm, 4)
    result["ms_per_step_eager"] = None if ms_per_step_eager is None else round(ms_per_step_eager, 4)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(c, key, logits_np, x_np, y_np, cap, align, rg, step_bytes,
                                              args.bf16_partials, args.fp8, fp8_block, args.backward)
    print(json.dumps(result), flush=True)


def _passes(run_once, min_seconds, min_passes=2, max_passes=8):
    """Runs the oracle pass until at least min_seconds of wall-clock time (2..8 passes); returns
    the best pass time, the number of passes and the total seconds."""
    times = []
    while len(times) < max_passes and (len(times) < min_passes or sum(times) < min_seconds):
        t0 = time.perf_counter()
        run_once()
        times.append(time.perf_counter() - t0)
    return min(times), len(times), sum(times)


def cpu_baseline(c, key, logits_np, x_np, y_np, cap, align, rg, step_bytes, bf16_partials=False, fp8=False,
                 fp8_block=128, backward=False):
    """The CPU oracle as it stands, over the same whole workload and mode as the GPU step (the
    forward: route, index, dispatch -- the FP8 one with --fp8 --, combine; or the backward on one
    saved forward index), timed twice: on all usable host cores (the oracle's per-token and
    per-row functions over disjoint slices on up to 16 threads; the index build stays one call)
    and on one thread. Passes repeat until a few seconds of wall-clock time; the best pass of
    each leg is reported, `value` from the all-cores leg."""
    import numpy as np

    import oracle
    import workloads as wl
    from oracle.parallel import Pool, Serial, cpu_model, usable_cores

    T, H, E, K, gs = c["T"], c["H"], c["E"], c["K"], c["group_size"]
    out_dt = np.uint16 if c["dtype"] == "bf16" else np.float32
    part_dt = np.uint16 if bf16_partials else np.float32
    if backward:
        idx0, w0 = Serial.route_topk(logits_np, K, gs, rg)
        ix0 = oracle.build_index(idx0, w0, E, capacity=cap, group_size=gs, alignment=align)
        rows = len(ix0["sorted_indices"])
        y_b = oracle.permute(x_np, ix0["sorted_indices"]) if y_np is None else y_np
        dout = wl.expert_outputs((*key, 7), T, H, c["dtype"])
        dxp = wl.expert_outputs((*key, 8), rows, H, c["dtype"])

    def run_once(o, st):
        """One pass; st[stage] collects the stage's seconds (route, index, dispatch, combine; or
        combine_bwd, dispatch_bwd, route_bwd)."""
        t = [time.perf_counter()]

        def lap(stage):
            now = time.perf_counter()
            st.setdefault(stage, []).append(now - t[0])
            t[0] = now

        if backward:
            _, dw = o.combine_backward(dout, y_b, ix0["row_of"], w0, out_dt)
            lap("combine_bwd")
            if gs:
                n = int(ix0["n_slots"][0])
                part = o.group_precombine(dxp, ix0["row_of"], None, idx0, E, gs, ix0["slot_of"], n, out_dtype=part_dt)
                o.unpermute_combine(part, ix0["slot_of"], None, out_dt)
            else:
                o.unpermute_combine(dxp, ix0["row_of"], None, out_dt)
            lap("dispatch_bwd")
            o.route_topk_backward(idx0, w0, dw, E)
            lap("route_bwd")
            return
        idx, w = o.route_topk(logits_np, K, gs, rg)
        lap("route")
        ix = oracle.build_index(idx, w, E, capacity=cap, group_size=gs, alignment=align)
        lap("index")
        maps = [ix["gsrc"], ix["esrc"]] if gs else [ix["sorted_indices"]]  # group mode: send, then receive
        if fp8:
            xp = None
            for a in o.quantize_fp8(x_np, fp8_block):  # the codes, then the scales, each moved like rows
                for mp in maps:
                    a = o.permute(a, mp)
        else:
            xp = x_np
            for mp in maps:
                xp = o.permute(xp, mp)
        lap("dispatch")
        y = xp if y_np is None else y_np
        if gs:
            n = int(ix["n_slots"][0])
            part = o.group_precombine(y, ix["row_of"], w, idx, E, gs, ix["slot_of"], n, out_dtype=part_dt)
            o.unpermute_combine(part, ix["slot_of"], None, out_dt)
        else:
            o.unpermute_combine(y, ix["row_of"], w, out_dt)
        lap("combine")

    def medians(st):
        return {k: round(float(np.median(v)), 4) for k, v in st.items()}

    st_all, st_one = {}, {}
    with Pool() as pool:
        best, n, total = _passes(lambda: run_once(pool, st_all), min_seconds=4.0)
        threads = pool.threads
    best1, n1, total1 = _passes(lambda: run_once(Serial(), st_one), min_seconds=6.0)
    what = ("the whole backward of the workload" if backward else "the whole workload") + f" ({c['name']}"
    what += (", FP8 dispatch" if fp8 else "") + (", bf16 partials" if bf16_partials else "") + ")"
    res = {"value": round(step_bytes / best / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
           "sample": f"{what} per pass, best of {n} passes ({total:.1f} s wall, {threads} threads); the "
                     f"oracle's per-token / per-row functions over disjoint slices, the index build in one call",
           "seconds_per_pass": round(best, 3), "stage_seconds_median": medians(st_all),
           "host": {"cpu_model": cpu_model(), "nproc": os.cpu_count(), "usable_cores": usable_cores(),
                    "threads_used": threads},
           "single_thread": {"value": round(step_bytes / best1 / 1e9, 3), "unit": "GB/s", "cores": 1,
                             "seconds_per_pass": round(best1, 3), "stage_seconds_median": medians(st_one),
                             "sample": f"{what} per pass, best of {n1} passes ({total1:.1f} s)"}}
    if not backward:
        res["routed_tokens_per_s"] = round(T * K / best, 1)
        res["single_thread"]["routed_tokens_per_s"] = round(T * K / best1, 1)
    return res


if __name__ == "__main__":
    main()
