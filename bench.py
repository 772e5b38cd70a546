"""Benchmark of the MoE routing + dispatch-layout hot path on one MI355X.

A step is one pass of the whole path over one batch of router logits already resident in HBM:
mep_route_layout_plan (routing, layout and plan in one call) on one stream.  On the default
workload that is two kernels: the sigmoid routing kernel, which also counts the plan tiles it
routes and forms every prefix in its epilogue, then the plan-tile kernel.  The default workload
is N=65536 tokens, E=256 experts, K=8, fp32 logits, sigmoid scoring with a per-expert bias,
8 groups keep 4 by top-2 sum, weights renormalised x2.5, alignment 128, R=8 virtual ranks with
one source shard per rank and 24 channels.

Input and output buffers rotate over several distinct sets (together larger than the 256 MB
Infinity Cache) so every step reads logits from HBM, not from the last-level cache.

The K timed steps are captured once into a HIP graph and the graph is replayed between two
events (`ms_per_step`, `value`): the path launches kernels only, so a replay does the work of the
eager calls without the host's per-launch cost.  `eager_ms_per_step` is the same K steps issued
call by call, and `path.latency` the per-step time from the routing kernel's start to the plan
kernel's end over at least 50 eager steps.

Prints one JSON line.  `roofline` describes the dominant kernel (routing + counting):
algorithmic bytes per launch / its average duration, timed inside the timed region with HIP
events that the kernel's launch on the bench stream stamps itself (mep_route_layout_plan_timed);
`roofline.path_frac` is the whole path's algorithmic bytes per step / the step time / peak.
`three_calls` times mep_route_topk + mep_build_layout + mep_plan.  `cpu_baseline` is the CPU
oracle timed on this host on a bounded sample (routing split over threads, layout and plan
serial).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
LLC_BYTES = 256 * 1024 * 1024  # MI355X Infinity Cache
CPU_THREADS_MAX = 16           # the CPU share of one GPU on the benchmark hosts


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dsv3")
    ap.add_argument("--legs", choices=("all", "step"), default="all",
                    help="'step': only the timed steps and the latency run (no three-call, "
                         "widening-row or CPU legs), for profiler runs")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time for the oracle baseline (0 disables it)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after the timed steps, copy MIB mebibytes device to device three times "
                         "(a plain copy kernel of known size, to scale HBM counters)")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU work: read two rocprofv3 counter CSVs (FETCH_SIZE, WRITE_SIZE) of "
                         "runs with --copy-calibration MIB (give the same MIB here) and write "
                         "profiles/route_traffic.json")
    return ap.parse_args()


def route_bytes(wl) -> int:
    """Compulsory HBM bytes of one routing launch: logits read once, bias read once, ids and
    weights written once."""
    b = 4 if wl.dtype == 0 else 2
    return wl.N * wl.E * b + (4 * wl.E if wl.score_fn == 1 else 0) + 8 * wl.N * wl.K


def path_bytes(wl, T: int, G: int, D: int) -> int:
    """Compulsory HBM bytes of the whole path (each input read once, each output written once)."""
    N, E, K, R, S, C = wl.N, wl.E, wl.K, wl.R, wl.S, wl.num_channels
    epn = E // R
    small = 4 * (E + (E + 1) + 2 * E)                              # layout per-expert outputs
    small += 4 * (S * R * 2 + S * E + S * R * C + R + R * (epn + 1) + 2 * E + 2 * R + 2 * (R + 1))
    return route_bytes(wl) + 4 * N * K + 4 * T + N * R + 4 * N * K + 12 * G + 4 * D + small


def route_kernel_name(wl) -> str:
    """The routing kernel the library launches for this workload (route_sig_kernel covers
    sigmoid scoring with one group of 32 experts per lane, or no group limit, K <= 8)."""
    lpt = wl.E // 32
    if (wl.score_fn == 1 and wl.E % 32 == 0 and lpt in (2, 4, 8, 16) and wl.K <= 8
            and (wl.n_group <= 1 or wl.n_group == lpt)):
        return "route_sig_kernel<%d, %s, %d>" % (lpt, "bf16" if wl.dtype else "fp32",
                                                 1 if wl.n_group > 1 else 0)
    return "route_fast_kernel"


# sources of the routing kernel (every file it includes, and the counting epilogue it runs) and
# the compile flags; a counter profile is valid only while all of them are unchanged
ROUTE_SOURCES = ["route.hip", "route_common.h", "route_sig.hip", "route_sig.h", "sigmoid_cr.h",
                 "route_fast.h", "route_fast.hip", "route_fast_f32.hip", "route_fast_bf16.hip",
                 "device_common.h", "host_common.h", "calls.h", "path.h"]
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "route_traffic.json")
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def route_sources_sha256() -> str:
    from expert_dispatch_layout_amd import build as hip_build

    h = hashlib.sha256()
    for name in ROUTE_SOURCES:
        h.update(open(os.path.join(ROOT, "expert_dispatch_layout_amd", "csrc", name), "rb").read())
    h.update(" ".join(hip_build.CFLAGS).encode())
    return h.hexdigest()


def traffic_from_profile():
    """Measured HBM bytes per routing launch, if a counter profile of the current routing
    sources was committed (profiles/route_traffic.json); None otherwise."""
    if not os.path.exists(TRAFFIC_JSON):
        return None
    rec = json.load(open(TRAFFIC_JSON))
    if rec.get("source_sha256") != route_sources_sha256():
        return None
    return rec.get("bytes_per_launch")


def read_counter_csv(path: str, counter: str):
    """Per-kernel lists of one counter's per-dispatch values (KiB) from a rocprofv3 CSV."""
    import csv

    per = {}
    for row in csv.DictReader(open(path)):
        if row["Counter_Name"] != counter:
            continue
        per.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return per


def record_traffic(fetch_csv: str, write_csv: str, copy_mib: int, wl):
    """Scale the routing kernel's FETCH_SIZE and WRITE_SIZE (KiB per dispatch) by what the same
    counters read for the plain copy kernel of --copy-calibration (known bytes), and store the
    result with the hash of the routing sources."""
    fetch = read_counter_csv(fetch_csv, "FETCH_SIZE")
    write = read_counter_csv(write_csv, "WRITE_SIZE")
    name = route_kernel_name(wl)
    rk = [k for k in fetch if name.split("<")[0] in k]
    assert len(rk) == 1, "routing kernel %s not unique in %s: %s" % (name, fetch_csv, list(fetch))
    rk = rk[0]
    # the copy kernel's dispatches of the calibration size are its largest ones
    cf = max(fetch[COPY_KERNEL])
    cw = max(write[COPY_KERNEL])
    copy_kib = copy_mib * 1024.0
    f_fac = copy_kib / cf
    w_fac = copy_kib / cw
    fk = sum(fetch[rk]) / len(fetch[rk])
    wk = sum(write[rk]) / len(write[rk])
    per = {}
    for k in fetch:
        if k in write and k != COPY_KERNEL:
            per[k] = {"fetch_bytes": 1024 * f_fac * sum(fetch[k]) / len(fetch[k]),
                      "write_bytes": 1024 * w_fac * sum(write[k]) / len(write[k]),
                      "dispatches": len(fetch[k])}
    rec = {"source_sha256": route_sources_sha256(), "kernel": rk,
           "fetch_kib_per_dispatch": fk, "write_kib_per_dispatch": wk,
           "copy_kib": copy_kib, "copy_fetch_kib": cf, "copy_write_kib": cw,
           "fetch_scale": f_fac, "write_scale": w_fac,
           "bytes_per_launch": 1024 * (fk * f_fac + wk * w_fac),
           "algorithmic_bytes_per_launch": route_bytes(wl), "kernels": per}
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps({k: rec[k] for k in rec if k != "kernels"}))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, inp, seconds: float):
    """The oracle on this host's cores, on the benchmark batch: one full pass (route, layout,
    plan) with the routing split over T threads (tokens are independent; layout and plan stay
    serial), and the same pass on one thread.  Each is the median of up to three passes,
    bounded by `seconds` of CPU work in all."""
    import oracle

    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    threads = max(1, min(avail or 1, CPU_THREADS_MAX))
    kw = dict(bias=inp.bias, score_fn=wl.score_fn, renormalize=wl.renormalize,
              n_group=wl.n_group, topk_group=wl.topk_group, group_topn=wl.group_topn,
              scale=wl.scale, dtype=wl.dtype)

    def one_pass(nthreads):
        t0 = time.perf_counter()
        if nthreads > 1:
            ids, _ = oracle.route_threads(inp.logits, wl.K, nthreads, **kw)
        else:
            ids, _ = oracle.route(inp.logits, wl.K, **kw)
        t1 = time.perf_counter()
        L = oracle.layout(ids, wl.E, wl.alignment)
        oracle.plan(ids, L.cu_seqlens, L.expanded_to_permuted, wl.E, wl.R, wl.S,
                    wl.num_channels, wl.NvS)
        t2 = time.perf_counter()
        return t2 - t0, t1 - t0

    t_start = time.perf_counter()
    multi = [one_pass(threads)]
    single = [one_pass(1)]
    while len(single) < 3 and time.perf_counter() - t_start + multi[0][0] + single[0][0] < seconds:
        multi.append(one_pass(threads))
        single.append(one_pass(1))
    m = statistics.median(p[0] for p in multi)
    s1 = statistics.median(p[0] for p in single)
    return {"value": wl.N / m, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "the whole %d-token batch, route + layout + plan; routing split over %d "
                      "threads, layout and plan serial; median of %d passes"
                      % (wl.N, threads, len(multi)),
            "single_thread": {"value": wl.N / s1, "unit": "tokens/s", "cores": 1,
                              "passes": len(single),
                              "route_s": statistics.median(p[1] for p in single)},
            "route_s": statistics.median(p[1] for p in multi),
            "host_cores_visible": avail, "cpu_model": cpu_model()}


def tile_map_leg(B, torch, L, wl, steps: int, stream):
    """Grouped-GEMM tile maps of the last step's histogram, timed on their own (not part of the
    step): `steps` back-to-back calls between two events on the launch stream."""
    N, E, K, A = wl.N, wl.E, wl.K, wl.alignment
    cap = B.tile_map_capacity(N * K, E, A)
    dev = L.tokens_per_expert.device
    c2e = torch.empty(cap, dtype=torch.int32, device=dev)
    lim = torch.empty(cap, dtype=torch.int32, device=dev)
    sc = torch.empty(2, dtype=torch.int32, device=dev)
    call = B.bound_tile_map(L.tokens_per_expert, N * K, A, c2e, lim, sc[:1], sc[1:], stream)
    for _ in range(3):
        call()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(steps):
        call()
    t1.record(stream)
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1e3 / steps
    tiles = int(sc[1].item())
    nbytes = 4 * E + 8 * tiles + 8   # counts in; expert and row limit per tile, two scalars out
    return {"us_per_call": us, "tiles": tiles, "algorithmic_bytes": nbytes,
            "GB_per_s": nbytes / (us * 1e-6) / 1e9}


HIDDEN = 7168   # DeepSeek-V3 hidden size, for the rows of the permute / combine leg


def rows_leg(B, torch, L, w, wl, steps: int, stream):
    """Local permute and weighted combine of bf16 hidden rows over the last step's layout, each
    timed on its own (not part of the step): `steps` back-to-back calls between two events."""
    N, E, K = wl.N, wl.E, wl.K
    dev = L.cu_seqlens.device
    T = int(L.cu_seqlens[E].item())
    row = HIDDEN * 2
    g = torch.Generator(device=dev).manual_seed(0)
    x = torch.randn((N, HIDDEN), generator=g, device=dev).to(torch.bfloat16)
    xp = torch.empty((T, HIDDEN), dtype=torch.bfloat16, device=dev)
    out = torch.empty((N, HIDDEN), dtype=torch.bfloat16, device=dev)
    legs = {
        "permute": (B.bound_permute_rows(x, L.expanded_to_permuted, K, L.zero_fill, xp, stream),
                    N * row + T * row + N * K * 4 + E * 8),
        "combine": (B.bound_combine_rows(xp, L.expanded_to_permuted, K, w, out, stream),
                    N * K * row + N * row + N * K * 8),
    }
    res = {"hidden": HIDDEN, "dtype": "bf16", "T": T}
    for name, (call, nbytes) in legs.items():
        for _ in range(2):
            call()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(stream)
        for _ in range(steps):
            call()
        t1.record(stream)
        torch.cuda.synchronize()
        us = t0.elapsed_time(t1) * 1e3 / steps
        gbs = nbytes / (us * 1e-6) / 1e9
        res[name] = {"us_per_call": us, "algorithmic_bytes": nbytes, "GB_per_s": gbs,
                     "frac_of_peak": gbs / HBM_PEAK_GBS}
    del x, xp, out
    return res


def balanced_leg(B, torch, ids, L, wl, steps: int, stream):
    """The plan with capacity rebalancing over the last step's ids and layout (R ranks, 4 copied
    experts per rank, groups padded to the layout alignment, capacity = the mean rank load),
    timed on its own: `steps` back-to-back calls between two events."""
    N, E, K, R, A = wl.N, wl.E, wl.K, wl.R, wl.alignment
    nb, cap = 4, N * K // R
    nvs = B.balanced_nvs(N, E, K, R, nb, A, cap)
    out = B.alloc_balanced(N, E, K, R, nb, ids.device)
    call = B.bound_plan_balanced(ids, L, E, R, nb, A, cap, nvs, out, stream)
    for _ in range(3):
        call()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(steps):
        call()
    t1.record(stream)
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1e3 / steps
    # ids, expanded_to_permuted read and dst written per slot; counts, offsets and the small
    # per-rank tables on top
    nbytes = 12 * N * K + 4 * (E + 1) + 4 * R * (R + 4 * E + 3 * (E + nb) + nb + 3)
    return {"us_per_call": us, "ranks": R, "copies_per_rank": nb, "capacity": cap,
            "moves": int((out.z > 0).sum().item()),
            "experts_copied": int((out.experts_to_copy >= 0).sum().item()),
            "algorithmic_bytes": nbytes, "GB_per_s": nbytes / (us * 1e-6) / 1e9}


def small_batch_leg(B, torch, synth, steps: int, stream):
    """Decode-size batches (the tiny and small workloads): mep_route_layout_plan (one kernel)
    against mep_route_topk followed by mep_layout_plan (three kernels), each timed over `steps`
    back-to-back calls between two events."""
    import numpy as np

    res = {}
    for name in ("tiny", "small"):
        wl = synth.WORKLOADS[name]
        inp = synth.make_inputs(wl)
        N, E, K, A, R, S, C = wl.N, wl.E, wl.K, wl.alignment, wl.R, wl.S, wl.num_channels
        dev = torch.device("cuda:0")
        x = torch.from_numpy(inp.logits.view(np.int16) if wl.dtype == synth.BF16 else inp.logits).to(dev)
        if wl.dtype == synth.BF16:
            x = x.view(torch.bfloat16)
        bias = torch.from_numpy(inp.bias).to(dev) if inp.bias is not None else None
        params = B.route_params(wl.score_fn, wl.renormalize, wl.n_group, wl.topk_group,
                                wl.group_topn, wl.scale)
        ids = torch.empty((N, K), dtype=torch.int32, device=dev)
        w = torch.empty((N, K), dtype=torch.float32, device=dev)
        L = B.alloc_layout(N, E, K, A, dev)
        P = B.alloc_plan(N, E, K, R, S, C, dev)
        ws = B.alloc_workspace(B.plan_workspace_size(N, E, K, R, S), dev)
        nvs = B.default_nvs(N, E, K, R, A)
        one = B.bound_route_layout_plan(x, K, bias, params, ids, w, A, L, R, S, C, nvs, P, ws, stream)
        r1 = B.bound_route_topk(x, K, bias, params, ids, w, stream)
        r2 = B.bound_layout_plan(ids, E, A, L, R, S, C, nvs, P, ws, stream)
        out = {}
        for label, fns in (("one_call_us", (one,)), ("three_kernels_us", (r1, r2))):
            for _ in range(5):
                for f in fns:
                    f()
            t0 = torch.cuda.Event(enable_timing=True)
            t1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            t0.record(stream)
            for _ in range(steps):
                for f in fns:
                    f()
            t1.record(stream)
            torch.cuda.synchronize()
            out[label] = t0.elapsed_time(t1) * 1e3 / steps
        out["tokens"] = N
        res[name] = out
    return res


def three_calls_leg(B, torch, sets, bias, params, wl, ws_l, ws_p, steps: int, stream):
    """mep_route_topk + mep_build_layout + mep_plan, back to back on one stream over the same
    rotating buffer sets, `steps` steps between two events (µs per step)."""
    N, E, K, A, R, S, C = wl.N, wl.E, wl.K, wl.alignment, wl.R, wl.S, wl.num_channels
    calls = []
    for x, ids, w, L, P in sets:
        calls.append((B.bound_route_topk(x, K, bias, params, ids, w, stream),
                      B.bound_build_layout(ids, E, A, L.tokens_per_expert, L.cu_seqlens,
                                           L.expanded_to_permuted, L.permuted_to_expanded,
                                           L.zero_fill, ws_l, stream),
                      B.bound_plan(ids, L.cu_seqlens, L.expanded_to_permuted, E, A, R, S, C,
                                   wl.NvS, P, ws_p, stream)))
    for i in range(3):
        for f in calls[i % len(calls)]:
            f()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(steps):
        for f in calls[i % len(calls)]:
            f()
    t1.record(stream)
    torch.cuda.synchronize()
    return {"us_per_step": t0.elapsed_time(t1) * 1e3 / steps, "steps": steps,
            "kernels": "routing, layout count + scatter, plan-tile counting + plan-tile kernel (5 launches)"}


def main():
    args = parse()
    if args.record_traffic:
        from expert_dispatch_layout_amd import synth

        assert args.copy_calibration > 0, "--record-traffic needs the --copy-calibration size of the run"
        record_traffic(*args.record_traffic, args.copy_calibration, synth.WORKLOADS[args.workload])
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from expert_dispatch_layout_amd import _binding as B
    from expert_dispatch_layout_amd import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    wl = synth.WORKLOADS[args.workload]
    inp = synth.make_inputs(wl)
    N, E, K, A, R, S, C = wl.N, wl.E, wl.K, wl.alignment, wl.R, wl.S, wl.num_channels
    logits_bytes = inp.logits.nbytes
    nsets = max(2, -(-(3 * LLC_BYTES // 2) // max(logits_bytes, 1)))   # > 1.5x the LLC
    nsets = min(nsets, 64)

    host = torch.from_numpy(inp.logits.view(np.int16) if wl.dtype == synth.BF16 else inp.logits)
    sets = []
    for _ in range(nsets):
        x = host.to(dev)
        if wl.dtype == synth.BF16:
            x = x.view(torch.bfloat16)
        ids = torch.empty((N, K), dtype=torch.int32, device=dev)
        w = torch.empty((N, K), dtype=torch.float32, device=dev)
        sets.append((x, ids, w, B.alloc_layout(N, E, K, A, dev), B.alloc_plan(N, E, K, R, S, C, dev)))
    bias = torch.from_numpy(inp.bias).to(dev) if inp.bias is not None else None
    params = B.route_params(wl.score_fn, wl.renormalize, wl.n_group, wl.topk_group,
                            wl.group_topn, wl.scale)
    ws_p = B.alloc_workspace(B.plan_workspace_size(N, E, K, R, S), dev)
    NvS = wl.NvS
    stream = torch.cuda.current_stream()

    def step_call(i, rt=None, pt=None, on=None):
        x, ids, w, L, P = sets[i % nsets]
        return B.bound_route_layout_plan(x, K, bias, params, ids, w, A, L, R, S, C, NvS, P, ws_p,
                                         on if on is not None else stream, route_timer=rt, plan_timer=pt)

    # one prepared call per step (arguments converted once); timed steps stamp two events per
    # kernel through their own launches (mep_route_layout_plan_timed)
    plain = [step_call(i) for i in range(nsets)]
    rts = [B.KernelTimer() for _ in range(args.steps)]
    pts = [B.KernelTimer() for _ in range(args.steps)]
    timed = [step_call(args.warmup + i, rts[i], pts[i]) for i in range(args.steps)]

    for i in range(args.warmup):
        plain[i % nsets]()
    torch.cuda.synchronize()

    # timed region: K steps bracketed by synchronisation
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        timed[i]()
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / args.steps
    ms_eager = ms_step

    # The same K steps captured once into a HIP graph and replayed: the host's per-launch cost
    # leaves the timed region (the path records kernels only, so a replay writes what the eager
    # calls write).  The graph's replay time is the headline; the eager loop is reported beside it.
    gstream = torch.cuda.Stream()
    gcalls = [step_call(args.warmup + i, on=gstream) for i in range(args.steps)]
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=gstream):
        for c in gcalls:
            c()
    with torch.cuda.stream(gstream):
        graph.replay()
    torch.cuda.synchronize()
    g_start = torch.cuda.Event(enable_timing=True)
    g_end = torch.cuda.Event(enable_timing=True)
    g_start.record(gstream)
    with torch.cuda.stream(gstream):
        graph.replay()
    g_end.record(gstream)
    torch.cuda.synchronize()
    ms_step = g_start.elapsed_time(g_end) / args.steps
    del graph

    route_us = [t.elapsed_ms() * 1e3 for t in rts]
    plan_us = [t.elapsed_ms() * 1e3 for t in pts]
    step_us = [B.event_elapsed_ms(r.start, p.stop) * 1e3 for r, p in zip(rts, pts)]

    # sizes of this batch's layout and dedup lists (for the whole-path byte count)
    L, P = sets[(args.warmup + args.steps - 1) % nsets][3:]
    T = int(L.cu_seqlens[E].item())
    G, D = [int(v) for v in P.dup_offsets[R].tolist()]
    rb = route_bytes(wl)
    route_mean = statistics.fmean(route_us)
    achieved = rb / (route_mean * 1e-6) / 1e9
    pb = path_bytes(wl, T, G, D)
    path_gbs = pb / (ms_step * 1e-3) / 1e9
    traffic = traffic_from_profile()

    # per-step latency over at least 50 steps (launch-stamped events: routing start to plan end)
    nlat = max(50, args.steps)
    lrt = [B.KernelTimer() for _ in range(nlat)]
    lpt = [B.KernelTimer() for _ in range(nlat)]
    lat_calls = [step_call(i, lrt[i], lpt[i]) for i in range(nlat)]
    torch.cuda.synchronize()
    for c in lat_calls:
        c()
    torch.cuda.synchronize()
    lat_us = sorted(B.event_elapsed_ms(r.start, p.stop) * 1e3 for r, p in zip(lrt, lpt))
    lat_route = sorted(t.elapsed_ms() * 1e3 for t in lrt)
    lat_plan = sorted(t.elapsed_ms() * 1e3 for t in lpt)

    def pct(v, q):
        return v[min(len(v) - 1, int(q * len(v)))]

    out = {
        "metric": "routed tokens/sec + achieved HBM GB/s (% of peak), N=65536 E=256 K=8",
        "value": N / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32,i32",
        "data": "synthetic",
        "config": {"workload": "%s: N=%d E=%d K=%d %s logits, %s, A=%d, R=%d, num_src=%d, "
                               "channels=%d" % (wl.name, N, E, K,
                                                "bf16" if wl.dtype else "fp32",
                                                "sigmoid+bias, 8 groups keep 4 (top-2 sum), "
                                                "renorm x2.5" if wl.score_fn else "softmax top-K",
                                                A, R, S, C),
                   "buffer_sets": nsets, "call": "mep_route_layout_plan",
                   "timed": "HIP graph of the K steps, replayed"},
        "eager_ms_per_step": ms_eager,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": route_kernel_name(wl) + " (routing + plan-tile counting)",
                     "bytes_per_launch": rb,
                     "path_frac": path_gbs / HBM_PEAK_GBS},
        "path": {"algorithmic_bytes": pb, "GB_per_s": path_gbs, "frac_of_peak": path_gbs / HBM_PEAK_GBS,
                 "slots_per_s": N * K / (ms_step * 1e-3), "T": T, "dedup_groups": G,
                 "dedup_dups": D, "host_wall_s": wall,
                 "route_us_mean": route_mean, "plan_us_mean": statistics.fmean(plan_us),
                 "step_us_mean_events": statistics.fmean(step_us),
                 "latency": {"steps": nlat, "step_us_median": pct(lat_us, 0.5),
                             "step_us_p10": pct(lat_us, 0.1), "step_us_p90": pct(lat_us, 0.9),
                             "route_us_median": pct(lat_route, 0.5),
                             "plan_us_median": pct(lat_plan, 0.5)}},
    }
    if args.legs == "all":
        ws_l = B.alloc_workspace(B.layout_workspace_size(N, E, K), dev)
        out["three_calls"] = three_calls_leg(B, torch, sets, bias, params, wl, ws_l, ws_p,
                                             max(50, args.steps), stream)
        ids_last, w_last = sets[(args.warmup + args.steps - 1) % nsets][1:3]
        out["next_rows"] = {"tile_map": tile_map_leg(B, torch, L, wl, args.steps, stream),
                            "balanced_plan": balanced_leg(B, torch, ids_last, L, wl, args.steps, stream),
                            "rows": rows_leg(B, torch, L, w_last, wl, min(args.steps, 20), stream),
                            "small_batch": small_batch_leg(B, torch, synth, 200, stream)}
    if args.copy_calibration > 0:
        nbytes = args.copy_calibration << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.cpu_seconds > 0 and args.legs == "all":
        out["cpu_baseline"] = cpu_baseline(wl, inp, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
