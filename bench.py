#!/usr/bin/env python3
"""Benchmark of the speculative verification step on one MI355X.

A step is one verification pass of every layer group over one batch of
synthetic input (ring write, resolution plan, host fetch of missing rows,
sparse attention, copy-back).  Inputs are resident in HBM / pinned host
memory before timing starts; the hot-cache state is restored from a device
snapshot before every step, outside the timed region, so each step resolves
at the workload's configured hit rate (``--retained`` skips the restore).

Prints one JSON line: verified query-tokens/s (whole job), the roofline of the
dominant kernel measured with HIP events on the streams the kernels run on,
every kernel's roofline, and the oracle timed on the host cores over a
bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_PCIE_GBS = 64.0           # PCIe 5.0 x16, one direction (host link of the MI355X)
CPU_SHARE_THREADS = 16         # host threads per GPU on the GPU host (worker pools are sized to it)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="mla128")
    ap.add_argument("--rho", type=float, default=0.0, help="static resident fraction of rows")
    ap.add_argument("--n-chunks", type=int, default=0)
    ap.add_argument("--fetch-cus", type=int, default=0, help="CUs reserved for the host fetch")
    ap.add_argument("--fetch-wgs", type=int, default=0, help="workgroups per chunk of the host fetch (0 = library default)")
    ap.add_argument("--retained", action="store_true", help="keep the cache state between steps")
    ap.add_argument("--timing-steps", type=int, default=3,
                    help="steps of the separate pass that times every kernel")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-requests", type=int, default=128,
                    help="requests per layer group the oracle resolves and attends in the CPU baseline")
    ap.add_argument("--cpu-groups", type=int, default=2,
                    help="layer groups the CPU baseline times (scaled to all groups of a step)")
    ap.add_argument("--load-step", action="store_true",
                    help="residency under a load step (low -> full -> low load), optional residency on and off")
    ap.add_argument("--load-lo", type=int, default=16, help="active requests at low load")
    ap.add_argument("--load-steps", default="20,20,40", help="steps of the low, full and recovery phases")
    ap.add_argument("--page-rows", type=int, default=64, help="rows per optional-history page")
    ap.add_argument("--populate-pages", type=int, default=512, help="population bound per step (pages)")
    ap.add_argument("--reserve-pages", type=int, default=64, help="admission reserve (pages)")
    ap.add_argument("--shared-source", action="store_true",
                    help="shared KV sources: selecting, re-selecting and reusing layers per source")
    ap.add_argument("--reuse-per-selection", type=int, default=2,
                    help="layers reusing each selection (shared-source run)")
    ap.add_argument("--reselect-new", type=float, default=0.25,
                    help="share of a re-selecting layer's entries that differ from the first selection")
    ap.add_argument("--rounds", type=int, default=0,
                    help="decode rounds with commits (fresh selections each round): host backup beside "
                         "the next step vs ahead of it")
    ap.add_argument("--recent", type=float, default=0.02,
                    help="rounds run: share of each list drawn from the last 128 rows")
    ap.add_argument("--drift", type=float, default=0.1,
                    help="rounds run: share of each list redrawn every round (the rest repeats round 0's)")
    ap.add_argument("--resolver", action="store_true",
                    help="resolver cost against the unique host-miss bytes of one call (mla32 shape): shared, "
                         "partial and disjoint selections across the queries, cold and retained caches")
    ap.add_argument("--resolver-reps", type=int, default=9, help="timings per resolver point")
    ap.add_argument("--copy-probe", action="store_true",
                    help="a plain 1 GiB device copy, three times after a 1 GiB fill: the reference reading "
                         "that scales the FETCH_SIZE / WRITE_SIZE counters to bytes")
    return ap.parse_args()


def resolver_sweep(args):
    """Resolution apart from the attention ("Adaptive DHiSparse" §4.3.3, Fig. 8a):
    one call of 32 requests x 8 queries (k = 2048, B = 4096, MLA rows) with
    selections shared by all queries, half shared, or disjoint, each against
    an empty hot cache (cold) or the cache one identical call left (retained).
    Resolver time = plan + host fetch + victim choice (per-kernel HIP events,
    one fetch chunk); host-miss bytes = distinct fetched rows x row bytes.  A
    least-squares line through the six points gives the rate."""
    import numpy as np
    import torch

    from hierarchical_sparse_kv_verify_amd import KV_FLAG_TIMING
    from workloads.load import device_inputs as to_device, load_library
    from workloads import WORKLOADS, make_step_inputs, shrink

    torch.cuda.set_device(0)
    base = shrink(WORKLOADS["mla32"], var_k=False, pad_frac=0.0, invalid_frac=0.0)
    patterns = [("shared", dict(f_sh=1.0)), ("partial", dict(f_sh=0.5)), ("disjoint", dict(f_sh=0.0, disjoint=True))]
    points = []
    for name, kw in patterns:
        w = shrink(base, **kw)
        ld = load_library(w, warm=False, lib_kw=dict(n_chunks=1))
        lib = ld.lib
        si = make_step_inputs(w, 0, 0, ld.hist_len)
        d = to_device(si)
        out = torch.zeros((w.n_req, w.q_max, w.n_heads, w.d_v), dtype=torch.int16, device="cuda")
        lib.set_flags(KV_FLAG_TIMING)
        lib.save_cache(0)                                   # empty hot caches
        for cache in ("cold", "retained"):
            if cache == "retained":
                lib.restore_cache(0)
                lib.verify_step(0, d["queries"], d["topk"], d["causal"], d["ring"], out)
                torch.cuda.synchronize()
                lib.save_cache(0)                           # the state one call left
            lib.restore_cache(0)                            # warm-up call
            lib.verify_step(0, d["queries"], d["topk"], d["causal"], d["ring"], out)
            torch.cuda.synchronize()
            ms, parts = [], []
            for _ in range(args.resolver_reps):
                lib.restore_cache(0)
                lib.reset_stats()
                torch.cuda.synchronize()
                lib.verify_step(0, d["queries"], d["topk"], d["causal"], d["ring"], out)
                torch.cuda.synchronize()
                last = lib.stats(0)[0]                      # this call alone (stats reset before it)
                part = (float(last["ms_plan"]), float(last["ms_gather"]), float(last["ms_victims"]))
                parts.append(part)
                ms.append(sum(part))
            mb = int(last["union_miss"]) * w.row_bytes / 1e6
            med = float(np.median(ms))
            pm = [float(np.median([p[i] for p in parts])) for i in range(3)]
            points.append(dict(pattern=name, cache=cache, union_rows=int(last["union_rows"]),
                               missed_rows=int(last["union_miss"]), miss_mb=round(mb, 2),
                               resolver_ms=dict(min=round(min(ms), 4), median=round(med, 4), max=round(max(ms), 4)),
                               plan_ms=round(pm[0], 4), fetch_ms=round(pm[1], 4), victims_ms=round(pm[2], 4)))
            log("bench: %-8s %-8s union %7d missed %7d  %8.2f MB  resolver %.3f ms (plan %.3f fetch %.3f "
                "victims %.3f)" % (name, cache, points[-1]["union_rows"], points[-1]["missed_rows"], mb, med,
                                   pm[0], pm[1], pm[2]))
        lib.set_flags(0)
        lib.close()
        del ld, lib
    x = np.array([p["miss_mb"] for p in points])
    y = np.array([p["resolver_ms"]["median"] for p in points])
    A = np.stack([x, np.ones_like(x)], axis=1)
    (slope, icpt), *_ = np.linalg.lstsq(A, y, rcond=None)
    pred = A @ np.array([slope, icpt])
    r2 = 1.0 - float(((y - pred) ** 2).sum()) / max(1e-30, float(((y - y.mean()) ** 2).sum()))
    cold = {p["pattern"]: p["resolver_ms"]["median"] for p in points if p["cache"] == "cold"}
    print(json.dumps({
        "metric": "resolver time against unique host-miss bytes per call", "workload": "mla32 (32 requests, Q=8, "
        "k=2048, B=4096, MLA rows of 1152 B)", "points": points,
        "fit": {"rate_GBs": round(1.0 / slope, 2) if slope > 0 else None, "intercept_ms": round(float(icpt), 4),
                "r2": round(r2, 5)},
        "disjoint_over_shared_cold": round(cold["disjoint"] / cold["shared"], 2)}))


def copy_probe():
    """Known traffic for counter calibration: 3 x 1 GiB read, 4 x 1 GiB written."""
    import torch
    a = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": a.numel() * 4, "copies": 3}))


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the verification "
              "step would shard by request, with no exchange between GPUs)", file=sys.stderr)
        sys.exit(2)

    if args.copy_probe:
        copy_probe()
        return
    if args.resolver:
        resolver_sweep(args)
        return
    if args.load_step:
        load_step(args)
        return
    if args.shared_source:
        shared_source(args)
        return
    if args.rounds > 0:
        rounds(args)
        return

    import numpy as np
    import torch

    from hierarchical_sparse_kv_verify_amd import KV_FLAG_SERIAL, KV_FLAG_TIMING, KV_FLAG_TIMING_ATTN
    from workloads.load import device_inputs as to_device, load_library
    from workloads import WORKLOADS, make_history, make_step_inputs, shrink
    from workloads.gen import make_hist_len

    w = WORKLOADS[args.workload]
    if args.rho > 0:
        w = shrink(w, rho=args.rho)
    torch.cuda.set_device(0)
    t_setup = time.perf_counter()
    log("bench: generating %s (%d requests x %d groups)" % (w.name, w.n_req, w.n_groups))
    hl = make_hist_len(w)
    hists = [make_history(w, g, hl, progress=log if w.n_prefix > 4 else None) for g in range(w.n_groups)]
    log("bench: host rows ready (%.1fs); creating the library state" % (time.perf_counter() - t_setup))
    ld = load_library(w, rho=args.rho, histories=hists,
                      lib_kw=dict(n_chunks=args.n_chunks, fetch_cus=args.fetch_cus, fetch_wgs=args.fetch_wgs))
    lib = ld.lib
    G = w.n_groups
    sis = [make_step_inputs(w, g, 0, hl) for g in range(G)]
    dev = [to_device(si) for si in sis]
    out = torch.zeros((w.n_req, w.q_max, w.n_heads, w.d_v), dtype=torch.int16, device="cuda")
    for g in range(G):
        lib.save_cache(g)
    torch.cuda.synchronize()
    log("bench: setup done in %.1fs; info %s" % (time.perf_counter() - t_setup, lib.info))

    def restore():
        if not args.retained:
            for g in range(G):
                lib.restore_cache(g)

    def step():
        for g in range(G):
            d = dev[g]
            lib.verify_step(g, d["queries"], d["topk"], d["causal"], d["ring"], out)

    # The attention (the roofline's kernel) is timed with HIP events bound to
    # its launches (the launch's own start and end, no marker on its stream)
    # during the timed steps themselves.  Every other kernel is timed in a
    # separate pass, whose events on the fetch stream would otherwise
    # lengthen the timed steps.
    lib.set_flags(KV_FLAG_TIMING_ATTN)
    for _ in range(args.warmup):
        restore()
        step()
    torch.cuda.synchronize()
    lib.reset_stats()
    times = []
    for i in range(args.steps):
        restore()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        step()
        torch.cuda.synchronize()
        times.append(time.perf_counter() - t0)
    ms = 1000.0 * float(np.mean(times))
    cum = [lib.stats(g)[0] for g in range(G)]
    log("bench: %d steps, %.3f ms/step (min %.3f, max %.3f)" %
        (args.steps, ms, 1000 * min(times), 1000 * max(times)))

    live = cum
    lib.set_flags(KV_FLAG_TIMING)
    lib.reset_stats()
    for _ in range(args.timing_steps):
        restore()
        step()
    torch.cuda.synchronize()
    tim = [lib.stats(g)[0] for g in range(G)]
    # the attention alone on the GPU: it starts after the step's whole fetch
    lib.set_flags(KV_FLAG_SERIAL | KV_FLAG_TIMING_ATTN)
    lib.reset_stats()
    for _ in range(args.timing_steps):
        restore()
        step()
    torch.cuda.synchronize()
    alone = [lib.stats(g)[0] for g in range(G)]
    lib.set_flags(0)

    row_bytes = 2 * w.row_elems
    queries_per_step = int(sum(int(c["active_queries"]) for c in cum)) // max(1, args.steps) // G
    sel_per_step = sum(int(c["selections"]) for c in cum) / args.steps
    union_per_step = sum(int(c["union_rows"]) for c in cum) / args.steps
    miss_per_step = sum(int(c["union_miss"]) for c in cum) / args.steps
    selmiss_per_step = sum(int(c["sel_miss"]) for c in cum) / args.steps
    value = queries_per_step / (ms / 1000.0)

    # algorithmic work of the steps the kernel durations cover
    T = args.timing_steps
    tot = lambda key: sum(float(t[key]) for t in tim)
    fetched = sum(int(t["union_miss"]) for t in tim) * row_bytes
    n_ring_rows = 0
    for si in sis:
        for r in range(w.n_req):
            n_r = int(si.causal_pos[r, 0])
            if n_r < 0:
                continue
            lo0 = max(0, n_r - w.ring_window + 1)
            for j in range(w.q_max):
                p = int(si.causal_pos[r, j])
                if p >= 0:
                    n_ring_rows += p - max(lo0, p - w.ring_window + 1, 0) + 1
    # attention work of one step: every selected row and ring row once per
    # query (bf16), the queries, the outputs and the location codes
    rows_per_step = sel_per_step + n_ring_rows
    attn_bytes_step = (rows_per_step * row_bytes + queries_per_step * G * w.n_heads * (w.d_qk + w.d_v) * 2 +
                       queries_per_step * G * w.topk * 4)
    attn_flops_step = 2.0 * w.n_heads * rows_per_step * (w.d_qk + w.d_v)
    # live: the timed steps themselves
    live_ms = lambda key: sum(float(c[key]) for c in live)
    ms_attn = live_ms("ms_attn") + live_ms("ms_combine")
    n_attn_live = max(1, int(sum(int(c["n_attn"]) for c in live)))
    attn_bytes = attn_bytes_step * args.steps
    attn_flops = attn_flops_step * args.steps
    ms_gather = tot("ms_gather")
    ms_plan = tot("ms_plan")
    ms_promote = tot("ms_promote")
    ms_victims = tot("ms_victims")
    n_launch = lambda key: max(1, int(sum(int(t[key]) for t in tim)))
    promote_bytes = 2 * sum(int(t["promoted"]) for t in tim) * row_bytes
    plan_bytes = (sum(int(t["active_queries"]) for t in tim) * w.topk * 4 * 3 +
                  sum(int(t["union_rows"]) for t in tim) * 4 * 4)

    def rl(bound, work, ms_total, launches, peak, unit, traffic=None):
        achieved = (work / (ms_total / 1000.0)) / (1e9 if unit == "GB/s" else 1e12) if ms_total > 0 else 0.0
        return {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4) if peak else None, "traffic": traffic,
                "avg_launch_ms": round(ms_total / launches, 5), "launches": launches,
                "work_per_launch": work / launches}

    rooflines = {
        "miss_gather": rl("host_link", fetched, ms_gather, n_launch("n_gather"), PEAK_PCIE_GBS, "GB/s"),
        "sparse_attn": rl("hbm", attn_bytes, ms_attn, n_attn_live, PEAK_HBM_GBS, "GB/s"),
        "sparse_attn_mfma": rl("mfma", attn_flops, ms_attn, n_attn_live, PEAK_BF16_TFLOPS, "TFLOP/s"),
        "sparse_attn_alone": rl("hbm", attn_bytes_step * T,
                                sum(float(c["ms_attn"]) + float(c["ms_combine"]) for c in alone),
                                max(1, int(sum(int(c["n_attn"]) for c in alone))), PEAK_HBM_GBS, "GB/s"),
        "plan": rl("hbm", plan_bytes, ms_plan, n_launch("n_plan"), PEAK_HBM_GBS, "GB/s"),
        "promote": rl("hbm", promote_bytes, ms_promote, n_launch("n_promote"), PEAK_HBM_GBS, "GB/s"),
    }
    h2d = measure_h2d(torch)
    rooflines["miss_gather"]["measured_h2d_GBs"] = round(h2d, 2)
    rooflines["miss_gather"]["frac_of_measured_h2d"] = round(rooflines["miss_gather"]["achieved"] / h2d, 4)
    kernel_ms = {"miss_gather": ms_gather, "sparse_attn": ms_attn * T / args.steps, "plan": ms_plan,
                 "plan_victims": ms_victims, "promote": ms_promote}
    # The host fetch runs longest but moves its bytes over the host link; the
    # dominant kernel bound by the GPU's own memory is the sparse attention.
    roofline = dict(rooflines["sparse_attn"])
    roofline["kernel"] = "sparse_attn"
    # the counters were taken on the default mla128 step (four 32-request chunks,
    # cold-to-restored caches, no residency): other launches get no figure
    same_launch = (args.workload == "mla128" and args.rho == 0 and not args.retained and args.n_chunks == 0
                   and args.fetch_cus == 0 and args.fetch_wgs == 0)
    roofline["traffic"] = attn_traffic(attn_bytes / n_attn_live) if same_launch else None
    roofline["timing"] = "HIP events bound to every attention launch (its start and end) during the timed steps"
    rooflines["sparse_attn"]["traffic"] = roofline["traffic"]
    # host-link bytes from the IO read counter: rows of the shared prefix that
    # two requests of a chunk both miss can be served on the GPU side
    mg = rooflines["miss_gather"]
    mg["traffic"] = link_traffic(mg["work_per_launch"]) if same_launch else None
    if mg["traffic"] is not None:
        link_gbs = mg["traffic"] / (mg["avg_launch_ms"] / 1000.0) / 1e9
        mg["link_achieved_GBs"] = round(link_gbs, 3)
        mg["link_frac_of_measured_h2d"] = round(link_gbs / h2d, 4)
    roofline_host = dict(mg)
    roofline_host["kernel"] = "miss_gather"

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, hists, hl, sis, args.cpu_requests, args.cpu_groups)

    line = {
        "metric": "verified query-tokens/s per GPU and selected-rows/s; % HBM and host-link peak",
        "value": round(value, 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_min_median_max": [round(1000 * min(times), 4), round(1000 * float(np.median(times)), 4),
                                       round(1000 * max(times), 4)],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "requests": w.n_req, "layer_groups": G, "q_max": w.q_max,
                   "topk": w.topk, "hot_slots": w.hot_slots, "ring_window": w.ring_window,
                   "heads": w.n_heads, "row_bytes": row_bytes, "history_rows": [int(hl.min()), int(hl.max())],
                   "resident_fraction": args.rho, "cache_state": "retained" if args.retained else "restored",
                   "n_chunks": lib.info["n_chunks"], "attn_splits": lib.info["attn_splits"],
                   "fetch_cus": args.fetch_cus, "fetch_wgs": args.fetch_wgs},
        "selected_rows_per_s": round(sel_per_step / (ms / 1000.0), 1),
        "unique_rows_per_s": round(union_per_step / (ms / 1000.0), 1),
        "fetched_rows_per_step": miss_per_step,
        "fetched_bytes_per_step": miss_per_step * row_bytes,
        "host_fetch_share_distinct": round(miss_per_step / max(1.0, union_per_step), 5),
        "host_fetch_share_selected": round(selmiss_per_step / max(1.0, sel_per_step), 5),
        "missing_selections_per_fetched_row": round(selmiss_per_step / max(1.0, miss_per_step), 4),
        "kernel_ms_per_step": {k: round(v / T, 4) for k, v in kernel_ms.items()},
        "roofline": roofline,
        "roofline_host_link": roofline_host,
        "rooflines": rooflines,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    lib.close()


def load_step(args):
    """Optional residency under a load step, at the level of the verification
    step ("Adaptive DHiSparse" §4.3.1, Figure 6, Table A1): the same selections
    and hot-cache state every step, while the load goes from a few requests
    (their whole imported history resident on admission) to every request slot
    (admissions reclaim whole requests, eq. 4) and back (completions free pages
    that a bounded round-robin population refills).  Reports, per phase and
    step, the share of selections fetched from host, the coverage (ready over
    eligible pages) and the step time, with residency on and off."""
    import math

    import numpy as np
    import torch

    from workloads.load import device_inputs as to_device, load_library
    from workloads import WORKLOADS, make_history, make_step_inputs
    from workloads.gen import make_hist_len

    w = WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    P, lo, N, G = args.page_rows, args.load_lo, w.n_req, w.n_groups
    s_lo, s_hi, s_rec = (int(x) for x in args.load_steps.split(","))
    hl = make_hist_len(w)
    hists = [make_history(w, g, hl) for g in range(G)]
    sis = [make_step_inputs(w, g, 0, hl) for g in range(G)]
    # required allocations of an admitted request, in pages: its hot cache and
    # its ring of R_d = p*ceil((W+p-1+K_max)/p) rows
    ring_rows = w.ring_page * math.ceil((w.ring_window + w.ring_page - 1 + w.q_max) / w.ring_page)
    required = math.ceil((w.hot_slots + ring_rows) / P)
    elig_max = int(hl.max()) // P
    M = lo * (elig_max + required) + args.reserve_pages     # low load: every history fits
    lo_set = np.arange(N) < lo
    everyone = np.ones(N, dtype=bool)
    report = {}
    for arm in ("on", "off"):
        kw = dict(resident_cap=M * P, opt_page_rows=P, opt_reserve=args.reserve_pages) if arm == "on" else {}
        log("load step: arm %s, pool %d pages of %d rows (%.2f GB per group)" %
            (arm, M if arm == "on" else 0, P, M * P * 2 * w.row_elems / 1e9 if arm == "on" else 0.0))
        ld = load_library(w, histories=hists, lib_kw=kw)
        lib = ld.lib
        assert lib.info["ring_rows"] == ring_rows
        dev = [to_device(si) for si in sis]
        causal = {}
        for name, mask in (("lo", lo_set), ("all", everyone)):
            cs = []
            for si in sis:
                c = si.causal_pos.copy()
                c[~mask] = -1
                cs.append(torch.from_numpy(c).cuda())
            causal[name] = cs
        out = torch.zeros((N, w.q_max, w.n_heads, w.d_v), dtype=torch.int16, device="cuda")
        for g in range(G):
            lib.save_cache(g)
        admitted = []
        waits = 0
        if arm == "on":
            # resident-first admission: the imported history is placed on the device
            for r in range(lo):
                assert lib.opt_admit(r, required, admitted) is not None
                admitted.append(r)
            while lib.opt_populate(4096):
                pass
            lib.opt_publish(wait=True)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        series, phases = [], []
        for phase, n_steps, act in (("low", s_lo, "lo"), ("full", s_hi, "all"), ("recovery", s_rec, "lo")):
            reclaimed = 0
            if arm == "on" and phase == "full":
                for r in range(lo, N):
                    q = lib.opt_admit(r, required, admitted)
                    if q is None:
                        waits += 1
                        continue
                    reclaimed += q
                    admitted.append(r)
            if arm == "on" and phase == "recovery":
                for r in range(lo, N):
                    if r in admitted:
                        lib.opt_complete(r)
                        admitted.remove(r)
            rows = []
            for i in range(n_steps):
                for g in range(G):
                    lib.restore_cache(g)
                torch.cuda.synchronize()
                if arm == "on" and phase != "low":
                    lib.opt_populate(args.populate_pages)    # runs beside the step
                ev0.record()
                for g in range(G):
                    d = dev[g]
                    lib.verify_step(g, d["queries"], d["topk"], causal[act][g], d["ring"], out)
                ev1.record()
                torch.cuda.synchronize()
                ms = ev0.elapsed_time(ev1)
                last = [lib.stats(g)[1] for g in range(G)]
                tot = {k: sum(int(x[k]) for x in last) for k in ("selections", "sel_miss", "union_rows",
                                                                 "union_miss", "active_queries")}
                cov = None
                if arm == "on":
                    inf = lib.opt_info()
                    cov = inf["ready_pages"] / max(1, inf["eligible_pages"])
                rows.append(dict(ms=ms, cov=cov, share_sel=tot["sel_miss"] / max(1, tot["selections"]),
                                 share_dist=tot["union_miss"] / max(1, tot["union_rows"]),
                                 tokens=tot["active_queries"] / G))
                series.append([phase, round(ms, 3), None if cov is None else round(cov, 4),
                               round(rows[-1]["share_sel"], 5)])
            mean = lambda k: float(np.mean([x[k] for x in rows])) if rows else None
            ph = dict(phase=phase, steps=n_steps, active_requests=int(lo if act == "lo" else N),
                      ms_per_step=round(mean("ms"), 4),
                      tokens_per_s=round(mean("tokens") / (mean("ms") / 1000.0), 1),
                      host_share_selected=round(mean("share_sel"), 5),
                      host_share_distinct=round(mean("share_dist"), 5))
            if arm == "on":
                ph.update(coverage_first=round(rows[0]["cov"], 4), coverage_last=round(rows[-1]["cov"], 4),
                          coverage_mean=round(mean("cov"), 4), requests_reclaimed=reclaimed)
            phases.append(ph)
            log("load step: arm %s phase %s: %s" % (arm, phase, ph))
        res = dict(phases=phases, series=series)
        if arm == "on":
            inf = lib.opt_info()
            res.update(admissions_waited=waits, pages_populated=inf["pages_populated"],
                       pages_reclaimed=inf["pages_reclaimed"], bytes_populated=inf["bytes_populated"])
        report[arm] = res
        lib.close()
        del ld, lib, dev, causal, out
        torch.cuda.empty_cache()
    line = {"metric": "host-fetched share of selections under a load step, optional residency on/off",
            "unit": "fraction", "n_gpus": 1, "data": "synthetic",
            "config": {"workload": w.name, "requests": N, "low_load_requests": lo, "layer_groups": G,
                       "page_rows": P, "pool_pages": M, "required_pages_per_request": required,
                       "reserve_pages": args.reserve_pages, "populate_pages_per_step": args.populate_pages,
                       "steps": [s_lo, s_hi, s_rec], "reclaim_order": "admission order (oldest first)"},
            "arms": report}
    print(json.dumps(line), flush=True)


def shared_source(args):
    """Shared KV sources ("Adaptive DHiSparse" §2 physical-source sharing, §3.2,
    Table 3): per source and step a selecting layer (resolve, fetch, attend), a
    re-selecting layer (a fresh top-k sharing most entries with the first,
    resolved against the state the first left: only absent rows are fetched) and, after
    each, layers that reuse the latest selection with their own queries.  Arm
    "reuse" runs those layers through kv_hier_verify_reuse; arm "resolve"
    resolves the same selection again for each of them (same outputs)."""
    import numpy as np
    import torch

    from workloads.load import device_inputs as to_device, load_library
    from workloads import WORKLOADS, make_history, make_step_inputs, shrink
    from workloads.gen import make_hist_len

    w = WORKLOADS["ds_shared"] if args.workload == "mla128" else WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    G, R = w.n_groups, args.reuse_per_selection
    hl = make_hist_len(w)
    hists = [make_history(w, g, hl) for g in range(G)]
    ld = load_library(w, histories=hists)
    lib = ld.lib
    dev = torch.device("cuda")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    layers = []          # per source: (selection A inputs, reindex topk, consumer query sets)
    for g in range(G):
        si = make_step_inputs(w, g, 0, hl)
        sb = make_step_inputs(w, g, 1, hl)
        # the re-selection keeps the first selection's entries except a seeded
        # share, which it takes from another draw of the same generator
        keep = np.random.default_rng([20261009, 6, g, 77]).random(si.topk.shape) >= args.reselect_new
        topk_b = np.where(keep, si.topk, sb.topk).astype(np.int32)
        qs = [t(make_step_inputs(w, g, 2 + i, hl).queries.view(np.int16)) for i in range(2 * R)]
        layers.append(dict(d=to_device(si), topk_b=t(topk_b), qb=t(sb.queries.view(np.int16)), qs=qs))
    out = torch.zeros((w.n_req, w.q_max, w.n_heads, w.d_v), dtype=torch.int16, device="cuda")
    for g in range(G):
        lib.save_cache(g)
    torch.cuda.synchronize()

    def step(arm):
        for g in range(G):
            L = layers[g]
            d = L["d"]
            lib.verify_step(g, d["queries"], d["topk"], d["causal"], d["ring"], out)
            for i in range(R):
                if arm == "reuse":
                    lib.verify_reuse(g, L["qs"][i], d["causal"], out)
                else:
                    lib.verify_step(g, L["qs"][i], d["topk"], d["causal"], None, out)
            lib.verify_step(g, L["qb"], L["topk_b"], d["causal"], None, out)
            for i in range(R, 2 * R):
                if arm == "reuse":
                    lib.verify_reuse(g, L["qs"][i], d["causal"], out)
                else:
                    lib.verify_step(g, L["qs"][i], L["topk_b"], d["causal"], None, out)

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    report = {}
    for arm in ("reuse", "resolve"):
        for _ in range(args.warmup):
            for g in range(G):
                lib.restore_cache(g)
            step(arm)
        torch.cuda.synchronize()
        lib.reset_stats()
        times = []
        for _ in range(args.steps):
            for g in range(G):
                lib.restore_cache(g)
            torch.cuda.synchronize()
            ev0.record()
            step(arm)
            ev1.record()
            torch.cuda.synchronize()
            times.append(ev0.elapsed_time(ev1))
        cum = [lib.stats(g)[0] for g in range(G)]
        ms = float(np.mean(times))
        calls = sum(int(c["calls"]) for c in cum) / args.steps
        fetched = sum(int(c["union_miss"]) for c in cum) / args.steps
        union = sum(int(c["union_rows"]) for c in cum) / args.steps
        tokens = w.n_req * w.q_max
        report[arm] = dict(ms_per_step=round(ms, 4), ms_min=round(min(times), 4), ms_max=round(max(times), 4),
                           query_tokens_per_s=round(tokens / (ms / 1000.0), 1),
                           resolver_calls_per_step=calls, attention_layers_per_step=G * (2 + 2 * R),
                           fetched_rows_per_step=fetched, fetched_mb_per_step=round(fetched * 2 * w.row_elems / 1e6, 2),
                           union_rows_per_step=union)
        log("shared source: arm %s: %s" % (arm, report[arm]))
    # the re-selecting layer alone: rows it fetches against those of the first selection
    lib.reset_stats()
    for g in range(G):
        lib.restore_cache(g)
    first, second = 0, 0
    for g in range(G):
        L = layers[g]
        d = L["d"]
        lib.verify_step(g, d["queries"], d["topk"], d["causal"], d["ring"], out)
        first += int(lib.stats(g)[1]["union_miss"])
        lib.verify_step(g, L["qb"], L["topk_b"], d["causal"], None, out)
        second += int(lib.stats(g)[1]["union_miss"])
    torch.cuda.synchronize()
    line = {"metric": "verified query-tokens/s with shared KV sources (reuse vs re-resolution)",
            "unit": "query-tokens/s", "n_gpus": 1, "data": "synthetic", "steps": args.steps,
            "warmup": args.warmup,
            "config": {"workload": w.name, "requests": w.n_req, "sources": G, "q_max": w.q_max, "topk": w.topk,
                       "hot_slots": w.hot_slots, "heads": w.n_heads, "row_bytes": 2 * w.row_elems,
                       "reuse_layers_per_selection": R, "reselect_new_share": args.reselect_new,
                       "layers_per_source": "select, %d reuse, re-select, %d reuse" % (R, R)},
            "arms": report,
            "reselect_fetched_rows": second, "select_fetched_rows": first}
    print(json.dumps(line), flush=True)
    lib.close()


def rounds(args):
    """Decode rounds over the hierarchy (Figure 3): every round verifies all
    layer groups, then commits (eq. 7); nothing is restored between rounds.
    Selections drift: each round redraws a seeded share of every list (a
    share of those from the most recent rows) and keeps the rest of the first
    round's, so the hot cache follows a slowly moving working set.  Arm
    "async": the committed rows' host backup runs beside the next round
    (those rows resolve from the tail meanwhile); arm "sync": it runs ahead of
    the next round on the caller's stream (KV_FLAG_SYNC_BACKUP)."""
    import numpy as np
    import torch

    from hierarchical_sparse_kv_verify_amd import KV_FLAG_SYNC_BACKUP
    from workloads.load import device_inputs as to_device, load_library
    from workloads import WORKLOADS, make_accepted, make_history, make_step_inputs, shrink
    from workloads.gen import make_hist_len

    w = shrink(WORKLOADS[args.workload], recent_frac=args.recent, recent_span=128)
    torch.cuda.set_device(0)
    G, R = w.n_groups, args.rounds
    hl = make_hist_len(w)
    hists = [make_history(w, g, hl) for g in range(G)]
    log("rounds: generating %d rounds of inputs" % (R + args.warmup))
    plan = []
    n = hl.copy()
    base = [make_step_inputs(w, g, 100, hl) for g in range(G)]
    for i in range(R + args.warmup):
        sis = [make_step_inputs(w, g, 101 + i, n) for g in range(G)]
        for g, si in enumerate(sis):
            keep = np.random.default_rng([20261009, 3, g, 500 + i]).random(si.topk.shape) >= args.drift
            si.topk = np.where(keep & (si.topk >= 0), base[g].topk, si.topk).astype(np.int32)
        acc = make_accepted(w, i, sis[0].k_active)
        plan.append(([to_device(si) for si in sis], acc))
        n = n + 1 + acc
    report = {}
    for arm in ("async", "sync"):
        ld = load_library(w, histories=hists,
                          lib_kw=dict(flags=KV_FLAG_SYNC_BACKUP if arm == "sync" else 0))
        lib = ld.lib
        out = torch.zeros((w.n_req, w.q_max, w.n_heads, w.d_v), dtype=torch.int16, device="cuda")
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        tails = sels = fetched = 0
        for i, (devs, acc) in enumerate(plan):
            if i == args.warmup:
                torch.cuda.synchronize()
                lib.reset_stats()
                ev0.record()
            for g in range(G):
                d = devs[g]
                lib.verify_step(g, d["queries"], d["topk"], d["causal"], d["ring"], out)
            lib.commit(acc)
        ev1.record()
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1) / R
        cum = [lib.stats(g)[0] for g in range(G)]
        tok = sum(int(c["active_queries"]) for c in cum) / G / R
        report[arm] = dict(ms_per_round=round(ms, 4), query_tokens_per_s=round(tok / (ms / 1000.0), 1),
                           tail_share_selected=round(sum(int(c["sel_tail"]) for c in cum) /
                                                     max(1, sum(int(c["selections"]) for c in cum)), 5),
                           host_share_distinct=round(sum(int(c["union_miss"]) for c in cum) /
                                                     max(1, sum(int(c["union_rows"]) for c in cum)), 5),
                           fetched_mb_per_round=round(sum(int(c["union_miss"]) for c in cum) * 2 * w.row_elems
                                                      / R / 1e6, 2))
        log("rounds: arm %s: %s" % (arm, report[arm]))
        lib.close()
        del ld, lib
        torch.cuda.empty_cache()
    print(json.dumps({"metric": "decode rounds with commits: host backup beside vs ahead of the next round",
                      "unit": "ms per round", "n_gpus": 1, "data": "synthetic", "rounds": R,
                      "warmup": args.warmup,
                      "config": {"workload": w.name, "requests": w.n_req, "layer_groups": G,
                                 "recent_share": args.recent, "recent_span": 128, "drift": args.drift},
                      "arms": report}), flush=True)


def measure_h2d(torch, mib=512, reps=3):
    """Best pinned host -> device copy rate (GB/s) of a bulk transfer."""
    src = torch.empty(mib << 20, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(mib << 20, dtype=torch.uint8, device="cuda")
    best = 0.0
    for _ in range(reps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        dst.copy_(src, non_blocking=True)
        torch.cuda.synchronize()
        best = max(best, src.numel() / (time.perf_counter() - t0) / 1e9)
    del src, dst
    return best


def _counter_ratio(profile, key, sources):
    """A counter-measured bytes-per-algorithmic-byte ratio from a committed
    rocprofv3 summary (its ``traffic:`` line), or None when a source file the
    counted traffic depends on changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", profile)
    try:
        text = open(path).read()
        digests = {os.path.splitext(src)[0] + "_sha256": hashlib.sha256(
            open(os.path.join(ROOT, "hierarchical_sparse_kv_verify_amd", "csrc", src), "rb").read()).hexdigest()
            for src in sources}
    except OSError:
        return None
    vals = {}
    for ln in text.splitlines():
        if ln.startswith("traffic:"):
            for kv in ln[len("traffic:"):].split():
                k, _, v = kv.partition("=")
                vals[k] = v
    if key not in vals or any(vals.get(tag) != d for tag, d in digests.items()):
        return None
    return float(vals[key])


def attn_traffic(algo_bytes_per_launch):
    """HBM bytes per attention launch of the default mla128 step: DRAM reads +
    writes from the TCC counters (profiles/sparse_attn_mla128_traffic.md)."""
    # the walk order of the lists (the order kernel) sets how much the L2 serves
    r = _counter_ratio("sparse_attn_mla128_traffic.md", "bytes_per_algo_byte", ("attn.hip", "plan.hip"))
    return None if r is None else round(r * algo_bytes_per_launch, 1)


def link_traffic(algo_bytes_per_launch):
    """Host-link bytes per fetch launch of the default mla128 step: the TCC IO
    read counter (profiles/miss_gather_mla128_host_link.md)."""
    r = _counter_ratio("miss_gather_mla128_host_link.md", "io_bytes_per_algo_byte", ("copy.hip",))
    return None if r is None else round(r * algo_bytes_per_launch, 1)


def _cpu_model():
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, hists, hl, sis, n_req_sample, n_groups_sample):
    """The oracle, as it stands, on the host cores over the first requests of
    the first layer groups (resolution + attention of all their queries)."""
    import oracle
    from workloads import make_hot_warm_set
    from workloads.load import prefill_rows

    # the host gives each GPU a share of 16 threads, whatever the affinity
    # mask shows: the oracle's worker pool is sized to that share
    online = len(os.sched_getaffinity(0))
    cores = min(online, CPU_SHARE_THREADS)
    reqs = list(range(min(n_req_sample, w.n_req)))
    groups = list(range(max(1, min(n_groups_sample, w.n_groups))))
    # no commit happens here, so the oracle may read the generator's rows in place
    ocfg = oracle.OracleConfig(
        n_req=w.n_req, n_groups=w.n_groups, hist_cap=w.hist_cap, n_prefix=w.n_prefix, prefix_len=w.prefix_len,
        row_elems=w.row_elems, d_qk=w.d_qk, v_off=w.v_off, d_v=w.d_v, n_heads=w.n_heads, q_max=w.q_max,
        topk=w.topk, hot_slots=w.hot_slots, ring_window=w.ring_window, ring_page=w.ring_page)
    orc = oracle.HierOracle(ocfg, hists, hl, requests=reqs)
    for g in groups:
        for r, hs in enumerate(make_hot_warm_set(w, g, hl, sis[g])):
            orc.set_hot(g, r, hs[0], hs[1])
        for r in reqs:
            first, rows = prefill_rows(hists[g], w, r, int(hl[r]))
            orc.ring_load(g, r, first, rows)
    log("bench: oracle on %d requests x %d queries x %d layer groups, %d threads" %
        (len(reqs), w.q_max, len(groups), cores))
    dt = 0.0
    for g in groups:
        si = sis[g]
        t0 = time.perf_counter()
        res = orc.verify_step(g, si.topk, si.causal_pos, si.queries, si.block_rows, n_threads=cores)
        dt += time.perf_counter() - t0
    nq = len(res.out)
    # one query token of a step passes through every layer group
    value = nq / (dt * w.n_groups / len(groups))
    log("bench: oracle %.2fs for %d query tokens of %d layer groups" % (dt, nq, len(groups)))
    return {"value": round(value, 3), "unit": "query-tokens/s", "cores": cores, "kind": "oracle",
            "online_cores": online, "cpu_model": _cpu_model(),
            "threads_note": "oracle threads = min(online cores, %d): the GPU host's CPU share per GPU"
                            % CPU_SHARE_THREADS,
            "sample": "%d requests x %d queries of layer groups 0..%d of %s (resolution + attention), "
                      "scaled to %d layer groups per step; %.2f s" % (len(reqs), w.q_max, len(groups) - 1,
                                                                      w.name, w.n_groups, dt)}


if __name__ == "__main__":
    main()
