"""Benchmark: one constrained coarsening level of a synthetic SNN-style
hypergraph on one MI355X.

Default workload: the 4,000,000-node block SNN graph (Poisson(250) fan-out
clipped to [2,4096], 90% of destinations in the source's aligned block of
65,536 ids, weights 1..8, Omega 1,024, Delta 16,384; about 1.0e9 pins), the
largest configuration, whose description asks for one timed level of rate +
match + contract.  `--workload 1..4` selects the smaller ones (the 100k-node
ring, the layered 1M-node graph and the 2M-node VLSI netlist run their whole
coarsening; the netlist evaluates its projected partition after every level).

One step = the whole hot path: build the canonical CSR and incidence (and
the neighbourhoods where they fit in 64 GB); coarsen level by level (rate,
handshake match, pair the nodes left without a partner, contract) until the
workload's stop rule; then evaluate the projected partition on the input
graph.  The input edge CSR is resident in HBM before timing starts.

value = pins processed by the coarsening levels (sum over levels of the
level's pin count) per second of whole-step time (build and evaluation
included).  The rating kernels' durations come from HIP events the library
records on its stream during the timed steps (only those kernels are
bracketed there); the per-kernel breakdown, the per-level times and the pin
visits per level come from one more step run after the timed ones.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
RATE_KERNELS = ("rate_big", "rate", "rate_inc", "rate_incq")
RATE_PASS = "+".join(RATE_KERNELS) + " (the rating pass)"
# Invalid neighbours are flagged by the rating and purged from the coarse
# neighbourhoods (the pages' coarsening does this; --no-purge turns it off).
PURGE = True
# Nodes left without a partner are paired best-effort, as the pages'
# coarsening does (--no-leftovers turns it off).
LEFTOVERS = True
# candidates kept per node; above 1, that many matching rounds (--pi)
PI = 1
# The driver stops after a level that pairs fewer than this fraction of its
# nodes (a stalled coarsening: each further level would cost a full pass for a
# handful of pairs).
MIN_PAIR_FRAC = 0.001
# workloads whose projected partition is evaluated after every level (the
# VLSI netlist's description asks for it), not only after the last
EVAL_EVERY_LEVEL = {4}
CSRC = os.path.join(ROOT, "constrained_hypergraph_partitioning_amd", "csrc")
RATE_SOURCES = [os.path.join(CSRC, f) for f in ("k_rate.hip", "k_rate_inc.hip", "k_rate_incq.hip",
                                                 "dev.h")]
COPY_REF_MIB = 256
# Pin visits per second the LDS can absorb: every visit is one 64-bit atomic
# add into an LDS slot; 256 CUs x 2.4 GHz x 128 bytes of LDS per clock per CU
# / 8 bytes per add (the derivation and its measurement are in the design
# notes).
LDS_VISIT_PEAK = 256 * 2.4e9 * 128 / 8


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--workload", type=int, default=5, help="workload index 1..5")
    p.add_argument("--nodes", type=int, default=None, help="shrink the workload (testing)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-nodes", type=int, default=None,
                   help="workloads 1-4: rate a smaller instance; workload 5: nodes of the "
                        "full graph the oracle rates")
    p.add_argument("--cpu-threads", type=int, default=None,
                   help="threads of the oracle's rating in the CPU baseline (default: "
                        "min(16, cpus) for workload 5, 1 otherwise)")
    p.add_argument("--copy-ref-mib", type=int, default=0,
                   help="run one plain device copy of this size first (a reference for "
                        "scaling hardware byte counters)")
    p.add_argument("--no-neighbour-lists", action="store_true",
                   help="build the graph without neighbour lists even where they fit")
    p.add_argument("--progress", action="store_true",
                   help="print a line per timed step to stderr (long workloads)")
    p.add_argument("--optimal-matching", action="store_true",
                   help="match by the exact maximum-weight matching of the proposal graph "
                        "instead of the greedy handshake")
    p.add_argument("--pi", type=int, default=1,
                   help="candidates kept per node (1..4); above 1 the matching takes that many "
                        "rounds over the top-pi lists")
    p.add_argument("--moves", action="store_true",
                   help="also time the refinement move proposal (Eq. 13) on the input graph "
                        "under the step's projected partition, Omega enforced")
    p.add_argument("--refine", type=int, default=0, metavar="THETA",
                   help="also time THETA refinement passes (proposal, chained sequence, "
                        "in-sequence gains, event validity, best prefix) on the input graph "
                        "from the step's projected partition, Omega enforced")
    p.add_argument("--vcycle", type=int, default=0, metavar="THETA",
                   help="also time the whole V-cycle: the coarsening as the step runs it, "
                        "then the coarsest nodes as partitions, THETA refinement passes per "
                        "level (the first half proposing without Omega) and projection down "
                        "to the input graph")
    p.add_argument("--no-leftovers", action="store_true",
                   help="do not pair the nodes left without a partner")
    p.add_argument("--no-purge", action="store_true",
                   help="keep invalid neighbours in the coarse neighbourhoods")
    p.add_argument("--counters", metavar="DIR", default=None,
                   help="no run: summarise the rocprofv3 FETCH_SIZE and WRITE_SIZE passes "
                        "under DIR/fetch and DIR/write into profiles/rating_counters_"
                        "<workload>.json")
    return p.parse_args()


def source_sha():
    """Hash of the rating kernels' sources (counter summaries are valid for
    them only)."""
    h = hashlib.sha256()
    for p in RATE_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def counters_json(workload):
    return os.path.join(ROOT, "profiles", "rating_counters_%s.json" % workload)


def kernel_base(name):
    """'void (anonymous namespace)::k_rate<...>(args)' -> 'k_rate'."""
    name = name.replace("(anonymous namespace)::", "").replace("void ", "")
    return name.split("(")[0].split("<")[0].strip()


def _counter_rows(d):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if len(files) != 1:
        raise SystemExit("expected one counter_collection.csv under %s, found %d" % (d, len(files)))
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def summarize_counters(d, workload):
    """HBM bytes per rating pass from two counter passes (FETCH_SIZE, then
    WRITE_SIZE; KiB per dispatch), each scaled by what the same counter read
    for the reference copy of COPY_REF_MIB MiB that the profiled run made
    first (its bytes read and written are known)."""
    out = {"source_sha256": source_sha(), "workload": workload,
           "copy_ref_bytes": COPY_REF_MIB << 20}
    for name, counter in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        rows = [r for r in _counter_rows(os.path.join(d, name)) if r["Counter_Name"] == counter]
        ref = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        rate = [r for r in rows
                if kernel_base(r["Kernel_Name"]) in ("k_rate", "k_rate_big", "k_rate_inc",
                                                     "k_rate_incq")]
        # one rating pass per level: a k_rate launch, or k_rate_inc where
        # every node of the level is rated from the incidence
        passes = max(sum(1 for r in rate if kernel_base(r["Kernel_Name"]) == k)
                     for k in ("k_rate", "k_rate_inc", "k_rate_incq"))
        if not ref or not passes:
            raise SystemExit("%s: no reference copy or no rating dispatch found" % name)
        kib = sum(float(r["Counter_Value"]) for r in rate)
        scale = (COPY_REF_MIB << 10) / max(ref)
        out[name] = {"counter": counter, "kib_per_pass": kib / passes, "passes": passes,
                     "copy_ref_kib": max(ref), "scale": scale}
    out["traffic_bytes_per_pass"] = 1024 * (out["fetch"]["kib_per_pass"] * out["fetch"]["scale"] +
                                            out["write"]["kib_per_pass"] * out["write"]["scale"])
    path = counters_json(workload)
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def measured_traffic(workload):
    """Bytes per rating pass from the committed counter summary, if it was
    taken on this workload with the current rating source; else None."""
    try:
        with open(counters_json(workload)) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("source_sha256") != source_sha() or c.get("workload") != workload:
        return None
    return c.get("traffic_bytes_per_pass")


# Neighbour lists above this many bytes are not materialised for the whole
# graph: the rating then builds them batch by batch (workload 5: ~1.9e11 ids).
NB_BYTES_MAX = 64 << 30


def run_step(chp, ctx, dev_edges, spec, rho_buf, with_nb=True, eval_every=False, detail=False):
    """One pass of the hot path.  Returns the per-level records (nodes, pins,
    pairs, neighbour entries, and with detail: ms and pin visits), the final
    evaluation summary and, with eval_every, the connectivity of the projected
    partition after each level."""
    import torch
    g0 = ctx.build_incidence(*dev_edges, spec.omega, spec.delta, with_nb)
    total_size = int(spec_total_size(dev_edges))
    floor_nodes = -(-total_size // spec.omega)
    levels = []
    level_conn = []
    g = g0
    rho = None
    for lvl in range(spec.levels):
        if spec.target_nodes and g.n_nodes < spec.target_nodes:
            break
        if g.n_nodes <= floor_nodes:
            break
        if detail:
            torch.cuda.synchronize()
            t_l = time.perf_counter()
        flags = ctx.new_flags(g) if PURGE and with_nb else None
        if PI > 1:
            tl, _, match, npairs = ctx.rate_top_and_match(g, PI, spec.omega, spec.delta, True,
                                                          spec.seed, flags=flags)
            tgt = tl[0]
        else:
            tgt, _, match, npairs = ctx.rate_and_match(g, spec.omega, spec.delta, True,
                                                       spec.seed, flags=flags)
        if LEFTOVERS:
            npairs += ctx.pair_leftovers(g, tgt, match, spec.omega, spec.delta)
        nb_total = g.nb_total if with_nb else ctx.last_rate_stats()[0]
        rec = [g.n_nodes, g.n_pins, npairs, nb_total]
        levels.append(rec)
        if npairs == 0:
            if detail:
                torch.cuda.synchronize()
                rec += [(time.perf_counter() - t_l) * 1e3, level_visits(g)]
            break
        gamma, cg = ctx.contract(g, match, with_nb, flags=flags)
        rho = gamma.long() if rho is None else gamma.long()[rho]
        if detail:
            torch.cuda.synchronize()
            rec += [(time.perf_counter() - t_l) * 1e3, level_visits(g)]
        if eval_every:
            rho_buf.copy_(rho.to(torch.int32))
            _, _, s_l = ctx.evaluate_partition(g0, rho_buf, cg.n_nodes, spec.omega, spec.delta)
            level_conn.append(int(s_l[0]))
        stalled = npairs < MIN_PAIR_FRAC * g.n_nodes
        if g is not g0:
            g.free()
        g = cg
        if stalled:
            break
    k = g.n_nodes
    if rho is None:
        rho = torch.arange(g0.n_nodes, device=ctx.device)
    rho_buf.copy_(rho.to(torch.int32))
    _, _, summ = ctx.evaluate_partition(g0, rho_buf, k, spec.omega, spec.delta)
    if g is not g0:
        g.free()
    g0.free()
    return levels, summ, level_conn


def level_visits(g):
    """Pin visits of a rating pass over g: every node visits every pin of
    every hyperedge it belongs to, so sum over hyperedges of |e|^2."""
    import torch
    sz = torch.diff(g.tensor("e_off")).double()
    return float((sz * sz).sum().item())


_size_cache = {}


def spec_total_size(dev_edges):
    key = dev_edges[4].data_ptr()
    if key not in _size_cache:
        _size_cache[key] = int(dev_edges[4].long().sum().item())
    return _size_cache[key]


def cpu_info():
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return os.cpu_count(), model


def cpu_baseline(h, spec, workload, sample_nodes, threads):
    """The CPU oracle on a bounded sample of the same workload.
    Workloads 1-4: level 0 (build incidence + neighbours, rate, match,
    contract) of the workload or of a smaller instance, single-threaded.
    Workload 5: the oracle builds the full graph's incidence (not timed), then
    rates nodes 0..R-1 (the level's dominant step) over `threads` threads; the
    value scales that rate to the level's pins (P * R / N per second)."""
    import oracle
    import synth
    nproc, model = cpu_info()
    if workload == 5:
        R = sample_nodes or 65536
        threads = threads or min(16, nproc or 1)
        g = oracle.build_incidence(h.e_off, h.e_nsrc, h.e_pins, h.e_w, h.n_size, spec.omega,
                                   spec.delta, False)
        tc = oracle.terms(g)
        t0 = time.perf_counter()
        oracle.rate(g, spec.omega, spec.delta, True, spec.seed, lo=0, hi=R, tc=tc,
                    threads=threads)
        dt = time.perf_counter() - t0
        del g
        return {"value": h.n_pins * (R / h.n_nodes) / dt, "unit": "pins/s", "cores": threads,
                "kind": "oracle", "nproc": nproc, "cpu_model": model,
                "sample": "oracle rating of nodes 0..%d of the full %s graph (%d nodes, %d "
                          "pins; the level's dominant step, incidence built beforehand, not "
                          "timed): %.1f s over %d threads, scaled to the level as P*R/N per "
                          "second" % (R - 1, h.spec.name, h.n_nodes, h.n_pins, dt, threads)}
    threads = threads or 1
    if sample_nodes and sample_nodes < h.n_nodes:
        h = synth.generate(synth.config(workload, n_nodes=sample_nodes))
    t0 = time.perf_counter()
    g = oracle.build_incidence(h.e_off, h.e_nsrc, h.e_pins, h.e_w, h.n_size, spec.omega,
                               spec.delta)
    oracle.level(g, spec.omega, spec.delta, True, spec.seed, threads=threads)
    dt = time.perf_counter() - t0
    return {"value": h.n_pins / dt, "unit": "pins/s", "cores": threads, "kind": "oracle",
            "nproc": nproc, "cpu_model": model,
            "sample": "level 0 (build incidence+neighbours, rate, match, contract) of %s: "
                      "%d nodes, %d pins, %.1f s, rating over %d thread(s)"
                      % (h.spec.name, h.n_nodes, h.n_pins, dt, threads)}


def main():
    args = parse()
    if args.counters:
        import synth
        summarize_counters(args.counters, synth.config(args.workload, n_nodes=args.nodes).name)
        return
    global PURGE, LEFTOVERS, PI
    PI = args.pi
    PURGE = not args.no_purge
    LEFTOVERS = not args.no_leftovers
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import constrained_hypergraph_partitioning_amd as chp
    import synth

    spec = synth.config(args.workload, n_nodes=args.nodes)
    h = synth.generate(spec)
    print("[bench] generated %s: %d pins" % (spec.name, h.n_pins), file=sys.stderr, flush=True)
    ctx = chp.Context(0)
    ctx.set_matching(args.optimal_matching)
    dev_edges = chp.upload_edges(h)
    rho_buf = torch.empty(h.n_nodes, dtype=torch.int32, device=ctx.device)
    if args.copy_ref_mib:
        src = torch.ones(args.copy_ref_mib << 18, dtype=torch.int32, device=ctx.device)
        dst = torch.empty_like(src)
        dst.copy_(src)
        del src, dst
    torch.cuda.synchronize()

    sz = np.diff(h.e_off).astype(np.float64)
    with_nb = float((sz * (sz - 1)).sum()) * 4 <= NB_BYTES_MAX and not args.no_neighbour_lists
    eval_every = args.workload in EVAL_EVERY_LEVEL
    for i in range(args.warmup):
        t_w = time.perf_counter()
        run_step(chp, ctx, dev_edges, spec, rho_buf, with_nb, eval_every)
        torch.cuda.synchronize()
        print("[bench] warmup step %d: %.3f s" % (i, time.perf_counter() - t_w), file=sys.stderr,
              flush=True)
    torch.cuda.synchronize()
    # timed steps: HIP events around the rating kernels only (events on every
    # launch would add their own host cost to the step time)
    ctx.reset_timings()
    ctx.set_timing_filter("rate")
    ctx.set_timing(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    pins = 0
    levels = None
    for i in range(args.steps):
        levels, summ, level_conn = run_step(chp, ctx, dev_edges, spec, rho_buf, with_nb,
                                            eval_every)
        pins += sum(lv[1] for lv in levels)
        if args.progress:
            print("[bench] step %d queued" % i, file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    timings = ctx.timings()
    # one more step, untimed, with every kernel timed: the per-kernel
    # breakdown; then one with a synchronisation around each level: the
    # per-level times and pin visits
    ctx.reset_timings()
    ctx.set_timing_filter(None)
    run_step(chp, ctx, dev_edges, spec, rho_buf, with_nb, eval_every)
    torch.cuda.synchronize()
    all_timings = ctx.timings()
    ctx.set_timing(False)
    detail, _, _ = run_step(chp, ctx, dev_edges, spec, rho_buf, with_nb, eval_every, True)
    torch.cuda.synchronize()

    # The rating pass (per level one launch of "rate_big", the nodes whose
    # neighbourhood exceeds one window of the small table, and one of
    # "rate", all other nodes) and its algorithmic bytes: each array it reads
    # or writes counted once per level.
    dom = max(all_timings.items(), key=lambda kv: kv[1][1])
    passes = len(levels) * args.steps  # one rating pass per level
    rate_ms = sum(timings.get(k, (0, 0.0))[1] for k in RATE_KERNELS)
    visits_per_step = sum(lv[5] for lv in detail)
    visits_s = visits_per_step * args.steps / (rate_ms / 1e3) if rate_ms else 0.0
    level_bytes = rate_level_bytes(levels, h, spec)
    rate_bytes_per_step = sum(level_bytes)
    achieved = rate_bytes_per_step * args.steps / (rate_ms / 1e3) / 1e9 if rate_ms else 0.0
    kern_ms = {k: round(v[1], 4) for k, v in
               sorted(all_timings.items(), key=lambda kv: -kv[1][1])[:12]}
    level_ms = sum(v[1] for k, v in all_timings.items())

    out = {
        "metric": "pins/s per constrained coarsening level (rate+match+contract); "
                  "HBM GB/s vs peak",
        "value": pins / dt,
        "unit": "pins/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": dt * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32/u64 (integer ids, 40-bit fixed-point ratings)",
        "data": "synthetic (seeded generator shaped like the pages' SNN workloads)",
        "config": {"workload": spec.name, "nodes": h.n_nodes, "hyperedges": h.n_edges,
                   "neighbourhoods": "whole graph" if with_nb else "built per node batch",
                   "purge": PURGE and with_nb, "leftover_pairing": LEFTOVERS,
                   "matching": "optimal" if args.optimal_matching else "handshake",
                   "candidates_pi": PI,
                   "pins": h.n_pins, "omega": spec.omega, "delta": spec.delta,
                   "levels": len(levels), "final_nodes": levels[-1][0] - levels[-1][2]
                   if levels else h.n_nodes, "connectivity": int(summ[0])},
        "roofline": {"bound": "hbm", "kernel": RATE_PASS,
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "avg_pass_ms": rate_ms / max(passes, 1),
                     "alg_bytes_per_pass": rate_bytes_per_step / max(len(levels), 1),
                     "traffic": measured_traffic(spec.name)},
        "roofline_visits": {"bound": "lds", "kernel": RATE_PASS,
                            "achieved": visits_s, "peak": LDS_VISIT_PEAK, "unit": "visits/s",
                            "frac": visits_s / LDS_VISIT_PEAK,
                            "visits_per_pass": visits_per_step / max(len(levels), 1)},
        "per_level": {"nodes": [lv[0] for lv in levels], "pins": [lv[1] for lv in levels],
                      "pairs": [lv[2] for lv in levels],
                      "neighbour_entries": [lv[3] for lv in levels],
                      "visits": [lv[5] for lv in detail],
                      "ms": [round(lv[4], 3) for lv in detail]},
        "kernel_ms_per_step": kern_ms,
        "kernel_sum_ms_per_step": level_ms,
        "dominant_kernel": dom[0],
        "cpu_baseline": None,
    }
    if eval_every:
        out["per_level"]["projected_connectivity"] = level_conn
    if args.moves:
        out["moves"] = time_moves(ctx, dev_edges, spec, rho_buf, out["config"]["final_nodes"], h)
    if args.refine:
        out["refine"] = time_refine(ctx, dev_edges, spec, rho_buf, out["config"]["final_nodes"],
                                    h, args.refine)
    if args.vcycle:
        out["vcycle"] = time_vcycle(ctx, dev_edges, spec, with_nb, args.vcycle)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(h, spec, args.workload, args.cpu_sample_nodes,
                                           args.cpu_threads)
    print(json.dumps(out))


def time_moves(ctx, dev_edges, spec, rho_buf, k, h, reps=5):
    """The Eq. 13 move proposal on the input graph under the projected
    partition of the last step (k parts), Omega enforced: ms per call (HIP
    events of the library, synchronised calls) and pins per second."""
    import torch
    g0 = ctx.build_incidence(*dev_edges, spec.omega, spec.delta, False)
    ctx.propose_moves(g0, rho_buf, k, spec.omega, True)
    torch.cuda.synchronize()
    ctx.reset_timings()
    ctx.set_timing(True)
    t0 = time.perf_counter()
    for _ in range(reps):
        mv, gn = ctx.propose_moves(g0, rho_buf, k, spec.omega, True)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    tm = ctx.timings()
    ctx.set_timing(False)
    improving = int((gn > 0).sum().item())
    g0.free()
    return {"parts": k, "ms_per_call": dt * 1e3, "pins_per_s": h.n_pins / dt,
            "improving_moves": improving,
            "kernel_ms_per_call": {kk: round(v[1] / reps, 4) for kk, v in
                                   sorted(tm.items(), key=lambda kv: -kv[1][1])[:8]}}


def time_refine(ctx, dev_edges, spec, rho_buf, k, h, theta):
    """theta refinement passes on the input graph from the projected partition
    of the last step (k parts), Omega enforced, chained move order: ms per
    pass (synchronised calls), the connectivity before and after, the moves
    applied, and the per-kernel breakdown (library HIP events, one extra run
    of the same passes)."""
    import torch
    g0 = ctx.build_incidence(*dev_edges, spec.omega, spec.delta, False)
    rho0 = rho_buf.clone()

    def run(timed):
        rho = rho0.clone()
        applied = gain = 0
        ms = []
        for _ in range(theta):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            _, na, ga = ctx.refine_pass(g0, rho, k, spec.omega, spec.delta, True)
            torch.cuda.synchronize()
            ms.append((time.perf_counter() - t0) * 1e3)
            applied += na
            gain += ga
        return rho, applied, gain, ms

    run(False)  # warm-up
    rho, applied, gain, ms = run(True)
    ctx.reset_timings()
    ctx.set_timing(True)
    run(False)
    tm = ctx.timings()
    ctx.set_timing(False)
    _, _, s0 = ctx.evaluate_partition(g0, rho0, k, spec.omega, spec.delta)
    _, _, s1 = ctx.evaluate_partition(g0, rho, k, spec.omega, spec.delta)
    g0.free()
    return {"passes": theta, "parts": k, "ms_per_pass": sum(ms) / theta,
            "ms_first_pass": ms[0], "moves_applied": applied, "gain": gain,
            "connectivity_before": int(s0[0]), "connectivity_after": int(s1[0]),
            "parts_over_omega": int(s1[2]), "parts_over_delta": int(s1[3]),
            "kernel_ms_per_pass": {kk: round(v[1] / theta, 4) for kk, v in
                                   sorted(tm.items(), key=lambda kv: -kv[1][1])[:10]}}


def time_vcycle(ctx, dev_edges, spec, with_nb, theta):
    """The whole multi-level scheme ([HP] Sec. III) on the input graph: the
    coarsening as run_step runs it (keeping every level), the coarsest nodes
    as the initial partitions, then from the coarsest level down theta
    refinement passes per level and the projection to the level below.
    Reports the two phases' times (synchronised), the time per level of the
    uncoarsening, and the connectivity after each phase."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g0 = ctx.build_incidence(*dev_edges, spec.omega, spec.delta, with_nb)
    floor_nodes = -(-int(spec_total_size(dev_edges)) // spec.omega)
    graphs, gammas = [g0], []
    for _ in range(spec.levels):
        g = graphs[-1]
        if (spec.target_nodes and g.n_nodes < spec.target_nodes) or g.n_nodes <= floor_nodes:
            break
        flags = ctx.new_flags(g) if PURGE and with_nb else None
        tgt, _, match, npairs = ctx.rate_and_match(g, spec.omega, spec.delta, True, spec.seed,
                                                   flags=flags)
        if LEFTOVERS:
            npairs += ctx.pair_leftovers(g, tgt, match, spec.omega, spec.delta)
        if npairs == 0:
            break
        gamma, cg = ctx.contract(g, match, with_nb, flags=flags)
        graphs.append(cg)
        gammas.append(gamma)
        if npairs < MIN_PAIR_FRAC * g.n_nodes:
            break
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    k = graphs[-1].n_nodes
    rho = torch.arange(k, dtype=torch.int32, device=ctx.device)
    _, _, s_init = ctx.evaluate_partition(graphs[-1], rho, k, spec.omega, spec.delta)
    applied = gain = 0
    level_ms = []
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for d in range(len(graphs) - 1, -1, -1):
        ta = time.perf_counter()
        na, ga = ctx.refine_level(graphs[d], rho, k, spec.omega, spec.delta, theta)
        applied += na
        gain += ga
        if d:
            rho = ctx.project_partition(gammas[d - 1], rho, graphs[d].n_nodes)
        torch.cuda.synchronize()
        level_ms.append(round((time.perf_counter() - ta) * 1e3, 3))
    t3 = time.perf_counter()
    _, _, s_fin = ctx.evaluate_partition(g0, rho, k, spec.omega, spec.delta)
    for g in graphs:
        g.free()
    return {"theta": theta, "levels": len(graphs) - 1, "parts": k,
            "coarsening_ms": (t1 - t0) * 1e3, "uncoarsening_ms": (t3 - t2) * 1e3,
            "uncoarsening_ms_per_level": level_ms, "moves_applied": applied, "gain": gain,
            "connectivity_initial": int(s_init[0]), "connectivity_final": int(s_fin[0]),
            "parts_over_omega": int(s_fin[2]), "parts_over_delta": int(s_fin[3])}


def rate_level_bytes(levels, h, spec):
    """Algorithmic bytes of the rating pass per level, each array read or
    written once: pins and incidence (4 B each per pin), neighbour lists
    (4 B per entry), per-hyperedge offsets, source counts and terms (20 B),
    per-node offsets, counts, sizes and outputs (40 B)."""
    return [8 * n_pins + 4 * nb_total + 20 * h.n_edges + 40 * n_nodes
            for n_nodes, n_pins, _, nb_total in levels]


if __name__ == "__main__":
    main()
