"""Expected values for the full-size parity tests of the 1M-node layered
SNN graph (workload 3), the 2M-node VLSI netlist (workload 4) and the
4M-node block SNN graph (workload 5).

At these sizes the CPU oracle takes from minutes to hours (the block graph's
rating alone costs about 9 ms per node on one core), far beyond what a GPU
test may spend.  So this script runs the oracle once, on the CPU, on the
seeded inputs of ``synth/`` and through ``oracle/`` only, and stores SHA-256
digests of every array the level produces in ``fullsize_<name>.json``; the
GPU tests hash the device's arrays the same way and compare.  No value here
comes from the GPU library.

    python tests/golden/fullsize.py 3 4 5 [--threads T]

What runs (the levels as ``bench.py`` runs each workload; the rating's
node loop is split over T threads, which does not change its result):

  3  the first two coarsening levels (rate, handshake, leftover pairing,
     contract), graphs without neighbour lists (the purge only removes
     invalid neighbours, so targets, matches and coarse graphs do not depend
     on it), and the projected partition evaluated on the input graph after
     each level;
  4  the whole coarsening (until at most ceil(sum size / Omega) nodes, a level
     without pairs, or a level that pairs fewer than 0.1% of its nodes), with
     neighbour lists, the invalid-neighbour flags and the purge, and the
     projected partition evaluated on the input graph after every level;
  5  one level without neighbour lists, and the projected partition
     evaluated on the input graph.

Every level records: node and pin counts, pairs, target and score (digests
per block of CHUNK nodes, so that a mismatch names its block), match (after
the leftover pairing), gamma, every array of the coarse graph, the flags
where the purge runs, and the evaluation summary with digests of the
per-part sizes and inbound counts.
"""
from __future__ import annotations

import hashlib
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))

CHUNK = 1 << 18
MIN_PAIR_FRAC = 0.001  # the benchmark's stall rule
RUNS = {
    3: dict(levels=2, neighbours=False, purge=False),
    4: dict(levels=64, neighbours=True, purge=True),
    5: dict(levels=1, neighbours=False, purge=False),
}
DTYPES = {"target": np.uint32, "score": np.uint64, "match": np.uint32, "gamma": np.uint32,
          "flags": np.uint8, "e_off": np.int64, "e_nsrc": np.uint32, "e_pins": np.uint32,
          "n_size": np.uint32, "n_off": np.int64, "n_nin": np.uint32, "n_inc": np.uint32,
          "nb_off": np.int64, "nb": np.uint32, "part_size": np.uint64, "part_inb": np.uint32}
COARSE = ("e_off", "e_nsrc", "e_pins", "n_size", "n_off", "n_nin", "n_inc")


def sha(name, a):
    """SHA-256 of the array's bytes in the canonical dtype of `name`."""
    a = np.ascontiguousarray(np.asarray(a).astype(DTYPES[name], copy=False))
    return hashlib.sha256(a.tobytes()).hexdigest()


def sha_chunks(name, a):
    return [sha(name, a[i:i + CHUNK]) for i in range(0, max(len(a), 1), CHUNK)]


def path_of(name):
    return os.path.join(HERE, "fullsize_%s.json" % name)


def load(name):
    with open(path_of(name)) as f:
        return json.load(f)


def _file_sha(p):
    with open(p, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def make(workload, threads):
    sys.path.insert(0, ROOT)
    import oracle
    import synth
    spec = synth.config(workload)
    run = RUNS[workload]
    t0 = time.time()
    h = synth.generate(spec)
    g0 = oracle.build_incidence(h.e_off, h.e_nsrc, h.e_pins, h.e_w, h.n_size, spec.omega,
                                spec.delta, run["neighbours"])
    print("[golden] %s: %d pins, built in %.0f s" % (spec.name, h.n_pins, time.time() - t0),
          flush=True)
    out = {"workload": workload, "name": spec.name, "nodes": h.n_nodes, "edges": h.n_edges,
           "pins": h.n_pins, "omega": spec.omega, "delta": spec.delta, "seed": spec.seed,
           "chunk": CHUNK, "run": run, "min_pair_frac": MIN_PAIR_FRAC,
           "command": "python tests/golden/fullsize.py %d" % workload,
           "oracle_source_sha256": _file_sha(os.path.join(ROOT, "oracle", "chp_oracle.c")),
           "synth_source_sha256": _file_sha(os.path.join(ROOT, "synth", "synth.c")),
           "levels": []}

    def on_level(i, g, lv, rho):
        rec = {"level": i, "n_nodes": g.n_nodes, "n_pins": g.n_pins, "n_pairs": lv.n_pairs,
               "target": sha_chunks("target", lv.target), "score": sha_chunks("score", lv.score),
               "match": sha("match", lv.match)}
        if lv.flags is not None:
            rec["flags"] = sha("flags", lv.flags)
        if lv.n_pairs:
            rec["gamma"] = sha("gamma", lv.gamma)
            names = COARSE + (("nb_off", "nb") if run["neighbours"] else ())
            rec["coarse"] = {"n_nodes": lv.coarse.n_nodes, "n_pins": lv.coarse.n_pins}
            for n in names:
                rec["coarse"][n] = sha(n, getattr(lv.coarse, n))
            k = lv.coarse.n_nodes
            ps, pi, summ = oracle.evaluate(g0, rho, k, spec.omega, spec.delta)
            rec["eval"] = {"k": k, "summary": [int(x) for x in summ],
                           "part_size": sha("part_size", ps), "part_inb": sha("part_inb", pi)}
        out["levels"].append(rec)
        print("[golden] level %d: %d nodes, %d pairs (%.0f s)"
              % (i, g.n_nodes, lv.n_pairs, time.time() - t0), flush=True)

    floor_target = spec.target_nodes
    oracle.coarsen(g0, spec.omega, spec.delta, floor_target, run["levels"], True, spec.seed,
                   purge_invalid=run["purge"], leftovers=True, min_pair_frac=MIN_PAIR_FRAC,
                   on_level=on_level, threads=threads, build_neighbors=run["neighbours"])
    out["oracle_seconds"] = round(time.time() - t0, 1)
    out["threads"] = threads
    with open(path_of(spec.name), "w") as f:
        json.dump(out, f, indent=1)
    print("[golden] wrote", path_of(spec.name), flush=True)


if __name__ == "__main__":
    args = sys.argv[1:]
    threads = 1
    if "--threads" in args:
        i = args.index("--threads")
        threads = int(args[i + 1])
        del args[i:i + 2]
    for w in args:
        make(int(w), threads)
