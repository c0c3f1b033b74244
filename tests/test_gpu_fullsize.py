"""Parity at the workloads' full sizes (needs a gfx950 GPU).

The device runs each workload as the benchmark runs it (full size, same
launch configuration: neighbour lists where they fit, the purge, the
leftover pairing, the projected partition evaluated on the input graph).

* The 100,000-node ring: the CPU oracle runs inline; levels 0 and 1 are
  compared array by array, flags included.
* The 1M-node layered graph (first two levels), the 2M-node VLSI netlist
  (its whole coarsening, evaluated after every level) and the 4M-node block
  graph (its one level): the oracle's outputs at these sizes take from
  minutes to hours of CPU time, so they are stored as SHA-256 digests in
  tests/golden/fullsize_<workload>.json, written by tests/golden/fullsize.py
  from the oracle alone.  Every array of every level is compared whole
  through its digest (target and score per block of 2^18 nodes).
"""
import os
import sys

import numpy as np
import pytest

import oracle
import synth
from gpu_common import assert_equal, assert_graph_equal, eval_pair

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def chp():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import constrained_hypergraph_partitioning_amd as m
    m.load_library()
    return m


@pytest.fixture(scope="module")
def ctx(chp):
    return chp.Context(0)


def say(*a):
    print("[case]", *a, flush=True)


def test_ring_100k_full_level(chp, ctx):
    """The benchmark's workload at full size, as the benchmark runs it (with
    the purge): level 0 and level 1 compared array by array with the oracle
    (flags included), then the projected partition."""
    spec = synth.config(2)
    say("ring 100k full")
    h = synth.generate(spec)
    dg = ctx.build_incidence(*chp.upload_edges(h), spec.omega, spec.delta)
    og = oracle.build_incidence(h.e_off, h.e_nsrc, h.e_pins, h.e_w, h.n_size, spec.omega,
                                spec.delta)
    assert_graph_equal(dg, og, "level 0")
    rho = np.arange(h.n_nodes, dtype=np.uint32)
    g0d, g0o = dg, og
    for lvl in range(2):
        # as the benchmark runs it: invalid neighbours flagged and purged
        flags = ctx.new_flags(dg)
        tgt, score, match, npairs = ctx.rate_and_match(dg, spec.omega, spec.delta, True,
                                                       spec.seed, flags=flags)
        lv = oracle.level(og, spec.omega, spec.delta, True, spec.seed, purge_invalid=True)
        assert_equal(chp.to_host(tgt, np.uint32), lv.target, "L%d target" % lvl)
        assert_equal(chp.to_host(score, np.uint64), lv.score, "L%d score" % lvl)
        assert_equal(chp.to_host(match, np.uint32), lv.match, "L%d match" % lvl)
        assert_equal(flags.cpu().numpy()[: og.nb.shape[0]], lv.flags, "L%d flags" % lvl)
        assert npairs == lv.n_pairs
        gamma, cg = ctx.contract(dg, match, flags=flags)
        assert_equal(chp.to_host(gamma, np.uint32), lv.gamma, "L%d gamma" % lvl)
        assert_graph_equal(cg, lv.coarse, "L%d coarse" % lvl)
        rho = lv.gamma[rho]
        dg, og = cg, lv.coarse
    eval_pair(chp, ctx, g0d, g0o, rho, og.n_nodes, spec.omega, spec.delta, "projected")


def test_ring_100k_top4_level(chp, ctx):
    """The ring at full size as `bench.py --pi 4` runs its first level: the
    top-4 lists of every node, the four matching rounds (with the purge
    flags and the leftover pairing) and the coarse graph, array by array."""
    spec = synth.config(2)
    say("ring 100k top-4")
    h = synth.generate(spec)
    dg = ctx.build_incidence(*chp.upload_edges(h), spec.omega, spec.delta)
    og = oracle.build_incidence(h.e_off, h.e_nsrc, h.e_pins, h.e_w, h.n_size, spec.omega,
                                spec.delta)
    flags = ctx.new_flags(dg)
    tl, sl, match, npairs = ctx.rate_top_and_match(dg, 4, spec.omega, spec.delta, True,
                                                   spec.seed, flags=flags)
    npairs += ctx.pair_leftovers(dg, tl[0], match, spec.omega, spec.delta)
    otl, osl = oracle.rate_top(og, spec.omega, spec.delta, True, spec.seed, 4)
    assert_equal(chp.to_host(tl, np.uint32).reshape(-1), otl.reshape(-1), "top-4 targets")
    assert_equal(chp.to_host(sl, np.uint64).reshape(-1), osl.reshape(-1), "top-4 scores")
    lv = oracle.level(og, spec.omega, spec.delta, True, spec.seed, purge_invalid=True,
                      leftovers=True, pi=4)
    assert_equal(chp.to_host(match, np.uint32), lv.match, "top-4 match")
    assert_equal(flags.cpu().numpy()[: og.nb.shape[0]], lv.flags, "top-4 flags")
    assert npairs == lv.n_pairs
    gamma, cg = ctx.contract(dg, match, flags=flags)
    assert_equal(chp.to_host(gamma, np.uint32), lv.gamma, "top-4 gamma")
    assert_graph_equal(cg, lv.coarse, "top-4 coarse")


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
sys.path.insert(0, GOLDEN)
import fullsize  # noqa: E402  (digest helpers and the stored records)

NB_BYTES_MAX = 64 << 30  # the benchmark's limit for whole-graph neighbour lists


def check_digests(rec, got, tag):
    """Compare one level's device outputs (host numpy arrays in `got`) with
    the oracle's stored digests."""
    assert got["n_nodes"] == rec["n_nodes"] and got["n_pins"] == rec["n_pins"], tag
    assert got["n_pairs"] == rec["n_pairs"], "%s pairs %d, oracle %d" % (
        tag, got["n_pairs"], rec["n_pairs"])
    for name in ("target", "score"):
        d = fullsize.sha_chunks(name, got[name])
        bad = [i for i, (a, b) in enumerate(zip(d, rec[name])) if a != b]
        assert len(d) == len(rec[name]) and not bad, "%s %s differs in node blocks %s (of %d)" % (
            tag, name, bad[:8], fullsize.CHUNK)
    assert fullsize.sha("match", got["match"]) == rec["match"], tag + " match"
    if "flags" in rec:
        assert fullsize.sha("flags", got["flags"]) == rec["flags"], tag + " flags"
    if not rec["n_pairs"]:
        return
    assert fullsize.sha("gamma", got["gamma"]) == rec["gamma"], tag + " gamma"
    c = rec["coarse"]
    assert got["coarse_n_nodes"] == c["n_nodes"] and got["coarse_n_pins"] == c["n_pins"], tag
    for name in fullsize.COARSE + ("nb_off", "nb"):
        if name in c:
            assert fullsize.sha(name, got["coarse"][name]) == c[name], "%s coarse %s" % (tag, name)
    ev = rec["eval"]
    assert got["k"] == ev["k"], tag
    assert [int(x) for x in got["summary"]] == ev["summary"], tag + " evaluation summary"
    assert fullsize.sha("part_size", got["part_size"]) == ev["part_size"], tag + " part sizes"
    assert fullsize.sha("part_inb", got["part_inb"]) == ev["part_inb"], tag + " part inbound"


@pytest.mark.parametrize("cfg", [3, 4, 5])
def test_fullsize_vs_stored_oracle(chp, ctx, cfg):
    """Workloads 3 (two levels), 4 (the whole coarsening) and 5 (one level)
    at full size, as the benchmark runs them, against the oracle's digests."""
    import torch
    spec = synth.config(cfg)
    path = fullsize.path_of(spec.name)
    if not os.path.exists(path):
        pytest.fail("no stored oracle record %s (python tests/golden/fullsize.py %d)"
                    % (path, cfg))
    gold = fullsize.load(spec.name)
    say("full size", spec.name)
    h = synth.generate(spec)
    assert h.n_pins == gold["pins"] and h.n_nodes == gold["nodes"]
    sz = np.diff(h.e_off).astype(np.float64)
    with_nb = float((sz * (sz - 1)).sum()) * 4 <= NB_BYTES_MAX
    g0 = ctx.build_incidence(*chp.upload_edges(h), spec.omega, spec.delta, with_nb)
    del sz
    say(spec.name, "built, lists" if with_nb else "built, no lists")
    floor_nodes = -(-int(h.n_size.astype(np.int64).sum()) // spec.omega)
    g = g0
    rho = None
    for i, rec in enumerate(gold["levels"]):
        assert not (spec.target_nodes and g.n_nodes < spec.target_nodes)
        assert g.n_nodes > floor_nodes
        flags = ctx.new_flags(g) if with_nb else None
        tgt, score, match, npairs = ctx.rate_and_match(g, spec.omega, spec.delta, True,
                                                       spec.seed, flags=flags)
        npairs += ctx.pair_leftovers(g, tgt, match, spec.omega, spec.delta)
        got = {"n_nodes": g.n_nodes, "n_pins": g.n_pins, "n_pairs": npairs,
               "target": chp.to_host(tgt, np.uint32), "score": chp.to_host(score, np.uint64),
               "match": chp.to_host(match, np.uint32)}
        if "flags" in rec:
            got["flags"] = flags.cpu().numpy()[: g.nb_total]
        if npairs:
            gamma, cg = ctx.contract(g, match, with_nb, flags=flags)
            rho = gamma.long() if rho is None else gamma.long()[rho]
            k = cg.n_nodes
            ps, pi, summ = ctx.evaluate_partition(g0, rho.to(torch.int32).contiguous(), k,
                                                  spec.omega, spec.delta)
            got.update(gamma=chp.to_host(gamma, np.uint32), coarse_n_nodes=cg.n_nodes,
                       coarse_n_pins=cg.n_pins, k=k, summary=summ,
                       part_size=chp.to_host(ps, np.uint64), part_inb=chp.to_host(pi, np.uint32),
                       coarse={n: cg.host(n) for n in fullsize.COARSE +
                               (("nb_off", "nb") if "nb" in rec["coarse"] else ())})
        say(spec.name, "level", i, "nodes", g.n_nodes, "pairs", npairs)
        check_digests(rec, got, "%s level %d" % (spec.name, i))
        del got
        if flags is not None:
            del flags
        if not npairs:
            break
        if g is not g0:
            g.free()
        g = cg
    if g is not g0:
        g.free()
    g0.free()
    torch.cuda.empty_cache()
