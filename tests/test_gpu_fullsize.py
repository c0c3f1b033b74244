"""Parity at the workloads' full sizes (needs a gfx950 GPU).

The device runs exactly what the benchmark runs (full-size level, same
launch configuration).  The CPU oracle, built from the same seeded arrays,
supplies what it can compute in seconds: everything for the 100,000-node
ring workload; sampled nodes (target, score, N(n)) plus the whole partition
evaluation for the 1M- and 2M-node workloads.  What the oracle cannot
produce per sample (the matching and the contraction of the whole graph) is
checked through properties that hold at any size.
"""
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


def check_match_properties(target, score, match, n_in, in_sets_of, sizes, omega, delta, rng,
                           n_check=2000):
    """The handshake's invariants: an involution; every pair is a proposal
    edge; two-cycles are matched; sampled pairs respect both limits."""
    N = target.shape[0]
    idx = np.arange(N, dtype=np.int64)
    assert np.array_equal(match[match.astype(np.int64)], idx.astype(np.uint32))
    paired = np.nonzero(match != idx)[0]
    m = match[paired].astype(np.int64)
    assert np.all((target[paired] == m) | (target[m] == paired))
    has = target != oracle.NONE
    t = target.astype(np.int64)
    roots = np.nonzero(has & (target[np.where(has, t, 0)] == idx))[0]
    assert np.array_equal(match[roots], target[roots])
    for a in rng.choice(paired, min(n_check, paired.size), replace=False):
        b = int(match[a])
        assert int(sizes[a]) + int(sizes[b]) <= omega
        assert len(in_sets_of(a) | in_sets_of(b)) <= delta


def check_coarse_properties(h, cg, gamma, match, sizes, omega, delta):
    """Contraction invariants on the device's coarse graph."""
    Nc = cg.n_nodes
    n_pairs = int(np.count_nonzero(match != np.arange(match.shape[0], dtype=np.uint32))) // 2
    assert Nc == h.n_nodes - n_pairs
    cs = cg.host("n_size").astype(np.int64)
    assert int(cs.sum()) == int(sizes.astype(np.int64).sum())
    assert int(cs.max()) <= omega
    assert int(cg.host("n_nin").max()) <= delta
    # gamma: ranks of the representatives (smallest member ids)
    rep = np.minimum(np.arange(match.shape[0], dtype=np.uint32), match)
    reps = np.nonzero(match >= np.arange(match.shape[0], dtype=np.uint32))[0]
    rank = np.empty(match.shape[0], np.int64)
    rank[reps] = np.arange(reps.size)
    assert np.array_equal(gamma.astype(np.int64), rank[rep])
    # coarse hyperedges: sorted distinct runs, src' and dst' disjoint, and
    # equal to gamma of the fine runs on a sample
    eo, ns, pins = cg.host("e_off"), cg.host("e_nsrc"), cg.host("e_pins")
    assert cg.n_edges == h.n_edges and cg.n_pins == int(eo[-1])
    rng = np.random.default_rng(1)
    for e in rng.choice(h.n_edges, 3000, replace=False):
        a, b, s = int(eo[e]), int(eo[e + 1]), int(ns[e])
        src, dst = pins[a:a + s], pins[a + s:b]
        fa, fb, fs = int(h.e_off[e]), int(h.e_off[e + 1]), int(h.e_nsrc[e])
        want_dst = np.unique(gamma[h.e_pins[fa + fs:fb]])
        want_src = np.setdiff1d(np.unique(gamma[h.e_pins[fa:fa + fs]]), want_dst)
        assert np.array_equal(dst, want_dst) and np.array_equal(src, want_src)
    # coarse incidence is the transpose of the coarse hyperedges
    E = cg.n_edges
    eid = np.repeat(np.arange(E, dtype=np.int64), np.diff(eo))
    pos = np.arange(cg.n_pins, dtype=np.int64) - np.repeat(eo[:-1], np.diff(eo))
    is_src = pos < np.repeat(ns.astype(np.int64), np.diff(eo))
    key = pins.astype(np.int64) * 2 + is_src
    order = np.lexsort((eid, key))
    no, nin, inc = cg.host("n_off"), cg.host("n_nin"), cg.host("n_inc")
    assert np.array_equal(inc, eid[order].astype(np.uint32))
    assert np.array_equal(np.diff(no), np.bincount(pins, minlength=Nc))
    assert np.array_equal(nin, np.bincount(pins[~is_src], minlength=Nc))


def sampled_rate_and_nb(chp, og, dg, tgt, score, spec, rng, n_sample):
    nodes = rng.choice(og.n_nodes, n_sample, replace=False)
    tc = oracle.terms(og)
    nbo, nb = dg.host("nb_off"), dg.host("nb")
    for n in nodes:
        n = int(n)
        t, s = oracle.rate(og, spec.omega, spec.delta, True, spec.seed, lo=n, hi=n + 1, tc=tc)
        assert int(tgt[n]) == int(t[n]) and int(score[n]) == int(s[n]), "node %d" % n
        # N(n) by definition from the oracle's incidence
        inc = og.n_inc[og.n_off[n]:og.n_off[n + 1]]
        want = set()
        for e in inc:
            want.update(og.e_pins[og.e_off[e]:og.e_off[e + 1]].tolist())
        want.discard(n)
        assert nb[nbo[n]:nbo[n + 1]].tolist() == sorted(want), "N(%d)" % n


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


@pytest.mark.parametrize("cfg,sample", [(3, 64), (4, 400)])
def test_large_workloads_sampled(chp, ctx, cfg, sample):
    """1M-node layered SNN and 2M-node VLSI netlist at full size."""
    spec = synth.config(cfg)
    say("full size", spec.name)
    h = synth.generate(spec)
    dg = ctx.build_incidence(*chp.upload_edges(h), spec.omega, spec.delta)
    og = oracle.build_incidence(h.e_off, h.e_nsrc, h.e_pins, h.e_w, h.n_size, spec.omega,
                                spec.delta, build_neighbors=False)
    for name in ("e_off", "e_nsrc", "e_pins", "n_off", "n_nin", "n_inc"):
        got, want = dg.host(name), getattr(og, name)
        assert np.array_equal(got.view(want.dtype), want), name
    tgt, score, match, npairs = ctx.rate_and_match(dg, spec.omega, spec.delta, True, spec.seed)
    tgt_h, score_h = chp.to_host(tgt, np.uint32), chp.to_host(score, np.uint64)
    match_h = chp.to_host(match, np.uint32)
    rng = np.random.default_rng(cfg)
    sampled_rate_and_nb(chp, og, dg, tgt_h, score_h, spec, rng, sample)

    def in_set(a):
        return set(og.n_inc[og.n_off[a]:og.n_off[a] + og.n_nin[a]].tolist())

    check_match_properties(tgt_h, score_h, match_h, og.n_nin, in_set, h.n_size, spec.omega,
                           spec.delta, rng)
    gamma, cg = ctx.contract(dg, match)
    gamma_h = chp.to_host(gamma, np.uint32)
    check_coarse_properties(h, cg, gamma_h, match_h, h.n_size, spec.omega, spec.delta)
    # the whole evaluation of a seeded partition against the oracle
    k = 1000
    rho = synth.uniform_u32(cfg, 11, h.n_nodes, k)
    eval_pair(chp, ctx, dg, og, rho, k, spec.omega, spec.delta, spec.name + " eval")


def test_block_4m_single_level(chp, ctx):
    """The 4M-node SNN workload (about 1e9 pins) at full size, as its
    description asks: one level of rate, match and contract.  Its
    neighbourhoods (about 1.9e11 entries) cannot be held at once, so the
    graph is built without them and the rating builds them batch by batch.
    Sampled nodes' target and score against the oracle; the matching and the
    coarse graph through the properties that hold at any size."""
    spec = synth.config(5)
    say("block 4m")
    h = synth.generate(spec)
    dg = ctx.build_incidence(*chp.upload_edges(h), spec.omega, spec.delta, False)
    say("block 4m built", dg.n_pins)
    tgt, score, match, npairs = ctx.rate_and_match(dg, spec.omega, spec.delta, True, spec.seed)
    say("block 4m rated", npairs)
    tgt_h, score_h = chp.to_host(tgt, np.uint32), chp.to_host(score, np.uint64)
    match_h = chp.to_host(match, np.uint32)
    og = oracle.build_incidence(h.e_off, h.e_nsrc, h.e_pins, h.e_w, h.n_size, spec.omega,
                                spec.delta, build_neighbors=False)
    say("block 4m oracle built")
    for name in ("e_off", "e_nsrc", "n_off", "n_nin"):
        got, want = dg.host(name), getattr(og, name)
        assert np.array_equal(got.view(want.dtype), want), name
    rng = np.random.default_rng(5)
    tc = oracle.terms(og)
    for n in rng.choice(h.n_nodes, 24, replace=False):
        n = int(n)
        t, s_ = oracle.rate(og, spec.omega, spec.delta, True, spec.seed, lo=n, hi=n + 1, tc=tc)
        assert int(tgt_h[n]) == int(t[n]) and int(score_h[n]) == int(s_[n]), "node %d" % n

    def in_set(a):
        return set(og.n_inc[og.n_off[a]:og.n_off[a] + og.n_nin[a]].tolist())

    check_match_properties(tgt_h, score_h, match_h, og.n_nin, in_set, h.n_size, spec.omega,
                           spec.delta, rng, n_check=200)
    gamma, cg = ctx.contract(dg, match, False)
    say("block 4m contracted", cg.n_nodes)
    gamma_h = chp.to_host(gamma, np.uint32)
    Nc = cg.n_nodes
    assert Nc == h.n_nodes - npairs
    cs = cg.host("n_size").astype(np.int64)
    assert int(cs.sum()) == int(h.n_size.astype(np.int64).sum()) and int(cs.max()) <= spec.omega
    assert int(cg.host("n_nin").max()) <= spec.delta
    rep = np.minimum(np.arange(h.n_nodes, dtype=np.uint32), match_h)
    reps = np.nonzero(match_h >= np.arange(h.n_nodes, dtype=np.uint32))[0]
    rank = np.empty(h.n_nodes, np.int64)
    rank[reps] = np.arange(reps.size)
    assert np.array_equal(gamma_h.astype(np.int64), rank[rep])
    eo, ns, pins = cg.host("e_off"), cg.host("e_nsrc"), cg.host("e_pins")
    for e in rng.choice(h.n_edges, 2000, replace=False):
        a, b, s0 = int(eo[e]), int(eo[e + 1]), int(ns[e])
        fa, fb, fs = int(h.e_off[e]), int(h.e_off[e + 1]), int(h.e_nsrc[e])
        want_dst = np.unique(gamma_h[h.e_pins[fa + fs:fb]])
        want_src = np.setdiff1d(np.unique(gamma_h[h.e_pins[fa:fa + fs]]), want_dst)
        assert np.array_equal(pins[a + s0:b], want_dst) and np.array_equal(pins[a:a + s0],
                                                                             want_src)
