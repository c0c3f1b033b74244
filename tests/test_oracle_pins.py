"""Pins of the CPU oracle against things other than itself.

* a hand-worked six-node example, every value derived on paper from the
  definitions (Eqs. 1, 2, 5, 6 of Ronzani & Silvano's TPDS paper and the
  handshake of their prototype paper, Sec. III-B3);
* the published splitmix64 output sequence (noise generator);
* brute force in pure Python (``tests/brute.py``: sets, exact rationals, full
  sorts, a literal sequential simulation of the handshake) on many tiny
  random hypergraphs;
* closed forms and invariants (symmetry, proposal-graph structure, Eq. 1 /
  Eq. 2 duality, projection invariance across levels).
"""
from fractions import Fraction

import numpy as np
import pytest

import brute
import oracle
import synth

NONE = oracle.NONE
BIG = 1 << 30


def load(h, omega=BIG, delta=BIG, neighbors=True):
    return oracle.build_incidence(h.e_off, h.e_nsrc, h.e_pins, h.e_w, h.n_size, omega, delta,
                                  neighbors)


# ---------------------------------------------------------------- hand-worked
# Six unit-size nodes, five h-edges (src | dst, weight):
#   e0: 0 | 1 2   w3     e1: 1 | 2 3   w2     e2: 3 | 4   w4
#   e3: 4 | 5 0   w1     e4: 2 | 1     w1
# Eq. 5 terms w/|e|: e0 1, e1 2/3, e2 2, e3 1/3, e4 1/2.
HAND_EDGES = [([0], [1, 2]), ([1], [2, 3]), ([3], [4]), ([4], [5, 0]), ([2], [1])]
HAND_W = [3, 2, 4, 1, 1]


def hand():
    return synth.from_lists(6, HAND_EDGES, HAND_W)


def test_hand_incidence_and_neighbors():
    g = load(hand())
    # in(n) = {e : n in dst(e)}, out(n) = {e : n in src(e)}; in-edges first
    want_in = [[3], [0, 4], [0, 1], [1], [2], [3]]
    want_out = [[0], [1], [4], [2], [3], []]
    for n in range(6):
        seg = g.n_inc[g.n_off[n]:g.n_off[n + 1]].tolist()
        k = int(g.n_nin[n])
        assert seg[:k] == want_in[n] and seg[k:] == want_out[n]
    want_nb = [[1, 2, 4, 5], [0, 2, 3], [0, 1, 3], [1, 2, 4], [0, 3, 5], [0, 4]]
    for n in range(6):
        assert g.nb[g.nb_off[n]:g.nb_off[n + 1]].tolist() == want_nb[n]
    # the src sub-list of e3 is {4}, dst sorted {0, 5}
    assert g.e_pins[g.e_off[3]:g.e_off[4]].tolist() == [4, 0, 5]


def fx(fr):
    return fr * (1 << 40)


def test_hand_rate_unconstrained():
    g = load(hand())
    t, cap = oracle.terms(g)
    assert t.tolist() == [(3 << 40) // 3, (2 << 40) // 3, (4 << 40) // 2, (1 << 40) // 3,
                          (1 << 40) // 2]
    target, score = oracle.rate(g, BIG, BIG, noise_on=False)
    # n0: eta(0,1) = eta(0,2) = 1 -> lowest id 1.  n1 <-> n2 at 1 + 1/2 + 2/3.
    # n3 <-> n4 at 2.  n5: eta(5,0) = eta(5,4) = 1/3 -> 0.
    assert target.tolist() == [1, 2, 1, 4, 3, 0]
    assert int(score[1]) == int(t[0] + t[4] + t[1]) == int(score[2])
    assert abs(Fraction(int(score[1]), 1 << 40) - Fraction(13, 6)) <= Fraction(3, 1 << 40)
    m, npairs = oracle.match(target, score)
    # roots {1,2}, {3,4}; 0 proposes to root 1 (never taken), 5 is 0's only
    # proposer and 0 is free, so 5 takes 0.
    assert m.tolist() == [5, 2, 1, 4, 3, 0] and npairs == 3


def test_hand_rate_delta_two():
    g = load(hand(), delta=2)
    target, score = oracle.rate(g, BIG, 2, noise_on=False)
    # |in(1) u in(2)| = |{e0,e4,e1}| = 3 > 2, |in(1) u in(0)| = 3, |in(1) u in(3)| = 3:
    # node 1 has no valid neighbour.  n2 -> 3 (|{e0,e1}| = 2).  n0: 1 and 2 invalid,
    # 4 and 5 tie at 1/3 -> 4.  n5 -> 0 (|{e3}| = 1).
    assert target.tolist() == [4, NONE, 3, 4, 3, 0]
    assert int(score[1]) == 0
    m, npairs = oracle.match(target, score)
    assert m.tolist() == [5, 1, 2, 4, 3, 0] and npairs == 2


def test_hand_contract_and_evaluate():
    g = load(hand())
    match = np.array([5, 2, 1, 4, 3, 0], np.uint32)
    gamma, cg = oracle.contract(g, match)
    assert gamma.tolist() == [0, 1, 1, 2, 2, 0]
    assert cg.n_size.tolist() == [2, 2, 2]
    lists = [cg.e_pins[cg.e_off[e]:cg.e_off[e + 1]].tolist() for e in range(5)]
    nsrc = cg.e_nsrc.tolist()
    # e0 {0}|{1}; e1 {}|{1,2} (src 1 is also a dst); e2 {}|{2}; e3 {2}|{0}; e4 {}|{1}
    assert lists == [[0, 1], [1, 2], [2], [2, 0], [1]]
    assert nsrc == [1, 0, 0, 1, 0]
    # Eq. 2: Score = sum w (|e| - |e'|) = 3 + 2 + 4 + 1 + 1 = 11;
    # Eq. 1 on gamma: 17 - 11 = 6; inbound per part: {e3}, {e0,e1,e4}, {e1,e2}
    ps, pi, summ = oracle.evaluate(g, gamma, 3, BIG, BIG)
    assert int(summ[0]) == 6 and int(summ[1]) == 6
    assert ps.tolist() == [2, 2, 2] and pi.tolist() == [1, 3, 2]
    ps2, pi2, summ2 = oracle.evaluate(cg, np.arange(3, dtype=np.uint32), 3, BIG, BIG)
    assert ps2.tolist() == ps.tolist() and pi2.tolist() == pi.tolist()
    assert int(summ2[0]) == 6


# ---------------------------------------------------------------- noise source
def test_splitmix64_published_sequence():
    # Vigna's splitmix64 from state 0: the first three outputs
    want = [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    gam = 0x9E3779B97F4A7C15
    for k, w in enumerate(want):
        state = (k * gam) & ((1 << 64) - 1)
        assert brute.splitmix64_once(state) == w
    # the oracle's noise is that output of state seed ^ (min << 32 | max), mod cap+1
    cap = (1 << 64) - 2
    assert oracle.noise(0, cap, 0, 0) == want[0] % (cap + 1)
    for seed, a, b in [(0, 1, 2), (7, 5, 3), (123456789, 10, 99999), (2 ** 63, 0, 4000000)]:
        for c in [0, 1, 17, 2 ** 34 + 5]:
            assert oracle.noise(seed, c, a, b) == brute.noise_fx(seed, c, a, b)
            assert oracle.noise(seed, c, a, b) == oracle.noise(seed, c, b, a)


# ---------------------------------------------------------------- brute force
def tiny_cases():
    cases = []
    for seed in range(60):
        n = 3 + seed % 17
        e = 1 + (seed * 7) % 23
        cases.append(dict(seed=seed, n_nodes=n, n_edges=e, max_src=seed % 3,
                          max_dst=1 + seed % 6, max_w=1 + seed % 9, max_size=1 + seed % 3))
    return cases


@pytest.mark.parametrize("kw", tiny_cases(), ids=lambda k: "s%d" % k["seed"])
def test_structures_vs_brute(kw):
    h = synth.tiny(**kw)
    g = load(h)
    edges = brute.edges_of(h.e_off, h.e_nsrc, h.e_pins)
    ins, outs = brute.incidence_sets(h.n_nodes, edges)
    nbs = brute.neighbor_sets(h.n_nodes, edges)
    for n in range(h.n_nodes):
        seg = g.n_inc[g.n_off[n]:g.n_off[n + 1]].tolist()
        k = int(g.n_nin[n])
        assert seg[:k] == sorted(ins[n]) and seg[k:] == sorted(outs[n])
        nb = g.nb[g.nb_off[n]:g.nb_off[n + 1]].tolist()
        assert nb == sorted(nbs[n])
        # |N(n)| <= sum over incident edges of (|e| - 1)
        assert len(nb) <= sum(len(edges[e][0] | edges[e][1]) - 1 for e in ins[n] | outs[n])
    for e in range(h.n_edges):
        a, b, s = int(g.e_off[e]), int(g.e_off[e + 1]), int(g.e_nsrc[e])
        assert g.e_pins[a:a + s].tolist() == sorted(edges[e][0])
        assert g.e_pins[a + s:b].tolist() == sorted(edges[e][1])


def constraint_grid(h):
    tot_in = max(1, int(np.bincount(h.e_pins[np.concatenate(
        [np.arange(h.e_off[e] + h.e_nsrc[e], h.e_off[e + 1]) for e in range(h.n_edges)])
        .astype(np.int64)], minlength=h.n_nodes).max()) if h.n_pins else 1)
    smax = int(h.n_size.max())
    return [(BIG, BIG), (2 * smax, BIG), (BIG, tot_in + 1), (smax + 1, tot_in)]


@pytest.mark.parametrize("kw", tiny_cases()[::2], ids=lambda k: "s%d" % k["seed"])
@pytest.mark.parametrize("noise_on", [False, True])
def test_rate_match_vs_brute(kw, noise_on):
    h = synth.tiny(**kw)
    edges = brute.edges_of(h.e_off, h.e_nsrc, h.e_pins)
    for omega, delta in constraint_grid(h):
        g = load(h, omega, delta)
        target, score = oracle.rate(g, omega, delta, noise_on=noise_on, seed=kw["seed"])
        bt, bs = brute.rate(h.n_nodes, edges, h.e_w, h.n_size, omega, delta, noise_on,
                            kw["seed"])
        assert target.tolist() == bt
        assert [int(x) for x in score] == bs
        m, npairs = oracle.match(target, score)
        assert m.tolist() == brute.handshake(bt, bs)
        assert npairs == sum(1 for n in range(h.n_nodes) if m[n] != n) // 2


@pytest.mark.parametrize("kw", tiny_cases()[1::3], ids=lambda k: "s%d" % k["seed"])
def test_fixed_point_vs_exact_eta(kw):
    """|eta_fx * 2^-40 - eta| <= (#shared edges) * 2^-40, and eta_fx symmetric."""
    h = synth.tiny(**kw)
    edges = brute.edges_of(h.e_off, h.e_nsrc, h.e_pins)
    exact = brute.eta_exact(h.n_nodes, edges, h.e_w)
    efx = brute.eta_fx(h.n_nodes, edges, h.e_w)
    for (n, m), v in exact.items():
        shared = sum(1 for (s, d) in edges if n in (s | d) and m in (s | d))
        assert abs(Fraction(efx[(n, m)], 1 << 40) - v) <= Fraction(shared, 1 << 40)
        assert efx[(n, m)] == efx[(m, n)]
        if v:
            assert abs(float(Fraction(efx[(n, m)], 1 << 40) / v) - 1.0) < 1e-6
    # the oracle's best score equals the brute-force fixed-point maximum
    g = load(h)
    target, score = oracle.rate(g, BIG, BIG, noise_on=False)
    for n in range(h.n_nodes):
        cands = [efx[(n, m)] for m in range(h.n_nodes) if (n, m) in efx]
        assert int(score[n]) == (max(cands) if cands else 0)


@pytest.mark.parametrize("kw", tiny_cases()[::3], ids=lambda k: "s%d" % k["seed"])
def test_contract_evaluate_vs_brute(kw):
    h = synth.tiny(**kw)
    edges = brute.edges_of(h.e_off, h.e_nsrc, h.e_pins)
    g = load(h)
    target, score = oracle.rate(g, BIG, BIG, noise_on=True, seed=3)
    m, _ = oracle.match(target, score)
    gamma, cg = oracle.contract(g, m)
    bg, bsize, bedges, bw = brute.contract(h.n_nodes, edges, h.e_w, h.n_size, m)
    assert gamma.tolist() == bg
    assert cg.n_size.tolist() == bsize
    for e, (s, d) in enumerate(bedges):
        a, b, ns = int(cg.e_off[e]), int(cg.e_off[e + 1]), int(cg.e_nsrc[e])
        assert cg.e_pins[a:a + ns].tolist() == sorted(s)
        assert cg.e_pins[a + ns:b].tolist() == sorted(d)
    # rebuilt incidence / neighbours of G' equal the definitions on G'
    ins, outs = brute.incidence_sets(cg.n_nodes, bedges)
    nbs = brute.neighbor_sets(cg.n_nodes, bedges)
    for c in range(cg.n_nodes):
        seg = cg.n_inc[cg.n_off[c]:cg.n_off[c + 1]].tolist()
        k = int(cg.n_nin[c])
        assert seg[:k] == sorted(ins[c]) and seg[k:] == sorted(outs[c])
        assert cg.nb[cg.nb_off[c]:cg.nb_off[c + 1]].tolist() == sorted(nbs[c])
    for k in [1, 2, 5, h.n_nodes]:
        rho = synth.uniform_u32(kw["seed"], 99, h.n_nodes, k)
        ps, pi, summ = oracle.evaluate(g, rho, k, BIG, BIG)
        conn, cut, bps, bpi, empty = brute.evaluate(h.n_nodes, edges, h.e_w, h.n_size, rho, k)
        assert (int(summ[0]), int(summ[1]), int(summ[4])) == (conn, cut, empty)
        assert ps.tolist() == bps and pi.tolist() == bpi


# ---------------------------------------------------------------- closed forms
@pytest.mark.parametrize("cfg", [1, 2])
def test_evaluate_closed_forms(cfg):
    h = synth.generate(synth.config(cfg, n_nodes=3000))
    g = load(h, neighbors=False)
    sizes = np.diff(g.e_off).astype(np.uint64)
    w = g.e_w.astype(np.uint64)
    n_dst = sizes - g.e_nsrc
    # k = 1: no cut; every edge with a destination is inbound to the only part
    ps, pi, summ = oracle.evaluate(g, np.zeros(g.n_nodes, np.uint32), 1, BIG, BIG)
    assert int(summ[0]) == 0 and int(summ[1]) == 0
    assert int(pi[0]) == int((n_dst > 0).sum()) and int(ps[0]) == int(g.n_size.sum())
    # identity partition: conn = sum w(|e|-1), inbound({n}) = |in(n)|
    ident = np.arange(g.n_nodes, dtype=np.uint32)
    ps, pi, summ = oracle.evaluate(g, ident, g.n_nodes, BIG, BIG)
    assert int(summ[0]) == int((w * (sizes - 1)).sum())
    assert int(summ[1]) == int(w[sizes > 1].sum())
    assert pi.tolist() == g.n_nin.tolist()
    assert int(summ[7]) == int(sizes.sum())


def proposal_invariants(target, score):
    N = target.shape[0]
    for n in range(N):
        t = int(target[n])
        if t == NONE:
            assert score[n] == 0
            continue
        # Sec. V-A: target(m) = n  =>  score(n) >= score(m)
        assert score[t] >= score[n]
        # only two-cycles
        tt = int(target[t])
        if tt != NONE and tt != n:
            assert int(target[tt]) != n


def match_invariants(target, score, m, g, omega, delta):
    N = target.shape[0]
    ins = [set(g.n_inc[g.n_off[n]:g.n_off[n] + g.n_nin[n]].tolist()) for n in range(N)]
    for n in range(N):
        p = int(m[n])
        assert int(m[p]) == n
        if p != n:
            # every pair is a proposal edge and a valid cluster
            assert int(target[n]) == p or int(target[p]) == n
            assert int(g.n_size[n]) + int(g.n_size[p]) <= omega
            assert len(ins[n] | ins[p]) <= delta
        t = int(target[n])
        if t != NONE:
            if int(target[t]) == n:
                assert p == t  # roots always match
            # every proposal edge has a matched endpoint
            assert p != n or int(m[t]) != t


@pytest.mark.parametrize("cfg,nn", [(1, None), (2, 20000), (3, 20000), (4, 20000), (5, 8192)])
def test_level_invariants_and_duality(cfg, nn):
    spec = synth.config(cfg, n_nodes=nn)
    h = synth.generate(spec)
    g = load(h, spec.omega, spec.delta)
    lv = oracle.level(g, spec.omega, spec.delta, noise_on=True, seed=spec.seed)
    proposal_invariants(lv.target, lv.score)
    match_invariants(lv.target, lv.score, lv.match, g, spec.omega, spec.delta)
    assert lv.n_pairs > 0
    cg = lv.coarse
    # sizes add up, limits hold, no duplicate pins, src' and dst' disjoint
    assert int(cg.n_size.astype(np.uint64).sum()) == int(h.n_size.astype(np.uint64).sum())
    assert int(cg.n_size.max()) <= spec.omega and int(cg.n_nin.max()) <= spec.delta
    assert cg.n_nodes == g.n_nodes - lv.n_pairs
    for e in range(0, cg.n_edges, max(1, cg.n_edges // 2000)):
        a, b, s = int(cg.e_off[e]), int(cg.e_off[e + 1]), int(cg.e_nsrc[e])
        src, dst = cg.e_pins[a:a + s], cg.e_pins[a + s:b]
        assert np.all(np.diff(src.astype(np.int64)) > 0) and np.all(np.diff(dst.astype(np.int64)) > 0)
        assert not set(src.tolist()) & set(dst.tolist())
    # Eq. 2 duality: Score(gamma) = sum w (|e| - |e'|) and
    # Conn_G(gamma) = Conn_G'(identity) = sum w (|e| - 1) - Score(gamma)
    w = g.e_w.astype(np.int64)
    sz = np.diff(g.e_off)
    csz = np.diff(cg.e_off)
    score_g = int((w * (sz - csz)).sum())
    _, _, s0 = oracle.evaluate(g, lv.gamma, cg.n_nodes, spec.omega, spec.delta)
    _, _, s1 = oracle.evaluate(cg, np.arange(cg.n_nodes, dtype=np.uint32), cg.n_nodes,
                               spec.omega, spec.delta)
    assert int(s0[0]) == int(s1[0]) == int((w * (sz - 1)).sum()) - score_g
    assert int(s0[2]) == 0 and int(s0[3]) == 0  # the clusters respect Omega and Delta


def test_multilevel_projection_invariance():
    """Coarsen a VLSI-style graph several levels; at every level the projected
    partition on G0 evaluates exactly like the identity on G_l."""
    spec = synth.config(4, n_nodes=6000)
    h = synth.generate(spec)
    g0 = load(h, spec.omega, spec.delta)
    cur = g0
    rho = np.arange(g0.n_nodes, dtype=np.uint32)
    for lvl in range(6):
        lv = oracle.level(cur, spec.omega, spec.delta, noise_on=True, seed=spec.seed)
        if lv.n_pairs == 0:
            break
        rho = lv.gamma[rho]
        cur = lv.coarse
        k = cur.n_nodes
        p0, i0, s0 = oracle.evaluate(g0, rho, k, spec.omega, spec.delta)
        p1, i1, s1 = oracle.evaluate(cur, np.arange(k, dtype=np.uint32), k, spec.omega,
                                     spec.delta)
        assert np.array_equal(p0, p1) and np.array_equal(i0, i1)
        assert np.array_equal(s0, s1)
        assert int(s0[2]) == 0 and int(s0[3]) == 0 and int(s0[4]) == 0
    assert lvl >= 3


def test_determinism():
    spec = synth.config(2, n_nodes=5000)
    h = synth.generate(spec)
    a = oracle.level(load(h, spec.omega, spec.delta), spec.omega, spec.delta)
    b = oracle.level(load(h, spec.omega, spec.delta), spec.omega, spec.delta)
    assert np.array_equal(a.target, b.target) and np.array_equal(a.score, b.score)
    assert np.array_equal(a.match, b.match) and np.array_equal(a.coarse.e_pins, b.coarse.e_pins)


@pytest.mark.parametrize("threads", [2, 3, 8])
def test_threaded_rating_is_the_single_threaded_one(threads):
    """The rating's node loop split over threads (each node is rated on its
    own accumulators) gives bit-identical top-pi lists for any thread count:
    on a scaled ring, a scaled block graph, every tiny graph, and node
    ranges; an overflowing node fails the same way."""
    for cfg, nn in ((2, 20000), (5, 4096)):
        spec = synth.config(cfg, n_nodes=nn)
        g = load(synth.generate(spec), spec.omega, spec.delta, neighbors=False)
        for pi in (1, 4):
            a = oracle.rate_top(g, spec.omega, spec.delta, True, spec.seed, pi)
            b = oracle.rate_top(g, spec.omega, spec.delta, True, spec.seed, pi, threads=threads)
            assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
        lo, hi = 1234, 3456
        a = oracle.rate(g, spec.omega, spec.delta, True, spec.seed, lo=lo, hi=hi)
        b = oracle.rate(g, spec.omega, spec.delta, True, spec.seed, lo=lo, hi=hi, threads=threads)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
        assert np.all(b[0][:lo] == NONE) and np.all(b[0][hi:] == NONE)
    for kw in tiny_cases()[::4]:
        g = load(synth.tiny(**kw), neighbors=False)
        a = oracle.rate_top(g, BIG, BIG, True, 3, 4)
        b = oracle.rate_top(g, BIG, BIG, True, 3, 4, threads=threads)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    # node 5 sits in two 2-pin hyperedges of weight 2^24 - 1: its terms sum
    # past 2^63
    edges = [([i], [i + 1]) for i in range(4)] + [([5], [6]), ([7], [5])]
    g = load(synth.from_lists(9, edges, [1, 1, 1, 1, (1 << 24) - 1, (1 << 24) - 1]),
             neighbors=False)
    for th in (1, threads):
        with pytest.raises(oracle.OracleError) as ei:
            oracle.rate(g, BIG, BIG, True, 0, threads=th)
        assert ei.value.code == oracle.EOVERFLOW


def test_coarsen_stall_rule():
    """The driver's stall rule: with min_pair_frac f the coarsening ends after
    the first level that pairs fewer than f of its nodes, and the levels up to
    it are the levels of the run without the rule."""
    spec = synth.config(2, n_nodes=5000)
    h = synth.generate(spec)
    full, _, _ = oracle.coarsen(load(h, spec.omega, spec.delta), spec.omega, spec.delta, 0, 64,
                                True, spec.seed, leftovers=True)
    for f in (0.02, 0.05, 0.2):
        stop = next((i for i, lv in enumerate(full)
                     if lv.n_pairs < f * lv.target.shape[0]), len(full) - 1)
        got, _, _ = oracle.coarsen(load(h, spec.omega, spec.delta), spec.omega, spec.delta, 0,
                                   64, True, spec.seed, leftovers=True, min_pair_frac=f)
        assert len(got) == stop + 1, (f, len(got), stop)
        for a, b in zip(got, full):
            assert np.array_equal(a.match, b.match) and a.n_pairs == b.n_pairs


@pytest.mark.parametrize("cfg,nn,theta", [(4, 2000, 4), (4, 3000, 8), (1, None, 4)])
def test_uncoarsen_invariants(cfg, nn, theta):
    """The uncoarsening driver against the evaluator: the coarsest level's
    identity partition is valid, projection keeps every partition's size,
    inbound count and the connectivity (evaluated on the finer graph), each
    level's refinement lowers the connectivity by exactly the gains it
    applied and never leaves a partition invalid."""
    spec = synth.config(cfg, n_nodes=nn)
    h = synth.generate(spec)
    g0 = load(h, spec.omega, spec.delta)
    levels, _, _ = oracle.coarsen(g0, spec.omega, spec.delta, spec.target_nodes, 64, True,
                                  spec.seed, leftovers=True)
    graphs = [g0] + [lv.coarse for lv in levels if lv.n_pairs]
    gammas = [lv.gamma for lv in levels if lv.n_pairs]
    k = graphs[-1].n_nodes
    rho = np.arange(k, dtype=np.uint32)
    prev = oracle.evaluate(graphs[-1], rho, k, spec.omega, spec.delta)
    assert int(prev[2][2]) == 0 and int(prev[2][3]) == 0
    seen = []
    for d in range(len(graphs) - 1, -1, -1):
        g = graphs[d]
        before = oracle.evaluate(g, rho, k, spec.omega, spec.delta)
        # projection keeps sizes, inbound counts and connectivity
        assert np.array_equal(before[0], prev[0]) and np.array_equal(before[1], prev[1])
        assert int(before[2][0]) == int(prev[2][0])
        rho2, applied, gain = oracle.refine_level(g, rho, k, spec.omega, spec.delta, theta)
        after = oracle.evaluate(g, rho2, k, spec.omega, spec.delta)
        assert int(before[2][0]) - int(after[2][0]) == gain and gain >= 0
        assert int(after[2][2]) == 0 and int(after[2][3]) == 0
        seen.append(rho2.copy())
        prev = after
        rho = rho2[gammas[d - 1]] if d else rho2
    # moves were applied somewhere (these workloads have improving moves)
    assert any(not np.array_equal(a, b) for a, b in zip(seen[1:], [
        r[gm] for r, gm in zip(seen[:-1], reversed(gammas))]))
    # the driver composes the same steps
    got, kk = oracle.uncoarsen(levels, g0, spec.omega, spec.delta, theta)
    assert kk == k and np.array_equal(got, rho)


# ---------------------------------------------------------------- error paths
def err_code(edges, n, w=None, sizes=None, omega=BIG, delta=BIG):
    h = synth.from_lists(n, edges, w, sizes)
    try:
        oracle.canonicalize(h.e_off, h.e_nsrc, h.e_pins, h.e_w, h.n_size, omega, delta)
        return 0
    except oracle.OracleError as ex:
        return ex.code


def test_validation_errors():
    assert err_code([([0], [1, 2])], 3) == 0
    assert err_code([([0], [1, 3])], 3) == oracle.EINVAL          # id out of range
    assert err_code([([0], [1, 1])], 3) == oracle.EINVAL          # duplicate pin
    assert err_code([([0], [0, 1])], 3) == oracle.EINVAL          # src and dst overlap
    assert err_code([([], [])], 3) == oracle.EINVAL               # empty h-edge
    assert err_code([([0], [1])], 3, w=[0]) == oracle.EINVAL      # zero weight
    assert err_code([([0], [1])], 3, w=[1 << 24]) == oracle.EOVERFLOW
    assert err_code([([0], [1])], 3, sizes=[1, 5, 1], omega=4) == oracle.EINFEASIBLE
    assert err_code([([0], [1]), ([2], [1])], 3, delta=1) == oracle.EINFEASIBLE
    assert err_code([([0], [1, 2])], 3, delta=1) == 0


# ---------------------------------------------------------------- purge (O10)
@pytest.mark.parametrize("kw", tiny_cases()[::3], ids=lambda k: "s%d" % k["seed"])
def test_flags_and_purge_vs_brute(kw):
    """Flags are the invalid pairs by Python set union; the purged coarse
    neighbourhood is the full one minus the coarse images of every flagged
    neighbour of a member, keeps every valid coarse neighbour, and leaves the
    level's own results unchanged."""
    h = synth.tiny(**kw)
    edges = brute.edges_of(h.e_off, h.e_nsrc, h.e_pins)
    ins, _ = brute.incidence_sets(h.n_nodes, edges)
    nbs = brute.neighbor_sets(h.n_nodes, edges)
    for omega, delta in constraint_grid(h):
        g = load(h, omega, delta)
        fl = oracle.flags(g, omega, delta)
        for n in range(h.n_nodes):
            for i in range(int(g.nb_off[n]), int(g.nb_off[n + 1])):
                assert bool(fl[i]) == (not brute.valid(n, int(g.nb[i]), h.n_size, ins, omega,
                                                       delta))
        full = oracle.level(load(h, omega, delta), omega, delta, False, kw["seed"])
        lv = oracle.level(load(h, omega, delta), omega, delta, False, kw["seed"],
                          purge_invalid=True)
        for k in ("target", "score", "match"):
            assert np.array_equal(getattr(full, k), getattr(lv, k))
        if lv.n_pairs == 0:
            continue
        gamma, csize, cedges, _ = brute.contract(h.n_nodes, edges, h.e_w, h.n_size, lv.match)
        nc = len(csize)
        cins, _ = brute.incidence_sets(nc, cedges)
        cnbs = brute.neighbor_sets(nc, cedges)
        killed = [set() for _ in range(nc)]
        for n in range(h.n_nodes):
            for m in nbs[n]:
                if not brute.valid(n, m, h.n_size, ins, omega, delta):
                    killed[gamma[n]].add(gamma[m])
        cg = lv.coarse
        for c in range(nc):
            got = cg.nb[cg.nb_off[c]:cg.nb_off[c + 1]].tolist()
            assert got == sorted(cnbs[c] - killed[c])
            for d in cnbs[c]:
                if brute.valid(c, d, csize, cins, omega, delta):
                    assert d in got
                else:
                    pass  # an invalid neighbour may stay (not flagged by a member)
            for d in cnbs[c] - set(got):
                assert not brute.valid(c, d, csize, cins, omega, delta)


def test_purge_multilevel_same_coarsening():
    """Over several levels with binding limits, purging leaves target, score,
    match, gamma and the coarse hyperedges unchanged, and only shrinks the
    neighbourhoods."""
    for cfg, nn, dslack in ((2, 2500, 8), (3, 3000, 16), (4, 6000, 0)):
        spec = synth.config(cfg, n_nodes=nn)
        h = synth.generate(spec)
        g0 = load(h, spec.omega, spec.delta)
        indeg = int(g0.n_nin.max())
        delta = indeg + dslack
        la, _, _ = oracle.coarsen(load(h, spec.omega, delta), spec.omega, delta, 0, 8, True,
                                  spec.seed)
        lb, _, _ = oracle.coarsen(load(h, spec.omega, delta), spec.omega, delta, 0, 8, True,
                                  spec.seed, purge_invalid=True)
        assert len(la) == len(lb)
        flagged = 0
        for x, y in zip(la, lb):
            for k in ("target", "score", "match", "gamma"):
                a, b = getattr(x, k), getattr(y, k)
                assert (a is None and b is None) or np.array_equal(a, b)
            flagged += int(y.flags.sum())
            if x.coarse is None:
                continue
            for k in ("e_off", "e_nsrc", "e_pins", "n_off", "n_inc", "n_size"):
                assert np.array_equal(getattr(x.coarse, k), getattr(y.coarse, k))
            # every pair dropped from a purged list is invalid on the coarse
            # graph (flags of the full lists, themselves pinned above)
            ff = oracle.flags(x.coarse, spec.omega, delta)
            for c in range(x.coarse.n_nodes):
                lo, hi = int(x.coarse.nb_off[c]), int(x.coarse.nb_off[c + 1])
                fa = x.coarse.nb[lo:hi].tolist()
                fb = y.coarse.nb[y.coarse.nb_off[c]:y.coarse.nb_off[c + 1]].tolist()
                assert set(fb) <= set(fa) and fb == sorted(fb)
                kept = set(fb)
                for i, d in enumerate(fa):
                    if d not in kept:
                        assert ff[lo + i] == 1
        assert flagged > 0  # the limits bind, so something was purged


# ---- O11: best-effort pairing of nodes left without a partner ([HP] Sec. V-C)
NONE = 0xFFFFFFFF


def _leftovers(sizes, nin, omega, delta, window=oracle.LEFTOVER_WINDOW, target=None, match=None):
    n = len(sizes)
    t = np.full(n, NONE, np.uint32) if target is None else np.asarray(target, np.uint32)
    m = np.arange(n, dtype=np.uint32) if match is None else np.asarray(match, np.uint32)
    return oracle.pair_leftovers(t, m, np.asarray(sizes, np.uint32), np.asarray(nin, np.uint32),
                                 omega, delta, window)


def _pairs(m):
    return sorted({tuple(sorted((i, int(j)))) for i, j in enumerate(m) if int(j) != i})


def test_leftovers_hand_examples():
    """Worked by hand from the reading: sort by (size, id), binary-search the
    slack, scan down for the first node within Delta, smallest claimer wins,
    a claimed node does not pair through its own claim."""
    # sizes 1,1,2,3 under Omega 4: 0 and 1 reach 3, 2 and 3 reach 1;
    # 3 goes to 0 (smaller id), 1 goes to 2 (2 is not claimed)
    m, k = _leftovers([1, 1, 2, 3], [1, 1, 1, 1], 4, 100)
    assert _pairs(m) == [(0, 3), (1, 2)] and k == 2
    # six equal nodes, Omega 2: all but 5 choose 5, 5 chooses 4; 0 wins 5,
    # and 5, being claimed, does not pair with 4
    m, k = _leftovers([1] * 6, [1] * 6, 2, 100)
    assert _pairs(m) == [(0, 5)] and k == 1
    # Delta binds: 0 and 1 (|in| 5) cannot join 3 (|in| 3) under Delta 7
    m, k = _leftovers([1, 1, 1, 1], [5, 5, 1, 3], 10, 7)
    assert _pairs(m) == [(0, 2)] and k == 1
    # a node whose slack fits nobody but itself stays single
    m, k = _leftovers([3, 3], [1, 1], 5, 100)
    assert k == 0 and _pairs(m) == []


def test_leftovers_window_bound():
    """Nodes 1..68 can only join node 0, at the bottom of the order and more
    than 64 positions below their slack position: they find nobody, and 0
    pairs with 69.  With a window covering everything they all choose 0,
    node 1 wins it, and 69 (which also wants 0) stays single."""
    n = 70
    nin = [10] * n
    nin[0] = 1
    m, k = _leftovers([1] * n, nin, 2, 11)
    assert _pairs(m) == [(0, 69)] and k == 1
    m, k = _leftovers([1] * n, nin, 2, 11, window=n)
    assert _pairs(m) == [(0, 1)] and k == 1


def test_leftovers_only_unmatched_without_target():
    """Nodes with a target, or already matched, are neither paired nor
    claimed; the existing pairs are kept."""
    t = [NONE, 5, NONE, NONE, NONE, 1]
    match = [0, 5, 2, 3, 4, 1]
    m, k = _leftovers([1] * 6, [1] * 6, 2, 100, target=t, match=match)
    assert m[1] == 5 and m[5] == 1
    assert _pairs(m) == [(0, 4), (1, 5)] and k == 1


@pytest.mark.parametrize("seed", range(40))
def test_leftovers_invariants(seed):
    """Random leftovers: the result is a matching that keeps every earlier
    pair, pairs only unmatched nodes without a target, and every new pair fits
    Omega and, with inbound sets counted as a sum, Delta."""
    rng = np.random.Generator(np.random.PCG64(seed))
    n = int(rng.integers(2, 400))
    sizes = rng.integers(1, 9, n).astype(np.uint32)
    nin = rng.integers(0, 20, n).astype(np.uint32)
    omega = int(rng.integers(8, 17))
    delta = int(rng.integers(10, 40))
    t = np.where(rng.random(n) < 0.6, NONE, 0).astype(np.uint32)
    match = np.arange(n, dtype=np.uint32)
    for i in range(0, n - 1, 7):  # some existing pairs
        if t[i] != NONE and t[i + 1] != NONE:
            match[i], match[i + 1] = i + 1, i
    m, k = _leftovers(sizes, nin, omega, delta, target=t, match=match)
    assert np.array_equal(m[m], np.arange(n))
    new = 0
    for i in range(n):
        j = int(m[i])
        if j == int(match[i]):
            continue
        assert int(match[i]) == i and int(match[j]) == j  # both were single
        assert t[i] == NONE and t[j] == NONE
        assert int(sizes[i]) + int(sizes[j]) <= omega
        assert int(nin[i]) + int(nin[j]) <= delta
        new += 1
    assert new == 2 * k


def test_leftovers_multilevel_invariants():
    """Coarsening with the leftover pairing keeps every coarse node within
    Omega and Delta, and its first level pairs at least as many nodes as the
    same level without it (same rating and matching, pairs only added)."""
    for cfg, nn in ((4, 6000), (1, None)):
        spec = synth.config(cfg, n_nodes=nn)
        h = synth.generate(spec)
        la, _, _ = oracle.coarsen(load(h, spec.omega, spec.delta), spec.omega, spec.delta, 0, 6,
                                  True, spec.seed)
        lb, _, _ = oracle.coarsen(load(h, spec.omega, spec.delta), spec.omega, spec.delta, 0, 6,
                                   True, spec.seed, leftovers=True)
        assert la[0].n_pairs <= lb[0].n_pairs
        for lv in lb:
            if lv.coarse is None:
                continue
            assert int(lv.coarse.n_size.max()) <= spec.omega
            assert int(lv.coarse.n_nin.max()) <= spec.delta


# ---- O12: refinement move proposal, Eq. 13 ([HP] Sec. VI-A/B)
def _hand_moves_graph():
    # e0: 0 -> {1, 2} weight 2; e1: 1 -> {3} weight 5
    return synth.from_lists(4, [([0], [1, 2]), ([1], [3])], weights=[2, 5])


def test_moves_hand_example():
    """Worked by hand: rho = [0, 0, 1, 1].  Node 1 leaves e1 with no pin in
    partition 0 (saving 5) and joins partition 1, where both hyperedges
    already have pins (loss 0); node 0 saves nothing; nodes 2 and 3 save 2 and
    5 and lose nothing in partition 0."""
    h = _hand_moves_graph()
    g = load(h)
    mv, gn = oracle.moves(g, np.array([0, 0, 1, 1], np.uint32), 2, BIG)
    assert mv.tolist() == [1, 1, 0, 0] and gn.tolist() == [0, 5, 2, 5]
    # an empty third partition: worse for everyone (it holds no pin)
    mv, gn = oracle.moves(g, np.array([0, 0, 1, 1], np.uint32), 3, BIG)
    assert mv.tolist() == [1, 1, 0, 0] and gn.tolist() == [0, 5, 2, 5]
    # Omega 2 with unit sizes: partitions 0 and 1 are full, only 2 is allowed
    mv, gn = oracle.moves(g, np.array([0, 0, 1, 1], np.uint32), 3, 2, enforce_omega=True)
    assert mv.tolist() == [2, 2, 2, 2] and gn.tolist() == [-2, -2, 0, 0]
    # a single partition: nowhere to go
    mv, gn = oracle.moves(g, np.zeros(4, np.uint32), 1, BIG)
    assert mv.tolist() == [0xFFFFFFFF] * 4 and gn.tolist() == [0] * 4


@pytest.mark.parametrize("kw", tiny_cases()[::2], ids=lambda k: "s%d" % k["seed"])
def test_moves_vs_brute(kw):
    h = synth.tiny(**kw)
    edges = brute.edges_of(h.e_off, h.e_nsrc, h.e_pins)
    g = load(h)
    for k in (1, 2, 3, h.n_nodes):
        rho = synth.uniform_u32(kw["seed"], 41, h.n_nodes, k)
        psize = np.bincount(rho, weights=h.n_size, minlength=k)
        for enforce, omega in ((False, BIG), (True, int(psize.max()) + 1), (True, 3)):
            mv, gn = oracle.moves(g, rho, k, omega, enforce)
            bm, bg = brute.moves(h.n_nodes, edges, h.e_w, h.n_size, rho.tolist(), k, omega,
                                 enforce)
            assert mv.tolist() == bm and gn.tolist() == bg


@pytest.mark.parametrize("seed", range(8))
def test_moves_identity_partition(seed):
    """Closed form: with every node alone (rho(n) = n), saving(n) is the whole
    weight of I(n), and the gain of joining m is the weight n and m share, so
    the move is the neighbour of largest shared weight (smallest id on ties),
    or, with no neighbour, the smallest other id at gain 0."""
    kw = tiny_cases()[seed * 7 % 60]
    h = synth.tiny(**kw)
    edges = brute.edges_of(h.e_off, h.e_nsrc, h.e_pins)
    n = h.n_nodes
    g = load(h)
    mv, gn = oracle.moves(g, np.arange(n, dtype=np.uint32), n, BIG)
    members = [set(s) | set(d) for s, d in edges]
    for v in range(n):
        shared = {}
        for e, mem in enumerate(members):
            if v in mem:
                for m in mem - {v}:
                    shared[m] = shared.get(m, 0) + int(h.e_w[e])
        if shared:
            best = max(shared.items(), key=lambda kv: (kv[1], -kv[0]))
            assert (int(mv[v]), int(gn[v])) == best
        else:
            assert (int(mv[v]), int(gn[v])) == (0 if v else 1, 0)


# ---- O13: exact matching on the proposal pseudo-forest ([HP] Sec. V-D)
def _total(match, score, target):
    tot = 0
    for v, m in enumerate(match.tolist()):
        if m > v:
            # the edge's weight: score of whichever endpoint proposed it
            tot += int(score[v]) if int(target[v]) == m else int(score[m])
    return tot


def test_match_dp_hand_examples():
    N = 0xFFFFFFFF
    # chain a -> b -> (c <-> d): pairing the roots (10) and then a with b (8)
    # beats b with c (9)
    tgt = np.array([1, 2, 3, 2], np.uint32)        # a=0, b=1, c=2, d=3
    sc = np.array([8, 9, 10, 10], np.uint64)
    m, k = oracle.match_dp(tgt, sc)
    assert m.tolist() == [1, 0, 3, 2] and k == 2
    # roots worth 5 with a child each worth 5: the roots stay apart and take
    # their children (10), where the handshake pairs the roots (5)
    tgt = np.array([1, 0, 0, 1], np.uint32)
    sc = np.array([5, 5, 5, 5], np.uint64)
    m, k = oracle.match_dp(tgt, sc)
    assert m.tolist() == [2, 3, 0, 1] and k == 2
    hm, hk = oracle.match(tgt, sc)
    assert hm.tolist() == [1, 0, 2, 3] and hk == 1
    # a tie between pairing the roots (5) and the root taking its child (5):
    # the roots pair only when strictly better
    tgt = np.array([1, 0, 0], np.uint32)
    sc = np.array([5, 5, 5], np.uint64)
    m, k = oracle.match_dp(tgt, sc)
    assert m.tolist() == [2, 1, 0] and k == 1
    # two equal children: the smaller id is taken; a node without a target
    # takes its best child
    tgt = np.array([N, 0, 0, N], np.uint32)
    sc = np.array([0, 7, 7, 0], np.uint64)
    m, k = oracle.match_dp(tgt, sc)
    assert m.tolist() == [1, 0, 2, 3] and k == 1


def _forest(rng, n):
    """A random proposal pseudo-forest: two-cycles and free tops as roots,
    every other node under a node of score at least its own."""
    target = np.full(n, 0xFFFFFFFF, np.uint32)
    score = np.zeros(n, np.uint64)
    order = rng.permutation(n)
    placed = []
    for v in order.tolist():
        r = rng.random()
        if not placed or r < 0.15:
            placed.append(v)  # a tree top without target
            continue
        if r < 0.3:
            # close a two-cycle with a free top
            tops = [u for u in placed if target[u] == 0xFFFFFFFF and score[u] == 0]
            if tops:
                u = tops[int(rng.integers(0, len(tops)))]
                s = int(rng.integers(1, 50))
                target[u], target[v] = v, u
                score[u] = score[v] = s
                placed.append(v)
                continue
        p = placed[int(rng.integers(0, len(placed)))]
        cap = int(score[p]) if target[p] != 0xFFFFFFFF else 50
        target[v] = p
        score[v] = int(rng.integers(1, max(cap, 1) + 1))
        placed.append(v)
    return target, score


@pytest.mark.parametrize("seed", range(60))
def test_match_dp_vs_brute(seed):
    """On random pseudo-forests of at most 16 nodes the matching reaches the
    largest total weight over all matchings of proposal edges."""
    rng = np.random.Generator(np.random.PCG64(seed))
    n = int(rng.integers(2, 17))
    tgt, sc = _forest(rng, n)
    m, k = oracle.match_dp(tgt, sc)
    assert np.array_equal(m[m], np.arange(n))
    for v in range(n):
        if int(m[v]) != v:
            assert int(tgt[v]) == int(m[v]) or int(tgt[int(m[v])]) == v
    best, _ = brute.max_weight_matching(tgt.tolist(), sc.tolist())
    assert _total(m, sc, tgt) == best


@pytest.mark.parametrize("kw", tiny_cases()[::3], ids=lambda k: "s%d" % k["seed"])
def test_match_dp_on_proposals(kw):
    """On the proposals of the tiny graphs (rating with noise): optimal, and
    never below the handshake's total."""
    h = synth.tiny(**kw)
    g = load(h)
    tgt, sc = oracle.rate(g, BIG, BIG, noise_on=True, seed=kw["seed"])
    m, _ = oracle.match_dp(tgt, sc)
    if h.n_nodes <= 18:
        best, _ = brute.max_weight_matching(tgt.tolist(), sc.tolist())
        assert _total(m, sc, tgt) == best
    hm, _ = oracle.match(tgt, sc)
    assert _total(m, sc, tgt) >= _total(hm, sc, tgt)


# ---- O14: one refinement pass ([HP] Sec. VI-A, VI-C, VI-D; Eqs. 14-15)
def test_refine_hand_example():
    """Worked by hand on the graph of the move example, rho = [0, 0, 1, 1]:
    proposals (1 -> 1, gain 5), (3 -> 0, 5), (2 -> 0, 2), (0 -> 1, 0).

    By gain alone the sequence is 1, 3, 2, 0.  Moving 1 first frees e1 of
    partition 0 (+5); then 3 re-enters partition 0 on e1, where 1 no longer is
    (-5 in sequence, +5 in isolation); 2 and 0 change no lambda.  Without
    limits the best prefix is the first move (connectivity 7 -> 2).

    As chains (|in| of nodes 0..3 is 0, 1, 1, 1; all sizes 1): 1 and 3 pick
    each other (grade 5e7 each; 0's bid for 3 is 1e-7 lower), 2's bid for 1
    ties 3's and loses to the larger id; next round 0 and 2 pick each other.
    Two swaps: [1, 3] (total 10), then [0, 2] (total 2), so 1, 3, 0, 2 with
    in-sequence gains 5, -5, 2, -2."""
    h = _hand_moves_graph()
    g = load(h)
    rho = np.array([0, 0, 1, 1], np.uint32)
    r = oracle.refine_pass(g, rho, 2, BIG, BIG, chained=False)
    assert r.seq.tolist() == [1, 3, 2, 0]
    assert r.seq_gain.tolist() == [5, -5, 0, 0]
    assert r.seq_viol.tolist() == [0, 0, 0, 0]
    assert (r.n_applied, r.gain) == (1, 5) and r.rho.tolist() == [0, 1, 1, 1]
    # Omega 2 (unit sizes): after the first move partition 1 holds 3; the
    # prefixes that are valid again gain nothing, so nothing is applied
    r = oracle.refine_pass(g, rho, 2, 2, BIG, chained=False)
    assert r.seq_viol.tolist() == [1, 0, 1, 0]
    assert (r.n_applied, r.gain) == (0, 0) and r.rho.tolist() == rho.tolist()
    # Delta 1: partition 1 starts with two inbound hyperedges (e0 by 2, e1 by
    # 3); after move 1, e0 has no destination left in partition 0; after move
    # 3, e1 is inbound to 0 and 1 keeps e0 (by 1 and 2); after move 2, e0 is
    # inbound to both
    r = oracle.refine_pass(g, rho, 2, BIG, 1, chained=False)
    assert r.seq_viol.tolist() == [1, 0, 1, 1]
    assert (r.n_applied, r.gain) == (0, 0)
    # the chained order
    r = oracle.refine_pass(g, rho, 2, BIG, BIG)
    assert r.seq.tolist() == [1, 3, 0, 2] and r.seq_chain.tolist() == [0, 0, 1, 1]
    assert r.seq_gain.tolist() == [5, -5, 2, -2]
    assert (r.n_applied, r.gain) == (1, 5)
    # Delta 1: moving source-only node 0 keeps both partitions at one inbound
    # hyperedge, so the prefix 1, 3, 0 is valid and gains 2
    r = oracle.refine_pass(g, rho, 2, BIG, 1)
    assert r.seq_viol.tolist() == [1, 0, 0, 1]
    assert (r.n_applied, r.gain) == (3, 2) and r.rho.tolist() == [1, 1, 1, 0]


def _chain(n, rho, move, gain, edges=(), sizes=None):
    h = synth.from_lists(n, list(edges), [1] * len(edges), sizes)
    g = load(h)
    k = max(max(rho), max(m for m in move if m != NONE)) + 1
    r = oracle.refine(g, np.array(rho, np.uint32), k, BIG, BIG,
                      np.array(move, np.uint32), np.array(gain, np.int64))
    return r.seq.tolist(), r.seq_chain.tolist()


def test_chain_hand_examples():
    """Chains worked by hand (unit sizes, no hyperedges, so grades are 1e7
    times the successor's gain).  Moves 0: 0->1 (5), 1: 1->0 (3), 2: 1->2 (4),
    3: 2->0 (1), 4: 0->2 (2).  Round 1: 0 picks 2; 4 and 2 both pick 3 (equal
    grades, the larger picker 4 wins); 1 and 3 both pick 0 (3 wins).  Round 2:
    1 picks 4, the only move out of partition 0 still without a predecessor;
    2 finds none.  One path 1, 4, 3, 0, 2."""
    seq, ch = _chain(5, [0, 1, 1, 2, 0], [1, 0, 2, 0, 2], [5, 3, 4, 1, 2])
    assert seq == [1, 4, 3, 0, 2] and ch == [0] * 5
    # a picker with two equal candidates takes the smaller id: 0 -> 1, then 2
    seq, ch = _chain(3, [0, 1, 1], [1, 2, 2], [0, 0, 0])
    assert seq == [0, 1, 2] and ch == [0, 0, 1]
    # a swap is a two-cycle, started at its smaller node
    seq, ch = _chain(2, [1, 0], [0, 1], [1, 1])
    assert seq == [0, 1] and ch == [0, 0]
    # moves 0: 0->1 (1), 1: 1->0 (2), 2: 2->3 (0), 3: 3->2 (3), 4: 4->0 (0),
    # 5: 5->4 (0).  1 and 4 both bid 1e7 for 0 and 4 wins; 2 and 3 swap.  The
    # path 5, 4, 0, 1 and the cycle 2, 3 both total 3: the cycle's first node
    # (2) is smaller, so it goes first
    seq, ch = _chain(6, [0, 1, 2, 3, 4, 5], [1, 0, 3, 2, 0, 4], [1, 2, 0, 3, 0, 0])
    assert seq == [2, 3, 5, 4, 0, 1] and ch == [0, 0, 1, 1, 1, 1]


def test_chain_window():
    """The window is the first 256 moves (by gain desc, id asc) leaving the
    destination.  Nodes 0..299 move 0 -> 1 with gain 0; node 300 moves 1 -> 0.
    Node 300 (size 100) picks, among ids 0..255, the closest size: 255 (102);
    256 (101) and 280 (100) lie outside.  Every move out of 0 bids for 300 and
    280 wins (grade 0).  One chain 280, 300, 255; the rest alone, by id."""
    n = 301
    sizes = [105] * n
    sizes[255], sizes[256], sizes[280], sizes[300] = 102, 101, 100, 100
    rho = [0] * 300 + [1]
    move = [1] * 300 + [0]
    seq, ch = _chain(n, rho, move, [0] * n, sizes=sizes)
    want = [v for v in range(280) if v != 255] + [280, 300, 255] + list(range(281, 300))
    assert seq == want
    assert ch[278:283] == [278, 279, 279, 279, 280]
    # the window holds the highest gains: nodes 200..299 gain 1 and come
    # first, then 0..155.  Node 300 picks 290 (gain 1, same size), 290 wins
    # the bids for 300: a two-cycle of total 1, ranked among the gain-1 nodes
    gain = [0] * 200 + [1] * 100 + [0]
    sizes = [105] * n
    sizes[290] = sizes[300] = 100
    seq, ch = _chain(n, rho, move, gain, sizes=sizes)
    assert seq == list(range(200, 290)) + [290, 300] + list(range(291, 300)) + list(range(200))


def test_chain_grade_weights():
    """The grade gain - 1e-6 |size diff| - 1e-7 ||in| diff|, exactly.  Node 0
    (size 10, |in| 0) moves 0 -> 1; candidates 1 and 2 move 1 -> 0 (gain 0)
    and node 3 holds the hyperedges that give |in|."""
    def case(size1, nin2, gain1=0):
        edges = [([3], [2])] * nin2
        sizes = [10, size1, 10, 1]
        return _chain(4, [0, 1, 1, 0], [1, 0, 0, 0xFFFFFFFF], [0, gain1, 0, 0],
                      edges, sizes)[0]
    # size off by 1 (-10e-7) against |in| off by 9 (-9e-7): 2 is closer
    assert case(11, 9) == [0, 2, 1]
    # against |in| off by 11: 1 is closer
    assert case(11, 11) == [0, 1, 2]
    # gain 1 (1e7 e-7) against a size gap of 1,000,001 (1e7 + 10 e-7): 2
    assert case(10 + 1000001, 0, gain1=1) == [1, 0, 2]


def _refine_brute_check(h, rho, k, omega, delta, enforce, chained):
    edges = brute.edges_of(h.e_off, h.e_nsrc, h.e_pins)
    g = load(h)
    r = oracle.refine_pass(g, rho, k, omega, delta, enforce, chained)
    mv, gn = oracle.moves(g, rho, k, omega, enforce)
    moving = [n for n in range(h.n_nodes) if mv[n] != NONE]
    seq = r.seq.tolist()
    assert sorted(seq) == moving
    if not chained:
        assert seq == sorted(moving, key=lambda n: (-int(gn[n]), n))
    else:
        # chains: consecutive members link (source of the next = destination
        # of the one before) to a successor within the window; chains ranked
        # by total gain desc, then first node asc
        srt = sorted(moving, key=lambda n: (int(rho[n]), -int(gn[n]), n))
        pos = {n: i for i, n in enumerate(srt)}
        first = {}
        for n in srt:
            first.setdefault(int(rho[n]), pos[n])
        ch = r.seq_chain.tolist()
        assert ch == sorted(ch) and (not ch or ch[0] == 0)
        for i in range(1, len(seq)):
            if ch[i] == ch[i - 1]:
                a, b = seq[i - 1], seq[i]
                assert int(rho[b]) == int(mv[a])
                assert pos[b] - first[int(rho[b])] < 256
        totals = {}
        heads = {}
        for c, n in zip(ch, seq):
            totals[c] = totals.get(c, 0) + int(gn[n])
            heads.setdefault(c, n)
        keys = [(-totals[c], heads[c]) for c in sorted(totals)]
        assert keys == sorted(keys)

    def state(part):
        conn, _, psize, pinb, _ = brute.evaluate(h.n_nodes, edges, h.e_w, h.n_size, part, k)
        return conn, sum(1 for p in range(k) if psize[p] > omega or pinb[p] > delta)

    cur = rho.tolist()
    conns = [state(cur)[0]]
    viols = []
    for i, n in enumerate(seq):
        cur[n] = int(mv[n])
        c, v = state(cur)
        conns.append(c)
        viols.append(v)
        assert int(r.seq_gain[i]) == conns[i] - conns[i + 1], (i, n)
        assert int(r.seq_viol[i]) == v, (i, n)
    # best prefix: largest connectivity drop with no violation, ties shortest
    best, blen = 0, 0
    for i in range(len(seq)):
        if viols[i] == 0 and conns[0] - conns[i + 1] > best:
            best, blen = conns[0] - conns[i + 1], i + 1
    assert (r.n_applied, r.gain) == (blen, best)
    out = rho.tolist()
    for n in seq[:blen]:
        out[n] = int(mv[n])
    assert r.rho.tolist() == out
    return r


@pytest.mark.parametrize("chained", [False, True])
@pytest.mark.parametrize("kw", tiny_cases()[::2], ids=lambda k: "s%d" % k["seed"])
def test_refine_vs_brute(kw, chained):
    """Every in-sequence gain equals the connectivity the move removes from the
    partition left by the moves before it, every violation count the invalid
    partitions then (both by the set-based evaluator), and the prefix applied
    is the best valid one; the order is by gain, or chains that link and are
    ranked as stated."""
    h = synth.tiny(**kw)
    grid = constraint_grid(h)
    for k in (1, 2, 3, max(2, h.n_nodes // 2)):
        rho = synth.uniform_u32(kw["seed"], 43, h.n_nodes, k)
        psize = np.bincount(rho, weights=h.n_size, minlength=k)
        for omega, delta in grid + [(int(psize.max()) + 1, BIG)]:
            for enforce in (False, True):
                _refine_brute_check(h, rho, k, omega, delta, enforce, chained)


@pytest.mark.parametrize("seed", range(6))
def test_refine_never_worsens(seed):
    """Repeated passes: connectivity never rises, a valid partition stays
    valid, and the applied gain is the connectivity drop the evaluator sees."""
    kw = tiny_cases()[seed * 11 % 60]
    h = synth.tiny(**kw)
    g = load(h)
    k = 3
    rho = synth.uniform_u32(seed, 47, h.n_nodes, k)
    psize = np.bincount(rho, weights=h.n_size, minlength=k)
    omega = int(psize.max()) + 2
    _, _, s0 = oracle.evaluate(g, rho, k, omega, BIG)
    for it in range(6):
        r = oracle.refine_pass(g, rho, k, omega, BIG, enforce_omega=True, chained=it % 2 == 0)
        _, _, s1 = oracle.evaluate(g, r.rho, k, omega, BIG)
        assert int(s1[0]) == int(s0[0]) - r.gain and r.gain >= 0
        assert int(s1[2]) == 0 and int(s1[3]) == 0
        rho, s0 = r.rho, s1


# ---- O16: top-Pi candidates and Pi matching rounds ([HP] Sec. V-D)
def _brute_rounds(lists, n, pi, optimal):
    """The rounds with the set-based handshake (or, for the exact matching,
    the brute-force best total checked per round): every unmatched node
    proposes to its first still-unmatched list entry."""
    match = list(range(n))
    totals = []
    for _ in range(pi):
        tg = [NONE] * n
        sc = [0] * n
        for v in range(n):
            if match[v] != v:
                continue
            for m, s in lists[v]:
                if match[m] == m:
                    tg[v], sc[v] = m, s
                    break
        if optimal:
            totals.append((tg, sc))
            mr, _ = oracle.match_dp(np.array(tg, np.uint32), np.array(sc, np.uint64))
            mr = mr.tolist()
        else:
            mr = brute.handshake(tg, sc)
        for v in range(n):
            if mr[v] != v:
                match[v] = mr[v]
    return match, totals


@pytest.mark.parametrize("kw", tiny_cases()[::2], ids=lambda k: "s%d" % k["seed"])
@pytest.mark.parametrize("noise_on", [False, True])
def test_rate_top_and_rounds_vs_brute(kw, noise_on):
    """The top-4 lists against a full sort of every node's valid neighbours;
    row 0 is the single-candidate rating; the rounds against the set-based
    handshake round by round, and (exact matching) each round's total against
    the brute-force best over its proposal edges."""
    h = synth.tiny(**kw)
    edges = brute.edges_of(h.e_off, h.e_nsrc, h.e_pins)
    for omega, delta in constraint_grid(h):
        g = load(h, omega, delta)
        tl, sl = oracle.rate_top(g, omega, delta, noise_on, kw["seed"], pi=4)
        want = brute.rate_top(h.n_nodes, edges, h.e_w, h.n_size, omega, delta, noise_on,
                              kw["seed"], 4)
        for v in range(h.n_nodes):
            got = [(int(tl[r, v]), int(sl[r, v])) for r in range(4) if tl[r, v] != NONE]
            assert got == want[v]
            assert all(tl[r, v] == NONE and sl[r, v] == 0 for r in range(len(got), 4))
        t1, s1 = oracle.rate(g, omega, delta, noise_on=noise_on, seed=kw["seed"])
        assert tl[0].tolist() == t1.tolist() and sl[0].tolist() == s1.tolist()
        for pi in (1, 2, 4):
            m, npairs = oracle.match_rounds(tl[:pi], sl[:pi])
            lists = [w[:pi] for w in want]
            bm, _ = _brute_rounds(lists, h.n_nodes, pi, False)
            assert m.tolist() == bm
            assert npairs == sum(1 for v in range(h.n_nodes) if m[v] != v) // 2
            if pi == 1:
                assert m.tolist() == oracle.match(t1, s1)[0].tolist()
            mo, _ = oracle.match_rounds(tl[:pi], sl[:pi], optimal=True)
            bo, graphs = _brute_rounds(lists, h.n_nodes, pi, True)
            assert mo.tolist() == bo
            if h.n_nodes <= 14:
                for tg, sc in graphs:
                    best, _ = brute.max_weight_matching(tg, sc)
                    mr, _ = oracle.match_dp(np.array(tg, np.uint32), np.array(sc, np.uint64))
                    assert _total(mr, np.array(sc), np.array(tg, np.uint32)) == best


def test_rounds_hand_example():
    """Unit sizes, Omega 2 (a node pairs once), every hyperedge of two pins
    (eta = w / 2).  A path 0 - 1 - 2 (weights 4, 2): 0 and 1 pick each other
    and pair; 2 picks 1, which is taken, and nobody picks 2; its list holds
    only 1, so round 2 adds nothing.

    Two stars: centre 1 with leaves 0 (eta 4) and 2 (eta 3), centre 4 with
    leaves 5 (4) and 3 (3), and 2 - 3 joined weakly (eta 1).  Round 1 pairs
    0-1 and 4-5; 2 and 3 picked their centres, were not picked, and stay
    alone.  Round 2: the first unmatched entries of 2's and 3's lists are each
    other: they pair."""
    h = synth.from_lists(3, [([0], [1]), ([1], [2])], [4, 2])
    g = load(h, 2, BIG)
    tl, sl = oracle.rate_top(g, 2, BIG, False, 0, pi=2)
    assert tl[0].tolist() == [1, 0, 1] and tl[1].tolist() == [NONE, 2, NONE]
    m, npairs = oracle.match_rounds(tl, sl)
    assert m.tolist() == [1, 0, 2] and npairs == 1
    h = synth.from_lists(6, [([0], [1]), ([2], [1]), ([5], [4]), ([3], [4]), ([2], [3])],
                         [8, 6, 8, 6, 2])
    g = load(h, 2, BIG)
    tl, sl = oracle.rate_top(g, 2, BIG, False, 0, pi=2)
    assert tl[0].tolist() == [1, 0, 1, 4, 5, 4]
    assert tl[1].tolist() == [NONE, 2, 3, 2, 3, NONE]
    m1, p1 = oracle.match_rounds(tl[:1], sl[:1])
    assert m1.tolist() == [1, 0, 2, 3, 5, 4] and p1 == 2
    m, npairs = oracle.match_rounds(tl, sl)
    assert m.tolist() == [1, 0, 3, 2, 5, 4] and npairs == 3
    mo, po = oracle.match_rounds(tl, sl, optimal=True)
    assert mo.tolist() == [1, 0, 3, 2, 5, 4] and po == 3


def test_rounds_more_pairs_multilevel():
    """Over several levels of a scaled workload: four rounds never pair fewer
    nodes on the first level than one, every pair is valid, and the
    coarsening reaches at most as many nodes after the same number of levels
    on that first level."""
    spec = synth.config(1)
    h = synth.generate(spec)
    g = load(h, spec.omega, spec.delta)
    l1 = oracle.level(g, spec.omega, spec.delta, True, 3)
    l4 = oracle.level(g, spec.omega, spec.delta, True, 3, pi=4)
    assert l4.n_pairs >= l1.n_pairs
    assert l4.target.tolist() == l1.target.tolist()
    m = l4.match
    assert np.array_equal(m[m], np.arange(h.n_nodes))
    for v in range(h.n_nodes):
        u = int(m[v])
        if u != v:
            assert int(h.n_size[v]) + int(h.n_size[u]) <= spec.omega
