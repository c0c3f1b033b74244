"""CPU oracle for one constrained coarsening level and the partition evaluator.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package; the GPU library
never does, and the two share no code.

``chp_oracle.c`` is a plain, single-threaded C statement of the definitions in
Ronzani & Silvano, "Hypergraph Partitioning on GPU with Distinct Incident
Hyperedges and Size Constraints" (Sec. II-V) and of the handshake matching of
their prototype paper "Incidence Constraints in Hypergraph Partitioning on GPU"
(Sec. III-A, III-B3).  This module only marshals numpy arrays through ctypes
and strings the per-level steps together (the level loop of Sec. III).

Pins of the oracle itself (brute force, closed forms, invariants) live in
``tests/test_oracle_*.py``.  Parity of every function is pinned there.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "chp_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

OK, EINVAL, ENOMEM, EOVERFLOW, EINFEASIBLE, ECYCLE, EINTERNAL = 0, -1, -2, -3, -4, -5, -7
NONE = 0xFFFFFFFF
FX_SHIFT = 40


class OracleError(RuntimeError):
    def __init__(self, code, what):
        super().__init__("%s failed with code %d" % (what, code))
        self.code = code


class _Edges(ctypes.Structure):
    _fields_ = [("n_nodes", ctypes.c_uint32), ("n_edges", ctypes.c_uint32),
                ("e_off", ctypes.c_void_p), ("e_nsrc", ctypes.c_void_p),
                ("e_pins", ctypes.c_void_p), ("e_w", ctypes.c_void_p),
                ("n_size", ctypes.c_void_p)]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no GPU code involved)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-shared", "-fPIC", "-std=gnu11", "-pthread", "-o", tmp,
                               _SRC])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        P, E = ctypes.c_void_p, ctypes.POINTER(_Edges)
        u32, u64, i32 = ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int
        sig = {
            "or_canonicalize": [E, u64, u32, P],
            "or_incidence": [E, P, P, P],
            "or_neighbors": [E, P, P, P, ctypes.POINTER(P), ctypes.POINTER(u64)],
            "or_terms": [E, P, ctypes.POINTER(u64)],
            "or_rate": [E, P, P, P, P, u64, u64, u32, i32, u64, u32, u32, P, P],
            "or_match": [u32, P, P, P, ctypes.POINTER(u64)],
            "or_contract": [E, P, P, ctypes.POINTER(u32), ctypes.POINTER(P), ctypes.POINTER(P),
                            ctypes.POINTER(P), ctypes.POINTER(P)],
            "or_evaluate": [E, P, u32, u64, u32, P, P, P],
            "or_flags": [E, P, P, P, P, P, u64, u32, P],
            "or_purge": [u32, P, P, P, P, P, u32, P, ctypes.POINTER(P), ctypes.POINTER(u64)],
            "or_pair_leftovers": [u32, P, P, P, u64, u32, u32, P, ctypes.POINTER(u64)],
            "or_moves": [E, P, P, P, u32, u64, i32, P, P],
            "or_match_dp": [u32, P, P, P, ctypes.POINTER(u64)],
            "or_rate_top": [E, P, P, P, P, u64, u64, u32, i32, u64, u32, P, P],
            "or_rate_top_mt": [E, P, P, P, P, u64, u64, u32, i32, u64, u32, u32, u32, u32, P,
                               P],
            "or_match_rounds": [u32, u32, P, P, i32, P, ctypes.POINTER(u64)],
            "or_refine": [E, P, P, P, P, u32, u64, u32, P, P, i32, P, P, P, P,
                          ctypes.POINTER(u32), ctypes.POINTER(u32),
                          ctypes.POINTER(ctypes.c_int64), P],
        }
        for name, args in sig.items():
            f = getattr(lib, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        lib.or_noise.argtypes = [u64, u64, u32, u32]
        lib.or_noise.restype = u64
        lib.or_free.argtypes = [P]
        lib.or_free.restype = None
        _lib = lib
    return _lib


def _p(a):
    return a.ctypes.data if a is not None and a.size else None


def _take(ptr, n, dtype):
    """Copy a malloc'd C array into numpy and free it."""
    lib = _load()
    if n == 0:
        lib.or_free(ptr)
        return np.zeros(0, dtype=dtype)
    buf = (ctypes.c_char * (n * np.dtype(dtype).itemsize)).from_address(ptr)
    out = np.frombuffer(buf, dtype=dtype).copy()
    lib.or_free(ptr)
    return out


@dataclasses.dataclass
class Graph:
    """One level of a hypergraph: canonical edge CSR, incidence, neighbours."""
    e_off: np.ndarray
    e_nsrc: np.ndarray
    e_pins: np.ndarray
    e_w: np.ndarray
    n_size: np.ndarray
    n_off: np.ndarray | None = None
    n_nin: np.ndarray | None = None
    n_inc: np.ndarray | None = None
    nb_off: np.ndarray | None = None
    nb: np.ndarray | None = None

    @property
    def n_nodes(self):
        return int(self.n_size.shape[0])

    @property
    def n_edges(self):
        return int(self.e_w.shape[0])

    @property
    def n_pins(self):
        return int(self.e_off[-1])

    def view(self):
        self._keep = [np.ascontiguousarray(a) for a in
                      (self.e_off, self.e_nsrc, self.e_pins, self.e_w, self.n_size)]
        k = self._keep
        return _Edges(self.n_nodes, self.n_edges, _p(k[0]), _p(k[1]), _p(k[2]), _p(k[3]), _p(k[4]))


def _check(rc, what):
    if rc != OK:
        raise OracleError(rc, what)


def canonicalize(e_off, e_nsrc, e_pins, e_w, n_size, omega, delta) -> Graph:
    """O1: sorted sub-lists + validation (raises OracleError on bad input)."""
    g = Graph(np.asarray(e_off, np.int64), np.asarray(e_nsrc, np.uint32),
              np.asarray(e_pins, np.uint32), np.asarray(e_w, np.uint32),
              np.asarray(n_size, np.uint32))
    out = np.empty(g.n_pins, dtype=np.uint32)
    v = g.view()
    _check(_load().or_canonicalize(ctypes.byref(v), omega, delta, _p(out)), "canonicalize")
    g.e_pins = out
    return g


def incidence(g: Graph) -> Graph:
    """O2: n_off, n_nin, n_inc (in-edges first, each list ascending)."""
    N = g.n_nodes
    g.n_off = np.empty(N + 1, np.int64)
    g.n_nin = np.empty(N, np.uint32)
    g.n_inc = np.empty(g.n_pins, np.uint32)
    v = g.view()
    _check(_load().or_incidence(ctypes.byref(v), _p(g.n_off), _p(g.n_nin), _p(g.n_inc)),
           "incidence")
    return g


def neighbors(g: Graph) -> Graph:
    """O3: nb_off, nb (sorted unique neighbours, n itself excluded)."""
    N = g.n_nodes
    g.nb_off = np.empty(N + 1, np.int64)
    ptr = ctypes.c_void_p()
    tot = ctypes.c_uint64()
    v = g.view()
    _check(_load().or_neighbors(ctypes.byref(v), _p(g.n_off), _p(g.n_inc), _p(g.nb_off),
                                ctypes.byref(ptr), ctypes.byref(tot)), "neighbors")
    g.nb = _take(ptr.value, tot.value, np.uint32)
    return g


def build_incidence(e_off, e_nsrc, e_pins, e_w, n_size, omega, delta, build_neighbors=True):
    g = canonicalize(e_off, e_nsrc, e_pins, e_w, n_size, omega, delta)
    incidence(g)
    if build_neighbors:
        neighbors(g)
    return g


def terms(g: Graph):
    """O4: t[E] (uint64 fixed point, scale 2^40) and the noise cap."""
    t = np.empty(g.n_edges, np.uint64)
    cap = ctypes.c_uint64()
    v = g.view()
    _check(_load().or_terms(ctypes.byref(v), _p(t), ctypes.byref(cap)), "terms")
    return t, int(cap.value)


def noise(seed: int, cap: int, n: int, m: int) -> int:
    return int(_load().or_noise(seed, cap, n, m))


def rate(g: Graph, omega, delta, noise_on=True, seed=0, lo=0, hi=None, tc=None, threads=1):
    """O5: target[N] (uint32, NONE if no valid neighbour) and score[N] (uint64).
    Only nodes lo..hi-1 are rated; other entries stay NONE / 0.  threads > 1
    splits the node loop (the result does not depend on it)."""
    t, s = rate_top(g, omega, delta, noise_on, seed, 1, lo, hi, tc, threads)
    return t[0], s[0]


def rate_top(g: Graph, omega, delta, noise_on=True, seed=0, pi=4, lo=0, hi=None, tc=None,
             threads=1):
    """Top-pi valid candidates of every node: (targets (pi, N) uint32, scores
    (pi, N) uint64), row r the (r+1)-th best by (score desc, id asc).  Only
    nodes lo..hi-1 are rated (the others stay NONE / 0), over `threads`
    threads."""
    N = g.n_nodes
    hi = N if hi is None else hi
    t, cap = terms(g) if tc is None else tc
    target = np.full((pi, N), NONE, np.uint32)
    score = np.zeros((pi, N), np.uint64)
    v = g.view()
    _check(_load().or_rate_top_mt(ctypes.byref(v), _p(g.n_off), _p(g.n_nin), _p(g.n_inc), _p(t),
                                  cap, omega, delta, 1 if noise_on else 0, seed, lo, hi, pi,
                                  threads, _p(target), _p(score)), "rate_top")
    return target, score


def match_rounds(targets, scores, optimal=False):
    """O16: pi matching rounds over the top-pi lists (match, number of pairs)."""
    tg = np.ascontiguousarray(targets, np.uint32)
    sc = np.ascontiguousarray(scores, np.uint64)
    pi, N = tg.shape
    m = np.empty(N, np.uint32)
    npairs = ctypes.c_uint64()
    _check(_load().or_match_rounds(N, pi, _p(tg), _p(sc), 1 if optimal else 0, _p(m),
                                   ctypes.byref(npairs)), "match_rounds")
    return m, int(npairs.value)


def match(target, score):
    """O6: match[N] (partner or self) and the number of pairs."""
    target = np.ascontiguousarray(target, np.uint32)
    score = np.ascontiguousarray(score, np.uint64)
    N = target.shape[0]
    m = np.empty(N, np.uint32)
    npairs = ctypes.c_uint64()
    _check(_load().or_match(N, _p(target), _p(score), _p(m), ctypes.byref(npairs)), "match")
    return m, int(npairs.value)


def contract(g: Graph, match_arr, build_neighbors=True):
    """O7: gamma[N] and the coarse graph G' (incidence and neighbours rebuilt
    from scratch on G' by O2/O3)."""
    match_arr = np.ascontiguousarray(match_arr, np.uint32)
    N = g.n_nodes
    gamma = np.empty(N, np.uint32)
    nc = ctypes.c_uint32()
    ps, po, pn, pp = ctypes.c_void_p(), ctypes.c_void_p(), ctypes.c_void_p(), ctypes.c_void_p()
    v = g.view()
    _check(_load().or_contract(ctypes.byref(v), _p(match_arr), _p(gamma), ctypes.byref(nc),
                               ctypes.byref(ps), ctypes.byref(po), ctypes.byref(pn),
                               ctypes.byref(pp)), "contract")
    E = g.n_edges
    n_c = int(nc.value)
    size = _take(ps.value, n_c, np.uint32)
    e_off = _take(po.value, E + 1, np.int64)
    nsrc = _take(pn.value, E, np.uint32)
    pins_full = _take(pp.value, g.n_pins, np.uint32)
    pins = pins_full[: int(e_off[-1])].copy()
    cg = Graph(e_off, nsrc, pins, g.e_w.copy(), size)
    incidence(cg)
    if build_neighbors:
        neighbors(cg)
    return gamma, cg


def evaluate(g: Graph, rho, k, omega, delta):
    """O8: part_size[k], part_inb[k] and the 8-entry summary
    (conn, cutnet, over_omega, over_delta, empty, max_size, max_inb, sum_lambda)."""
    rho = np.ascontiguousarray(rho, np.uint32)
    ps = np.empty(k, np.uint64)
    pi = np.empty(k, np.uint32)
    summ = np.zeros(8, np.uint64)
    v = g.view()
    _check(_load().or_evaluate(ctypes.byref(v), _p(rho), k, omega, delta, _p(ps), _p(pi),
                               _p(summ)), "evaluate")
    return ps, pi, summ


def flags(g: Graph, omega, delta):
    """O10: flag[nb_total] (uint8): 1 where (n, nb[i]) is not a valid pair."""
    f = np.empty(g.nb.shape[0], np.uint8)
    v = g.view()
    _check(_load().or_flags(ctypes.byref(v), _p(g.n_off), _p(g.n_nin), _p(g.n_inc), _p(g.nb_off),
                            _p(g.nb), omega, delta, _p(f)), "flags")
    return f


def purge(g: Graph, flag, match_arr, gamma, cg: Graph) -> Graph:
    """O10: cg's neighbourhoods built from the members' current lists in g,
    without every coarse neighbour that a member flagged (cg.nb_off / cg.nb
    replaced)."""
    nc = cg.n_nodes
    off = np.empty(nc + 1, np.int64)
    ptr = ctypes.c_void_p()
    tot = ctypes.c_uint64()
    _check(_load().or_purge(g.n_nodes, _p(g.nb_off), _p(g.nb), _p(np.ascontiguousarray(flag)),
                            _p(np.ascontiguousarray(match_arr, np.uint32)),
                            _p(np.ascontiguousarray(gamma, np.uint32)), nc, _p(off),
                            ctypes.byref(ptr), ctypes.byref(tot)), "purge")
    cg.nb_off = off
    cg.nb = _take(ptr.value, tot.value, np.uint32)
    return cg


def match_dp(target, score):
    """O13: exact maximum-weight matching on the proposal pseudo-forest
    (match array, number of pairs)."""
    t = np.ascontiguousarray(target, np.uint32)
    sc = np.ascontiguousarray(score, np.uint64)
    m = np.empty(t.shape[0], np.uint32)
    npairs = ctypes.c_uint64()
    _check(_load().or_match_dp(t.shape[0], _p(t), _p(sc), _p(m), ctypes.byref(npairs)),
           "match_dp")
    return m, int(npairs.value)


def moves(g: Graph, rho, k, omega, enforce_omega=False):
    """O12: (move[N] uint32, gain[N] int64) of Eq. 13 for partition rho."""
    N = g.n_nodes
    mv = np.empty(N, np.uint32)
    gn = np.empty(N, np.int64)
    v = g.view()
    _check(_load().or_moves(ctypes.byref(v), _p(g.n_off), _p(g.n_inc),
                            _p(np.ascontiguousarray(rho, np.uint32)), k, omega,
                            1 if enforce_omega else 0, _p(mv), _p(gn)), "moves")
    return mv, gn


@dataclasses.dataclass
class Refinement:
    rho: np.ndarray        # the partition after the pass
    seq: np.ndarray        # nodes in sequence order
    seq_chain: np.ndarray  # rank of each position's chain
    seq_gain: np.ndarray   # in-sequence gain of each move (int64)
    seq_viol: np.ndarray   # invalid partitions after each move
    n_applied: int         # length of the prefix applied
    gain: int              # its summed in-sequence gain


def refine(g: Graph, rho, k, omega, delta, move, gain, chained=True) -> Refinement:
    """O14: sequence the proposed moves (as chains, O15, or by gain alone),
    take their in-sequence gains and the violations after every prefix, and
    apply the best valid prefix."""
    N = g.n_nodes
    r = np.ascontiguousarray(rho, np.uint32)
    seq = np.empty(N, np.uint32)
    sc = np.empty(N, np.uint32)
    sg = np.empty(N, np.int64)
    sv = np.empty(N, np.uint32)
    out = np.empty(N, np.uint32)
    m, na, ga = ctypes.c_uint32(), ctypes.c_uint32(), ctypes.c_int64()
    v = g.view()
    _check(_load().or_refine(ctypes.byref(v), _p(g.n_off), _p(g.n_nin), _p(g.n_inc), _p(r), k,
                             omega, delta, _p(np.ascontiguousarray(move, np.uint32)),
                             _p(np.ascontiguousarray(gain, np.int64)), 1 if chained else 0,
                             _p(seq), _p(sc), _p(sg), _p(sv),
                             ctypes.byref(m), ctypes.byref(na), ctypes.byref(ga), _p(out)),
           "refine")
    M = int(m.value)
    return Refinement(out if N else r.copy(), seq[:M], sc[:M], sg[:M], sv[:M], int(na.value),
                      int(ga.value))


def refine_pass(g: Graph, rho, k, omega, delta, enforce_omega=False,
                chained=True) -> Refinement:
    """One pass of refinement: propose (O12), then sequence and apply (O14)."""
    mv, gn = moves(g, rho, k, omega, enforce_omega)
    return refine(g, rho, k, omega, delta, mv, gn, chained)


def refine_level(g: Graph, rho, k, omega, delta, theta=16, chained=True):
    """The refinement of one level ([P1] Sec. VI-A: theta repetitions of
    proposal and application; Sec. VI-B: the first half proposes without the
    size limit, the second half within it).  Returns (rho after the passes,
    moves applied, summed gain)."""
    r = np.ascontiguousarray(rho, np.uint32)
    applied = gain = 0
    for p in range(theta):
        ref = refine_pass(g, r, k, omega, delta, enforce_omega=p >= theta // 2, chained=chained)
        r = ref.rho
        applied += ref.n_applied
        gain += ref.gain
    return r, applied, gain


def uncoarsen(levels, g0: Graph, omega, delta, theta=16, on_level=None):
    """The uncoarsening phase of [P1] Sec. III: the coarsest level's nodes are
    the initial partitions (rho = identity there, k their number); each level
    from the coarsest down is refined (refine_level), then its partition is
    projected to the level below through that level's coarsening map.
    `levels` is coarsen()'s list (its last entry may have no pairs).
    on_level(depth, graph, rho) after each level's refinement.  Returns the
    partition of g0 and k."""
    graphs = [g0] + [lv.coarse for lv in levels if lv.n_pairs]
    gammas = [lv.gamma for lv in levels if lv.n_pairs]
    top = graphs[-1]
    k = top.n_nodes
    rho = np.arange(k, dtype=np.uint32)
    for d in range(len(graphs) - 1, -1, -1):
        rho, _, _ = refine_level(graphs[d], rho, k, omega, delta, theta)
        if on_level:
            on_level(d, graphs[d], rho)
        if d:
            rho = rho[gammas[d - 1]]
    return rho, k


LEFTOVER_WINDOW = 64  # positions a leftover node scans below its slack position


def pair_leftovers(target, match_arr, n_size, n_nin, omega, delta, window=LEFTOVER_WINDOW):
    """O11: best-effort pairing of the unmatched nodes without a target.
    Returns (new match array, number of new pairs)."""
    m = np.array(match_arr, dtype=np.uint32, copy=True)
    t = np.ascontiguousarray(target, np.uint32)
    npairs = ctypes.c_uint64()
    _check(_load().or_pair_leftovers(t.shape[0], _p(t), _p(np.ascontiguousarray(n_size, np.uint32)),
                                     _p(np.ascontiguousarray(n_nin, np.uint32)), omega, delta,
                                     window, _p(m), ctypes.byref(npairs)), "pair_leftovers")
    return m, int(npairs.value)


@dataclasses.dataclass
class Level:
    target: np.ndarray
    score: np.ndarray
    match: np.ndarray
    n_pairs: int
    gamma: np.ndarray | None
    coarse: Graph | None
    flags: np.ndarray | None = None


def level(g: Graph, omega, delta, noise_on=True, seed=0, build_neighbors=True,
          purge_invalid=False, leftovers=False, optimal=False, pi=1, threads=1) -> Level:
    """One coarsening level: rate, match, contract.  With purge_invalid the
    neighbour flags of g are computed (Level.flags) and the coarse
    neighbourhoods are purged of flagged neighbours (O10); with leftovers the
    unmatched nodes without a target are paired best-effort (O11); with
    optimal the matching is the exact one of O13 instead of the handshake;
    with pi > 1 the matching takes pi rounds over the top-pi candidates (O16)
    and target/score are the best candidates.  threads splits the rating's
    node loop (the result does not depend on it)."""
    if pi > 1:
        tl, sl = rate_top(g, omega, delta, noise_on, seed, pi, threads=threads)
        target, score = tl[0].copy(), sl[0].copy()
        m, npairs = match_rounds(tl, sl, optimal)
    else:
        target, score = rate(g, omega, delta, noise_on, seed, threads=threads)
        m, npairs = match_dp(target, score) if optimal else match(target, score)
    if leftovers:
        m, extra = pair_leftovers(target, m, g.n_size, g.n_nin, omega, delta)
        npairs += extra
    fl = flags(g, omega, delta) if purge_invalid else None
    if npairs == 0:
        return Level(target, score, m, 0, None, None, fl)
    gamma, cg = contract(g, m, build_neighbors)
    if purge_invalid and build_neighbors:
        purge(g, fl, m, gamma, cg)
    return Level(target, score, m, npairs, gamma, cg, fl)


def coarsen(g: Graph, omega, delta, target_nodes=0, max_levels=64, noise_on=True, seed=0,
            purge_invalid=False, leftovers=False, min_pair_frac=0.0, on_level=None,
            threads=1, build_neighbors=True):
    """O9: the level loop of [P1] Sec. III.  Stops at the first of: fewer than
    target_nodes nodes; at most ceil(sum size / Omega) nodes (the lowest valid
    count); a level with no pair; max_levels levels; after a level that pairs
    fewer than min_pair_frac of its nodes (a stalled coarsening: 0 = never).
    on_level(index, fine graph, Level, rho) is called after each level.
    Returns the list of Levels and the projection rho = gamma_l o ... o
    gamma_1 onto the finest nodes."""
    levels = []
    rho = np.arange(g.n_nodes, dtype=np.uint32)
    floor_nodes = -(-int(g.n_size.astype(np.uint64).sum()) // omega)
    cur = g
    for _ in range(max_levels):
        if cur.n_nodes < target_nodes or cur.n_nodes <= floor_nodes:
            break
        lv = level(cur, omega, delta, noise_on, seed, build_neighbors=build_neighbors,
                   purge_invalid=purge_invalid, leftovers=leftovers, threads=threads)
        levels.append(lv)
        if lv.n_pairs == 0:
            if on_level:
                on_level(len(levels) - 1, cur, lv, rho)
            break
        rho = lv.gamma[rho]
        if on_level:
            on_level(len(levels) - 1, cur, lv, rho)
        stalled = lv.n_pairs < min_pair_frac * cur.n_nodes
        cur = lv.coarse
        if stalled:
            break
    return levels, rho, cur
