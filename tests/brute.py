"""Brute-force statements of the definitions, in pure Python (tiny inputs only).

Written independently of ``oracle/chp_oracle.c`` to pin it: Python sets,
exact rationals (``fractions.Fraction``) and exhaustive sorts.  Sources:
Ronzani & Silvano, "Hypergraph Partitioning on GPU with Distinct Incident
Hyperedges and Size Constraints" (Sec. II-A/B Eqs. 1, 5, 6; Sec. III Eq. 2;
Sec. V-A/E) and the handshake of "Incidence Constraints in Hypergraph
Partitioning on GPU" (Sec. III-A, III-B3).
"""
from __future__ import annotations

from fractions import Fraction

NONE = 0xFFFFFFFF
SCALE = 1 << 40


def edges_of(e_off, e_nsrc, e_pins):
    """[(src_set, dst_set)] from an edge CSR."""
    out = []
    for e in range(len(e_off) - 1):
        a, b = int(e_off[e]), int(e_off[e + 1])
        ns = int(e_nsrc[e])
        out.append((set(int(x) for x in e_pins[a:a + ns]), set(int(x) for x in e_pins[a + ns:b])))
    return out


def incidence_sets(n_nodes, edges):
    ins = [set() for _ in range(n_nodes)]
    outs = [set() for _ in range(n_nodes)]
    for e, (src, dst) in enumerate(edges):
        for n in dst:
            ins[n].add(e)
        for n in src:
            outs[n].add(e)
    return ins, outs


def neighbor_sets(n_nodes, edges):
    ins, outs = incidence_sets(n_nodes, edges)
    nb = []
    for n in range(n_nodes):
        s = set()
        for e in ins[n] | outs[n]:
            s |= edges[e][0] | edges[e][1]
        s.discard(n)
        nb.append(s)
    return nb


def eta_exact(n_nodes, edges, weights):
    """Eq. 5 with exact rationals: {(n, m): sum over shared e of w/|e|}."""
    ins, outs = incidence_sets(n_nodes, edges)
    eta = {}
    for n in range(n_nodes):
        for e in ins[n] | outs[n]:
            pins = edges[e][0] | edges[e][1]
            for m in pins:
                if m != n:
                    eta[(n, m)] = eta.get((n, m), Fraction(0)) + Fraction(int(weights[e]), len(pins))
    return eta


def term_fx(w, size):
    return (int(w) * SCALE) // int(size)


def cap_fx(edges, weights):
    tot = sum(term_fx(weights[e], len(s | d)) for e, (s, d) in enumerate(edges))
    return tot // (10 * len(edges)) if edges else 0


def splitmix64_once(state):
    """One output of Vigna's splitmix64 generator from the given state."""
    mask = (1 << 64) - 1
    z = (state + 0x9E3779B97F4A7C15) & mask
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & mask
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & mask
    return z ^ (z >> 31)


def noise_fx(seed, cap, n, m):
    a, b = min(n, m), max(n, m)
    return splitmix64_once(seed ^ ((a << 32) | b)) % (cap + 1)


def eta_fx(n_nodes, edges, weights, noise_on=False, seed=0):
    """Fixed-point eta: sum of floor(w * 2^40 / |e|), plus noise once per pair."""
    ins, outs = incidence_sets(n_nodes, edges)
    cap = cap_fx(edges, weights)
    eta = {}
    for n in range(n_nodes):
        for e in ins[n] | outs[n]:
            pins = edges[e][0] | edges[e][1]
            t = term_fx(weights[e], len(pins))
            for m in pins:
                if m != n:
                    eta[(n, m)] = eta.get((n, m), 0) + t
    if noise_on:
        for k in list(eta):
            eta[k] += noise_fx(seed, cap, *k)
    return eta


def valid(n, m, sizes, ins, omega, delta):
    """Eq. 6 by Python set union."""
    return int(sizes[n]) + int(sizes[m]) <= omega and len(ins[n] | ins[m]) <= delta


def rate(n_nodes, edges, weights, sizes, omega, delta, noise_on=False, seed=0):
    """Eq. 6: best valid neighbour by (eta desc, id asc), via a full sort."""
    ins, _ = incidence_sets(n_nodes, edges)
    eta = eta_fx(n_nodes, edges, weights, noise_on, seed)
    per = [[] for _ in range(n_nodes)]
    for (n, m), v in eta.items():
        per[n].append((v, m))
    target = [NONE] * n_nodes
    score = [0] * n_nodes
    for n in range(n_nodes):
        for v, m in sorted(per[n], key=lambda x: (-x[0], x[1])):
            if valid(n, m, sizes, ins, omega, delta):
                target[n], score[n] = m, v
                break
    return target, score


def rate_top(n_nodes, edges, weights, sizes, omega, delta, noise_on, seed, pi):
    """The pi best valid neighbours of every node, by (eta desc, id asc), via
    a full sort of all neighbours: lists of (m, eta)."""
    ins, _ = incidence_sets(n_nodes, edges)
    eta = eta_fx(n_nodes, edges, weights, noise_on, seed)
    per = [[] for _ in range(n_nodes)]
    for (n, m), v in eta.items():
        per[n].append((v, m))
    out = []
    for n in range(n_nodes):
        top = [(m, v) for v, m in sorted(per[n], key=lambda x: (-x[0], x[1]))
               if valid(n, m, sizes, ins, omega, delta)]
        out.append(top[:pi])
    return out


def handshake(target, score):
    """The prototype's matching procedure, simulated literally and sequentially.

    Upward phase: from every leaf, each node on the path places its score on
    its candidate; the candidate keeps the best proposal (higher score, ties to
    the smaller id); the walk stops at a two-cycle or a node without candidate.
    Two-cycles match by default.  Downward phase: every path is retraced from
    its top; a node locks its candidate iff the candidate still holds that
    node's proposal."""
    N = len(target)
    tg = [int(x) for x in target]
    sc = [int(x) for x in score]
    slot = list(range(N))  # match(n), initially n

    def better(c, cur, t):
        if cur == t:
            return True
        return sc[c] > sc[cur] or (sc[c] == sc[cur] and c < cur)

    def is_root(n):
        return tg[n] != NONE and tg[tg[n]] == n

    has_child = [False] * N
    for n in range(N):
        if tg[n] != NONE:
            has_child[tg[n]] = True
    paths = []
    for leaf in range(N):
        if has_child[leaf]:
            continue
        path = []
        v = leaf
        seen = set()
        while v != NONE and v not in seen:
            seen.add(v)
            path.append(v)
            if is_root(v):
                break
            t = tg[v]
            if t != NONE and better(v, slot[t], t):
                slot[t] = v
            v = t
        paths.append(path)
    # every node lies on some leaf-to-top path, except pure cycles (roots
    # whose only children are each other): visit those too
    for n in range(N):
        if is_root(n):
            slot[n] = tg[n]
    for path in paths:
        for v in reversed(path):
            if is_root(v):
                continue
            t = tg[v]
            if t != NONE and slot[t] == v:
                slot[v] = t
    return slot


def contract(n_nodes, edges, weights, sizes, match):
    """E' = {gamma(e)}; coarse ids = rank of the smallest member."""
    reps = sorted({min(n, int(match[n])) for n in range(n_nodes)})
    rank = {r: i for i, r in enumerate(reps)}
    gamma = [rank[min(n, int(match[n]))] for n in range(n_nodes)]
    csize = [0] * len(reps)
    for n in range(n_nodes):
        csize[gamma[n]] += int(sizes[n])
    cedges = []
    for src, dst in edges:
        d = {gamma[n] for n in dst}
        s = {gamma[n] for n in src} - d
        cedges.append((s, d))
    return gamma, csize, cedges, list(weights)


def evaluate(n_nodes, edges, weights, sizes, rho, k):
    part_size = [0] * k
    count = [0] * k
    for n in range(n_nodes):
        part_size[int(rho[n])] += int(sizes[n])
        count[int(rho[n])] += 1
    part_inb = [0] * k
    conn = cut = 0
    for e, (src, dst) in enumerate(edges):
        parts = {int(rho[n]) for n in src | dst}
        lam = len(parts)
        conn += int(weights[e]) * (lam - 1)
        cut += int(weights[e]) if lam > 1 else 0
        for p in {int(rho[n]) for n in dst}:
            part_inb[p] += 1
    empty = sum(1 for c in count if c == 0)
    return conn, cut, part_size, part_inb, empty


def moves(n_nodes, edges, weights, sizes, rho, k, omega, enforce_omega):
    """Eq. 13 by sets: pins(p, e) counted over e's members, every partition
    tried, ties to the smallest partition id."""
    members = [set(s) | set(d) for s, d in edges]
    inc = [[e for e in range(len(edges)) if n in members[e]] for n in range(n_nodes)]
    psize = [0] * k
    for n in range(n_nodes):
        psize[rho[n]] += int(sizes[n])

    def pins(p, e):
        return sum(1 for m in members[e] if rho[m] == p)

    mv, gn = [], []
    for n in range(n_nodes):
        saving = sum(int(weights[e]) for e in inc[n] if pins(rho[n], e) == 1)
        best, bg = None, 0
        for p in range(k):
            if p == rho[n] or (enforce_omega and psize[p] + int(sizes[n]) > omega):
                continue
            loss = sum(int(weights[e]) for e in inc[n] if pins(p, e) == 0)
            if best is None or saving - loss > bg:
                best, bg = p, saving - loss
        mv.append(0xFFFFFFFF if best is None else best)
        gn.append(0 if best is None else bg)
    return mv, gn


def max_weight_matching(target, score):
    """Largest total weight of a matching made of proposal edges {n, target(n)}
    (weight score(n); a two-cycle is one edge), by enumerating edge subsets."""
    n = len(target)
    edges = {}
    for v in range(n):
        t = target[v]
        if t != 0xFFFFFFFF:
            edges[tuple(sorted((v, t)))] = int(score[v])
    el = list(edges.items())
    best = 0
    for mask in range(1 << len(el)):
        used, total, ok = set(), 0, True
        for i, ((a, b), w) in enumerate(el):
            if mask >> i & 1:
                if a in used or b in used:
                    ok = False
                    break
                used.add(a), used.add(b)
                total += w
        if ok and total > best:
            best = total
    return best, edges
