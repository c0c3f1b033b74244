"""Seeded synthetic hypergraphs (inputs only; no partitioner arithmetic).

The five workload shapes stand in for the data sets of Ronzani & Silvano,
"Hypergraph Partitioning on GPU with Distinct Incident Hyperedges and Size
Constraints": SNN-style hypergraphs shaped like its Table I (one outbound
hyperedge per neuron, fan-outs of tens to thousands) and a VLSI-style netlist
shaped like its Table III (ISPD98-like pin counts).  The real data sets are not
used.  ``config(i)`` gives the full-size spec of workload ``i`` (1..5) and
``config(i, n_nodes=...)`` a structurally identical smaller one.

The C source (``synth.c``) draws every value from a counter-based generator,
so the arrays depend only on the spec and never on the thread count.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")

UNIFORM, RING, LAYERED, VLSI, BLOCK = 1, 2, 3, 4, 5


class _Spec(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32),
        ("n_nodes", ctypes.c_uint32),
        ("n_edges", ctypes.c_uint32),
        ("kmin", ctypes.c_uint32),
        ("kmax", ctypes.c_uint32),
        ("wmax", ctypes.c_uint32),
        ("smax", ctypes.c_uint32),
        ("window", ctypes.c_uint32),
        ("grid_w", ctypes.c_uint32),
        ("pad_", ctypes.c_uint32),
        ("lam", ctypes.c_double),
        ("sigma", ctypes.c_double),
        ("p_local", ctypes.c_double),
        ("seed", ctypes.c_uint64),
    ]


def build(force: bool = False) -> str:
    """Compile synth.c into libsynth.so (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        lib.synth_edge_sizes.argtypes = [ctypes.POINTER(_Spec), P]
        lib.synth_edge_sizes.restype = ctypes.c_int
        lib.synth_fill.argtypes = [ctypes.POINTER(_Spec), P, P, P, P, P]
        lib.synth_fill.restype = ctypes.c_int
        lib.synth_permutation.argtypes = [ctypes.c_uint64, ctypes.c_uint32, P]
        lib.synth_permutation.restype = None
        lib.synth_uniform_u32.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                          ctypes.c_uint32, P]
        lib.synth_uniform_u32.restype = None
        _lib = lib
    return _lib


@dataclasses.dataclass
class Spec:
    name: str
    kind: int
    n_nodes: int
    n_edges: int
    kmin: int
    kmax: int
    wmax: int
    smax: int
    omega: int
    delta: int
    seed: int
    window: int = 0
    grid_w: int = 0
    lam: float = 0.0
    sigma: float = 0.0
    p_local: float = 0.0
    target_nodes: int = 0      # coarsening stops below this node count (0 = one level)
    levels: int = 1            # level cap used by the driver for this workload

    def as_c(self) -> _Spec:
        return _Spec(self.kind, self.n_nodes, self.n_edges, self.kmin, self.kmax, self.wmax,
                     self.smax, self.window, self.grid_w, 0, self.lam, self.sigma,
                     self.p_local, self.seed)


@dataclasses.dataclass
class Hypergraph:
    """Edge CSR of a directed hypergraph (sources first in each segment)."""
    spec: Spec
    e_off: np.ndarray   # int64 [E+1]
    e_nsrc: np.ndarray  # uint32 [E]
    e_pins: np.ndarray  # uint32 [P]
    e_w: np.ndarray     # uint32 [E]
    n_size: np.ndarray  # uint32 [N]

    @property
    def n_nodes(self) -> int:
        return int(self.n_size.shape[0])

    @property
    def n_edges(self) -> int:
        return int(self.e_w.shape[0])

    @property
    def n_pins(self) -> int:
        return int(self.e_off[-1])


def config(i: int, n_nodes: int | None = None, seed: int | None = None) -> Spec:
    """Workload ``i`` (1..5).  ``n_nodes`` shrinks it keeping its structure."""
    if i == 1:
        N = n_nodes or 2000
        s = Spec("snn-uniform-2k", UNIFORM, N, N, 2, min(16, N - 1), 8, 1, 16, 64, 0)
        s.target_nodes, s.levels = 0, 1
    elif i == 2:
        N = n_nodes or 100_000
        s = Spec("snn-ring-100k", RING, N, N, 2, min(256, N - 1), 8, 1, 64, 1024, 1,
                 window=min(512, max(1, N // 4)), lam=32.0, p_local=0.8)
        s.target_nodes, s.levels = 10_000 if n_nodes is None else max(2, N // 10), 64
    elif i == 3:
        N = n_nodes or 1_000_000
        L = 10
        N = (N // L) * L
        per = N // L
        s = Spec("snn-layered-1m", LAYERED, N, N, 2, min(2048, per), 16, 1, 256, 4096, 2,
                 window=L, lam=64.0, sigma=0.6)
        s.target_nodes, s.levels = 10_000 if n_nodes is None else max(2, N // 100), 64
    elif i == 4:
        if n_nodes is None:
            W, H = 1600, 1250
        else:
            H = max(4, int(math.sqrt(n_nodes * 1250 / 1600)))
            W = max(4, n_nodes // H)
        N = W * H
        E = N * 11 // 10
        if n_nodes is None:
            sig, kmax = 50.0, 1000
        else:  # keep the largest net well inside its Gaussian neighbourhood
            sig = max(3.0, 50.0 * (N / 2_000_000) ** 0.25)
            kmax = max(4, min(1000, int(2 * sig * sig), N // 4))
        s = Spec("vlsi-grid-2m", VLSI, N, E, 2, kmax, 1, 4, 128, 512, 3,
                 grid_w=W, lam=2.5, sigma=sig)
        s.target_nodes, s.levels = 0, 64
    elif i == 5:
        N = n_nodes or 4_000_000
        B = 65536 if n_nodes is None else max(64, min(65536, N // 8))
        s = Spec("snn-block-4m", BLOCK, N, N, 2, min(4096, N - 1), 8, 1, 1024, 16384, 4,
                 window=B, lam=250.0 if n_nodes is None else min(250.0, B / 8), p_local=0.9)
        s.target_nodes, s.levels = 0, 1
    else:
        raise ValueError("workload index is 1..5")
    if n_nodes is not None:
        s.name += "-n%d" % s.n_nodes
    if seed is not None:
        s.seed = seed
    return s


def custom(kind: int, n_nodes: int, n_edges: int, kmin: int, kmax: int, wmax: int, smax: int,
           omega: int, delta: int, seed: int, **kw) -> Spec:
    """A free-form spec (used for constraint-stress inputs in tests)."""
    return Spec("custom-k%d-n%d-s%d" % (kind, n_nodes, seed), kind, n_nodes, n_edges, kmin, kmax,
                wmax, smax, omega, delta, seed, **kw)


def generate(spec: Spec) -> Hypergraph:
    lib = _load()
    cs = spec.as_c()
    E = spec.n_edges
    sizes = np.empty(E, dtype=np.uint32)
    if lib.synth_edge_sizes(ctypes.byref(cs), sizes.ctypes.data) != 0:
        raise RuntimeError("synth_edge_sizes failed")
    e_off = np.zeros(E + 1, dtype=np.int64)
    np.cumsum(sizes, out=e_off[1:])
    del sizes
    P = int(e_off[-1])
    e_pins = np.empty(P, dtype=np.uint32)
    e_nsrc = np.empty(E, dtype=np.uint32)
    e_w = np.empty(E, dtype=np.uint32)
    n_size = np.empty(spec.n_nodes, dtype=np.uint32)
    rc = lib.synth_fill(ctypes.byref(cs), e_off.ctypes.data, e_nsrc.ctypes.data,
                        e_pins.ctypes.data, e_w.ctypes.data, n_size.ctypes.data)
    if rc != 0:
        raise RuntimeError("synth_fill failed (%d)" % rc)
    return Hypergraph(spec, e_off, e_nsrc, e_pins, e_w, n_size)


def permutation(seed: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint32)
    _load().synth_permutation(seed, n, out.ctypes.data)
    return out


def uniform_u32(seed: int, stream: int, n: int, bound: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint32)
    _load().synth_uniform_u32(seed, stream, n, bound, out.ctypes.data)
    return out


def fixed_partition(n_nodes: int, k: int, seed: int = 0) -> np.ndarray:
    """rho(n) = pi(n) mod k for a seeded permutation pi: every part holds
    floor or ceil of n/k nodes, none is empty when k <= n."""
    return (permutation(seed, n_nodes) % np.uint32(k)).astype(np.uint32)


def from_lists(n_nodes: int, edges, weights=None, sizes=None, name="explicit",
               omega=1 << 30, delta=1 << 30) -> Hypergraph:
    """Build an edge CSR from explicit (src_list, dst_list) pairs, unsorted allowed."""
    offs = [0]
    pins, nsrc = [], []
    for src, dst in edges:
        pins.extend(src)
        pins.extend(dst)
        nsrc.append(len(src))
        offs.append(len(pins))
    E = len(edges)
    spec = Spec(name, 0, n_nodes, E, 0, 0, 0, 0, omega, delta, 0)
    w = np.asarray(weights if weights is not None else [1] * E, dtype=np.uint32)
    s = np.asarray(sizes if sizes is not None else [1] * n_nodes, dtype=np.uint32)
    return Hypergraph(spec, np.asarray(offs, dtype=np.int64), np.asarray(nsrc, dtype=np.uint32),
                      np.asarray(pins, dtype=np.uint32), w, s)


def tiny(seed: int, n_nodes: int, n_edges: int, max_src: int = 2, max_dst: int = 4,
         max_w: int = 5, max_size: int = 1, omega: int = 1 << 30, delta: int = 1 << 30,
         name: str = "tiny") -> Hypergraph:
    """A small random hypergraph for brute-force comparisons (PCG64 seeded).
    Each edge draws 0..max_src sources and 1..max_dst destinations, disjoint."""
    rng = np.random.Generator(np.random.PCG64(seed))
    edges = []
    for _ in range(n_edges):
        k = int(rng.integers(1, max_dst + 1))
        s = int(rng.integers(0, max_src + 1))
        k = min(k, n_nodes)
        s = min(s, n_nodes - k)
        pick = rng.permutation(n_nodes)[: k + s]
        src = [int(x) for x in pick[:s]]
        dst = [int(x) for x in pick[s:]]
        rng.shuffle(src)
        rng.shuffle(dst)
        edges.append((src, dst))
    w = rng.integers(1, max_w + 1, size=n_edges).tolist()
    sz = rng.integers(1, max_size + 1, size=n_nodes).tolist()
    return from_lists(n_nodes, edges, w, sz, name="%s-s%d" % (name, seed), omega=omega,
                      delta=delta)
