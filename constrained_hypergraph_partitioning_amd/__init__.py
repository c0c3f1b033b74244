"""Python binding of the gfx950 constrained hypergraph coarsening library.

Argument marshalling only: every step runs in the HIP kernels of
``libchp.so`` (C ABI declared in ``include/chp.h``).  PyTorch provides the
device memory (the library allocates through callbacks that create torch
tensors, so torch's caching allocator owns every buffer) and the stream (the
current torch stream when the context is created).

The library must be built first (``python -m
constrained_hypergraph_partitioning_amd._build`` or ``__graft_entry__.build()``);
importing this package never falls back to anything else.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libchp.so")

OK, EINVAL, ENOMEM, EOVERFLOW, EINFEASIBLE, ECYCLE, EDEVICE = 0, -1, -2, -3, -4, -5, -6
NONE = 0xFFFFFFFF
FX_SHIFT = 40
_NAMES = {EINVAL: "EINVAL", ENOMEM: "ENOMEM", EOVERFLOW: "EOVERFLOW",
          EINFEASIBLE: "EINFEASIBLE", ECYCLE: "ECYCLE", EDEVICE: "EDEVICE"}

EXPORTS = ["chp_create", "chp_destroy", "chp_last_error", "chp_build_incidence",
           "chp_rate_and_match", "chp_contract", "chp_evaluate_partition", "chp_hgraph_free",
           "chp_set_timing", "chp_get_timings", "chp_reset_timings", "chp_set_batch_entries",
           "chp_last_rate_stats", "chp_set_incidence_rating", "chp_pair_leftovers",
           "chp_propose_moves", "chp_set_matching", "chp_set_timing_filter",
           "chp_refine_moves", "chp_set_move_order", "chp_rate_top_and_match",
           "chp_evaluate_partition_noalloc", "chp_set_incidence_bins", "chp_project_partition",
           "chp_refine_level"]


class ChpError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("%s (%d): %s" % (_NAMES.get(code, "?"), code, msg))
        self.code = code


class Edges(ctypes.Structure):
    _fields_ = [("n_nodes", ctypes.c_uint32), ("n_edges", ctypes.c_uint32),
                ("n_pins", ctypes.c_uint64),
                ("e_off", ctypes.c_void_p), ("e_nsrc", ctypes.c_void_p),
                ("e_pins", ctypes.c_void_p), ("e_w", ctypes.c_void_p),
                ("n_size", ctypes.c_void_p)]


class HGraphC(ctypes.Structure):
    _fields_ = [("n_nodes", ctypes.c_uint32), ("n_edges", ctypes.c_uint32),
                ("n_pins", ctypes.c_uint64),
                ("e_off", ctypes.c_void_p), ("e_nsrc", ctypes.c_void_p),
                ("e_pins", ctypes.c_void_p), ("e_w", ctypes.c_void_p),
                ("n_size", ctypes.c_void_p),
                ("n_off", ctypes.c_void_p), ("n_nin", ctypes.c_void_p),
                ("n_inc", ctypes.c_void_p),
                ("nb_off", ctypes.c_void_p), ("nb", ctypes.c_void_p),
                ("nb_total", ctypes.c_uint64)]


class Params(ctypes.Structure):
    _fields_ = [("omega", ctypes.c_uint64), ("delta", ctypes.c_uint32),
                ("noise_on", ctypes.c_uint32), ("noise_seed", ctypes.c_uint64)]


class Timing(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("launches", ctypes.c_uint64),
                ("total_ms", ctypes.c_double)]


ALLOC_FN = ctypes.CFUNCTYPE(ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p)
FREE_FN = ctypes.CFUNCTYPE(None, ctypes.c_void_p, ctypes.c_void_p)

_lib = None


def load_library(path: str = LIB_PATH):
    """Load libchp.so and declare its signatures (no GPU needed)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError("libchp.so is not built (%s); run the build step first" % path)
    lib = ctypes.CDLL(path)
    P, I = ctypes.c_void_p, ctypes.c_int
    lib.chp_create.argtypes = [ctypes.POINTER(P), P, ALLOC_FN, FREE_FN, P]
    lib.chp_create.restype = I
    lib.chp_destroy.argtypes = [P]
    lib.chp_destroy.restype = None
    lib.chp_last_error.argtypes = [P]
    lib.chp_last_error.restype = ctypes.c_char_p
    lib.chp_build_incidence.argtypes = [P, ctypes.POINTER(Edges), ctypes.POINTER(Params), I,
                                        ctypes.POINTER(HGraphC)]
    lib.chp_build_incidence.restype = I
    lib.chp_rate_and_match.argtypes = [P, ctypes.POINTER(HGraphC), ctypes.POINTER(Params), P, P,
                                       P, ctypes.POINTER(ctypes.c_uint32), P]
    lib.chp_rate_and_match.restype = I
    lib.chp_rate_top_and_match.argtypes = [P, ctypes.POINTER(HGraphC), ctypes.POINTER(Params),
                                           ctypes.c_uint32, P, P, P,
                                           ctypes.POINTER(ctypes.c_uint32), P]
    lib.chp_rate_top_and_match.restype = I
    lib.chp_contract.argtypes = [P, ctypes.POINTER(HGraphC), P, P, I, ctypes.POINTER(HGraphC),
                                 P]
    lib.chp_contract.restype = I
    lib.chp_set_batch_entries.argtypes = [P, ctypes.c_uint64]
    lib.chp_set_batch_entries.restype = I
    lib.chp_last_rate_stats.argtypes = [P, ctypes.POINTER(ctypes.c_uint64),
                                        ctypes.POINTER(ctypes.c_uint32),
                                        ctypes.POINTER(ctypes.c_uint32)]
    lib.chp_last_rate_stats.restype = I
    lib.chp_set_timing_filter.argtypes = [P, ctypes.c_char_p]
    lib.chp_set_timing_filter.restype = I
    lib.chp_set_matching.argtypes = [P, I]
    lib.chp_set_matching.restype = I
    lib.chp_propose_moves.argtypes = [P, ctypes.POINTER(HGraphC), P, ctypes.c_uint32,
                                      ctypes.POINTER(Params), I, P, P]
    lib.chp_propose_moves.restype = I
    lib.chp_refine_moves.argtypes = [P, ctypes.POINTER(HGraphC), P, ctypes.c_uint32,
                                     ctypes.POINTER(Params), P, P, P, P, P,
                                     ctypes.POINTER(ctypes.c_uint32),
                                     ctypes.POINTER(ctypes.c_uint32),
                                     ctypes.POINTER(ctypes.c_int64)]
    lib.chp_refine_moves.restype = I
    lib.chp_set_move_order.argtypes = [P, I]
    lib.chp_set_move_order.restype = I
    lib.chp_pair_leftovers.argtypes = [P, ctypes.POINTER(HGraphC), ctypes.POINTER(Params), P, P,
                                       ctypes.POINTER(ctypes.c_uint32)]
    lib.chp_pair_leftovers.restype = I
    lib.chp_set_incidence_rating.argtypes = [P, ctypes.c_uint64, ctypes.c_uint32]
    lib.chp_set_incidence_rating.restype = I
    lib.chp_set_incidence_bins.argtypes = [P, I]
    lib.chp_set_incidence_bins.restype = I
    lib.chp_project_partition.argtypes = [P, ctypes.c_uint32, P, ctypes.c_uint32, P, P]
    lib.chp_project_partition.restype = I
    lib.chp_refine_level.argtypes = [P, ctypes.POINTER(HGraphC), P, ctypes.c_uint32,
                                     ctypes.POINTER(Params), ctypes.c_uint32,
                                     ctypes.POINTER(ctypes.c_uint32),
                                     ctypes.POINTER(ctypes.c_int64)]
    lib.chp_refine_level.restype = I
    lib.chp_evaluate_partition.argtypes = [P, ctypes.POINTER(HGraphC), P, ctypes.c_uint32,
                                           ctypes.POINTER(Params), P, P,
                                           ctypes.POINTER(ctypes.c_uint64)]
    lib.chp_evaluate_partition.restype = I
    lib.chp_evaluate_partition_noalloc.argtypes = lib.chp_evaluate_partition.argtypes
    lib.chp_evaluate_partition_noalloc.restype = I
    lib.chp_hgraph_free.argtypes = [P, ctypes.POINTER(HGraphC)]
    lib.chp_hgraph_free.restype = None
    lib.chp_set_timing.argtypes = [P, I]
    lib.chp_set_timing.restype = I
    lib.chp_get_timings.argtypes = [P, ctypes.POINTER(Timing), I]
    lib.chp_get_timings.restype = I
    lib.chp_reset_timings.argtypes = [P]
    lib.chp_reset_timings.restype = None
    _lib = lib
    return lib


def _ptr(t):
    return t.data_ptr() if t is not None and t.numel() else None


def to_device(a, device="cuda"):
    """numpy array -> torch tensor on the GPU with the same bytes
    (uint32 travels as int32, uint64 as int64)."""
    a = np.ascontiguousarray(a)
    m = {np.dtype(np.uint32): np.int32, np.dtype(np.uint64): np.int64}
    if a.dtype in m:
        a = a.view(m[a.dtype])
    return torch.from_numpy(a).to(device)


def to_host(t, dtype):
    """torch tensor -> numpy array reinterpreted as dtype."""
    return t.detach().cpu().numpy().view(dtype)


@dataclasses.dataclass
class Params_:
    omega: int
    delta: int
    noise_on: bool = True
    seed: int = 0

    def c(self):
        return Params(self.omega, self.delta, 1 if self.noise_on else 0, self.seed)


class HGraph:
    """A library-owned level (canonical edge CSR, incidence, neighbours)."""

    def __init__(self, ctx: "Context", g: HGraphC):
        self.ctx = ctx
        self.c = g

    @property
    def n_nodes(self):
        return int(self.c.n_nodes)

    @property
    def n_edges(self):
        return int(self.c.n_edges)

    @property
    def n_pins(self):
        return int(self.c.n_pins)

    @property
    def nb_total(self):
        return int(self.c.nb_total)

    _LEN = {"e_off": ("E1", torch.int64), "e_nsrc": ("E", torch.int32),
            "e_pins": ("P", torch.int32), "e_w": ("E", torch.int32),
            "n_size": ("N", torch.int32), "n_off": ("N1", torch.int64),
            "n_nin": ("N", torch.int32), "n_inc": ("P", torch.int32),
            "nb_off": ("N1", torch.int64), "nb": ("NB", torch.int32)}

    def tensor(self, name):
        """A torch view of one library-owned array (shares its memory)."""
        kind, dt = self._LEN[name]
        n = {"E1": self.n_edges + 1, "E": self.n_edges, "P": self.n_pins,
             "N": self.n_nodes, "N1": self.n_nodes + 1, "NB": self.nb_total}[kind]
        ptr = getattr(self.c, name)
        if ptr is None:
            return None
        return self.ctx._view(ptr, n, dt)

    def host(self, name):
        t = self.tensor(name)
        if t is None:
            return None
        np_dt = {torch.int64: np.int64, torch.int32: np.uint32}[t.dtype]
        return to_host(t, np_dt)

    def free(self):
        if self.ctx is not None and self.c is not None:
            self.ctx.lib.chp_hgraph_free(self.ctx.h, ctypes.byref(self.c))
            self.c = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


class Context:
    """One library context on a GPU and a torch stream.

    Every buffer the library needs is a torch uint8 tensor created by the
    allocation callback and kept in ``self._blocks`` until the library frees
    it."""

    def __init__(self, device: int = 0, stream: torch.cuda.Stream | None = None):
        if not torch.cuda.is_available():
            raise RuntimeError("no GPU visible: the HIP library needs one")
        self.lib = load_library()
        self.device = torch.device("cuda", device)
        torch.cuda.set_device(self.device)
        self.stream = stream if stream is not None else torch.cuda.current_stream(self.device)
        self._blocks = {}
        self.n_allocs = 0  # calls of the allocation callback so far

        def _alloc(nbytes, user):
            self.n_allocs += 1
            try:
                with torch.cuda.stream(self.stream):
                    t = torch.empty(int(nbytes), dtype=torch.uint8, device=self.device)
            except RuntimeError:
                return None
            p = t.data_ptr()
            self._blocks[p] = t
            return p

        def _free(ptr, user):
            self._blocks.pop(ptr, None)

        self._alloc_cb = ALLOC_FN(_alloc)
        self._free_cb = FREE_FN(_free)
        h = ctypes.c_void_p()
        rc = self.lib.chp_create(ctypes.byref(h), ctypes.c_void_p(self.stream.cuda_stream),
                                 self._alloc_cb, self._free_cb, None)
        if rc != OK:
            raise ChpError(rc, "chp_create")
        self.h = h

    def close(self):
        if getattr(self, "h", None):
            self.lib.chp_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _check(self, rc, what):
        if rc != OK:
            raise ChpError(rc, "%s: %s" % (what, self.lib.chp_last_error(self.h).decode()))

    def _view(self, ptr, n, dtype):
        """Typed view of n elements at ptr inside a library-owned block."""
        base = self._blocks.get(ptr)
        if base is None:
            raise KeyError("pointer not allocated by this context")
        itemsize = torch.empty(0, dtype=dtype).element_size()
        return base[: n * itemsize].view(dtype)

    # ---- entry points -------------------------------------------------------
    def build_incidence(self, e_off, e_nsrc, e_pins, e_w, n_size, omega, delta,
                        neighbors=True) -> HGraph:
        """Tensors on this context's device: e_off int64 [E+1], the others
        int32 carrying uint32 values."""
        E = int(e_w.shape[0])
        N = int(n_size.shape[0])
        P = int(e_pins.shape[0])
        ed = Edges(N, E, P, _ptr(e_off), _ptr(e_nsrc), _ptr(e_pins), _ptr(e_w), _ptr(n_size))
        prm = Params(omega, delta, 0, 0)
        g = HGraphC()
        self._check(self.lib.chp_build_incidence(self.h, ctypes.byref(ed), ctypes.byref(prm),
                                                 1 if neighbors else 0, ctypes.byref(g)),
                    "build_incidence")
        return HGraph(self, g)

    def rate_and_match(self, g: HGraph, omega, delta, noise_on=True, seed=0, out=None,
                       flags=None):
        """target, score, match, n_pairs; with flags (a uint8 tensor of
        g.nb_total entries) the invalid-neighbour flags are written too."""
        N = g.n_nodes
        if out is None:
            out = (torch.empty(N, dtype=torch.int32, device=self.device),
                   torch.empty(N, dtype=torch.int64, device=self.device),
                   torch.empty(N, dtype=torch.int32, device=self.device))
        target, score, match = out
        prm = Params(omega, delta, 1 if noise_on else 0, seed)
        npairs = ctypes.c_uint32()
        self._check(self.lib.chp_rate_and_match(self.h, ctypes.byref(g.c), ctypes.byref(prm),
                                                _ptr(target), _ptr(score), _ptr(match),
                                                ctypes.byref(npairs),
                                                _ptr(flags) if flags is not None else None),
                    "rate_and_match")
        return target, score, match, int(npairs.value)

    def rate_top_and_match(self, g: HGraph, pi, omega, delta, noise_on=True, seed=0, out=None,
                           flags=None):
        """target and score as (pi, N) tensors (row r: every node's (r+1)-th
        best valid neighbour), match after pi matching rounds, n_pairs."""
        N = g.n_nodes
        if out is None:
            out = (torch.empty((pi, N), dtype=torch.int32, device=self.device),
                   torch.empty((pi, N), dtype=torch.int64, device=self.device),
                   torch.empty(N, dtype=torch.int32, device=self.device))
        target, score, match = out
        if target.numel() < pi * N or score.numel() < pi * N or match.numel() < N:
            raise ValueError("target and score need pi * N entries, match N")
        prm = Params(omega, delta, 1 if noise_on else 0, seed)
        npairs = ctypes.c_uint32()
        self._check(self.lib.chp_rate_top_and_match(self.h, ctypes.byref(g.c), ctypes.byref(prm),
                                                    pi, _ptr(target), _ptr(score), _ptr(match),
                                                    ctypes.byref(npairs),
                                                    _ptr(flags) if flags is not None else None),
                    "rate_top_and_match")
        return target, score, match, int(npairs.value)

    def set_timing_filter(self, prefix=None):
        """Time only kernels whose name starts with prefix (None = all)."""
        self._check(self.lib.chp_set_timing_filter(self.h, prefix.encode() if prefix else None),
                    "set_timing_filter")

    def set_matching(self, optimal=False):
        """Matching of rate_and_match: the greedy handshake (default) or the
        exact maximum-weight matching of the proposal pseudo-forest."""
        self._check(self.lib.chp_set_matching(self.h, 1 if optimal else 0), "set_matching")

    def propose_moves(self, g: HGraph, rho, k, omega, enforce_omega=False):
        """Eq. 13 move proposal for partition rho: (move int32, gain int64)."""
        N = g.n_nodes
        move = torch.empty(max(N, 1), dtype=torch.int32, device=self.device)
        gain = torch.empty(max(N, 1), dtype=torch.int64, device=self.device)
        prm = Params(omega, 0, 0, 0)
        self._check(self.lib.chp_propose_moves(self.h, ctypes.byref(g.c), _ptr(rho), int(k),
                                               ctypes.byref(prm), 1 if enforce_omega else 0,
                                               _ptr(move), _ptr(gain)), "propose_moves")
        return move[:N], gain[:N]

    def set_move_order(self, chained=True):
        """Sequence moves as chains (the default) or by gain alone."""
        self._check(self.lib.chp_set_move_order(self.h, 0 if chained else 1), "set_move_order")

    def refine_moves(self, g: HGraph, rho, k, omega, delta, move, gain, details=False):
        """One refinement pass over the proposed moves (rho updated in place).
        Returns (moves in the sequence, prefix length applied, its gain), and
        with details also the device arrays (seq, seq_gain, seq_viol)."""
        N = g.n_nodes
        prm = Params(omega, delta, 0, 0)
        seq = sg = sv = None
        if details:
            seq = torch.empty(max(N, 1), dtype=torch.int32, device=self.device)
            sg = torch.empty(max(N, 1), dtype=torch.int64, device=self.device)
            sv = torch.empty(max(N, 1), dtype=torch.int32, device=self.device)
        m, na = ctypes.c_uint32(), ctypes.c_uint32()
        ga = ctypes.c_int64()
        self._check(self.lib.chp_refine_moves(self.h, ctypes.byref(g.c), _ptr(rho), int(k),
                                              ctypes.byref(prm), _ptr(move), _ptr(gain),
                                              _ptr(seq), _ptr(sg), _ptr(sv), ctypes.byref(m),
                                              ctypes.byref(na), ctypes.byref(ga)),
                    "refine_moves")
        M = int(m.value)
        out = (M, int(na.value), int(ga.value))
        if details:
            return out + (seq[:M], sg[:M], sv[:M])
        return out

    def refine_pass(self, g: HGraph, rho, k, omega, delta, enforce_omega=False, details=False):
        """Propose (Eq. 13) then sequence and apply: one pass of refinement."""
        move, gain = self.propose_moves(g, rho, k, omega, enforce_omega)
        return self.refine_moves(g, rho, k, omega, delta, move, gain, details)

    def pair_leftovers(self, g: HGraph, target, match, omega, delta):
        """Best-effort pairing of the unmatched nodes without a target (match
        updated in place); returns the number of new pairs."""
        prm = Params(omega, delta, 0, 0)
        npairs = ctypes.c_uint32()
        self._check(self.lib.chp_pair_leftovers(self.h, ctypes.byref(g.c), ctypes.byref(prm),
                                                _ptr(target), _ptr(match), ctypes.byref(npairs)),
                    "pair_leftovers")
        return int(npairs.value)

    def new_flags(self, g: HGraph):
        """A uint8 device tensor for g's invalid-neighbour flags."""
        return torch.empty(max(g.nb_total, 1), dtype=torch.uint8, device=self.device)

    def contract(self, g: HGraph, match, neighbors=True, gamma=None, flags=None):
        """gamma and the coarse graph; with flags (from rate_and_match on g)
        the coarse neighbourhoods are purged of flagged neighbours."""
        N = g.n_nodes
        if gamma is None:
            gamma = torch.empty(N, dtype=torch.int32, device=self.device)
        cg = HGraphC()
        self._check(self.lib.chp_contract(self.h, ctypes.byref(g.c), _ptr(match), _ptr(gamma),
                                          1 if neighbors else 0, ctypes.byref(cg),
                                          _ptr(flags) if flags is not None else None),
                    "contract")
        return gamma, HGraph(self, cg)

    def evaluate_partition(self, g: HGraph, rho, k, omega, delta):
        part_size = torch.empty(max(k, 1), dtype=torch.int64, device=self.device)
        part_inb = torch.empty(max(k, 1), dtype=torch.int32, device=self.device)
        summ = (ctypes.c_uint64 * 8)()
        prm = Params(omega, delta, 0, 0)
        self._check(self.lib.chp_evaluate_partition(self.h, ctypes.byref(g.c), _ptr(rho), k,
                                                    ctypes.byref(prm), _ptr(part_size),
                                                    _ptr(part_inb), summ), "evaluate_partition")
        return part_size[:k], part_inb[:k], np.array(list(summ), dtype=np.uint64)

    def evaluate_partition_noalloc(self, g: HGraph, rho, k, omega, delta, part_size, part_inb):
        """chp_evaluate_partition_noalloc: the evaluation into caller-owned
        part_size (int64, >= k) and part_inb (int32, >= k), with the
        library's fixed scratch (no device allocation); returns the summary."""
        summ = (ctypes.c_uint64 * 8)()
        prm = Params(omega, delta, 0, 0)
        self._check(self.lib.chp_evaluate_partition_noalloc(
            self.h, ctypes.byref(g.c), _ptr(rho), k, ctypes.byref(prm), _ptr(part_size),
            _ptr(part_inb), summ), "evaluate_partition_noalloc")
        return np.array(list(summ), dtype=np.uint64)

    def project_partition(self, gamma, rho_coarse, n_coarse):
        """rho of the finer level: rho_coarse[gamma[n]] (a new int32 tensor)."""
        n = int(gamma.numel())
        out = torch.empty(max(n, 1), dtype=torch.int32, device=self.device)
        self._check(self.lib.chp_project_partition(self.h, n, _ptr(gamma), n_coarse,
                                                   _ptr(rho_coarse), _ptr(out)),
                    "project_partition")
        return out[:n]

    def refine_level(self, g: HGraph, rho, k, omega, delta, theta=16):
        """theta refinement passes on g (rho updated in place): (moves
        applied, summed gain)."""
        na = ctypes.c_uint32()
        ga = ctypes.c_int64()
        prm = Params(omega, delta, 0, 0)
        self._check(self.lib.chp_refine_level(self.h, ctypes.byref(g.c), _ptr(rho), k,
                                              ctypes.byref(prm), theta, ctypes.byref(na),
                                              ctypes.byref(ga)), "refine_level")
        return int(na.value), int(ga.value)

    def set_batch_entries(self, entries=0):
        """Neighbour entries per rating batch for graphs without neighbours
        (0 = the library default)."""
        self._check(self.lib.chp_set_batch_entries(self.h, int(entries)), "set_batch_entries")

    def last_rate_stats(self):
        """(neighbour entries built batch by batch, batches, nodes rated
        straight from the incidence) of the last rate_and_match; all 0 when
        the graph carried its neighbourhoods."""
        n = ctypes.c_uint64()
        b = ctypes.c_uint32()
        f = ctypes.c_uint32()
        self._check(self.lib.chp_last_rate_stats(self.h, ctypes.byref(n), ctypes.byref(b),
                                                 ctypes.byref(f)), "last_rate_stats")
        return int(n.value), int(b.value), int(f.value)

    def set_incidence_bins(self, bits=32):
        """Bins of the rating from the incidence: 32 (quantised sums, exact
        eta for the neighbours in reach; the default) or 64 (exact eta)."""
        mode = {32: 0, 64: 1}[bits]
        self._check(self.lib.chp_set_incidence_bins(self.h, mode), "set_incidence_bins")

    def set_incidence_rating(self, min_visits=0, hash_keys=0):
        """Incident pins from which a node of a graph without neighbour lists
        is rated straight from the incidence (0 = default, 2**64-1 = never),
        and the keys a sparse window may claim (0 = its capacity)."""
        self._check(self.lib.chp_set_incidence_rating(self.h, int(min_visits), int(hash_keys)),
                    "set_incidence_rating")

    # ---- timing ---------------------------------------------------------------
    def set_timing(self, on=True):
        self._check(self.lib.chp_set_timing(self.h, 1 if on else 0), "set_timing")

    def timings(self):
        n = self.lib.chp_get_timings(self.h, None, 0)
        arr = (Timing * max(n, 1))()
        n = self.lib.chp_get_timings(self.h, arr, n)
        return {arr[i].name.decode(): (int(arr[i].launches), float(arr[i].total_ms))
                for i in range(n)}

    def reset_timings(self):
        self.lib.chp_reset_timings(self.h)


def upload_edges(h, device="cuda"):
    """Device tensors for an edge CSR held in numpy (e.g. a synth Hypergraph)."""
    return (to_device(h.e_off, device), to_device(h.e_nsrc, device), to_device(h.e_pins, device),
            to_device(h.e_w, device), to_device(h.n_size, device))
