// Candidate proposal and handshake matching of one coarsening level.
//
// Rating: "Hypergraph Partitioning on GPU with Distinct Incident Hyperedges
// and Size Constraints", Sec. V-A (Eqs. 5-6) and Sec. V-C (inline inter(n,m)
// counter, symmetric noise).  eta is held in fixed point with 40 fractional
// bits, one rounded-down term per hyperedge, so every sum is exact and
// eta(n,m) = eta(m,n) bit for bit; the best valid candidate is the argmax of
// (eta, -id) over neighbours that pass both limits, which equals taking
// candidates in (eta desc, id asc) order and stopping at the first valid one.
//
// Matching: the greedy handshake of "Incidence Constraints in Hypergraph
// Partitioning on GPU", Sec. III-A and III-B3.
#include "dev.h"
#include "kernels.h"

namespace {

// ---------------------------------------------------------------------------
// per-hyperedge term t(e) = floor(w(e) * 2^40 / |e|) and 128-bit partial sums
constexpr int TB = 256;

__global__ __launch_bounds__(TB) void k_terms(u32 E, const i64 *e_off, const u32 *e_w, u64 *t,
                                              u64 *partials) {
  __shared__ u64 lo_s[TB], hi_s[TB];
  u32 e = blockIdx.x * TB + threadIdx.x;
  u64 v = 0;
  if (e < E) {
    u64 sz = (u64)(e_off[e + 1] - e_off[e]);
    v = ((u64)e_w[e] << FX_SHIFT) / sz;
    t[e] = v;
  }
  lo_s[threadIdx.x] = v;
  hi_s[threadIdx.x] = 0;
  __syncthreads();
  for (int s = TB / 2; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) {
      u64 a = lo_s[threadIdx.x], b = lo_s[threadIdx.x + s];
      u64 r = a + b;
      hi_s[threadIdx.x] += hi_s[threadIdx.x + s] + (r < a ? 1 : 0);
      lo_s[threadIdx.x] = r;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    partials[2 * blockIdx.x] = lo_s[0];
    partials[2 * blockIdx.x + 1] = hi_s[0];
  }
}

// cap = floor(sum t / (10 |E|)), d = cap + 1, magic = floor((2^64-1)/d).
// One workgroup adds the 128-bit partial sums, thread 0 divides.
__global__ __launch_bounds__(TB) void k_cap(u32 nparts, const u64 *partials, u32 E,
                                            u64 *capinfo) {
  __shared__ u64 lo_s[TB], hi_s[TB];
  u64 lo = 0, hi = 0;
  for (u32 i = threadIdx.x; i < nparts; i += TB) {
    const u64 r = lo + partials[2 * i];
    hi += partials[2 * i + 1] + (r < lo ? 1 : 0);
    lo = r;
  }
  lo_s[threadIdx.x] = lo;
  hi_s[threadIdx.x] = hi;
  __syncthreads();
  for (int st = TB / 2; st > 0; st >>= 1) {
    if ((int)threadIdx.x < st) {
      const u64 a = lo_s[threadIdx.x], b = lo_s[threadIdx.x + st];
      const u64 r = a + b;
      hi_s[threadIdx.x] += hi_s[threadIdx.x + st] + (r < a ? 1 : 0);
      lo_s[threadIdx.x] = r;
    }
    __syncthreads();
  }
  if (threadIdx.x != 0) return;
  lo = lo_s[0];
  hi = hi_s[0];
  u64 cap = 0;
  if (E) {
    const u64 dv = 10ull * E;
    u64 rem = 0, q = 0;
    for (int bit = 127; bit >= 0; --bit) {
      const u64 b = bit >= 64 ? (hi >> (bit - 64)) & 1 : (lo >> bit) & 1;
      rem = (rem << 1) | b;
      u64 qb = 0;
      if (rem >= dv) {
        rem -= dv;
        qb = 1;
      }
      if (bit < 64) q |= qb << bit;
    }
    cap = q;
  }
  capinfo[0] = cap;
  capinfo[1] = cap + 1;
  capinfo[2] = cap + 1 >= 2 ? (~0ull) / (cap + 1) : 0;
  capinfo[3] = 0;
}

// ---------------------------------------------------------------------------
// rating
// Nodes by |N(n)| and |I(n)|: light (|N(n)| <= small_cap and at most one
// chunk of light_ech hyperedges, so that a wave's pin visits stay short) are
// queued by id in list[0]; the others with their record: heavy (<= heavy_cap,
// at most big_ech hyperedges: more pins are visited faster by the 1024
// threads of the large-table kernel) in recs[]
// from the front; huge (above big_cap, at most heavy_ech hyperedges) in
// recs[] from the back; big (the rest) in big[].  A huge node takes several
// windows of either table; with one chunk of hyperedges a window costs the
// small table little, and four of its workgroups share a CU.  A node without
// neighbours gets no candidate here.
// (nodes lo .. hi - 1; recs must hold hi - lo records)
__global__ __launch_bounds__(256) void k_rate_classify(RateArgs A, u32 lo, u32 hi, NbLists nl,
                                                       NodeRec *recs, NodeRec *big,
                                                       u32 small_cap, u32 heavy_cap, u32 big_cap,
                                                       u32 heavy_ech, u32 light_ech,
                                                       u32 big_ech) {
  __shared__ u32 s_app[4 * (256 / WAVE) + 4];
  const u32 n = lo + blockIdx.x * blockDim.x + threadIdx.x;
  u64 K = 0, deg = 0;
  if (n < hi) {
    K = (u64)(A.nb_off[n + 1] - A.nb_off[n]);
    deg = (u64)(A.n_off[n + 1] - A.n_off[n]);
    if (K == 0) {
      for (u32 r = 0; r < A.pi; ++r) {
        A.target[(u64)r * A.N + n] = NONE32;
        A.score[(u64)r * A.N + n] = 0;
      }
    }
  }
  const int c = (n >= hi || K == 0)               ? 4
                : K <= small_cap && deg <= light_ech  ? 0
                : K <= heavy_cap && deg <= big_ech    ? 1
                : K > big_cap && deg <= heavy_ech     ? 3
                                                      : 2;
  const u32 slot = block_append<256, 4>(nl.cnt, c, s_app);
  if (c == 0) nl.list[0][slot] = n;
  if (c >= 1 && c <= 3) {
    NodeRec r;
    r.n = n;
    r.K = (u32)K;
    r.nin = A.n_nin[n];
    r.size = A.n_size[n];
    r.i0 = A.n_off[n];
    r.deg = (u32)deg;
    r.nb0 = A.nb_off[n];
    r.pad0 = r.pad1 = r.pad2 = 0;
    if (c == 1) recs[slot] = r;
    else if (c == 2) big[slot] = r;
    else recs[hi - lo - 1 - slot] = r;
  }
}

template <int BLOCK>
__device__ __forceinline__ u64 wg_sat_sum(u64 v, u64 *lds) {
  constexpr int NW = BLOCK / WAVE;
#pragma unroll
  for (int d = WAVE / 2; d > 0; d >>= 1) v = sat_add(v, __shfl_xor(v, d, WAVE));
  if (NW == 1) return v;
  if (lane_id() == 0) lds[wave_id()] = v;
  __syncthreads();
  u64 t = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) t = sat_add(t, lds[w]);
  __syncthreads();
  return t;
}

// ---------------------------------------------------------------------------
// Rating: two launches per level.  A node with at most RATE_SMALL_CAP
// neighbours ("light") takes one wave; a larger one a workgroup, either of
// 256 threads with a 2048-slot table, four to a CU ("Heavy"), or, for nodes
// whose neighbourhood would need several windows of that table, of 1024
// threads with an 8192-slot table that fills most of the CU's LDS ("Big").
// Every node is pulled from a work counter.
//
// Per node the neighbour list N(n) is loaded, a window of at most CAP ids at a
// time, into an LDS hash table whose slots are the bins of m in N(n):
//   eta  u64  eta(n,m) in fixed point; bit 63 set when size(n)+size(m) > Omega
//             (free: a node whose terms plus the noise cap reach 2^63 is an
//             overflow error anyway),
//   rem  u32  |in(m)| - inter(n,m) = |in(m) \ in(n)|, so the inbound limit is
//             |in(n)| + rem <= Delta.
// Both limits are read together with the ids, so judging a candidate needs
// no further memory access.  A node's header comes from a 48-byte record the
// classification writes; its first window's ids and its first hyperedges'
// incidence entries are loaded together, then their sizes, inbound counts and
// descriptors, so that the opening costs two memory round trips.  The ids of
// a window are inserted with all home-slot compare-and-swaps issued at once.
//
// Incident hyperedges are taken a chunk at a time; each brings a source run
// and a destination run of its pin list (for a windowed node, the stretch of
// each run inside the window, see rate_heavy).  A scan lays the runs end to
// end and every thread loads up to IMAX consecutive pins, then reads their
// home slots and their runs' terms (the destination run of an inbound
// hyperedge carries a flag in its term), then adds t(e) to the bin of each
// pin m != n and, for a flagged run, takes one from rem.  The candidate scan
// keeps, per thread, the best valid bin by (eta desc, id asc), skipping a bin
// whose upper bound eta + cap cannot beat the largest raw eta of a valid bin
// before its noise is computed; it empties each slot it reads, so the table
// is clean for the next window or node.
// A heavy-path shape: B threads per node, T hash slots (T = 2^(32-SHIFT)),
// at most CAP neighbours per window (load 0.75), ECH hyperedges per chunk.
template <int B_, u32 T_, u32 SHIFT_, u32 CAP_, int ECH_>
struct HCfg {
  static constexpr int B = B_, W = B_ / WAVE, ECH = ECH_;
  static constexpr u32 T = T_, SHIFT = SHIFT_, CAP = CAP_, UNR = CAP_ / B_;
  static_assert(CAP_ % B_ == 0 && (1ull << (32 - SHIFT_)) == T_ && CAP_ * 4 <= T_ * 3, "shape");
};
// four workgroups of 256 per CU, a node of at most 1536 neighbours each
using Heavy = HCfg<256, 2048, 21, 1536, 128>;
// one workgroup of 1024 per CU (the table takes most of the LDS), windows of
// 6144 neighbours: for the nodes that would need several windows above
using Big = HCfg<1024, 8192, 19, 6144, 512>;
constexpr int RB = Heavy::B;
constexpr int RW = Heavy::W;
constexpr u32 L_T = 512, L_SHIFT = 23;   // hash slots per wave, light path
constexpr int L_ECH = 32;
constexpr u32 IMAX = 8;  // pins per thread per round, at most
constexpr u32 L_UNR = RATE_SMALL_CAP / WAVE;  // window ids per lane, light path
constexpr u32 EMPTY = 0xFFFFFFFFu;
constexpr u64 INB = 1ull << 63;  // term flag: destination run of an inbound hyperedge
constexpr u64 BAD = 1ull << 63;  // bin flag: the pair breaks Omega
static_assert(RATE_SMALL_CAP <= L_T * 3 / 4, "light window must fit its table");

template <class C>
struct HeavySmem {
  u64 eta[C::T];
  u32 key[C::T];
  u32 rem[C::T];
  u64 rs[2 * C::ECH];
  u64 rt[2 * C::ECH];
  u32 pre[2 * C::ECH + 1];
  u32 red32[C::W + 1];
  u64 red64[C::W + 1];
  u64 rede[C::W + 1];
  u32 redi[C::W + 1];
};
struct LightWave {
  u64 eta[L_T];
  u32 key[L_T];
  u32 rem[L_T];
  u64 rs[2 * L_ECH];
  u64 rt[2 * L_ECH];
  u32 pre[2 * L_ECH + 1];
};
union RateSmem {
  HeavySmem<Heavy> h;
  LightWave l[RW];
};

__device__ __forceinline__ u32 hslot(u32 m, u32 shift) { return (m * 0x9E3779B1u) >> shift; }

// Insert the ids m[0, UNR) (EMPTY = none; all distinct and absent) with
// their limit data: every id first tries its home slot (the compare-and-swaps
// are issued together), then the ones that collided probe on.
template <u32 UNR>
__device__ __forceinline__ void insert_bins(u32 *key, u64 *eta, u32 *rem, u32 mask, u32 shift,
                                            const u32 *m, const bool *bad, const u32 *ni) {
  u32 s[UNR], got[UNR];
#pragma unroll
  for (u32 k = 0; k < UNR; ++k) {
    s[k] = hslot(m[k], shift);
    got[k] = m[k] != EMPTY ? atomicCAS(&key[s[k]], EMPTY, m[k]) : EMPTY;
  }
#pragma unroll
  for (u32 k = 0; k < UNR; ++k) {
    if (m[k] == EMPTY) continue;
    if (got[k] != EMPTY) {
      u32 q = (s[k] + 1) & mask;
      for (u32 p = 0; p < mask; ++p) {
        if (atomicCAS(&key[q], EMPTY, m[k]) == EMPTY) break;
        q = (q + 1) & mask;
      }
      s[k] = q;
    }
    eta[s[k]] = bad[k] ? BAD : 0;
    rem[s[k]] = ni[k];
  }
}

__device__ __forceinline__ u32 h_find(const u32 *key, u32 mask, u32 shift, u32 m) {
  u32 s = hslot(m, shift);
  u32 k = key[s];
  u32 p = 0;
#pragma unroll 1
  while (k != m && k != EMPTY && p < mask) {
    s = (s + 1) & mask;
    k = key[s];
    ++p;
  }
  return k == m ? s : EMPTY;
}

// Walk the pins of runs [0, nruns) (flat length tot), LANES threads, t = this
// thread's index among them.  The pins are dealt in rounds of up to IMAX
// consecutive pins per thread, as few per thread as lets one round cover
// them all, so that no lane is left with a second round (and a second
// memory round trip) that the others would wait for at the next barrier.
// Each thread first issues the loads of its pins, then updates their bins.
template <u32 LANES>
__device__ __forceinline__ void visit_runs(const u32 *__restrict__ pins,
                                           const u32 *__restrict__ key, u32 mask, u32 shift,
                                           u64 *__restrict__ eta, u32 *__restrict__ rem,
                                           const u64 *__restrict__ rs, const u64 *__restrict__ rt,
                                           const u32 *__restrict__ pre, u32 nruns, u32 tot, u32 n,
                                           u32 t) {
  const u32 need = (tot + LANES - 1) / LANES;
  const u32 per = need < IMAX ? need : IMAX;
  for (u32 base = t * per; base < tot; base += LANES * per) {
    // the run of the first pin, its end and the pin index of flat index 0
    // in it are kept in registers; LDS is read again only at a run boundary
    u32 r = run_of(pre, nruns + 1, base);
    u32 end = pre[r + 1];
    i64 org = (i64)rs[r] - (i64)pre[r];
    u32 m[IMAX];
    u32 rr[IMAX];
#pragma unroll
    for (u32 k = 0; k < IMAX; ++k) {
      const u32 idx = base + k;
      m[k] = n;  // n marks "no pin": it is skipped below
      rr[k] = r;
      if (k < per && idx < tot) {
        while (idx >= end) {
          ++r;
          end = pre[r + 1];
          org = (i64)rs[r] - (i64)pre[r];
        }
        rr[k] = r;
        m[k] = pins[org + idx];
      }
    }
    // without branches, every pin's home slot and its run's term (with the
    // inbound flag) are read together; a pin not at its home slot probes on
    u32 sl[IMAX], kk[IMAX];
    u64 tf[IMAX];
#pragma unroll
    for (u32 k = 0; k < IMAX; ++k) {
      sl[k] = hslot(m[k], shift);
      kk[k] = key[sl[k]];
      tf[k] = rt[rr[k]];
    }
#pragma unroll
    for (u32 k = 0; k < IMAX; ++k)
      if (kk[k] != m[k] && m[k] != n) sl[k] = h_find(key, mask, shift, m[k]);
#pragma unroll
    for (u32 k = 0; k < IMAX; ++k) {
      if (m[k] == n || sl[k] == EMPTY) continue;  // EMPTY cannot happen for a valid N(n)
      atomicAdd(&eta[sl[k]], tf[k] & ~INB);
      if (tf[k] & INB) atomicSub(&rem[sl[k]], 1u);
    }
  }
}

// Insert the window nb[0, cw) into the table: UNR neighbour ids are loaded,
// then their sizes and inbound counts, then the slots are claimed.
template <u32 LANES>
__device__ __forceinline__ void insert_window(const RateArgs &A, const u32 *nb, u32 cw, u64 size_n,
                                              u32 *key, u64 *eta, u32 *rem, u32 mask, u32 shift,
                                              u32 t) {
  constexpr u32 UNR = 4;
  for (u32 b0 = t; b0 < cw; b0 += LANES * UNR) {
    u32 m[UNR], sz[UNR], ni[UNR];
#pragma unroll
    for (u32 k = 0; k < UNR; ++k) {
      const u32 i = b0 + k * LANES;
      m[k] = i < cw ? nb[i] : EMPTY;
    }
#pragma unroll
    for (u32 k = 0; k < UNR; ++k) {  // branch-free: an absent id reads entry 0
      const u32 mk = m[k] != EMPTY ? m[k] : 0;
      sz[k] = A.n_size[mk];
      ni[k] = A.n_nin[mk];
    }
    bool bad[UNR];
#pragma unroll
    for (u32 k = 0; k < UNR; ++k) bad[k] = size_n + sz[k] > A.omega;
    insert_bins<UNR>(key, eta, rem, mask, shift, m, bad, ni);
  }
}

// r1 = first index in a[lo1, hi1) with a[i] > v, r2 likewise in [lo2, hi2):
// two binary searches in lockstep, so that each step costs one memory round
// trip for both (a finished search reads a[0], which always exists).
__device__ __forceinline__ void upper_bound2(const u32 *a, i64 lo1, i64 hi1, i64 lo2, i64 hi2,
                                             u32 v, i64 &r1, i64 &r2) {
  while (lo1 < hi1 || lo2 < hi2) {
    const i64 m1 = lo1 + ((hi1 - lo1) >> 1), m2 = lo2 + ((hi2 - lo2) >> 1);
    const u32 x1 = a[lo1 < hi1 ? m1 : 0];
    const u32 x2 = a[lo2 < hi2 ? m2 : 0];
    if (lo1 < hi1) {
      if (x1 <= v) lo1 = m1 + 1;
      else hi1 = m1;
    }
    if (lo2 < hi2) {
      if (x2 <= v) lo2 = m2 + 1;
      else hi2 = m2;
    }
  }
  r1 = lo1;
  r2 = lo2;
}

struct EdgeDesc {
  i64 a, b, dm;
  u64 te;
};

__device__ __forceinline__ EdgeDesc load_edge(const RateArgs &A, i64 j) {
  const u32 e = A.n_inc[j];
  EdgeDesc d;
  d.a = A.e_off[e];
  d.b = A.e_off[e + 1];
  d.dm = d.a + A.e_nsrc[e];
  d.te = A.t[e];
  return d;
}

__device__ __forceinline__ bool bin_valid(const RateArgs &A, u32 nin, u64 v, u32 rem) {
  return !(v & BAD) && (u64)nin + rem <= (u64)A.delta;
}

// Invalid-neighbour flags of a window ([HP] Sec. V-C): entry i of the
// window nb[w0, w0 + cw) gets 1 when its bin breaks a limit.  Reads the bins
// only; it must follow the window's last visit and precede the candidate
// scan, whose barrier orders it before the bins are emptied.
template <u32 LANES, u32 UNR>
__device__ __forceinline__ void flag_window(const RateArgs &A, const u32 *key, const u64 *eta,
                                            const u32 *rem, u32 mask, u32 shift, i64 w0, u32 cw,
                                            u32 nin, u32 t) {
  for (u32 b0 = 0; b0 < cw; b0 += LANES * UNR) {
    u32 m[UNR];
#pragma unroll
    for (u32 k = 0; k < UNR; ++k) {  // branch-free: past the end reads the last id
      const u32 i = b0 + t + k * LANES;
      m[k] = A.nb[w0 + (i < cw ? i : cw - 1)];
    }
#pragma unroll
    for (u32 k = 0; k < UNR; ++k) {
      const u32 i = b0 + t + k * LANES;
      if (i >= cw) continue;
      const u32 sl = h_find(key, mask, shift, m[k]);
      A.flag[w0 + i] = (sl != EMPTY && bin_valid(A, nin, eta[sl], rem[sl])) ? 0 : 1;
    }
  }
}

// A valid bin can win only if eta + cap reaches floor, the largest raw eta
// of a valid bin (that bin's total is at least floor); the others are
// skipped before their noise is computed.
// With MP > 1 the floor is 0 and only the thread's own list prunes.
template <int MP>
__device__ __forceinline__ void consider(const RateArgs &A, u32 n, u32 nin, u32 m, u64 v, u32 rem,
                                         u64 ub_add, u64 floor, u64 dmod, u64 magic,
                                         TopList<MP> &b) {
  if (!bin_valid(A, nin, v, rem) || v + ub_add < floor) return;
  if (!b.admits(v + ub_add, m)) return;
  const u64 tv = A.noise_on ? v + pair_noise(A.seed, n, m, dmod, magic) : v;
  if (b.admits(tv, m)) b.insert(tv, m);
}

template <int BLOCK>
__device__ __forceinline__ u64 wg_max_u64(u64 v, u64 *lds) {
  constexpr int NW = BLOCK / WAVE;
#pragma unroll
  for (int d = WAVE / 2; d > 0; d >>= 1) {
    const u64 o = __shfl_xor(v, d, WAVE);
    v = o > v ? o : v;
  }
  if (NW == 1) return v;
  if (lane_id() == 0) lds[wave_id()] = v;
  __syncthreads();
  u64 m = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) m = lds[w] > m ? lds[w] : m;
  __syncthreads();
  return m;
}


// The opening of a heavy node, loaded in two stages so that each costs one
// memory round trip: this thread's incidence entry of the first chunk and its
// share of the first window's ids, then that hyperedge's descriptor and the
// ids' sizes and inbound counts.
template <class C>
__device__ __forceinline__ void open_node(const RateArgs &A, const NodeRec &h, u32 t,
                                          EdgeDesc &d0, u32 *m, u32 *sz, u32 *ni) {
  const u32 ne0 = h.deg < (u32)C::ECH ? h.deg : (u32)C::ECH;
  const u32 cw = h.K < C::CAP ? h.K : C::CAP;
  const u32 e0 = t < ne0 ? A.n_inc[h.i0 + t] : EMPTY;
#pragma unroll
  for (u32 k = 0; k < C::UNR; ++k) {
    const u32 i = t + k * C::B;
    m[k] = i < cw ? A.nb[h.nb0 + i] : EMPTY;
  }
  // second stage without branches (an absent item reads entry 0), so that
  // every load is issued before the first is waited for
  const u32 e = e0 != EMPTY ? e0 : 0;
  d0.a = A.e_off[e];
  d0.b = A.e_off[e + 1];
  d0.dm = d0.a + A.e_nsrc[e];
  d0.te = A.t[e];
#pragma unroll
  for (u32 k = 0; k < C::UNR; ++k) {
    const u32 mk = m[k] != EMPTY ? m[k] : 0;
    sz[k] = A.n_size[mk];
    ni[k] = A.n_nin[mk];
  }
}

template <class C, int MP>
__device__ void rate_heavy(const RateArgs &A, HeavySmem<C> &S, const NodeRec &h, u64 cap, u64 dmod,
                           u64 magic) {
  const u32 tid = threadIdx.x;
  const u32 n = h.n, K = h.K, nin = h.nin;
  const i64 nb0 = h.nb0, i0 = h.i0, i1 = h.i0 + h.deg;
  const u64 size_n = h.size;
  const u64 ub_add = A.noise_on ? cap : 0;
  TopList<MP> best;
  best.clear();
  u64 tsum = 0;
  EdgeDesc d0;
  {
    u32 m[C::UNR], sz[C::UNR], ni[C::UNR];
    open_node<C>(A, h, tid, d0, m, sz, ni);
    bool bad[C::UNR];
#pragma unroll
    for (u32 k = 0; k < C::UNR; ++k) bad[k] = size_n + sz[k] > A.omega;
    insert_bins<C::UNR>(S.key, S.eta, S.rem, C::T - 1, C::SHIFT, m, bad, ni);
  }
  // Windows cover N(n) in id order.  The pins of a sorted run that fall in
  // window w form the stretch from where window w-1 stopped (its cursor)
  // to the first pin above the window's last id; between two windows lies
  // no neighbour, only n itself, which the visit skips.  So a window needs
  // one upper-bound search per run (none for the last window), started at
  // the cursor.  Cursors of a node whose hyperedges fit one chunk stay in
  // registers; otherwise they are kept per incidence entry in A.cur (as the
  // number of pins left in the run).
  const bool one_chunk = h.deg <= (u32)C::ECH;
  i64 cs0 = 0, cd0 = 0;
  for (u32 s0 = 0; s0 < K; s0 += C::CAP) {
    const u32 cw = (K - s0) < C::CAP ? (K - s0) : C::CAP;
    const bool last = s0 + C::CAP >= K;
    if (s0 > 0)
      insert_window<C::B>(A, A.nb + nb0 + s0, cw, size_n, S.key, S.eta, S.rem, C::T - 1, C::SHIFT,
                        tid);
    const u32 hi = A.nb[nb0 + s0 + cw - 1];
    __syncthreads();
    for (i64 c0 = i0; c0 < i1; c0 += C::ECH) {
      const u32 ne = (u32)((i1 - c0) < C::ECH ? (i1 - c0) : C::ECH);
      u32 ls = 0, ld = 0;
      if (tid < ne) {
        const EdgeDesc d = c0 == i0 ? d0 : load_edge(A, c0 + tid);
        if (s0 == 0 && d.b - d.a >= 2) tsum = sat_add(tsum, d.te);
        const i64 j = c0 + tid;
        i64 sa = d.a, da = d.dm;
        if (s0 > 0) {
          if (one_chunk) {
            sa = cs0;
            da = cd0;
          } else {
            sa = d.dm - A.cur[2 * j];
            da = d.b - A.cur[2 * j + 1];
          }
        }
        i64 sb = d.dm, db = d.b;
        if (!last) {
          upper_bound2(A.e_pins, sa, d.dm, da, d.b, hi, sb, db);
          if (one_chunk) {
            cs0 = sb;
            cd0 = db;
          } else {
            A.cur[2 * j] = (u32)(d.dm - sb);
            A.cur[2 * j + 1] = (u32)(d.b - db);
          }
        }
        S.rs[2 * tid] = (u64)sa;
        S.rs[2 * tid + 1] = (u64)da;
        S.rt[2 * tid] = d.te;
        S.rt[2 * tid + 1] = d.te | ((u64)(j - i0) < (u64)nin ? INB : 0);
        ls = (u32)(sb - sa);
        ld = (u32)(db - da);
      }
      u32 tot;
      const u32 off = wg_excl_scan<C::B>(ls + ld, S.red32, &tot);
      if (tid < ne) {
        S.pre[2 * tid] = off;
        S.pre[2 * tid + 1] = off + ls;
      }
      if (tid == 0) S.pre[2 * ne] = tot;
      __syncthreads();
      visit_runs<C::B>(A.e_pins, S.key, C::T - 1, C::SHIFT, S.eta, S.rem, S.rs, S.rt, S.pre, 2 * ne,
                     tot, n, tid);
      __syncthreads();
    }
    if (A.flag) {
      flag_window<C::B, C::UNR>(A, S.key, S.eta, S.rem, C::T - 1, C::SHIFT, nb0 + s0, cw, nin,
                                tid);
      // without the floor's reduction, a barrier orders the flag reads
      // before the candidate scan empties the slots
      if (MP > 1) __syncthreads();
    }
    u64 floor = 0;
    if (MP == 1) {
      for (u32 i = tid; i < C::T; i += C::B) {
        const u64 v = S.eta[i];
        if (S.key[i] != EMPTY && bin_valid(A, nin, v, S.rem[i]) && v > floor) floor = v;
      }
      floor = wg_max_u64<C::B>(floor, S.red64);
    }
    for (u32 i = tid; i < C::T; i += C::B) {
      const u32 m = S.key[i];
      if (m != EMPTY) {
        consider(A, n, nin, m, S.eta[i], S.rem[i], ub_add, floor, dmod, magic, best);
        S.key[i] = EMPTY;
        S.eta[i] = 0;
      }
    }
    // after the last window the reduction's barrier orders these clears
    // before the next node's inserts
    if (s0 + C::CAP < K) __syncthreads();
  }
  if (MP > 1) {
    tsum = wg_sat_sum<C::B>(tsum, S.red64);
    if (tid == 0 && sat_add(tsum, cap) >= (1ull << 63)) atomicOr(A.flags, FLAG_EOVERFLOW);
    emit_top<C::B, MP>(best, A.pi, S.rede, S.redi, tid == 0, A.target, A.score, A.N, n);
    return;
  }
  // term sum and best candidate: per wave by shuffles, then thread 0
  // combines the waves' partials
  u64 be = best.e[0];
  u32 bi = best.i[0];
#pragma unroll
  for (int d = WAVE / 2; d > 0; d >>= 1) {
    tsum = sat_add(tsum, __shfl_xor(tsum, d, WAVE));
    const u64 oe = __shfl_xor(be, d, WAVE);
    const u32 oi = __shfl_xor(bi, d, WAVE);
    if (better(oe, oi, be, bi)) be = oe, bi = oi;
  }
  if (lane_id() == 0) {
    S.red64[wave_id()] = tsum;
    S.rede[wave_id()] = be;
    S.redi[wave_id()] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    tsum = 0;
    be = 0;
    bi = NONE32;
#pragma unroll
    for (int w = 0; w < C::W; ++w) {
      tsum = sat_add(tsum, S.red64[w]);
      if (better(S.rede[w], S.redi[w], be, bi)) be = S.rede[w], bi = S.redi[w];
    }
    if (sat_add(tsum, cap) >= (1ull << 63)) atomicOr(A.flags, FLAG_EOVERFLOW);
    A.target[n] = bi;
    A.score[n] = bi == NONE32 ? 0 : be;
  }
}

template <int MP>
__device__ void rate_light(const RateArgs &A, LightWave &S, u32 n, u64 cap, u64 dmod,
                           u64 magic) {
  const u32 l = lane_id();
  const i64 nb0 = A.nb_off[n];
  const u32 K = (u32)(A.nb_off[n + 1] - nb0);
  const i64 i0 = A.n_off[n], i1 = A.n_off[n + 1];
  const u32 nin = A.n_nin[n];
  const u64 size_n = A.n_size[n];
  const u64 ub_add = A.noise_on ? cap : 0;
  const u32 ne0 = (u32)((i1 - i0) < L_ECH ? (i1 - i0) : L_ECH);
  TopList<MP> best;
  best.clear();
  u64 tsum = 0;
  EdgeDesc d0{0, 0, 0, 0};
  if (l < ne0) d0 = load_edge(A, i0 + l);
  // the wave's table is empty on entry (see the candidate scan)
  insert_window<WAVE>(A, A.nb + nb0, K, size_n, S.key, S.eta, S.rem, L_T - 1, L_SHIFT, l);
  wave_sync();
  for (i64 c0 = i0; c0 < i1; c0 += L_ECH) {
    const u32 ne = (u32)((i1 - c0) < L_ECH ? (i1 - c0) : L_ECH);
    u32 ls = 0, ld = 0;
    if (l < ne) {
      const EdgeDesc d = c0 == i0 ? d0 : load_edge(A, c0 + l);
      if (d.b - d.a >= 2) tsum = sat_add(tsum, d.te);
      S.rs[2 * l] = (u64)d.a;
      S.rs[2 * l + 1] = (u64)d.dm;
      S.rt[2 * l] = d.te;
      S.rt[2 * l + 1] = d.te | ((u64)(c0 + l - i0) < (u64)nin ? INB : 0);
      ls = (u32)(d.dm - d.a);
      ld = (u32)(d.b - d.dm);
    }
    const u32 v = ls + ld;
    const u32 inc = wave_incl_scan(v);
    const u32 tot = __shfl(inc, WAVE - 1, WAVE);
    if (l < ne) {
      S.pre[2 * l] = inc - v;
      S.pre[2 * l + 1] = inc - v + ls;
    }
    if (l == 0) S.pre[2 * ne] = tot;
    wave_sync();
    visit_runs<WAVE>(A.e_pins, S.key, L_T - 1, L_SHIFT, S.eta, S.rem, S.rs, S.rt, S.pre,
                     2 * ne, tot, n, l);
    wave_sync();
  }
  if (A.flag) {
    flag_window<WAVE, L_UNR>(A, S.key, S.eta, S.rem, L_T - 1, L_SHIFT, nb0, K, nin, l);
    if (MP > 1) wave_sync();
  }
  u64 floor = 0;
  if (MP == 1) {
    for (u32 i = l; i < L_T; i += WAVE) {
      const u64 v = S.eta[i];
      if (S.key[i] != EMPTY && bin_valid(A, nin, v, S.rem[i]) && v > floor) floor = v;
    }
    floor = wg_max_u64<WAVE>(floor, nullptr);
  }
  for (u32 i = l; i < L_T; i += WAVE) {
    const u32 m = S.key[i];
    if (m != EMPTY) {
      consider(A, n, nin, m, S.eta[i], S.rem[i], ub_add, floor, dmod, magic, best);
      S.key[i] = EMPTY;
      S.eta[i] = 0;
    }
  }
  tsum = wg_sat_sum<WAVE>(tsum, nullptr);
  if (l == 0 && sat_add(tsum, cap) >= (1ull << 63)) atomicOr(A.flags, FLAG_EOVERFLOW);
  emit_top<WAVE, MP>(best, A.pi, nullptr, nullptr, l == 0, A.target, A.score, A.N, n);
}

__device__ __forceinline__ u32 rfl(u32 v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ NodeRec rec_from_lds(const u32 *w) {
  NodeRec h;
  h.n = rfl(w[0]);
  h.K = rfl(w[1]);
  h.nin = rfl(w[2]);
  h.size = rfl(w[3]);
  h.deg = rfl(w[4]);
  h.nb0 = (i64)((u64)rfl(w[6]) | ((u64)rfl(w[7]) << 32));
  h.i0 = (i64)((u64)rfl(w[8]) | ((u64)rfl(w[9]) << 32));
  return h;
}

// Work items: cnt[0] light nodes in light[]; records of cnt[1] heavy nodes
// (one window of Heavy) at the front of recs[nrec] and of cnt[3] huge ones (more
// than one window of Big, one chunk of Heavy) at its back; cnt[2] big ones in
// big[]; work[0..2] are zeroed work counters (the caller zeroes them).
// k_rate_big rates the big nodes, a workgroup of Big per node; k_rate the
// huge then the heavy ones, a workgroup of Heavy per node, HB at a time (one
// counter access and one load of the records per batch), then the light
// ones, a wave per node.  Every node is taken from a counter (node costs are
// heavy tailed, so a static deal leaves some workgroups far behind), the
// costliest kinds first.  Work indices are scalars (readfirstlane) and each
// loop body ends with a barrier (a wave barrier for the light loop), so every
// lane reconverges before the back edge: without that the compiler may route
// thread 0, which alone takes the next item, around the other lanes, which
// then re-enter the loop on the stale item and never leave.
constexpr u32 HB = 2;  // heavy nodes per counter access
// Light nodes per counter access: one while the light queue is short (a
// batch would leave waves idle at its end), up to LB_MAX when it holds many
// times more nodes than there are waves (each access is an atomic on one
// shared word, which millions of light nodes would otherwise serialise).
constexpr u32 LB_MAX = 8, LB_PER_WAVE = 16;
static_assert(HB * 12 <= RB, "record words of a batch");

// rec(j) is the record of item j < nh
template <class C, u32 NB, int MP, typename RecAt>
__device__ __forceinline__ void heavy_loop(const RateArgs &A, HeavySmem<C> &S, u32 *s_item,
                                           u32 *s_rec, RecAt rec, u32 nh, u32 *work, u64 cap,
                                           u64 dmod, u64 magic) {
  const u32 tid = threadIdx.x;
  if (nh == 0) return;  // uniform: no table to clear for an empty queue
  for (u32 i = tid; i < C::T; i += C::B) {
    S.key[i] = EMPTY;
    S.eta[i] = 0;
  }
  for (;;) {
    if (tid == 0) *s_item = atomicAdd(work, NB);
    __syncthreads();
    const u32 w = rfl(*s_item);
    if (w >= nh) break;
    const u32 nb_ = nh - w < NB ? nh - w : NB;
    if (tid < nb_ * 12) s_rec[tid] = reinterpret_cast<const u32 *>(rec(w + tid / 12))[tid % 12];
    __syncthreads();
    for (u32 j = 0; j < nb_; ++j)
      rate_heavy<C, MP>(A, S, rec_from_lds(s_rec + j * 12), cap, dmod, magic);
    __syncthreads();
  }
}

template <int MP>
__global__ __launch_bounds__(1024) void k_rate_big(RateArgs A, const NodeRec *big,
                                                   const u32 *cnt, u32 *work) {
  __shared__ HeavySmem<Big> S;
  __shared__ u32 s_item;
  __shared__ u32 s_rec[12];
  const u64 cap = A.capinfo[0], dmod = A.capinfo[1], magic = A.capinfo[2];
  heavy_loop<Big, 1, MP>(A, S, &s_item, s_rec, [&](u32 j) { return big + j; }, cnt[2], &work[2], cap,
                     dmod, magic);
}

template <int MP>
__global__ __launch_bounds__(RB, 4) void k_rate(RateArgs A, const u32 *light, const NodeRec *recs,
                                             u32 nrec, const u32 *cnt, u32 *work) {
  __shared__ RateSmem sm;
  __shared__ u32 s_item;
  __shared__ u32 s_rec[HB * 12];
  const u32 nl = cnt[0], nhuge = cnt[3];
  const u64 cap = A.capinfo[0], dmod = A.capinfo[1], magic = A.capinfo[2];
  heavy_loop<Heavy, HB, MP>(
      A, sm.h, &s_item, s_rec,
      [&](u32 j) { return j < nhuge ? recs + (nrec - 1 - j) : recs + (j - nhuge); },
      cnt[1] + nhuge, &work[0], cap, dmod, magic);
  LightWave &S = sm.l[wave_id()];
  for (u32 i = lane_id(); i < L_T; i += WAVE) {
    S.key[i] = EMPTY;
    S.eta[i] = 0;
  }
  wave_sync();
  const u32 q = nl / (gridDim.x * RW * LB_PER_WAVE);
  const u32 lb = rfl(q < 1 ? 1 : q > LB_MAX ? LB_MAX : q);
  u32 lw = 0;
  if (lane_id() == 0) lw = atomicAdd(&work[1], lb);
  lw = __builtin_amdgcn_readfirstlane(__shfl(lw, 0, WAVE));
  for (;;) {
    if (lw >= nl) break;
    u32 nxt = 0;
    if (lane_id() == 0) nxt = atomicAdd(&work[1], lb);
    const u32 end = rfl(nl - lw < lb ? nl : lw + lb);
    for (u32 j = lw; j < end; ++j) {
      rate_light<MP>(A, S, light[j], cap, dmod, magic);
      wave_sync();
    }
    lw = __builtin_amdgcn_readfirstlane(__shfl(nxt, 0, WAVE));
  }
}

// ---------------------------------------------------------------------------
// handshake matching
__global__ void k_bc_score(u32 N, const u32 *target, const u64 *score, u64 *bscore, u32 *bid,
                           u32 *flags) {
  u32 n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= N) return;
  u32 t = target[n];
  if (t == NONE32) return;
  if (t >= N || t == n) {
    atomicOr(flags, FLAG_EINVAL);
    return;
  }
  if (target[t] == n) return;  // a two-cycle: matched by default, not a proposer
  atomicMax((unsigned long long *)&bscore[t], (unsigned long long)score[n]);
}

// best proposer: highest score, smallest id among equals
__global__ void k_bc_id(u32 N, const u32 *target, const u64 *score, const u64 *bscore, u32 *bid) {
  u32 n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= N) return;
  u32 t = target[n];
  if (t == NONE32 || t >= N || t == n || target[t] == n) return;
  if (score[n] == bscore[t]) atomicMin(&bid[t], n);
}

// taken(v) = v in R, or (target(v) != none, bc(target(v)) = v and not
// taken(target(v))).  Each node walks its chain of winning links upward to
// the first node without one; taken(n) = top value XOR parity of the length.
constexpr u32 WALK_LIMIT = 256;

__global__ void k_taken(u32 N, const u32 *target, const u32 *bid, uint8_t *tk, u32 *flags) {
  u32 n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= N) return;
  u32 v = n, parity = 0, top = 0;
  bool done = false;
  for (u32 step = 0; step < WALK_LIMIT; ++step) {
    const u32 t = target[v];
    if (t == NONE32) {  // no candidate: top of its tree, never taken
      done = true;
      break;
    }
    if (target[t] == v) {  // v in R: matched by default
      top = 1;
      done = true;
      break;
    }
    if (bid[t] != v) {  // v is not t's best proposer: not taken
      done = true;
      break;
    }
    v = t;
    parity ^= 1;
  }
  if (!done) {
    tk[n] = 2;
    atomicOr(flags, FLAG_LONGCHAIN);
  } else {
    tk[n] = (uint8_t)(top ^ parity);
  }
}

// Fallback for chains longer than WALK_LIMIT: pointer jumping over the
// winning links, taken(v) = taken(p(v)) XOR x(v) until p(v) is none.
__global__ void k_jump_init(u32 N, const u32 *target, const u32 *bid, u32 *p, uint8_t *x) {
  u32 v = blockIdx.x * blockDim.x + threadIdx.x;
  if (v >= N) return;
  const u32 t = target[v];
  if (t == NONE32) {
    p[v] = NONE32;
    x[v] = 0;
  } else if (target[t] == v) {
    p[v] = NONE32;
    x[v] = 1;
  } else if (bid[t] != v) {
    p[v] = NONE32;
    x[v] = 0;
  } else {
    p[v] = t;
    x[v] = 1;
  }
}

__global__ void k_jump_round(u32 N, const u32 *p_in, const uint8_t *x_in, u32 *p_out,
                             uint8_t *x_out) {
  u32 v = blockIdx.x * blockDim.x + threadIdx.x;
  if (v >= N) return;
  const u32 q = p_in[v];
  if (q == NONE32) {
    p_out[v] = NONE32;
    x_out[v] = x_in[v];
  } else {
    p_out[v] = p_in[q];
    x_out[v] = x_in[v] ^ x_in[q];
  }
}

__global__ void k_jump_finish(u32 N, const u32 *p, const uint8_t *x, uint8_t *tk, u32 *flags) {
  u32 v = blockIdx.x * blockDim.x + threadIdx.x;
  if (v >= N) return;
  if (p[v] != NONE32) atomicOr(flags, FLAG_ECYCLE);
  tk[v] = x[v];
}

// Pi matching rounds ([HP] Sec. V-D): in each round a node still unmatched
// proposes to the first entry of its top-pi list (rows of target/score,
// stride N) that is still unmatched, with that entry's score; a matched node
// proposes nothing.  Along a cycle of these proposals the scores could not
// fall and the ids would have to fall strictly, so each round's proposal
// graph again has no cycle longer than two.  The round's matching gives mr;
// its pairs join match.  Before the first round match is the identity.
__global__ void k_round_prep(u32 N, u32 pi, const u32 *target, const u64 *score,
                             const u32 *match, u32 *tr, u64 *sr) {
  const u32 n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= N) return;
  u32 t = NONE32;
  u64 sc = 0;
  if (match[n] == n) {
    for (u32 j = 0; j < pi; ++j) {
      const u32 m = target[(u64)j * N + n];
      if (m == NONE32) break;  // rows are filled best first
      if (match[m] == m) {
        t = m;
        sc = score[(u64)j * N + n];
        break;
      }
    }
  }
  tr[n] = t;
  sr[n] = sc;
}

__global__ void k_round_merge(u32 N, const u32 *mr, u32 *match) {
  const u32 n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n < N && mr[n] != n) match[n] = mr[n];
}

__global__ void k_iota(u32 N, u32 *p) {
  const u32 n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n < N) p[n] = n;
}

// match(n) = target(n) if taken(n); else its best proposer if any; else n.
__global__ __launch_bounds__(256) void k_match(u32 N, const u32 *target, const u32 *bid,
                                               const uint8_t *tk, u32 *match, u32 *npairs) {
  __shared__ u32 red[256 / WAVE + 1];
  u32 n = blockIdx.x * blockDim.x + threadIdx.x;
  u32 pair = 0;
  if (n < N) {
    u32 m;
    if (tk[n]) m = target[n];
    else if (bid[n] != NONE32) m = bid[n];
    else m = n;
    match[n] = m;
    pair = m > n ? 1 : 0;
  }
  u32 s = wg_sum<256>(pair, red);
  if (threadIdx.x == 0 && s) atomicAdd(npairs, s);
}

}  // namespace

u32 terms_partials(u32 E) { return E ? (E + TB - 1) / TB : 1; }

void launch_terms(chp_ctx *c, u32 E, const i64 *e_off, const u32 *e_w, u64 *t, u64 *partials,
                  u32 nparts, u64 *capinfo) {
  if (E)
    CHP_LAUNCH(c, "terms", k_terms, nparts, TB, 0, E, e_off, e_w, t, partials);
  CHP_LAUNCH(c, "cap", k_cap, 1, TB, 0, E ? nparts : 0u, (const u64 *)partials, E, capinfo);
}

void launch_rate_classify(chp_ctx *c, const RateArgs &a, u32 lo, u32 hi, NbLists nl,
                          NodeRec *recs, NodeRec *big) {
  if (hi <= lo) return;
  CHP_LAUNCH(c, "rate_classify", k_rate_classify, grid_for(hi - lo, 256), 256, 0, a, lo, hi, nl,
             recs, big,
             RATE_SMALL_CAP, Heavy::CAP, Big::CAP, (u32)Heavy::ECH, (u32)L_ECH, (u32)Big::ECH);
}

void launch_rate(chp_ctx *c, const RateArgs &a, NbLists nl, const NodeRec *recs, u32 nrec,
                 const NodeRec *big, u32 *work) {
  if (a.pi > 1) {  // top-pi lists (pi <= RATE_MAX_PI)
    CHP_LAUNCH(c, "rate_big", k_rate_big<RATE_MAX_PI>, c->n_cu, Big::B, 0, a, big,
               (const u32 *)nl.cnt, work);
    CHP_LAUNCH(c, "rate", k_rate<RATE_MAX_PI>, c->n_cu * 4, RB, 0, a, (const u32 *)nl.list[0],
               recs, nrec, (const u32 *)nl.cnt, work);
    return;
  }
  CHP_LAUNCH(c, "rate_big", k_rate_big<1>, c->n_cu, Big::B, 0, a, big, (const u32 *)nl.cnt, work);
  CHP_LAUNCH(c, "rate", k_rate<1>, c->n_cu * 4, RB, 0, a, (const u32 *)nl.list[0], recs, nrec,
             (const u32 *)nl.cnt, work);
}

void launch_match(chp_ctx *c, u32 N, const u32 *target, const u64 *score, MatchScratch ms,
                  u32 *match, u32 *npairs) {
  if (N == 0) return;
  const u32 g = grid_for(N, 256);
  CHP_LAUNCH(c, "bc_score", k_bc_score, g, 256, 0, N, target, score, ms.bscore, ms.bid, c->flags);
  CHP_LAUNCH(c, "bc_id", k_bc_id, g, 256, 0, N, target, score, (const u64 *)ms.bscore, ms.bid);
  CHP_LAUNCH(c, "taken", k_taken, g, 256, 0, N, target, (const u32 *)ms.bid, ms.tk, c->flags);
}

void launch_match_jump(chp_ctx *c, u32 N, const u32 *target, MatchScratch ms) {
  const u32 g = grid_for(N, 256);
  CHP_LAUNCH(c, "jump_init", k_jump_init, g, 256, 0, N, target, (const u32 *)ms.bid, ms.p0, ms.x0);
  u32 *pa = ms.p0, *pb = ms.p1;
  uint8_t *xa = ms.x0, *xb = ms.x1;
  for (int r = 0; r < 33; ++r) {
    CHP_LAUNCH(c, "jump_round", k_jump_round, g, 256, 0, N, (const u32 *)pa, (const uint8_t *)xa,
               pb, xb);
    u32 *tp = pa;
    pa = pb;
    pb = tp;
    uint8_t *tx = xa;
    xa = xb;
    xb = tx;
  }
  CHP_LAUNCH(c, "jump_finish", k_jump_finish, g, 256, 0, N, (const u32 *)pa, (const uint8_t *)xa,
             ms.tk, c->flags);
}

void launch_match_write(chp_ctx *c, u32 N, const u32 *target, MatchScratch ms, u32 *match,
                        u32 *npairs) {
  if (N == 0) return;
  CHP_LAUNCH(c, "match", k_match, grid_for(N, 256), 256, 0, N, target, (const u32 *)ms.bid,
             (const uint8_t *)ms.tk, match, npairs);
}

void launch_round_prep(chp_ctx *c, u32 N, u32 pi, const u32 *target, const u64 *score,
                       const u32 *match, u32 *tr, u64 *sr) {
  if (N == 0) return;
  CHP_LAUNCH(c, "round_prep", k_round_prep, grid_for(N, 256), 256, 0, N, pi, target, score, match,
             tr, sr);
}

void launch_round_merge(chp_ctx *c, u32 N, const u32 *mr, u32 *match) {
  if (N == 0) return;
  CHP_LAUNCH(c, "round_merge", k_round_merge, grid_for(N, 256), 256, 0, N, mr, match);
}

void launch_iota(chp_ctx *c, u32 N, u32 *p) {
  if (N == 0) return;
  CHP_LAUNCH(c, "iota", k_iota, grid_for(N, 256), 256, 0, N, p);
}
