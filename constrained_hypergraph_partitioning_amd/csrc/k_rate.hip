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
__global__ void k_rate_classify(u32 N, const i64 *nb_off, NbLists nl, u32 *target, u64 *score,
                                u32 small_cap) {
  const u32 n = blockIdx.x * blockDim.x + threadIdx.x;
  u64 K = 0;
  if (n < N) {
    K = (u64)(nb_off[n + 1] - nb_off[n]);
    if (K == 0) {
      target[n] = NONE32;
      score[n] = 0;
    }
  }
  const int c = (n >= N || K == 0) ? 2 : (K <= small_cap ? 0 : 1);
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const u32 slot = wave_append(&nl.cnt[k], c == k);
    if (c == k) nl.list[k][slot] = n;
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
// Rating kernel: one launch per level.  A node with more than RATE_SMALL_CAP
// neighbours ("heavy") takes a whole workgroup, a "light" node one wave; both
// pull nodes from a work counter, heavy ones first.
//
// Per node the neighbour list N(n) is loaded, a window of at most H_CAP ids at
// a time (a light node's list always fits one), into an LDS hash table whose
// slots are the bins of m in N(n):
//   eta  u64  eta(n,m) in fixed point; bit 63 set when size(n)+size(m) > Omega
//             (free: a node whose terms plus the noise cap reach 2^63 is an
//             overflow error anyway),
//   rem  u32  |in(m)| - inter(n,m) = |in(m) \ in(n)|, so the inbound limit is
//             |in(n)| + rem <= Delta.
// Both limits are read together with the ids, so judging a candidate needs
// no further memory access.  Incident hyperedges are taken a chunk at a time;
// each brings a source run and a destination run of its pin list (for a
// windowed node, clipped by binary search to the window's id interval, as the
// runs and N(n) are sorted).  A scan lays the runs end to end and every thread
// walks ITEMS consecutive pins with one run lookup, adding t(e) to the bin of
// each pin m != n and, for a destination pin of an inbound hyperedge, taking
// one from rem.  The candidate scan keeps, per thread, the best valid bin by
// (eta desc, id asc), skipping a bin whose upper bound eta + cap cannot beat
// it before its noise is computed; it empties each slot it reads, so the
// table is clean for the next window or node.
constexpr int RB = 256;
constexpr int RW = RB / WAVE;
constexpr u32 H_T = 2048, H_SHIFT = 21;  // hash slots of the heavy path
constexpr u32 H_CAP = 1536;              // neighbours per window (load 0.75)
constexpr int H_ECH = 128;               // hyperedges per chunk
constexpr u32 L_T = 512, L_SHIFT = 23;   // hash slots per wave, light path
constexpr int L_ECH = 32;
constexpr u32 ITEMS = 4;
constexpr u32 EMPTY = 0xFFFFFFFFu;
constexpr u64 INB = 1ull << 63;  // run flag: destination run of an inbound hyperedge
constexpr u64 BAD = 1ull << 63;  // bin flag: the pair breaks Omega
static_assert(RATE_SMALL_CAP <= L_T * 3 / 4, "light window must fit its table");

struct HeavySmem {
  u64 eta[H_T];
  u32 key[H_T];
  u32 rem[H_T];
  u64 rs[2 * H_ECH];
  u64 rt[2 * H_ECH];
  u32 pre[2 * H_ECH + 1];
  u32 red32[RW + 1];
  u64 red64[RW + 1];
  u32 redi[RW + 1];
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
  HeavySmem h;
  LightWave l[RW];
};

// LDS writes of this wave become visible to its other lanes
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

__device__ __forceinline__ u32 hslot(u32 m, u32 shift) { return (m * 0x9E3779B1u) >> shift; }

// Insert neighbour m (not yet present; linear probing, bounded) into an empty
// table slot together with its limit data.
__device__ __forceinline__ void h_insert_bin(u32 *key, u64 *eta, u32 *rem, u32 mask, u32 shift,
                                             u32 m, bool bad, u32 nin_m) {
  u32 s = hslot(m, shift);
  for (u32 p = 0; p <= mask; ++p) {
    if (atomicCAS(&key[s], EMPTY, m) == EMPTY) {
      eta[s] = bad ? BAD : 0;
      rem[s] = nin_m;
      return;
    }
    s = (s + 1) & mask;
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
// thread's index among them.  Each thread first issues the loads of its
// ITEMS consecutive pins, then updates their bins.
template <u32 LANES>
__device__ __forceinline__ void visit_runs(const u32 *pins, const u32 *key, u32 mask, u32 shift,
                                           u64 *eta, u32 *rem, const u64 *rs, const u64 *rt,
                                           const u32 *pre, u32 nruns, u32 tot, u32 n, u32 t) {
  for (u32 base = t * ITEMS; base < tot; base += LANES * ITEMS) {
    u32 r = run_of(pre, nruns + 1, base);
    u32 m[ITEMS];
    u32 rr[ITEMS];
#pragma unroll
    for (u32 k = 0; k < ITEMS; ++k) {
      const u32 idx = base + k;
      m[k] = n;  // n marks "no pin": it is skipped below
      rr[k] = r;
      if (idx < tot) {
        while (idx >= pre[r + 1]) ++r;
        rr[k] = r;
        m[k] = pins[(i64)(rs[r] & ~INB) + (idx - pre[r])];
      }
    }
#pragma unroll
    for (u32 k = 0; k < ITEMS; ++k) {
      if (m[k] == n) continue;
      const u32 slot = h_find(key, mask, shift, m[k]);
      if (slot == EMPTY) continue;  // cannot happen for a valid N(n)
      atomicAdd(&eta[slot], rt[rr[k]]);
      if (rs[rr[k]] & INB) atomicSub(&rem[slot], 1u);
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
    for (u32 k = 0; k < UNR; ++k) {
      sz[k] = 0;
      ni[k] = 0;
      if (m[k] != EMPTY) {
        sz[k] = A.n_size[m[k]];
        ni[k] = A.n_nin[m[k]];
      }
    }
#pragma unroll
    for (u32 k = 0; k < UNR; ++k)
      if (m[k] != EMPTY)
        h_insert_bin(key, eta, rem, mask, shift, m[k], size_n + sz[k] > A.omega, ni[k]);
  }
}

// Hyperedge segment [a, b) with destinations from dm: its source and
// destination runs, clipped to [lo, hi] if clip.
__device__ __forceinline__ void edge_runs(const u32 *pins, i64 a, i64 b, i64 dm, u64 te, bool isin,
                                          bool clip, u32 lo, u32 hi, u64 *rs, u64 *rt, u32 &ls,
                                          u32 &ld) {
  i64 sa = a, sb = dm, da = dm, db = b;
  if (clip) {
    sa = lower_bound_i(pins, a, dm, lo);
    sb = upper_bound_i(pins, sa, dm, hi);
    da = lower_bound_i(pins, dm, b, lo);
    db = upper_bound_i(pins, da, b, hi);
  }
  rs[0] = (u64)sa;
  rs[1] = (u64)da | (isin ? INB : 0);
  rt[0] = te;
  rt[1] = te;
  ls = (u32)(sb - sa);
  ld = (u32)(db - da);
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

struct NodeBest {
  u64 e;
  u32 i;
};

__device__ __forceinline__ bool bin_valid(const RateArgs &A, u32 nin, u64 v, u32 rem) {
  return !(v & BAD) && (u64)nin + rem <= (u64)A.delta;
}

// A valid bin can win only if eta + cap reaches floor, the largest raw eta
// of a valid bin (that bin's total is at least floor); the others are
// skipped before their noise is computed.
__device__ __forceinline__ void consider(const RateArgs &A, u32 n, u32 nin, u32 m, u64 v, u32 rem,
                                         u64 ub_add, u64 floor, u64 dmod, u64 magic,
                                         NodeBest &b) {
  if (!bin_valid(A, nin, v, rem) || v + ub_add < floor) return;
  if (!better(v + ub_add, m, b.e, b.i)) return;
  const u64 tv = A.noise_on ? v + pair_noise(A.seed, n, m, dmod, magic) : v;
  if (better(tv, m, b.e, b.i)) {
    b.e = tv;
    b.i = m;
  }
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

__device__ void rate_heavy(const RateArgs &A, HeavySmem &S, u32 n, u64 cap, u64 dmod,
                           u64 magic) {
  const u32 tid = threadIdx.x;
  const i64 nb0 = A.nb_off[n];
  const u32 K = (u32)(A.nb_off[n + 1] - nb0);
  const i64 i0 = A.n_off[n], i1 = A.n_off[n + 1];
  const u32 nin = A.n_nin[n];
  const u64 size_n = A.n_size[n];
  const u64 ub_add = A.noise_on ? cap : 0;
  const bool clip = K > H_CAP;
  const u32 ne0 = (u32)((i1 - i0) < H_ECH ? (i1 - i0) : H_ECH);
  NodeBest best{0, NONE32};
  u64 tsum = 0;
  for (u32 s0 = 0; s0 < K; s0 += H_CAP) {
    const u32 cw = (K - s0) < H_CAP ? (K - s0) : H_CAP;
    // this thread's hyperedge of the first chunk, loaded ahead of the inserts
    EdgeDesc d0{0, 0, 0, 0};
    if (tid < ne0) d0 = load_edge(A, i0 + tid);
    insert_window<RB>(A, A.nb + nb0 + s0, cw, size_n, S.key, S.eta, S.rem, H_T - 1, H_SHIFT,
                      tid);
    const u32 lo = A.nb[nb0 + s0], hi = A.nb[nb0 + s0 + cw - 1];
    __syncthreads();
    for (i64 c0 = i0; c0 < i1; c0 += H_ECH) {
      const u32 ne = (u32)((i1 - c0) < H_ECH ? (i1 - c0) : H_ECH);
      u32 ls = 0, ld = 0;
      if (tid < ne) {
        const EdgeDesc d = c0 == i0 ? d0 : load_edge(A, c0 + tid);
        if (s0 == 0 && d.b - d.a >= 2) tsum = sat_add(tsum, d.te);
        edge_runs(A.e_pins, d.a, d.b, d.dm, d.te, (u64)(c0 + tid - i0) < (u64)nin, clip, lo, hi,
                  &S.rs[2 * tid], &S.rt[2 * tid], ls, ld);
      }
      u32 tot;
      const u32 off = wg_excl_scan<RB>(ls + ld, S.red32, &tot);
      if (tid < ne) {
        S.pre[2 * tid] = off;
        S.pre[2 * tid + 1] = off + ls;
      }
      if (tid == 0) S.pre[2 * ne] = tot;
      __syncthreads();
      visit_runs<RB>(A.e_pins, S.key, H_T - 1, H_SHIFT, S.eta, S.rem, S.rs, S.rt, S.pre, 2 * ne,
                     tot, n, tid);
      __syncthreads();
    }
    u64 floor = 0;
    for (u32 i = tid; i < H_T; i += RB) {
      const u64 v = S.eta[i];
      if (S.key[i] != EMPTY && bin_valid(A, nin, v, S.rem[i]) && v > floor) floor = v;
    }
    floor = wg_max_u64<RB>(floor, S.red64);
    for (u32 i = tid; i < H_T; i += RB) {
      const u32 m = S.key[i];
      if (m != EMPTY) {
        consider(A, n, nin, m, S.eta[i], S.rem[i], ub_add, floor, dmod, magic, best);
        S.key[i] = EMPTY;
        S.eta[i] = 0;
      }
    }
    __syncthreads();
  }
  tsum = wg_sat_sum<RB>(tsum, S.red64);
  wg_best<RB>(best.e, best.i, S.red64, S.redi);
  if (tid == 0) {
    if (sat_add(tsum, cap) >= (1ull << 63)) atomicOr(A.flags, FLAG_EOVERFLOW);
    A.target[n] = best.i;
    A.score[n] = best.i == NONE32 ? 0 : best.e;
  }
}

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
  NodeBest best{0, NONE32};
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
      edge_runs(A.e_pins, d.a, d.b, d.dm, d.te, (u64)(c0 + l - i0) < (u64)nin, false, 0, 0,
                &S.rs[2 * l], &S.rt[2 * l], ls, ld);
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
  u64 floor = 0;
  for (u32 i = l; i < L_T; i += WAVE) {
    const u64 v = S.eta[i];
    if (S.key[i] != EMPTY && bin_valid(A, nin, v, S.rem[i]) && v > floor) floor = v;
  }
  floor = wg_max_u64<WAVE>(floor, nullptr);
  for (u32 i = l; i < L_T; i += WAVE) {
    const u32 m = S.key[i];
    if (m != EMPTY) {
      consider(A, n, nin, m, S.eta[i], S.rem[i], ub_add, floor, dmod, magic, best);
      S.key[i] = EMPTY;
      S.eta[i] = 0;
    }
  }
  tsum = wg_sat_sum<WAVE>(tsum, nullptr);
  wg_best<WAVE>(best.e, best.i, nullptr, nullptr);
  if (l == 0) {
    if (sat_add(tsum, cap) >= (1ull << 63)) atomicOr(A.flags, FLAG_EOVERFLOW);
    A.target[n] = best.i;
    A.score[n] = best.i == NONE32 ? 0 : best.e;
  }
}

// cnt[0] light nodes in light[], cnt[1] heavy nodes in heavy[]; work[0..1]
// are zeroed work counters.  Heavy nodes are taken one per workgroup, then
// light ones one per wave, each from its counter (node costs are heavy
// tailed, so a static deal leaves some workgroups far behind).  The work
// index is a scalar (readfirstlane) and each loop body ends with a barrier (a
// wave barrier for the light loop), so every lane reconverges before the
// back edge: without that the compiler may route thread 0, which alone takes
// the next item, around the other lanes, which then re-enter the loop on the
// stale item and never leave.
__global__ __launch_bounds__(RB) void k_rate(RateArgs A, const u32 *light, const u32 *heavy,
                                             const u32 *cnt, u32 *work) {
  __shared__ RateSmem sm;
  __shared__ u32 s_item;
  const u32 nl = cnt[0], nh = cnt[1];
  const u64 cap = A.capinfo[0], dmod = A.capinfo[1], magic = A.capinfo[2];
  for (u32 i = threadIdx.x; i < H_T; i += RB) {
    sm.h.key[i] = EMPTY;
    sm.h.eta[i] = 0;
  }
  for (;;) {
    if (threadIdx.x == 0) s_item = atomicAdd(&work[0], 1u);
    __syncthreads();
    const u32 w = __builtin_amdgcn_readfirstlane(s_item);
    __syncthreads();
    if (w >= nh) break;
    rate_heavy(A, sm.h, heavy[w], cap, dmod, magic);
    __syncthreads();
  }
  LightWave &S = sm.l[wave_id()];
  for (u32 i = lane_id(); i < L_T; i += WAVE) {
    S.key[i] = EMPTY;
    S.eta[i] = 0;
  }
  wave_sync();
  for (;;) {
    u32 w = 0;
    if (lane_id() == 0) w = atomicAdd(&work[1], 1u);
    w = __builtin_amdgcn_readfirstlane(__shfl(w, 0, WAVE));
    if (w >= nl) break;
    rate_light(A, S, light[w], cap, dmod, magic);
    wave_sync();
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

void launch_rate_classify(chp_ctx *c, u32 N, const i64 *nb_off, NbLists nl, u32 *target,
                          u64 *score) {
  if (N == 0) return;
  CHP_LAUNCH(c, "rate_classify", k_rate_classify, grid_for(N, 256), 256, 0, N, nb_off, nl, target,
             score, RATE_SMALL_CAP);
}

void launch_rate(chp_ctx *c, const RateArgs &a, NbLists nl, u32 *work) {
  launch_fill_u32(c, work, 2, 0);
  CHP_LAUNCH(c, "rate", k_rate, c->n_cu * 4, RB, 0, a, (const u32 *)nl.list[0],
             (const u32 *)nl.list[1], (const u32 *)nl.cnt, work);
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
