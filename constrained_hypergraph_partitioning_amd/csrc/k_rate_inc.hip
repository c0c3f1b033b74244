// Rating straight from the incidence: candidate proposal ("Hypergraph
// Partitioning on GPU with Distinct Incident Hyperedges and Size
// Constraints", Sec. V-A Eqs. 5-6 and Sec. V-C) for nodes of a graph whose
// neighbour lists are not held in memory (Sec. VII-C: their total does not
// fit).  The result is the one the list-based rating gives: eta(n,m) in 40-bit
// fixed point summed exactly over the hyperedges n and m share, inter(n,m)
// over n's inbound hyperedges with m among their destinations, and the argmax
// of (eta + noise, -id) over the neighbours m that pass both limits.
//
// N(n) is materialised one id window at a time, in LDS, by the pins
// themselves: every incident hyperedge brings a sorted source run and a sorted
// destination run, and a pass over [lo, hi) visits the stretch of each run
// that falls in the window, adding t(e) into the slot of each pin m != n.
// Two kinds of window share the LDS:
//   direct  hi - lo <= 8192 ids (eta and inter) or 12288 (eta alone, when
//           Delta cannot reject any neighbour of n), slot m - lo, no keys
//           and no probing; taken where the pins are dense,
//   hash    a linear-probing table of FHS slots keyed by m + 1 that claims at
//           most about FCAP keys; taken where they are sparse.  A visit that
//           finds the table full lowers fail_min; keys below fail_min are
//           complete (a key is either claimed before its first visit or never),
//           the others are dropped, the next window starts at fail_min and the
//           id span of hash windows is halved (so a window of one id, which
//           always fits, bounds the restarts).
// Where the windows go comes from a sample of each run, the first and the
// last pin of every block of 2^sh consecutive pins, held in LDS: it bounds each
// run's stretch for a window to whole blocks (so no search in global memory)
// and gives estimated visits per id bucket (each block's pins spread evenly
// between its first and last pin), from which each window picks its kind and
// its end.  These choices only steer the work; the sums and the argmax do not
// depend on them.
#include "dev.h"
#include "kernels.h"

namespace {

constexpr int FB = 1024;           // threads per node
constexpr int FW = FB / WAVE;
constexpr u32 FD = 8192;           // ids of a direct window (eta and inter)
constexpr u32 FD2 = 12288;         // ids of a direct window (eta alone)
constexpr u32 FHS = 6144;          // slots of the hash table (the same LDS)
constexpr u32 FCAP = 4608;         // keys a hash pass claims before it reports full
constexpr u32 FRUNS = 768;         // runs: a source and a destination run per hyperedge
constexpr u32 FSMAX = 3072;        // sampled blocks
constexpr u32 FNHB = 2048;         // histogram buckets
constexpr u32 FBS_MIN = 11;        // log2 of the narrowest bucket (FD / 4 ids)
constexpr u32 FHTGT = FCAP * 3 / 4;  // estimated visits a hash pass aims at
constexpr u32 FEST = 16;           // estimates count sixteenths of a visit
constexpr u32 FU = 12;             // pins per thread per chunk
constexpr u32 FCH = FB * FU;       // pins per chunk
constexpr u32 FNBLK = FCH / WAVE;  // wave blocks per chunk
constexpr u64 FINB = 1ull << 63;   // term flag: destination run of an inbound hyperedge
static_assert(FD * 12 == FHS * 16 && FD2 * 8 == FD * 12, "the windows fill the same LDS");
static_assert(FB - 1 + FCAP < FHS, "claims in flight never fill the table");
static_assert(FRUNS / 2 <= FB && FNBLK <= FB && FNHB <= 2 * FB, "one item per thread");
static_assert(FNHB == 64 * 32, "two-level dense bitmap");
static_assert((FD / FB) % 4 == 0 && (FD2 / FB) % 4 == 0 && (FHS / FB) % 3 == 0,
              "candidate groups");

struct IncSmem {
  union {
    struct {
      u64 eta[FD];
      u32 inter[FD];
    } d;
    struct {
      u64 eta[FD2];
    } e;
    struct {
      u64 eta[FHS];
      u32 inter[FHS];
      u32 key[FHS];  // m + 1, 0 = empty
    } h;
  } t;
  i64 rstart[FRUNS];   // first pin of each run in e_pins
  u64 rt[FRUNS];       // t(e), with FINB on the destination run of an inbound hyperedge
  u32 rlen[FRUNS];
  u32 rsp[FRUNS + 1];  // first sample of each run
  u32 rs[FRUNS];       // this window: first pin of each run's stretch
  u32 nxt[FRUNS];      // after a window: each run's first pin at or above its end
  u32 pre[FRUNS + 1];  // this window: stretch offsets
  u32 sfirst[FSMAX];
  u32 slast[FSMAX];
  u32 cum[FNHB + 1];   // estimated visits below each bucket (sixteenths)
  u32 dbits[64];       // bucket b starts a dense window
  u32 dsum[2];         // dbits word w is not zero
  u32 rfirst[FNBLK];   // run of the first pin of each wave block of a chunk
  u64 red64[FW];
  u64 rede[FW];
  u32 redi[FW];
  u32 red32[FW + 1];
  u32 fail_min;
  u32 nkeys;
  u32 item;
};
static_assert(sizeof(IncSmem) <= 160 * 1024, "LDS");

__device__ __forceinline__ u32 rfl(u32 v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ u32 hslot(u32 m) {
  return (u32)(((u64)(m * 0x9E3779B1u) * FHS) >> 32);
}

// Slot of m in the hash table, claimed if absent; FAIL when the table has
// reached its claim limit hcap (<= FCAP) and m is not in it.
constexpr u32 FAIL = 0xFFFFFFFFu;
__device__ __forceinline__ u32 h_insert(IncSmem &S, u32 m, u32 hcap) {
  const u32 k = m + 1;
  u32 s = hslot(m);
  for (;;) {
    const u32 cur = S.t.h.key[s];
    if (cur == k) return s;
    if (cur == 0) {
      if (__hip_atomic_load(&S.nkeys, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= hcap)
        return FAIL;
      const u32 old = atomicCAS(&S.t.h.key[s], 0u, k);
      if (old == 0) {
        atomicAdd(&S.nkeys, 1u);
        return s;
      }
      if (old == k) return s;
    }
    s = s + 1 == FHS ? 0 : s + 1;
  }
}

// first index in a[lo, hi) with a[i] >= v (LDS)
__device__ __forceinline__ u32 lds_lower_bound(const u32 *a, u32 lo, u32 hi, u32 v) {
  while (lo < hi) {
    const u32 mid = (lo + hi) >> 1;
    if (a[mid] < v) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

// first bucket >= b that starts a dense window, else nbk
__device__ __forceinline__ u32 first_dense(const IncSmem &S, u32 b, u32 nbk) {
  if (b >= nbk) return nbk;
  u32 w = b >> 5;
  u32 m = S.dbits[w] & (~0u << (b & 31));
  if (!m) {
    const u32 ws = w + 1;
    if (ws >= 64) return nbk;
    u32 m2 = S.dsum[ws >> 5] & (~0u << (ws & 31));
    if (m2) {
      w = (ws & ~31u) + (u32)__builtin_ctz(m2);
    } else if (ws < 32 && S.dsum[1]) {
      w = 32 + (u32)__builtin_ctz(S.dsum[1]);
    } else {
      return nbk;
    }
    m = S.dbits[w];
  }
  const u32 r = (w << 5) + (u32)__builtin_ctz(m);
  return r < nbk ? r : nbk;
}

template <typename T, typename Op>
__device__ __forceinline__ T wg_reduce(T v, T *lds, Op op) {
#pragma unroll
  for (int d = WAVE / 2; d > 0; d >>= 1) v = op(v, (T)__shfl_xor(v, d, WAVE));
  if (lane_id() == 0) lds[wave_id()] = v;
  __syncthreads();
  T r = lds[0];
#pragma unroll
  for (int w = 1; w < FW; ++w) r = op(r, lds[w]);
  __syncthreads();
  return r;
}

// m with raw eta v and inter c: judged and, if it can still enter the
// thread's list, noised
template <int MP>
__device__ __forceinline__ void take(const RateArgs &A, u32 n, u64 size_n, u32 nin, bool om,
                                     bool de, u32 m, u64 v, u32 c, u32 sz, u32 ni, u64 ub,
                                     u64 dmod, u64 magic, TopList<MP> &b) {
  if (om && size_n + sz > A.omega) return;
  if (de && (u64)nin + ni - c > (u64)A.delta) return;
  if (!b.admits(v + ub, m)) return;
  const u64 tv = A.noise_on ? v + pair_noise(A.seed, n, m, dmod, magic) : v;
  if (b.admits(tv, m)) b.insert(tv, m);
}

template <int MP>
__device__ void rate_inc_node(const RateArgs &A, IncSmem &S, const NodeRec &h, u32 max_size,
                              u32 max_nin, u32 hcap, u64 cap, u64 dmod, u64 magic) {
  const u32 tid = threadIdx.x, lane = lane_id(), wid = wave_id();
  const u32 n = h.n, deg = h.deg, nin = h.nin, nr = 2 * deg;
  const u64 size_n = h.size, W = (u64)h.nb0;
  const bool om = size_n + max_size > A.omega;        // Omega can reject a neighbour
  const bool de = (u64)nin + max_nin > (u64)A.delta;  // Delta can reject a neighbour
  const u64 ub = A.noise_on ? cap : 0;
  // -- runs of the incident hyperedges (inbound ones first in n_inc)
  u64 tsum = 0;
  u32 l0 = 0, l1 = 0;
  if (tid < deg) {
    const u32 e = A.n_inc[h.i0 + tid];
    const i64 a = A.e_off[e], b = A.e_off[e + 1];
    const u32 ns = A.e_nsrc[e];
    const u64 te = A.t[e];
    if (b - a >= 2) tsum = te;
    l0 = ns;
    l1 = (u32)(b - a) - ns;
    S.rstart[2 * tid] = a;
    S.rstart[2 * tid + 1] = a + ns;
    S.rlen[2 * tid] = l0;
    S.rlen[2 * tid + 1] = l1;
    S.rt[2 * tid] = te;
    S.rt[2 * tid + 1] = te | (tid < nin ? FINB : 0);
  }
  // -- samples: blocks of 2^sh pins, so that at most FSMAX blocks are needed
  u32 sh = 0;
  while (((u64)(FSMAX - nr) << sh) < W) ++sh;
  const u32 c0 = (l0 + (1u << sh) - 1) >> sh, c1 = (l1 + (1u << sh) - 1) >> sh;
  u32 ts;
  const u32 so = wg_excl_scan<FB>(c0 + c1, S.red32, &ts);
  if (tid < deg) {
    S.rsp[2 * tid] = so;
    S.rsp[2 * tid + 1] = so + c0;
  }
  if (tid == 0) S.rsp[nr] = ts;
  __syncthreads();
  constexpr u32 SPT = FSMAX / FB;
  u32 sf[SPT], sl[SPT], sw[SPT];
  u32 mn = 0xFFFFFFFFu, mx = 0;
#pragma unroll
  for (u32 k = 0; k < SPT; ++k) {
    const u32 g = tid + k * FB;
    sf[k] = 0;
    sl[k] = 0;
    sw[k] = 0;
    if (g < ts) {
      const u32 r = run_of(S.rsp, nr, g);
      const u32 bk = g - S.rsp[r], len = S.rlen[r];
      const u32 p0 = bk << sh;
      const u32 p1 = (p0 + (1u << sh) < len ? p0 + (1u << sh) : len) - 1;
      const i64 base = S.rstart[r];
      sf[k] = A.e_pins[base + p0];
      sl[k] = A.e_pins[base + p1];
      sw[k] = p1 + 1 - p0;
    }
  }
#pragma unroll
  for (u32 k = 0; k < SPT; ++k) {
    const u32 g = tid + k * FB;
    if (g < ts) {
      S.sfirst[g] = sf[k];
      S.slast[g] = sl[k];
      mn = sf[k] < mn ? sf[k] : mn;
      mx = sl[k] > mx ? sl[k] : mx;
    }
  }
  mn = wg_reduce(mn, S.red32, [](u32 a, u32 b) { return a < b ? a : b; });
  mx = wg_reduce(mx, S.red32, [](u32 a, u32 b) { return a > b ? a : b; });
  // -- estimated visits over buckets of 2^bs ids from mn, in 1/16 of a
  // visit: each block's pins spread evenly over the buckets from its first
  // pin's to its last pin's (a difference array, then two scans)
  u32 bs = FBS_MIN;
  while (((mx - mn) >> bs) >= FNHB) ++bs;
  const u32 nbk = ((mx - mn) >> bs) + 1;
  for (u32 b = tid; b <= FNHB; b += FB) S.cum[b] = 0;
  __syncthreads();
#pragma unroll
  for (u32 k = 0; k < SPT; ++k) {
    const u32 g = tid + k * FB;
    if (g < ts) {
      const u32 bf = (sf[k] - mn) >> bs, bl = (sl[k] - mn) >> bs;
      const u32 unit = sw[k] * FEST, span = bl - bf + 1;
      const u32 q = unit / span, r = unit - q * span;  // density q, the rest at bf
      atomicAdd(&S.cum[bf], q + r);
      atomicSub(&S.cum[bf + 1], r);
      atomicSub(&S.cum[bl + 1], q);
    }
  }
  __syncthreads();
  {
    const u32 d0 = S.cum[2 * tid], d1 = S.cum[2 * tid + 1];
    u32 tot;
    const u32 e = wg_excl_scan<FB>(d0 + d1, S.red32, &tot);  // mod 2^32: the sums are exact
    const u32 v0 = e + d0, v1 = e + d0 + d1;                  // estimates of the two buckets
    const u32 off = wg_excl_scan<FB>(v0 + v1, S.red32, &tot);
    S.cum[2 * tid] = off;
    S.cum[2 * tid + 1] = off + v0;
    if (tid == 0) S.cum[FNHB] = tot;
  }
  __syncthreads();
  // a direct window holds eta and inter, or eta alone when Delta cannot bind
  const u32 fd = de ? FD : FD2;
  const u32 dense = fd / 8 * FEST;  // estimated visits that make a window direct
  {
    const u32 wb = (fd >> bs) > 0 ? (fd >> bs) : 1;  // buckets of a direct window
#pragma unroll
    for (u32 k = 0; k < 2; ++k) {
      const u32 b = tid + k * FB;
      const u32 bend = b + wb < nbk ? b + wb : nbk;
      const bool dn = b < nbk && S.cum[bend] - S.cum[b] >= dense;
      const u64 bal = __ballot(dn);
      if (lane == 0) {
        S.dbits[(b >> 5)] = (u32)bal;
        S.dbits[(b >> 5) + 1] = (u32)(bal >> 32);
      }
    }
    __syncthreads();
    if (wid == 0) {
      const u64 bal = __ballot(S.dbits[lane] != 0);
      if (lane == 0) {
        S.dsum[0] = (u32)bal;
        S.dsum[1] = (u32)(bal >> 32);
      }
    }
    if (tid == 0) {
      S.fail_min = 0xFFFFFFFFu;
      S.nkeys = 0;
    }
    __syncthreads();
  }
  // -- windows over [mn, mx]
  TopList<MP> best;
  best.clear();
  const u64 end = (u64)mx + 1;
  u64 lo = mn;
  // id span a hash window may take: halved after a window that filled up,
  // doubled after one that did not, so a misjudged stretch costs a few
  // windows and a window of one id always fits
  u64 hspan = end - mn;
  u64 last_hi = ~0ull;  // end of the last window, if it did not fill up (then nxt is exact)
  while (lo < end) {
    // the window: all threads take the same decision from the estimates
    const u32 b0 = (u32)((lo - mn) >> bs);
    const u64 dhi = lo + fd < end ? lo + fd : end;
    const u32 bde = (u32)((dhi - 1 - mn) >> bs) + 1;
    const u32 est = S.cum[bde < nbk ? bde : nbk] - S.cum[b0];
    const bool direct =
        rfl(est >= dense || S.cum[b0 + 1] - S.cum[b0] > FHTGT * FEST ? 1u : 0u) != 0;
    u64 hi = dhi;
    if (!direct) {
      // the last bucket boundary with at most FHTGT estimated visits, no
      // further than the next dense window, and within hspan ids
      u32 l = b0 + 1, r = nbk;
      while (l < r) {
        const u32 mid = (l + r + 1) >> 1;
        if (S.cum[mid] - S.cum[b0] <= FHTGT * FEST) l = mid;
        else r = mid - 1;
      }
      const u32 bd = first_dense(S, b0 + 1, nbk);
      const u32 b1 = bd < l ? bd : l;
      hi = b1 >= nbk ? end : (u64)mn + ((u64)b1 << bs);
      if (hi - lo > hspan) hi = lo + hspan;
    }
    const u32 lo32 = (u32)lo, hi32 = (u32)(hi < 0xFFFFFFFFull ? hi : 0xFFFFFFFFull);
    // each run's stretch: whole sampled blocks that can hold a pin in [lo, hi),
    // from the run's exact position when the last window ended at lo
    u32 L = 0;
    if (tid < nr) {
      const u32 g0 = S.rsp[tid], g1 = S.rsp[tid + 1];
      const u32 ks = lds_lower_bound(S.slast, g0, g1, lo32);
      const u32 ke = lds_lower_bound(S.sfirst, g0, g1, hi32);  // one past the last block
      u32 s0 = 0, e0 = 0;
      if (ks < ke) {
        s0 = (ks - g0) << sh;
        if (lo == last_hi && S.nxt[tid] > s0) s0 = S.nxt[tid];
        e0 = ((ke - g0) << sh) < S.rlen[tid] ? ((ke - g0) << sh) : S.rlen[tid];
        L = e0 > s0 ? e0 - s0 : 0;
      }
      S.rs[tid] = s0;
      S.nxt[tid] = L ? e0 : 0;  // lowered below to the first pin >= hi, 0 = unknown
    }
    u32 T;
    const u32 po = wg_excl_scan<FB>(L, S.red32, &T);
    T = rfl(T);
    if (tid < nr) S.pre[tid] = po;
    if (tid == 0) {
      S.pre[nr] = T;
      S.fail_min = 0xFFFFFFFFu;
      S.nkeys = 0;
    }
    __syncthreads();
    for (u32 c = 0; c < T; c += FCH) {
      const u32 cn = T - c < FCH ? T - c : FCH;
      const u32 nblk = (cn + WAVE - 1) / WAVE;
      if (tid < nblk) S.rfirst[tid] = run_of(S.pre, nr, c + tid * WAVE);
      __syncthreads();
      u32 v[FU], rr[FU];
#pragma unroll
      for (u32 u = 0; u < FU; ++u) {
        const u32 q = u * FW + wid;
        const u32 i = c + q * WAVE + lane;
        const bool ok = q < nblk && i < T;
        u32 r = ok ? S.rfirst[q] : 0;
        if (ok)
          while (S.pre[r + 1] <= i) ++r;
        rr[u] = r;
        const i64 pos = ok ? S.rstart[r] + S.rs[r] + (i - S.pre[r]) : 0;
        const u32 x = A.e_pins[pos];
        v[u] = ok ? x : 0xFFFFFFFFu;
      }
      // the first pin >= hi of each run's stretch (one lane per run and wave block)
#pragma unroll
      for (u32 u = 0; u < FU; ++u) {
        const bool bey = v[u] != 0xFFFFFFFFu && v[u] >= hi32;
        const u32 tag = bey ? rr[u] : 0xFFFFFFFFu;
        const u32 ptag = __shfl_up(tag, 1, WAVE);
        if (bey && (lane == 0 || ptag != rr[u])) {
          const u32 r = rr[u];
          const u32 i = c + (u * FW + wid) * WAVE + lane;
          atomicMin(&S.nxt[r], S.rs[r] + (i - S.pre[r]));
        }
      }
      if (direct && de) {
#pragma unroll
        for (u32 u = 0; u < FU; ++u) {
          const u32 x = v[u];
          if (x >= lo32 && x < hi32 && x != n) {
            const u64 te = S.rt[rr[u]];
            const u32 s = x - lo32;
            atomicAdd((unsigned long long *)&S.t.d.eta[s], (unsigned long long)(te & ~FINB));
            if (te & FINB) atomicAdd(&S.t.d.inter[s], 1u);
          }
        }
      } else if (direct) {
#pragma unroll
        for (u32 u = 0; u < FU; ++u) {
          const u32 x = v[u];
          if (x >= lo32 && x < hi32 && x != n)
            atomicAdd((unsigned long long *)&S.t.e.eta[x - lo32],
                      (unsigned long long)(S.rt[rr[u]] & ~FINB));
        }
      } else {
#pragma unroll
        for (u32 u = 0; u < FU; ++u) {
          const u32 x = v[u];
          if (x >= lo32 && x < hi32 && x != n) {
            const u32 s = h_insert(S, x, hcap);
            if (s == FAIL) {
              atomicMin(&S.fail_min, x);
              continue;
            }
            const u64 te = S.rt[rr[u]];
            atomicAdd((unsigned long long *)&S.t.h.eta[s], (unsigned long long)(te & ~FINB));
            if (de && (te & FINB)) atomicAdd(&S.t.h.inter[s], 1u);
          }
        }
      }
      __syncthreads();
    }
    // candidates of the window; every slot is read and left empty
    const u32 fmin = rfl(S.fail_min);
    if (direct) {
      constexpr u32 G = 4;  // slots per group (registers)
#pragma unroll 1
      for (u32 k0 = 0; k0 < fd / FB; k0 += G) {
        u64 ev[G];
        u32 cv[G], szv[G], niv[G];
#pragma unroll
        for (u32 k = 0; k < G; ++k) {
          const u32 s = tid + (k0 + k) * FB;
          if (de) {
            ev[k] = S.t.d.eta[s];
            cv[k] = S.t.d.inter[s];
            S.t.d.eta[s] = 0;
            S.t.d.inter[s] = 0;
          } else {
            ev[k] = S.t.e.eta[s];
            cv[k] = 0;
            S.t.e.eta[s] = 0;
          }
        }
#pragma unroll
        for (u32 k = 0; k < G; ++k) {
          const u32 mm = ev[k] ? lo32 + tid + (k0 + k) * FB : n;  // in range when untouched
          szv[k] = om ? A.n_size[mm] : 0;
          niv[k] = de ? A.n_nin[mm] : 0;
        }
#pragma unroll
        for (u32 k = 0; k < G; ++k)
          if (ev[k])
            take(A, n, size_n, nin, om, de, lo32 + tid + (k0 + k) * FB, ev[k], cv[k], szv[k],
                 niv[k], ub, dmod, magic, best);
      }
    } else {
      constexpr u32 G = 3;
#pragma unroll 1
      for (u32 k0 = 0; k0 < FHS / FB; k0 += G) {
        u64 ev[G];
        u32 mv[G], cv[G], szv[G], niv[G];
#pragma unroll
        for (u32 k = 0; k < G; ++k) {
          const u32 s = tid + (k0 + k) * FB;
          const u32 key = S.t.h.key[s];
          mv[k] = key - 1;
          ev[k] = (key != 0 && key - 1 < fmin) ? S.t.h.eta[s] : 0;
          cv[k] = S.t.h.inter[s];
          S.t.h.key[s] = 0;
          S.t.h.eta[s] = 0;
          S.t.h.inter[s] = 0;
        }
#pragma unroll
        for (u32 k = 0; k < G; ++k) {
          const u32 mm = ev[k] ? mv[k] : n;
          szv[k] = om ? A.n_size[mm] : 0;
          niv[k] = de ? A.n_nin[mm] : 0;
        }
#pragma unroll
        for (u32 k = 0; k < G; ++k)
          if (ev[k])
            take(A, n, size_n, nin, om, de, mv[k], ev[k], cv[k], szv[k], niv[k], ub, dmod, magic,
                 best);
      }
    }
    const bool full = !direct && fmin < hi32;
    last_hi = full ? ~0ull : hi;
    if (!direct) {
      if (full) {
        hspan = (hi - fmin) / 2 > 0 ? (hi - fmin) / 2 : 1;
      } else if (hspan < end - mn) {
        hspan *= 2;
      }
    }
    const u64 nx = full ? (u64)fmin : hi;
    lo = ((u64)rfl((u32)(nx >> 32)) << 32) | rfl((u32)nx);
    hspan = ((u64)rfl((u32)(hspan >> 32)) << 32) | rfl((u32)hspan);
    // the next window's first barrier orders these slot clears before its
    // visits, and the reads of fail_min before its reset
  }
  if (MP > 1) {
#pragma unroll
    for (int d = WAVE / 2; d > 0; d >>= 1) tsum = sat_add(tsum, __shfl_xor(tsum, d, WAVE));
    if (lane == 0) S.red64[wid] = tsum;
    __syncthreads();
    if (tid == 0) {
      tsum = 0;
#pragma unroll
      for (int w = 0; w < FW; ++w) tsum = sat_add(tsum, S.red64[w]);
      if (sat_add(tsum, cap) >= (1ull << 63)) atomicOr(A.flags, FLAG_EOVERFLOW);
    }
    emit_top<FB, MP>(best, A.pi, S.rede, S.redi, tid == 0, A.target, A.score, A.N, n);
    return;
  }
  // -- term sum and best candidate: per wave by shuffles, then thread 0
  u64 be = best.e[0];
  u32 bi = best.i[0];
#pragma unroll
  for (int d = WAVE / 2; d > 0; d >>= 1) {
    tsum = sat_add(tsum, __shfl_xor(tsum, d, WAVE));
    const u64 oe = __shfl_xor(be, d, WAVE);
    const u32 oi = __shfl_xor(bi, d, WAVE);
    if (better(oe, oi, be, bi)) be = oe, bi = oi;
  }
  if (lane == 0) {
    S.red64[wid] = tsum;
    S.rede[wid] = be;
    S.redi[wid] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    tsum = 0;
    be = 0;
    bi = NONE32;
#pragma unroll
    for (int w = 0; w < FW; ++w) {
      tsum = sat_add(tsum, S.red64[w]);
      if (better(S.rede[w], S.redi[w], be, bi)) be = S.rede[w], bi = S.redi[w];
    }
    if (sat_add(tsum, cap) >= (1ull << 63)) atomicOr(A.flags, FLAG_EOVERFLOW);
    A.target[n] = bi;
    A.score[n] = bi == NONE32 ? 0 : be;
  }
}

// Nodes are taken one at a time from a counter (thread 0 takes the item, a
// barrier publishes it, and the loop body ends with a barrier so that every
// lane reconverges before the back edge).
template <int MP>
__global__ __launch_bounds__(FB) void k_rate_inc(RateArgs A, const NodeRec *recs, const u32 *cnt,
                                                 const u32 *gmax, u32 *work, u32 hcap) {
  __shared__ IncSmem S;
  const u32 tid = threadIdx.x;
  const u64 cap = A.capinfo[0], dmod = A.capinfo[1], magic = A.capinfo[2];
  const u32 max_size = gmax[0], max_nin = gmax[1];
  const u32 total = *cnt;
  for (u32 i = tid; i < FD; i += FB) {
    S.t.d.eta[i] = 0;
    S.t.d.inter[i] = 0;
  }
  for (;;) {
    if (tid == 0) S.item = atomicAdd(work, 1u);
    __syncthreads();
    const u32 w = rfl(S.item);
    if (w >= total) break;
    NodeRec h = recs[w];
    h.n = rfl(h.n);
    h.deg = rfl(h.deg);
    h.nin = rfl(h.nin);
    h.size = rfl(h.size);
    rate_inc_node<MP>(A, S, h, max_size, max_nin, hcap, cap, dmod, magic);
    __syncthreads();
  }
}

// Nodes of [0, N) with 1..FRUNS/2 incident hyperedges and min_visits to
// 2^27 - 1 pins over them (the estimates in sixteenths stay below 2^31) go to
// the list (record: n, nin, size, deg, i0 and the pin count in nb0) and get
// skip[n] = 1; gmax = {max size, max |in|} over all.  Thread n holds node n;
// the pin counts are summed by the whole wave, node after node.
__global__ void k_inc_classify(RateArgs A, u64 min_visits, uint8_t *skip, NodeRec *recs,
                               u32 *cnt, u32 *gmax) {
  const u32 n = blockIdx.x * blockDim.x + threadIdx.x;
  const u32 l = lane_id();
  bool take_it = false;
  u32 sz = 0, ni = 0, deg = 0;
  u64 w = 0;
  i64 a = 0;
  if (n < A.N) {
    a = A.n_off[n];
    deg = (u32)(A.n_off[n + 1] - a);
    sz = A.n_size[n];
    ni = A.n_nin[n];
  }
  const bool counted = n < A.N && deg >= 1 && deg <= FRUNS / 2;
  u64 todo = __ballot(counted);
  while (todo) {
    const u32 i = (u32)__builtin_ctzll(todo);
    todo &= todo - 1;
    const u32 di = (u32)__builtin_amdgcn_readlane((int)deg, (int)i);
    const i64 ai = (i64)((u64)(u32)__builtin_amdgcn_readlane((int)(u32)((u64)a >> 32), (int)i)
                             << 32 |
                         (u32)__builtin_amdgcn_readlane((int)(u32)(u64)a, (int)i));
    u64 part = 0;
    for (u32 j = l; j < di; j += WAVE) {
      const u32 e = A.n_inc[ai + j];
      part += (u64)(A.e_off[e + 1] - A.e_off[e]);
    }
    part = wave_sum(part);
    if (l == i) w = part;
  }
  if (n < A.N) {
    take_it = counted && w >= min_visits && w < (1ull << 27);
    skip[n] = take_it ? 1 : 0;
  }
  u32 msz = sz, mni = ni;
#pragma unroll
  for (int d = WAVE / 2; d > 0; d >>= 1) {
    const u32 o1 = __shfl_xor(msz, d, WAVE), o2 = __shfl_xor(mni, d, WAVE);
    msz = o1 > msz ? o1 : msz;
    mni = o2 > mni ? o2 : mni;
  }
  if (lane_id() == 0) {
    atomicMax(gmax + 0, msz);
    atomicMax(gmax + 1, mni);
  }
  const u32 s = wave_append(cnt, take_it);
  if (take_it) {
    NodeRec r;
    r.n = n;
    r.K = 0;
    r.nin = ni;
    r.size = sz;
    r.deg = deg;
    r.pad0 = r.pad1 = r.pad2 = 0;
    r.nb0 = (i64)w;
    r.i0 = a;
    recs[s] = r;
  }
}

}  // namespace

void launch_inc_classify(chp_ctx *c, const RateArgs &a, u64 min_visits, uint8_t *skip,
                         NodeRec *recs, u32 *cnt, u32 *gmax) {
  if (a.N == 0) return;
  CHP_LAUNCH(c, "inc_classify", k_inc_classify, grid_for(a.N, 256), 256, 0, a, min_visits, skip,
             recs, cnt, gmax);
}

void launch_rate_inc(chp_ctx *c, const RateArgs &a, const NodeRec *recs, const u32 *cnt,
                     const u32 *gmax, u32 *work, u32 host_count, u32 hash_keys) {
  if (!host_count) return;
  const u32 g = host_count < c->n_cu ? host_count : c->n_cu;
  // (at least 2: a window of one id then never fills)
  const u32 hcap = hash_keys && hash_keys < FCAP ? (hash_keys < 2 ? 2 : hash_keys) : FCAP;
  if (a.pi > 1)
    CHP_LAUNCH(c, "rate_inc", k_rate_inc<RATE_MAX_PI>, g, FB, 0, a, recs, cnt, gmax, work, hcap);
  else
    CHP_LAUNCH(c, "rate_inc", k_rate_inc<1>, g, FB, 0, a, recs, cnt, gmax, work, hcap);
}
