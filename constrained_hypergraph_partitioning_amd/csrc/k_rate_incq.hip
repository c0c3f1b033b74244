// Rating straight from the incidence with 32-bit bins: candidate proposal
// ("Hypergraph Partitioning on GPU with Distinct Incident Hyperedges and Size
// Constraints", Sec. V-A Eqs. 5-6 and Sec. V-C) for nodes of a graph whose
// neighbour lists are not held in memory (Sec. VII-C), when Delta cannot reject
// any neighbour of the node (so no per-neighbour inbound count is needed).
//
// Windows over the node's neighbour ids are visited as in k_rate_inc.hip (a
// sample of every run steers dense windows, slot m - lo, and sparse ones, a
// hash table), but a bin holds a 32-bit sum of the quantised terms
// q(e) = t(e) >> s, where s is the smallest shift that keeps the node's whole
// term sum below 2^32.  A bin is then twice as small as an exact 64-bit eta,
// so a window covers twice the ids.  The bins only bound eta: with V the bin
// and c the number of hyperedges n and m share (at most V / q_min),
//     V << s  <=  eta(n, m)  <=  (V << s) + c * (2^s - 1).
// Each window keeps every valid neighbour whose upper bound (noise at most the
// cap) can still reach the best lower bound seen so far: the contenders.  At
// the node's end the contenders still in reach get their exact eta, the sum of
// t(e) over the hyperedges of I(m) that are also in I(n) (both incidence lists
// sorted), and the best of them by (eta + noise desc, id asc) is the node's
// target.  The result is the exact argmax of the definition; the bounds only
// decide how few neighbours need their exact sum.
//
// Run stretches are exact at their start: every run carries its cursor, the
// first pin at or above the window's low end, found during the visits of the
// window before (the first pin at or above that window's end).  Only the end
// of a stretch is rounded up to a sampled block.  Stretches are compacted
// (empty ones dropped) before the pins are dealt to the threads.
//
// A node whose terms cannot be quantised without losing a hyperedge (q = 0),
// whose Delta may bind, or whose contenders overflow their list is handed to
// k_rate_inc (appended to a spill list) before or after its windows; the bins
// are left empty either way.
#include "dev.h"
#include "kernels.h"

namespace {

constexpr int QB = 1024;              // threads per node
constexpr int QW = QB / WAVE;
constexpr u32 QD = 24576;             // ids of a direct window (one u32 bin each)
constexpr u32 QHS = QD / 2;           // slots of the hash table (key, bin)
constexpr u32 QCAP = QHS * 3 / 4;     // keys a hash window claims before it reports full
constexpr u32 QE = 384;               // incident hyperedges
constexpr u32 QRUNS = 2 * QE;         // a source and a destination run per hyperedge
constexpr u32 QSMAX = 4096;           // sampled blocks
constexpr u32 QNHB = 1024;            // estimate buckets
constexpr u32 QBS_MIN = 12;           // log2 of the narrowest bucket
constexpr u32 QHTGT = QCAP * 3 / 4;   // estimated visits a hash window aims at
constexpr u32 QEST = 16;              // estimates count sixteenths of a visit
constexpr u32 QU = 16;                // pins per thread per chunk
constexpr u32 QCH = QB * QU;          // pins per chunk
constexpr u32 QNBLK = QCH / WAVE;     // wave blocks per chunk
constexpr u32 QCONT = 256;            // contenders a node may keep
constexpr u32 QFAIL = 0xFFFFFFFFu;
static_assert(QB - 1 + QCAP < QHS, "claims in flight never fill the table");
static_assert(QRUNS <= QB && QNBLK <= QB && QNHB <= QB, "one item per thread");
static_assert(QNHB == 32 * 32, "two-level dense bitmap");
static_assert(QD % QB == 0 && QHS % QB == 0 && QSMAX % QB == 0, "slots per thread");

struct QSmem {
  union {
    u32 bin[QD];
    struct {
      u32 key[QHS];  // m + 1, 0 = empty
      u32 bin[QHS];
    } h;
  } t;
  // incident hyperedge k (n_inc order: inbound ones first, each part sorted)
  i64 eoff[QE];
  u64 tx[QE];    // exact t(e)
  u32 eid[QE];
  u32 ens[QE];   // source pins
  u32 elen[QE];  // pins
  u32 q[QE];     // t(e) >> s
  // run r: sources (r even) or destinations (r odd) of hyperedge r / 2
  u32 rcur[QRUNS];     // exact: first pin at or above the window's low end
  u32 rsp[QRUNS + 1];  // first sample of each run
  u32 sfirst[QSMAX];   // first pin of each sampled block
  // the window's non-empty stretches
  i64 caddr[QRUNS];    // e_pins index of flat position 0 of stretch k
  u32 cpre[QRUNS + 1];
  u32 cq[QRUNS];
  u32 cnext[QRUNS];    // stretch index of its first pin at or above the window's end
  u32 bfirst[QNBLK];   // stretch of the first pin of each wave block of a chunk
  u32 cum[QNHB + 1];   // estimated visits below each bucket (sixteenths)
  u32 dbits[32];       // bucket b starts a dense window
  u32 dsum;            // dbits word w is not zero
  u32 cid[QCONT];      // contenders: id, upper bound of eta + noise
  u64 cub[QCONT];
  u64 red64[QW];
  u32 redi[QW];
  u32 red32[QW + 1];
  u32 fail_min;
  u32 nkeys;
  u32 ncont;
  u32 item;
};
static_assert(sizeof(QSmem) <= 160 * 1024, "LDS");

__device__ __forceinline__ u32 rfl(u32 v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ u64 rfl64(u64 v) {
  return ((u64)rfl((u32)(v >> 32)) << 32) | rfl((u32)v);
}

__device__ __forceinline__ u32 qslot(u32 m) { return (u32)(((u64)(m * 0x9E3779B1u) * QHS) >> 32); }

// Slot of m in the hash table, claimed if absent; QFAIL when the table has
// reached its claim limit hcap and m is not in it.
__device__ __forceinline__ u32 q_insert(QSmem &S, u32 m, u32 hcap) {
  const u32 k = m + 1;
  u32 s = qslot(m);
  for (;;) {
    const u32 cur = S.t.h.key[s];
    if (cur == k) return s;
    if (cur == 0) {
      if (__hip_atomic_load(&S.nkeys, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= hcap)
        return QFAIL;
      const u32 old = atomicCAS(&S.t.h.key[s], 0u, k);
      if (old == 0) {
        atomicAdd(&S.nkeys, 1u);
        return s;
      }
      if (old == k) return s;
    }
    s = s + 1 == QHS ? 0 : s + 1;
  }
}

// first index in a[lo, hi) with a[i] >= v (LDS)
__device__ __forceinline__ u32 q_lower_bound(const u32 *a, u32 lo, u32 hi, u32 v) {
  while (lo < hi) {
    const u32 mid = (lo + hi) >> 1;
    if (a[mid] < v) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

// first bucket >= b that starts a dense window, else nbk
__device__ __forceinline__ u32 q_first_dense(const QSmem &S, u32 b, u32 nbk) {
  if (b >= nbk) return nbk;
  u32 w = b >> 5;
  u32 m = S.dbits[w] & (~0u << (b & 31));
  if (!m) {
    const u32 ws = w + 1;
    if (ws >= 32) return nbk;
    const u32 m2 = S.dsum & (~0u << ws);
    if (!m2) return nbk;
    w = (u32)__builtin_ctz(m2);
    m = S.dbits[w];
  }
  const u32 r = (w << 5) + (u32)__builtin_ctz(m);
  return r < nbk ? r : nbk;
}

template <typename T, typename Op>
__device__ __forceinline__ T q_reduce(T v, T *lds, Op op) {
#pragma unroll
  for (int d = WAVE / 2; d > 0; d >>= 1) v = op(v, (T)__shfl_xor(v, d, WAVE));
  if (lane_id() == 0) lds[wave_id()] = v;
  __syncthreads();
  T r = lds[0];
#pragma unroll
  for (int w = 1; w < QW; ++w) r = op(r, lds[w]);
  __syncthreads();
  return r;
}

__device__ __forceinline__ u64 umax64(u64 a, u64 b) { return a > b ? a : b; }

// One candidate m with bin value V (valid, V > 0): judged against the
// threshold T; a contender is appended, the thread's best lower bound kept.
__device__ __forceinline__ void q_judge(const RateArgs &A, QSmem &S, u32 n, u32 m, u32 V, u32 s,
                                        u32 qmin, u64 errunit, u64 ub, u64 T, u64 dmod, u64 magic,
                                        u64 &bl) {
  const u64 lo = (u64)V << s;
  const u64 err = (u64)(V / qmin) * errunit;
  if (lo + err + ub < T) return;
  const u64 nz = A.noise_on ? pair_noise(A.seed, n, m, dmod, magic) : 0;
  const u64 lb = lo + nz, up = lb + err;
  bl = lb > bl ? lb : bl;
  if (up >= T) {
    const u32 j = atomicAdd(&S.ncont, 1u);
    if (j < QCONT) {
      S.cid[j] = m;
      S.cub[j] = up;
    }
  }
}

// Rates node h; false (and nothing written, the bins left empty) when the
// node must go to k_rate_inc instead.
__device__ bool rate_node_q(const RateArgs &A, QSmem &S, const NodeRec &h, u32 max_size,
                            u32 max_nin, u32 hcap, u64 cap, u64 dmod, u64 magic) {
  const u32 tid = threadIdx.x, lane = lane_id(), wid = wave_id();
  const u32 n = h.n, deg = h.deg, nin = h.nin, nr = 2 * deg;
  const u64 size_n = h.size, W = (u64)h.nb0;
  const bool om = size_n + max_size > A.omega;  // Omega can reject a neighbour
  if ((u64)nin + max_nin > (u64)A.delta || deg > QE) return false;
  const u64 ub = A.noise_on ? cap : 0;
  // -- incident hyperedges; the term sum and the smallest term decide s
  u64 te = 0;
  u32 l0 = 0, l1 = 0;
  bool counts = false;
  if (tid < deg) {
    const u32 e = A.n_inc[h.i0 + tid];
    const i64 a = A.e_off[e], b = A.e_off[e + 1];
    const u32 ns = A.e_nsrc[e];
    te = A.t[e];
    counts = b - a >= 2;
    l0 = ns;
    l1 = (u32)(b - a) - ns;
    S.eoff[tid] = a;
    S.tx[tid] = te;
    S.eid[tid] = e;
    S.ens[tid] = ns;
    S.elen[tid] = (u32)(b - a);
  }
  const u64 tsum = q_reduce<u64>(counts ? te : 0, S.red64, [](u64 x, u64 y) { return sat_add(x, y); });
  const u64 tmin = q_reduce<u64>(counts ? te : ~0ull, S.red64,
                                 [](u64 x, u64 y) { return x < y ? x : y; });
  if (sat_add(tsum, cap) >= (1ull << 63)) {
    if (tid == 0) {
      atomicOr(A.flags, FLAG_EOVERFLOW);
      A.target[n] = NONE32;
      A.score[n] = 0;
    }
    return true;
  }
  // the bit length of tsum >> 32, so that tsum >> s < 2^32
  const u32 s = tsum >> 32 ? 64u - (u32)__builtin_clzll(tsum >> 32) : 0u;
  const u32 qmin = (u32)(tmin >> s);
  if (tsum && qmin == 0) return false;
  const u64 errunit = (1ull << s) - 1;
  if (tid < deg) S.q[tid] = (u32)(te >> s);
  // -- samples: blocks of 2^sh pins, so that at most QSMAX blocks are needed
  u32 sh = 0;
  while (((u64)(QSMAX - nr) << sh) < W) ++sh;
  const u32 c0 = (l0 + (1u << sh) - 1) >> sh, c1 = (l1 + (1u << sh) - 1) >> sh;
  u32 ts;
  const u32 so = wg_excl_scan<QB>(c0 + c1, S.red32, &ts);
  if (tid < deg) {
    S.rsp[2 * tid] = so;
    S.rsp[2 * tid + 1] = so + c0;
  }
  if (tid < nr) S.rcur[tid] = 0;  // every pin is >= the first window's low end
  if (tid == 0) S.rsp[nr] = ts;
  for (u32 b = tid; b <= QNHB; b += QB) S.cum[b] = 0;
  __syncthreads();
  constexpr u32 SPT = QSMAX / QB;
  u32 sf[SPT], sl[SPT], sw[SPT];
  u32 mn = 0xFFFFFFFFu, mx = 0;
#pragma unroll
  for (u32 k = 0; k < SPT; ++k) {
    const u32 g = tid + k * QB;
    sf[k] = 0;
    sl[k] = 0;
    sw[k] = 0;
    if (g < ts) {
      const u32 r = run_of(S.rsp, nr, g);
      const u32 ke = r >> 1;
      const u32 len = (r & 1) ? S.elen[ke] - S.ens[ke] : S.ens[ke];
      const i64 base = S.eoff[ke] + ((r & 1) ? S.ens[ke] : 0);
      const u32 p0 = (g - S.rsp[r]) << sh;
      const u32 p1 = (p0 + (1u << sh) < len ? p0 + (1u << sh) : len) - 1;
      sf[k] = A.e_pins[base + p0];
      sl[k] = A.e_pins[base + p1];
      sw[k] = p1 + 1 - p0;
    }
  }
#pragma unroll
  for (u32 k = 0; k < SPT; ++k) {
    const u32 g = tid + k * QB;
    if (g < ts) {
      S.sfirst[g] = sf[k];
      mn = sf[k] < mn ? sf[k] : mn;
      mx = sl[k] > mx ? sl[k] : mx;
    }
  }
  mn = q_reduce<u32>(mn, S.red32, [](u32 a, u32 b) { return a < b ? a : b; });
  mx = q_reduce<u32>(mx, S.red32, [](u32 a, u32 b) { return a > b ? a : b; });
  // -- estimated visits over buckets of 2^bs ids from mn, in 1/16 of a visit:
  // each block's pins spread evenly over the buckets from its first pin's to
  // its last pin's (a difference array, then two scans)
  u32 bs = QBS_MIN;
  while (((mx - mn) >> bs) >= QNHB) ++bs;
  const u32 nbk = ((mx - mn) >> bs) + 1;
#pragma unroll
  for (u32 k = 0; k < SPT; ++k) {
    const u32 g = tid + k * QB;
    if (g < ts) {
      const u32 bf = (sf[k] - mn) >> bs, bl = (sl[k] - mn) >> bs;
      const u32 unit = sw[k] * QEST, span = bl - bf + 1;
      const u32 qd = unit / span, rem = unit - qd * span;
      atomicAdd(&S.cum[bf], qd + rem);
      atomicSub(&S.cum[bf + 1], rem);
      atomicSub(&S.cum[bl + 1], qd);
    }
  }
  __syncthreads();
  {
    const u32 d0 = tid < QNHB ? S.cum[tid] : 0;
    u32 tot;
    const u32 e = wg_excl_scan<QB>(d0, S.red32, &tot);  // mod 2^32: the sums are exact
    const u32 v0 = e + d0;                               // estimate of bucket tid
    const u32 off = wg_excl_scan<QB>(v0, S.red32, &tot);
    if (tid < QNHB) S.cum[tid] = off;
    if (tid == 0) S.cum[QNHB] = tot;
  }
  __syncthreads();
  const u32 dense = QD / 8 * QEST;  // estimated visits that make a window direct
  {
    const u32 wb = (QD >> bs) > 0 ? (QD >> bs) : 1;  // buckets of a direct window
    const u32 b = tid;
    const u32 bend = b + wb < nbk ? b + wb : nbk;
    const bool dn = b < nbk && S.cum[bend] - S.cum[b] >= dense;
    const u64 bal = __ballot(dn);
    if (lane == 0 && wid < QNHB / WAVE) {
      S.dbits[2 * wid] = (u32)bal;
      S.dbits[2 * wid + 1] = (u32)(bal >> 32);
    }
    __syncthreads();
    if (wid == 0) {
      const u64 b2 = __ballot(lane < 32 && S.dbits[lane & 31] != 0);
      if (lane == 0) S.dsum = (u32)b2;
    }
    if (tid == 0) S.ncont = 0;
    __syncthreads();
  }
  // -- windows over [mn, mx]
  u64 lstar = 0;  // best lower bound of eta + noise so far (a valid neighbour's)
  const u64 end = (u64)mx + 1;
  u64 lo = mn;
  u64 hspan = end - mn;  // id span a hash window may take (halved after one fills)
  u64 last_hi = mn;      // end of the last window if it did not fill (cursors exact)
  while (lo < end) {
    const u32 b0 = (u32)((lo - mn) >> bs);
    const u64 dhi = lo + QD < end ? lo + QD : end;
    const u32 bde = (u32)((dhi - 1 - mn) >> bs) + 1;
    const u32 est = S.cum[bde < nbk ? bde : nbk] - S.cum[b0];
    const bool direct =
        rfl(est >= dense || S.cum[b0 + 1] - S.cum[b0] > QHTGT * QEST ? 1u : 0u) != 0;
    u64 hi = dhi;
    if (!direct) {
      u32 l = b0 + 1, r = nbk;
      while (l < r) {
        const u32 mid = (l + r + 1) >> 1;
        if (S.cum[mid] - S.cum[b0] <= QHTGT * QEST) l = mid;
        else r = mid - 1;
      }
      const u32 bd = q_first_dense(S, b0 + 1, nbk);
      const u32 b1 = bd < l ? bd : l;
      hi = b1 >= nbk ? end : (u64)mn + ((u64)b1 << bs);
      if (hi - lo > hspan) hi = lo + hspan;
    }
    hi = rfl64(hi);
    const u32 lo32 = (u32)lo, hi32 = (u32)(hi < 0xFFFFFFFFull ? hi : 0xFFFFFFFFull);
    const bool exact = lo == last_hi;
    // each run's stretch: from its cursor (or, after a window that filled, the
    // sampled block holding its first pin >= lo) to the first sampled block
    // starting at or above hi
    u32 L = 0, cur = 0;
    if (tid < nr) {
      const u32 g0 = S.rsp[tid], g1 = S.rsp[tid + 1];
      const u32 ke = tid >> 1;
      const u32 len = (tid & 1) ? S.elen[ke] - S.ens[ke] : S.ens[ke];
      if (exact) {
        cur = S.rcur[tid];
      } else {
        const u32 kb = q_lower_bound(S.sfirst, g0, g1, lo32);
        cur = kb > g0 ? (kb - 1 - g0) << sh : 0;
      }
      const u32 kh = q_lower_bound(S.sfirst, g0, g1, hi32);
      const u32 e0 = ((kh - g0) << sh) < len ? ((kh - g0) << sh) : len;
      L = e0 > cur ? e0 - cur : 0;
    }
    u32 T, K;
    const u32 po = wg_excl_scan<QB>(L, S.red32, &T);
    const u32 ko = wg_excl_scan<QB>(L ? 1u : 0u, S.red32, &K);
    T = rfl(T);
    K = rfl(K);
    if (L) {
      const u32 ke = tid >> 1;
      S.caddr[ko] = S.eoff[ke] + ((tid & 1) ? S.ens[ke] : 0) + cur - (i64)po;
      S.cpre[ko] = po;
      S.cq[ko] = S.q[ke];
      S.cnext[ko] = L;
    }
    if (tid == 0) {
      S.cpre[K] = T;
      S.fail_min = 0xFFFFFFFFu;
      S.nkeys = 0;
    }
    __syncthreads();
    for (u32 c = 0; c < T; c += QCH) {
      const u32 cn = T - c < QCH ? T - c : QCH;
      const u32 nblk = (cn + WAVE - 1) / WAVE;
      if (tid < nblk) S.bfirst[tid] = run_of(S.cpre, K, c + tid * WAVE);
      __syncthreads();
      u32 v[QU], kk[QU];
#pragma unroll
      for (u32 u = 0; u < QU; ++u) {
        const u32 qb = u * QW + wid;
        const u32 i = c + qb * WAVE + lane;
        const bool ok = qb < nblk && i < T;
        u32 k = ok ? S.bfirst[qb] : 0;
        if (ok)
          while (S.cpre[k + 1] <= i) ++k;
        kk[u] = k;
        const i64 pos = ok ? S.caddr[k] + (i64)i : 0;
        const u32 x = A.e_pins[pos];
        v[u] = ok ? x : 0xFFFFFFFFu;
      }
      // the first pin >= hi of each stretch (one lane per stretch and wave block)
#pragma unroll
      for (u32 u = 0; u < QU; ++u) {
        const bool bey = v[u] != 0xFFFFFFFFu && v[u] >= hi32;
        const u32 tag = bey ? kk[u] : 0xFFFFFFFFu;
        const u32 ptag = __shfl_up(tag, 1, WAVE);
        if (bey && (lane == 0 || ptag != kk[u])) {
          const u32 i = c + (u * QW + wid) * WAVE + lane;
          atomicMin(&S.cnext[kk[u]], i - S.cpre[kk[u]]);
        }
      }
      if (direct) {
#pragma unroll
        for (u32 u = 0; u < QU; ++u) {
          const u32 x = v[u];
          if (x >= lo32 && x < hi32 && x != n) atomicAdd(&S.t.bin[x - lo32], S.cq[kk[u]]);
        }
      } else {
#pragma unroll
        for (u32 u = 0; u < QU; ++u) {
          const u32 x = v[u];
          if (x >= lo32 && x < hi32 && x != n) {
            const u32 sl2 = q_insert(S, x, hcap);
            if (sl2 == QFAIL) {
              atomicMin(&S.fail_min, x);
              continue;
            }
            atomicAdd(&S.t.h.bin[sl2], S.cq[kk[u]]);
          }
        }
      }
      __syncthreads();
    }
    // next cursors: exact first pin >= hi of every run
    if (tid < nr) S.rcur[tid] = L ? cur + S.cnext[ko] : cur;
    const u32 fmin = rfl(S.fail_min);
    // candidates of the window: the largest valid bin, then the valid bins
    // that can still reach it; every slot is read and left empty
    u64 bl = 0;
    if (direct) {
      // pass 1: the largest valid bin (validity kept as a bit per slot)
      constexpr u32 NS = QD / QB;
      u32 vmax = 0, bad = 0;
#pragma unroll 4
      for (u32 j = 0; j < NS; ++j) {
        const u32 V = S.t.bin[tid + j * QB];
        bool ok = V != 0;
        if (om && ok) ok = size_n + A.n_size[lo32 + tid + j * QB] <= A.omega;
        if (!ok) bad |= 1u << j;
        else vmax = V > vmax ? V : vmax;
      }
      vmax = q_reduce<u32>(vmax, S.red32, [](u32 a, u32 b) { return a > b ? a : b; });
      const u64 T2 = umax64((u64)vmax << s, lstar);
      // pass 2: the bins that can still reach it; every slot left empty
#pragma unroll 4
      for (u32 j = 0; j < NS; ++j) {
        const u32 sl2 = tid + j * QB;
        const u32 V = S.t.bin[sl2];
        S.t.bin[sl2] = 0;
        if (!((bad >> j) & 1u))
          q_judge(A, S, n, lo32 + sl2, V, s, qmin, errunit, ub, T2, dmod, magic, bl);
      }
    } else {
      constexpr u32 NS = QHS / QB;
      u32 vmax = 0, bad = 0;
#pragma unroll 4
      for (u32 j = 0; j < NS; ++j) {
        const u32 sl2 = tid + j * QB;
        const u32 key = S.t.h.key[sl2];
        const u32 V = S.t.h.bin[sl2];
        bool ok = key != 0 && key - 1 < fmin && V != 0;
        if (om && ok) ok = size_n + A.n_size[key - 1] <= A.omega;
        if (!ok) bad |= 1u << j;
        else vmax = V > vmax ? V : vmax;
      }
      vmax = q_reduce<u32>(vmax, S.red32, [](u32 a, u32 b) { return a > b ? a : b; });
      const u64 T2 = umax64((u64)vmax << s, lstar);
#pragma unroll 4
      for (u32 j = 0; j < NS; ++j) {
        const u32 sl2 = tid + j * QB;
        const u32 key = S.t.h.key[sl2];
        const u32 V = S.t.h.bin[sl2];
        S.t.h.key[sl2] = 0;
        S.t.h.bin[sl2] = 0;
        if (!((bad >> j) & 1u)) q_judge(A, S, n, key - 1, V, s, qmin, errunit, ub, T2, dmod, magic, bl);
      }
    }
    lstar = umax64(lstar, q_reduce<u64>(bl, S.red64, [](u64 a, u64 b) { return umax64(a, b); }));
    const bool full = !direct && fmin < hi32;
    last_hi = full ? ~0ull : hi;
    if (!direct) {
      if (full) {
        hspan = (hi - fmin) / 2 > 0 ? (hi - fmin) / 2 : 1;
      } else if (hspan < end - mn) {
        hspan *= 2;
      }
    }
    lo = rfl64(full ? (u64)fmin : hi);
    hspan = rfl64(hspan);
    // the reduction's barriers order the slot clears before the next window's
    // visits and the reads of fail_min before its reset
  }
  const u32 nc = rfl(S.ncont);
  if (nc > QCONT) return false;
  // -- exact eta of the contenders still in reach: t(e) summed over the
  // hyperedges of I(m) that are in I(n); the best by (eta + noise, -id)
  u64 be = 0;
  u32 bi = NONE32;
  for (u32 j = wid; j < nc; j += QW) {
    const u32 m = S.cid[j];
    if (S.cub[j] < lstar) continue;
    const i64 a = A.n_off[m], b = A.n_off[m + 1];
    u64 sum = 0;
    for (i64 p = a + lane; p < b; p += WAVE) {
      const u32 e = A.n_inc[p];
      u32 k = q_lower_bound(S.eid, 0, nin, e);
      if (k == nin || S.eid[k] != e) k = q_lower_bound(S.eid, nin, deg, e);
      if (k < deg && S.eid[k] == e) sum += S.tx[k];
    }
#pragma unroll
    for (int d = WAVE / 2; d > 0; d >>= 1) sum += __shfl_xor(sum, d, WAVE);
    const u64 key = sum + (A.noise_on ? pair_noise(A.seed, n, m, dmod, magic) : 0);
    if (better(key, m, be, bi)) be = key, bi = m;
  }
  if (lane == 0) {
    S.red64[wid] = be;
    S.redi[wid] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    be = 0;
    bi = NONE32;
#pragma unroll
    for (int w = 0; w < QW; ++w)
      if (better(S.red64[w], S.redi[w], be, bi)) be = S.red64[w], bi = S.redi[w];
    A.target[n] = bi;
    A.score[n] = bi == NONE32 ? 0 : be;
  }
  return true;
}

// Nodes are taken one at a time from a counter (thread 0 takes the item, a
// barrier publishes it, and the loop body ends with a barrier so that every
// lane reconverges before the back edge).  A node this kernel cannot rate is
// appended to `spill` for k_rate_inc.
__global__ __launch_bounds__(QB) void k_rate_incq(RateArgs A, const NodeRec *recs, const u32 *cnt,
                                                  const u32 *gmax, u32 *work, u32 hcap,
                                                  NodeRec *spill, u32 *spill_cnt) {
  __shared__ QSmem S;
  const u32 tid = threadIdx.x;
  const u64 cap = A.capinfo[0], dmod = A.capinfo[1], magic = A.capinfo[2];
  const u32 max_size = gmax[0], max_nin = gmax[1];
  const u32 total = *cnt;
  for (u32 i = tid; i < QD; i += QB) S.t.bin[i] = 0;
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
    const bool done = rate_node_q(A, S, h, max_size, max_nin, hcap, cap, dmod, magic);
    if (!done && tid == 0) spill[atomicAdd(spill_cnt, 1u)] = recs[w];
    __syncthreads();
  }
}

}  // namespace

void launch_rate_incq(chp_ctx *c, const RateArgs &a, const NodeRec *recs, const u32 *cnt,
                      const u32 *gmax, u32 *work, u32 host_count, u32 hash_keys, NodeRec *spill,
                      u32 *spill_cnt) {
  if (!host_count) return;
  const u32 g = host_count < c->n_cu ? host_count : c->n_cu;
  const u32 hcap = hash_keys && hash_keys < QCAP ? hash_keys : QCAP;
  CHP_LAUNCH(c, "rate_incq", k_rate_incq, g, QB, 0, a, recs, cnt, gmax, work, hcap, spill,
             spill_cnt);
}
