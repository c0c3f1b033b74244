// Rating straight from the incidence with quantised bins: candidate proposal
// ("Hypergraph Partitioning on GPU with Distinct Incident Hyperedges and Size
// Constraints", Sec. V-A Eqs. 5-6 and Sec. V-C) for nodes of a graph whose
// neighbour lists are not held in memory (Sec. VII-C), when Delta cannot reject
// any neighbour of the node (so no per-neighbour inbound count is needed).
//
// Windows over the node's neighbour ids are visited as in k_rate_inc.hip (a
// sample of every run steers dense windows, slot m - lo, and sparse ones, a
// hash table), but a bin holds a sum of the quantised terms q(e) = t(e) >> s,
// where s is the smallest shift that keeps the node's whole term sum below
// 2^16.  A direct window's bin then takes 16 bits, two ids to a 32-bit word,
// so it covers four times the ids of an exact 64-bit eta (the hash and sketch
// windows keep 32-bit bins).  The bins only bound eta: with V the bin and c
// the number of hyperedges n and m share (at most V / q_min),
//     V << s  <=  eta(n, m)  <=  (V << s) + c * (2^s - 1).
// Each window keeps every valid neighbour whose upper bound (noise at most the
// cap) can still reach the best lower bound seen so far: the contenders.  At
// the node's end the contenders still in reach get their exact eta, the sum of
// t(e) over the hyperedges of I(m) that are also in I(n) (both incidence lists
// sorted), and the best of them by (eta + noise desc, id asc) is the node's
// target.  The result is the exact argmax of the definition; the bounds only
// decide how few neighbours need their exact sum.
//
// The windows run from the first dense one to the largest id, then from the
// smallest id up to that window, so that in most graphs the neighbours that
// share the most hyperedges with n (the dense ids) bound the winner first.
// Once a valid neighbour's lower bound is known, a sparse window is a sketch:
// its bins are indexed by a hash of the id and hold no keys, and a bin's sum
// bounds the quantised sum of every id that falls in it.  When no bin can
// reach the best lower bound, no id of the window can win and the window is
// done; otherwise the same window is visited again with a hash table.
//
// The samples of a run are the first pins of its blocks of 2^sh pins.  Where
// sh >= QSG they come from a per-level array holding every 2^QSG-th pin of
// each run (k_samples_fill), so that a run's samples lie within a line or two
// instead of one line each.
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
constexpr u32 QD = 24576;             // 32-bit words of the bins
constexpr u32 QDD = 2 * QD;           // ids of a direct window (a 16-bit bin each)
constexpr u32 QHS = QD / 2;           // slots of the hash table (key, bin)
constexpr u32 QCAP = QHS * 3 / 4;     // keys a hash window claims before it reports full
constexpr u32 QE = 384;               // incident hyperedges
constexpr u32 QRUNS = 2 * QE;         // a source and a destination run per hyperedge
constexpr u32 QSMAX = 4096;           // sampled blocks
constexpr u32 QSG = 4;                // log2 of the per-level sample array's step
constexpr u32 QNHB = 1024;            // estimate buckets
constexpr u32 QBS_MIN = 12;           // log2 of the narrowest bucket
constexpr u32 QHTGT = QCAP * 3 / 4;   // estimated visits a hash window aims at
constexpr u32 QEST = 16;              // estimates count sixteenths of a visit
constexpr u32 QSK = 16384;            // estimated visits a sketch window aims at
// (on the 4M-node block level, with direct windows from 2 visits per 16 ids,
// 8,192, 12,288 and 16,384 took 1,072, 988 and 972 ms per pass; from 4 per
// 16 ids, 12,288, 16,384 and 24,576 took 955, 938 and 939 ms)
constexpr u32 QU = 16384 / QB;        // pins per thread per chunk
constexpr u32 QCH = QB * QU;          // pins per chunk
constexpr u32 QNBLK = QCH / WAVE;     // wave blocks per chunk
constexpr u32 QCONT = 256;            // contenders a node may keep
constexpr u32 QFAIL = 0xFFFFFFFFu;
static_assert(QB - 1 + QCAP < QHS, "claims in flight never fill the table");
static_assert(QE <= QB && QNBLK <= QB, "one hyperedge (its two runs) and one block per thread");
constexpr u32 QBPT = QNHB / QB;       // estimate buckets per thread
static_assert(QNHB % QB == 0 && QBPT <= 2 && QNHB == 32 * 32,
              "one or two buckets per thread; two-level dense bitmap");
static_assert(QD % QB == 0 && QHS % QB == 0 && QSMAX % QB == 0, "slots per thread");
static_assert(QSMAX <= QD, "the samples' run table fits the bins");
static_assert(QD % (4 * QB) == 0 && QHS % (4 * QB) == 0, "four slots per thread and step");

typedef unsigned short q_u16x2 __attribute__((ext_vector_type(2)));
// the slots (4 words from w0, 16-byte aligned) read and left empty
__device__ __forceinline__ uint4 q_take4(u32 *a, u32 w0) {
  const uint4 x = *reinterpret_cast<const uint4 *>(a + w0);
  *reinterpret_cast<uint4 *>(a + w0) = make_uint4(0u, 0u, 0u, 0u);
  return x;
}
// some 16-bit half of w is above vt (packed saturating subtraction)
__device__ __forceinline__ bool q_half_above(u32 w, u32 vt) {
  const q_u16x2 t = {(unsigned short)vt, (unsigned short)vt};
  return __builtin_bit_cast(u32, __builtin_elementwise_sub_sat(__builtin_bit_cast(q_u16x2, w), t)) != 0;
}

struct QSmem {
  union alignas(16) {
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
  u32 soff[QE];  // its first entry in the per-level sample array
  u32 ens[QE];   // source pins
  u32 elen[QE];  // pins
  u32 q[QE];     // t(e) >> s
  // run r: sources (r even) or destinations (r odd) of hyperedge r / 2
  u32 rcur[QRUNS];     // exact: first pin at or above the window's low end
  u32 rsp[QRUNS + 1];  // first sample of each run
  u32 sfirst[QSMAX];   // first pin of each sampled block
  // the window's non-empty stretches
  i32 caddr[QRUNS];    // e_pins index of flat position 0 of stretch k (fewer than 2^31 pins)
  u32 cpre[QRUNS + 1];
  u32 cq[QRUNS];
  u32 cnext[QRUNS];    // flat position of stretch k's first pin at or above the window's end
  // two buffers: chunk c's and, built while chunk c is visited, chunk c + 1's
  u32 bfirst[2][QNBLK];  // stretch of the first pin of each wave block of a chunk
  u64 sbits[2][QNBLK];   // bit p of word b: a stretch starts at chunk position 64 b + p
  u32 cum[QNHB + 1];   // estimated visits below each bucket (sixteenths)
  u32 dbits[32];       // bucket b starts a dense window

  u32 cid[QCONT];      // contenders: id, upper bound of eta + noise
  u64 cub[QCONT];
  u64 red64[QW + 1];
  u64 wbl[2][QW];      // per wave: best lower bound of a window (by window parity)
  u32 wvmax[QW];       // per wave: largest bin a window's visits left
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

// a value known to be the same on every lane, moved to scalar registers
__device__ __forceinline__ u32 uni(u32 v) { return rfl(v); }
__device__ __forceinline__ u64 uni(u64 v) { return rfl64(v); }

// Row operations on the 16 lanes of a DPP row (one per wave of the
// workgroup): a value moved from another lane of the row, zero where the
// source lies outside it.
static_assert(QW == 16, "one DPP row holds a value per wave");
template <int C>
__device__ __forceinline__ u32 q_dpp(u32 v) {
  return (u32)__builtin_amdgcn_update_dpp(0, (int)v, C, 0xF, 0xF, true);
}
template <int C>
__device__ __forceinline__ u64 q_dpp(u64 v) {
  return (u64)q_dpp<C>((u32)(v >> 32)) << 32 | q_dpp<C>((u32)v);
}
// every lane of a row ends with op over the row's 16 values
template <typename T, typename Op>
__device__ __forceinline__ T q_row_reduce(T v, Op op) {
  v = op(v, q_dpp<0xB1>(v));   // quad_perm [1,0,3,2]
  v = op(v, q_dpp<0x4E>(v));   // quad_perm [2,3,0,1]
  v = op(v, q_dpp<0x141>(v));  // row_half_mirror
  v = op(v, q_dpp<0x140>(v));  // row_mirror
  return v;
}
// lane i of a row ends with the sum of the row's values 0 .. i
template <typename T>
__device__ __forceinline__ T q_row_scan(T v) {
  v += q_dpp<0x111>(v);  // row_shr:1
  v += q_dpp<0x112>(v);  // row_shr:2
  v += q_dpp<0x114>(v);  // row_shr:4
  v += q_dpp<0x118>(v);  // row_shr:8
  return v;
}
// inclusive prefix over the whole wave: the row prefix, then row 0's total
// into row 1 and row 2's into row 3 (row_bcast:15), then the total of rows
// 0-1 into rows 2 and 3 (row_bcast:31); rows left out keep their value
__device__ __forceinline__ u32 q_wave_scan(u32 v) {
  v = q_row_scan(v);
  v += (u32)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);
  v += (u32)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);
  return v;
}
// the same for two independent 32-bit halves (their sums never carry)
__device__ __forceinline__ u64 q_wave_scan(u64 v) {
  return (u64)q_wave_scan((u32)(v >> 32)) << 32 | q_wave_scan((u32)v);
}
__device__ __forceinline__ u32 q_lane(u32 v, u32 l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ u64 q_lane(u64 v, u32 l) {
  return (u64)(u32)__builtin_amdgcn_readlane((u32)(v >> 32), l) << 32 |
         (u32)__builtin_amdgcn_readlane((u32)v, l);
}
// op over the 16 per-wave values of a[], in every lane
template <typename T, typename Op>
__device__ __forceinline__ T q_fold(const T *a, Op op) {
  return q_lane(q_row_reduce(a[lane_id() & (QW - 1)], op), 0u);
}

__device__ __forceinline__ u32 qslot(u32 m) { return (u32)(((u64)(m * 0x9E3779B1u) * QHS) >> 32); }
__device__ __forceinline__ u32 qsketch(u32 m) { return (u32)(((u64)(m * 0x9E3779B1u) * QD) >> 32); }

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

// The node's hyperedges, hashed into the emptied bins for the contenders'
// exact sums: slot i is the 16 bytes from word 4 i, (e + 1, 0, t(e) low, high)
constexpr u32 QEH = 2048;
static_assert(4 * QEH <= QD && QE <= QEH / 4, "the hyperedge table fits the bins, a quarter full");
__device__ __forceinline__ u32 q_eslot(u32 e) { return (e * 0x9E3779B1u) >> 21; }
static_assert(QEH == 1u << 11, "slot hash");

// e's slot, claimed (the hyperedges of a node are distinct)
__device__ __forceinline__ u32 q_einsert(QSmem &S, u32 e, u64 te) {
  u32 i = q_eslot(e);
  while (atomicCAS(&S.t.bin[4 * i], 0u, e + 1) != 0) i = (i + 1) & (QEH - 1);
  S.t.bin[4 * i + 2] = (u32)te;
  S.t.bin[4 * i + 3] = (u32)(te >> 32);
  return i;
}

// t(e) if e is one of the node's hyperedges, else 0
__device__ __forceinline__ u64 q_efind(const QSmem &S, u32 e) {
  for (u32 i = q_eslot(e);; i = (i + 1) & (QEH - 1)) {
    const uint4 x = *reinterpret_cast<const uint4 *>(&S.t.bin[4 * i]);
    if (x.x == e + 1) return (u64)x.w << 32 | x.z;
    if (x.x == 0) return 0;
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

// largest i in [0, n) with pre[i] <= v (pre[0] <= v, pre ascending, n <= 2^STEPS),
// in STEPS fixed steps
template <u32 STEPS>
__device__ __forceinline__ u32 q_run_of(const u32 *pre, u32 n, u32 v) {
  u32 lo = 0;
#pragma unroll
  for (int b = (int)STEPS - 1; b >= 0; --b) {
    const u32 mid = lo + (1u << b);
    if (mid < n && pre[mid] <= v) lo = mid;
  }
  return lo;
}
constexpr u32 QRUN_STEPS = 10;
static_assert(QRUNS <= (1u << QRUN_STEPS), "stretches in QRUN_STEPS steps");

// first bucket >= b that starts a dense window, else nbk
__device__ __forceinline__ u32 q_first_dense(const QSmem &S, u32 dsum, u32 b, u32 nbk) {
  if (b >= nbk) return nbk;
  u32 w = b >> 5;
  u32 m = S.dbits[w] & (~0u << (b & 31));
  if (!m) {
    const u32 ws = w + 1;
    if (ws >= 32) return nbk;
    const u32 m2 = dsum & (~0u << ws);
    if (!m2) return nbk;
    w = (u32)__builtin_ctz(m2);
    m = S.dbits[w];
  }
  const u32 r = (w << 5) + (u32)__builtin_ctz(m);
  return r < nbk ? r : nbk;
}

// Workgroup reductions and scans over the per-wave partials in lds.  With
// TRAIL false they end without the barrier that protects lds from the next
// writer: the caller then uses another buffer before the next barrier.
template <bool TRAIL = true, typename T, typename Op>
__device__ __forceinline__ T q_reduce(T v, T *lds, Op op) {
#pragma unroll
  for (int d = WAVE / 2; d > 0; d >>= 1) v = op(v, (T)__shfl_xor(v, d, WAVE));
  if (lane_id() == 0) lds[wave_id()] = v;
  __syncthreads();
  const T r = q_fold(lds, op);
  if (TRAIL) __syncthreads();
  return r;
}

// exclusive prefix of v over the workgroup, *total the sum (lds: QW entries);
// a 64-bit v is two 32-bit counts whose sums stay below 2^32
template <typename T>
__device__ __forceinline__ T q_scan(T v, T *lds, T *total) {
  const T inc = q_wave_scan(v);
  if (lane_id() == WAVE - 1) lds[wave_id()] = inc;
  __syncthreads();
  const T x = q_row_scan(lds[lane_id() & (QW - 1)]);
  const u32 ws = rfl(wave_id());
  *total = q_lane(x, QW - 1);
  return (ws ? q_lane(x, ws - 1) : (T)0) + inc - v;
}

__device__ __forceinline__ u64 umax64(u64 a, u64 b) { return a > b ? a : b; }

// Two reductions over the workgroup with one pair of barriers; lds holds 2 QW.
template <bool TRAIL = true, typename T, typename Op1, typename Op2>
__device__ __forceinline__ void q_reduce2(T &v1, T &v2, T *lds, Op1 op1, Op2 op2) {
#pragma unroll
  for (int d = WAVE / 2; d > 0; d >>= 1) {
    v1 = op1(v1, (T)__shfl_xor(v1, d, WAVE));
    v2 = op2(v2, (T)__shfl_xor(v2, d, WAVE));
  }
  if (lane_id() == 0) {
    lds[wave_id()] = v1;
    lds[QW + wave_id()] = v2;
  }
  __syncthreads();
  v1 = q_fold(lds, op1);
  v2 = q_fold(lds + QW, op2);
  if (TRAIL) __syncthreads();
}

// A bin value below which no bin can reach T: every V < q_vthr(...) has
// (V << s) + floor(V / qmin) * errunit + ub < T.  The real bound
// V * (2^s + errunit / qmin) + ub is at least that sum, so V below
// x = (T - ub) / (2^s + errunit / qmin) cannot reach T; floor(x) - 1 keeps
// the double's rounding of x on the safe side.  Bins at or above it are
// judged exactly.
__device__ __forceinline__ u32 q_vthr(u64 T, u32 s, u32 qmin, u64 errunit, u64 ub) {
  if (T <= ub) return 0;
  const double x = (double)(T - ub) / ((double)(1ull << s) + (double)errunit / (double)qmin);
  const double f = floor(x) - 1.0;
  return f <= 0.0 ? 0u : f >= 4294967295.0 ? 0xFFFFFFFFu : (u32)f;
}

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
                            u32 max_nin, u32 hcap, u64 cap, u64 dmod, u64 magic,
                            const i64 *samp_off, const u32 *samp) {
  // the thread index is re-read per node through an empty asm, so that the
  // compiler recomputes the slot addresses derived from it inside each node
  // instead of holding dozens of them in registers across the node loop
  u32 tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  u32 lane = tid & (WAVE - 1), wid = tid / WAVE;
  const u32 n = h.n, deg = h.deg, nin = h.nin, nr = 2 * deg;
  const u64 size_n = h.size, W = (u64)h.nb0;
  const bool om = size_n + max_size > A.omega;  // Omega can reject a neighbour
  if ((u64)nin + max_nin > (u64)A.delta || deg > QE) return false;
  const u64 ub = A.noise_on ? cap : 0;
  // -- incident hyperedges; the term sum and the smallest term decide s
  u64 te = 0;
  u32 l0 = 0, l1 = 0;
  i64 a = 0, b = 0;
  bool counts = false;
  if (tid < deg) {
    const u32 e = A.n_inc[h.i0 + tid];
    a = A.e_off[e];
    b = A.e_off[e + 1];
    const u32 ns = A.e_nsrc[e];
    te = A.t[e];
    counts = b - a >= 2;
    l0 = ns;
    l1 = (u32)(b - a) - ns;
    S.eoff[tid] = a;
    S.tx[tid] = te;
    S.eid[tid] = e;
    if (samp) S.soff[tid] = (u32)samp_off[e];
    S.ens[tid] = ns;
    S.elen[tid] = (u32)(b - a);
  }
  u64 tsum = counts ? te : 0, tmin = counts ? te : ~0ull;
  // (the buffers of consecutive reductions and scans alternate, so that no
  // barrier is needed after each)
  q_reduce2<false>(tsum, tmin, S.cub, [](u64 x, u64 y) { return sat_add(x, y); },
                   [](u64 x, u64 y) { return x < y ? x : y; });
  if (sat_add(tsum, cap) >= (1ull << 63)) {
    if (tid == 0) {
      atomicOr(A.flags, FLAG_EOVERFLOW);
      A.target[n] = NONE32;
      A.score[n] = 0;
    }
    return true;
  }
  // the bit length of tsum >> 16, so that tsum >> s < 2^16: no id's sum of
  // quantised terms reaches 2^16, so a direct window packs two ids' bins in
  // each 32-bit word (its adds never carry from one half into the other)
  const u32 s = tsum >> 16 ? 64u - (u32)__builtin_clzll(tsum >> 16) : 0u;
  const u32 qmin = (u32)(tmin >> s);
  if (tsum && qmin == 0) return false;
  const u64 errunit = (1ull << s) - 1;
  if (tid < deg) S.q[tid] = (u32)(te >> s);
  // -- samples: blocks of 2^sh pins, so that at most QSMAX blocks are needed
  u32 sh = 0;
  while (((u64)(QSMAX - nr) << sh) < W) ++sh;
  const u32 c0 = (l0 + (1u << sh) - 1) >> sh, c1 = (l1 + (1u << sh) - 1) >> sh;
  u32 ts;
  const u32 so = q_scan<u32>(c0 + c1, S.red32, &ts);
  ts = rfl(ts);
  if (tid < deg) {
    S.rsp[2 * tid] = so;
    S.rsp[2 * tid + 1] = so + c0;
    // the run of every sample, in the (empty) bins until the samples are read
    for (u32 g = so; g < so + c0 + c1; ++g) S.t.bin[g] = g < so + c0 ? 2 * tid : 2 * tid + 1;
  }
  if (tid < deg) {  // every pin is >= the first window's low end
    S.rcur[2 * tid] = 0;
    S.rcur[2 * tid + 1] = 0;
  }
  if (tid == 0) S.rsp[nr] = ts;
  for (u32 b = tid; b <= QNHB; b += QB) S.cum[b] = 0;
  __syncthreads();
  // (only the first pin of a block is read; a block's pins then lie between
  // it and the next block's first pin, or the run's last pin, read by the
  // run's thread into rlast, which is cnext until the windows)
  u32 *const rlast = S.cnext;
  constexpr u32 SPT = QSMAX / QB;
  const bool from_samp = samp && sh >= QSG;
  u32 sf[SPT], sw[SPT], sr[SPT];
  u32 mn = 0xFFFFFFFFu, mx = 0;
  if (tid < deg) {
    if (l0) mx = rlast[2 * tid] = A.e_pins[a + l0 - 1];
    if (l1) {
      const u32 x = A.e_pins[b - 1];
      rlast[2 * tid + 1] = x;
      mx = x > mx ? x : mx;
    }
  }
#pragma unroll
  for (u32 k = 0; k < SPT; ++k) {
    const u32 g = tid + k * QB;
    sf[k] = 0;
    sw[k] = 0;
    sr[k] = 0;
    if (g < ts) {
      const u32 r = S.t.bin[g];
      S.t.bin[g] = 0;  // (the bins are empty again before the windows)
      const u32 ke = r >> 1;
      const u32 len = (r & 1) ? S.elen[ke] - S.ens[ke] : S.ens[ke];
      const i64 base = S.eoff[ke] + ((r & 1) ? S.ens[ke] : 0);
      const u32 p0 = (g - S.rsp[r]) << sh;
      const u32 p1 = (p0 + (1u << sh) < len ? p0 + (1u << sh) : len) - 1;
      sf[k] = from_samp ? samp[S.soff[ke] + ((r & 1) ? (S.ens[ke] + (1u << QSG) - 1) >> QSG : 0u) +
                               (p0 >> QSG)]
                        : A.e_pins[base + p0];
      sw[k] = p1 + 1 - p0;
      sr[k] = r;
    }
  }
#pragma unroll
  for (u32 k = 0; k < SPT; ++k) {
    const u32 g = tid + k * QB;
    if (g < ts) {
      S.sfirst[g] = sf[k];
      mn = sf[k] < mn ? sf[k] : mn;
    }
  }
  q_reduce2<false>(mn, mx, S.cid, [](u32 a, u32 b) { return a < b ? a : b; },
                 [](u32 a, u32 b) { return a > b ? a : b; });
  // -- estimated visits over buckets of 2^bs ids from mn, in 1/16 of a visit:
  // each block's pins spread evenly over the buckets from its first pin's to
  // its last pin's bound (a difference array, then two scans)
  u32 bs = QBS_MIN;
  while (((mx - mn) >> bs) >= QNHB) ++bs;
  const u32 nbk = ((mx - mn) >> bs) + 1;
#pragma unroll
  for (u32 k = 0; k < SPT; ++k) {
    const u32 g = tid + k * QB;
    if (g < ts) {
      const u32 r = sr[k];
      const u32 last = g + 1 < S.rsp[r + 1] ? S.sfirst[g + 1] - 1 : rlast[r];
      const u32 bf = (sf[k] - mn) >> bs, bl = (last - mn) >> bs;
      const u32 unit = sw[k] * QEST, span = bl - bf + 1;
      // floor(unit / span) from a reciprocal (unit < 2^20: one step of
      // correction either way makes it exact)
      u32 qd = (u32)((float)unit * __builtin_amdgcn_rcpf((float)span));
      qd -= qd * span > unit ? 1u : 0u;
      qd += (qd + 1) * span <= unit ? 1u : 0u;
      const u32 rem = unit - qd * span;
      atomicAdd(&S.cum[bf], qd + rem);
      atomicSub(&S.cum[bf + 1], rem);
      atomicSub(&S.cum[bl + 1], qd);
    }
  }
  __syncthreads();
  {
    const u32 d0 = S.cum[QBPT * tid], d1 = QBPT > 1 ? S.cum[QBPT * tid + 1] : 0;
    u32 tot;
    const u32 e = q_scan<u32>(d0 + d1, S.red32, &tot);  // mod 2^32: the sums are exact
    const u32 v0 = e + d0, v1 = e + d0 + d1;                  // estimates of the buckets
    const u32 off = q_scan<u32>(QBPT > 1 ? v0 + v1 : v0, S.cid, &tot);
    S.cum[QBPT * tid] = off;
    if (QBPT > 1) S.cum[QBPT * tid + 1] = off + v0;
    if (tid == 0) S.cum[QNHB] = tot;
  }
  __syncthreads();
  // estimated visits that make a window direct: 6 per 16 ids.  On the
  // 4M-node block level, with sketches of 16,384 estimated visits, 3, 4, 5
  // and 6 per 16 ids took 946, 938, 926 and 917 ms per pass and 8 per 16
  // ids 1,480 ms; 2 per 16 with sketches of 12,288 took 988 ms
  const u32 dense = QDD * 3 / 8 * QEST;
  {
    const u32 wb = (QDD >> bs) > 0 ? (QDD >> bs) : 1;  // buckets of a direct window
#pragma unroll
    for (u32 h2 = 0; h2 < QBPT; ++h2) {
      const u32 b = tid + h2 * QB;
      const u32 bend = b + wb < nbk ? b + wb : nbk;
      const bool dn = b < nbk && S.cum[bend] - S.cum[b] >= dense;
      const u64 bal = __ballot(dn);
      if (lane == 0) {
        S.dbits[(b >> 5)] = (u32)bal;
        S.dbits[(b >> 5) + 1] = (u32)(bal >> 32);
      }
    }
    if (tid == 0) S.ncont = 0;
    if (tid < 2 * QW) S.wbl[tid / QW][tid % QW] = 0;
    __syncthreads();
  }
  // bit w: dense bits word w is not zero (each wave finds it)
  const u32 dsum = (u32)__builtin_amdgcn_ballot_w64(lane < 32 && S.dbits[lane & 31] != 0);
  // -- windows over [mn, mx]: from the first dense window to mx, then from mn
  // up to that window, so that the dense ones (in most graphs the best
  // neighbours) set a high bound before the sparse ones are visited
  u64 lstar = 0;  // best lower bound of eta + noise so far (a valid neighbour's)
  const u64 end = (u64)mx + 1;
  const u32 bd0 = q_first_dense(S, dsum, 0, nbk);
  const u64 start = bd0 < nbk ? (u64)mn + ((u64)bd0 << bs) : (u64)mn;
  u64 lo = start, wend = end;
  bool wrapped = start == mn;
  u64 hspan = end - mn;  // id span a hash window may take (halved after one fills)
  u64 last_hi = start == mn ? mn : ~0ull;  // end of the last window if it did not fill
  u32 par = 0;           // parity of the window (the wbl buffer it writes)
  bool redo = false;     // the last window was a sketch with a hot slot: hash it
  for (;;) {
    if (lo >= wend) {
      if (wrapped) break;
      wrapped = true;
      lo = mn;
      wend = start;
      last_hi = mn;
      if (tid < deg) {  // every pin is >= mn: the cursors restart at the runs' starts
        S.rcur[2 * tid] = 0;
        S.rcur[2 * tid + 1] = 0;
      }
    }
    // (the same re-read per window: what derives from the thread index is
    // recomputed here rather than held across windows)
    asm volatile("" : "+v"(tid));
    lane = tid & (WAVE - 1);
    wid = tid / WAVE;
    const u32 b0 = (u32)((lo - mn) >> bs);
    const u64 dhi = lo + QDD < wend ? lo + QDD : wend;
    const u32 bde = (u32)((dhi - 1 - mn) >> bs) + 1;
    const u32 est = S.cum[bde < nbk ? bde : nbk] - S.cum[b0];
    const bool direct =
        rfl(est >= dense || S.cum[b0 + 1] - S.cum[b0] > QHTGT * QEST ? 1u : 0u) != 0;
    // a sparse window is a sketch (bins indexed by a hash of the id, no keys)
    // once some valid neighbour bounds the winner from below: every id of a
    // slot whose sum cannot reach that bound is out of the running
    const bool sk0 = !direct && lstar != 0 && !redo;
    u64 hi = dhi;
    if (!direct) {
      // the last bucket l in [b0 + 1, nbk] whose estimate from b0 stays within
      // tgt (b0 + 1 when none does), 64 candidates a step, one per lane (the
      // estimates grow with l, so the lanes that hold are a prefix)
      const u32 tgt = (sk0 ? QSK : QHTGT) * QEST;
      const u32 cb0 = S.cum[b0];
      u32 l = b0 + 1, r = nbk;
      while (l < r) {
        const u32 step = (r - l + WAVE) / WAVE;
        const u32 idx = l + lane * step;
        const u32 cnt = (u32)__builtin_popcountll(
            __builtin_amdgcn_ballot_w64(idx <= r && S.cum[idx] - cb0 <= tgt));
        if (cnt == 0) break;
        l += (cnt - 1) * step;
        r = l + step - 1 < r ? l + step - 1 : r;
        if (step == 1) break;
      }
      const u32 bd = q_first_dense(S, dsum, b0 + 1, nbk);
      const u32 b1 = bd < l ? bd : l;
      hi = b1 >= nbk ? wend : (u64)mn + ((u64)b1 << bs);
      hi = hi < wend ? hi : wend;
      if (!sk0 && hi - lo > hspan) hi = lo + hspan;
    }
    hi = rfl64(hi);
    const u32 lo32 = (u32)lo, hi32 = (u32)(hi < 0xFFFFFFFFull ? hi : 0xFFFFFFFFull);
    const bool exact = lo == last_hi;
    // each run's stretch: from its cursor (or, after a window that filled, the
    // sampled block holding its first pin >= lo) to the first sampled block
    // starting at or above hi
    // (thread tid holds hyperedge tid's source run 2 tid and destination run
    // 2 tid + 1)
    u32 L[2] = {0, 0}, cur[2] = {0, 0};
    if (tid < deg) {
#pragma unroll
      for (u32 j = 0; j < 2; ++j) {
        const u32 r = 2 * tid + j;
        const u32 g0 = S.rsp[r], g1 = S.rsp[r + 1];
        const u32 len = j ? S.elen[tid] - S.ens[tid] : S.ens[tid];
        if (exact) {
          cur[j] = S.rcur[r];
        } else {
          const u32 kb = q_lower_bound(S.sfirst, g0, g1, lo32);
          cur[j] = kb > g0 ? (kb - 1 - g0) << sh : 0;
        }
        const u32 kh = q_lower_bound(S.sfirst, g0, g1, hi32);
        const u32 e0 = ((kh - g0) << sh) < len ? ((kh - g0) << sh) : len;
        L[j] = e0 > cur[j] ? e0 - cur[j] : 0;
      }
    }
    // one scan of (pins << 32 | non-empty): offsets and compacted indices
    u64 tk;
    const u64 pk = q_scan<u64>(((u64)(L[0] + L[1]) << 32) |
                                             ((L[0] ? 1u : 0u) + (L[1] ? 1u : 0u)),
                                         S.red64, &tk);
    const u32 T = rfl((u32)(tk >> 32)), K = rfl((u32)tk);
    // a sketch slot's sum stays below 2^32: each of fewer than 2^16 pins adds
    // less than 2^16 (otherwise the window takes the hash table)
    const bool sk = sk0 && T < (1u << 16);
    u32 po[2], ko[2];
    po[0] = (u32)(pk >> 32);
    ko[0] = (u32)pk;
    po[1] = po[0] + L[0];
    ko[1] = ko[0] + (L[0] ? 1u : 0u);
    // (and the first chunk's stretch starts: the wave blocks whose first
    // position the stretch holds, and its start bit; the words are clear)
#pragma unroll
    for (u32 j = 0; j < 2; ++j) {
      if (L[j]) {
        S.caddr[ko[j]] = (i32)(S.eoff[tid] + (j ? S.ens[tid] : 0) + cur[j] - (i64)po[j]);
        S.cpre[ko[j]] = po[j];
        S.cq[ko[j]] = S.q[tid];
        S.cnext[ko[j]] = po[j] + L[j];
        const u32 pe = po[j] + L[j];
        for (u32 b = (po[j] + WAVE - 1) / WAVE; b < QNBLK && b * WAVE < pe; ++b)
          S.bfirst[0][b] = ko[j];
        if (po[j] < QCH)
          atomicOr((unsigned long long *)&S.sbits[0][po[j] >> 6], 1ull << (po[j] & 63));
      }
    }
    if (tid == 0) {
      S.cpre[K] = T;
      S.fail_min = 0xFFFFFFFFu;
      S.nkeys = 0;
    }
    if (tid < QW) S.wvmax[tid] = 0;
    __syncthreads();
    u32 vmax = 0;  // largest bin left by this thread's visits (Omega cannot bind)
    u32 cb = 0;    // buffer of this chunk's stretch starts
    for (u32 c = 0; c < T; c += QCH, cb ^= 1) {
      const u32 cn = T - c < QCH ? T - c : QCH;
      const u32 nblk = (cn + WAVE - 1) / WAVE;
      // where the stretches start in the next chunk, into the other buffer
      // (cleared by the lanes that read it, two chunks ago): the stretch of
      // position i is the one holding its wave block's first position plus
      // the starts after that position and up to i
      if (c + QCH < T) {
        const u32 c2 = c + QCH, cn2 = T - c2 < QCH ? T - c2 : QCH;
        if (tid < (cn2 + WAVE - 1) / WAVE)
          S.bfirst[cb ^ 1][tid] = q_run_of<QRUN_STEPS>(S.cpre, K, c2 + tid * WAVE);
        for (u32 k = tid; k < K; k += QB) {
          const u32 p = S.cpre[k];
          if (p >= c2 && p - c2 < cn2)
            atomicOr((unsigned long long *)&S.sbits[cb ^ 1][(p - c2) >> 6],
                     1ull << ((p - c2) & 63));
        }
      }
      // lane u (< QU) of the wave reads the first stretch and the start bits of
      // the wave's block of u; every u then takes them from that lane into
      // scalar registers, so one LDS read per pin remains (its stretch's
      // address) and all of them issue before the first wait
      static_assert(QU <= WAVE, "one lane per u");
      const u32 myq = lane * QW + wid;
      const u32 myc = lane < QU && myq < nblk ? myq : 0;
      const u32 bf_l = S.bfirst[cb][myc];
      const u64 sb_l = S.sbits[cb][myc];
      if (lane < QU && myq < nblk) S.sbits[cb][myq] = 0;  // read once: left clear
      // phase by phase for all u: stretch of each pin, its address, the pin.
      // The block of u starts at flat position pbase(u) = c + (u QW + ws) 64
      // (a scalar value)
      const u32 ws = rfl(wid);
      auto pbase = [&](u32 u) { return c + (u * QW + ws) * WAVE; };
      // a lane's position is in the chunk when it is below T (the blocks of
      // u all lie below c + QCH)
      auto lim = [&](u32 u) { return (int)(T - pbase(u)); };
      // (a lane outside the chunk gets some stretch of the chunk, read but
      // unused; its load is redirected and its pin reads as hi: in no
      // window, and past the end of every stretch of the chunk)
      u32 kk[QU], v[QU];
#pragma unroll
      for (u32 u = 0; u < QU; ++u) {
        const u32 k0 = __builtin_amdgcn_readlane(bf_l, u);
        // starts at block positions 1 .. lane: the set bits of bits >> 1 below
        // this lane (the lane-mask count)
        const u64 sb = ((u64)(u32)__builtin_amdgcn_readlane((u32)(sb_l >> 32), u) << 32 |
                        (u32)__builtin_amdgcn_readlane((u32)sb_l, u)) >> 1;
        const u32 k = k0 + __builtin_amdgcn_mbcnt_hi((u32)(sb >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((u32)sb, 0u));
        kk[u] = k;
      }
      i32 ca[QU];
#pragma unroll
      for (u32 u = 0; u < QU; ++u) ca[u] = S.caddr[kk[u]];
#pragma unroll
      for (u32 u = 0; u < QU; ++u)
        v[u] = A.e_pins[(int)lane < lim(u) ? (u32)(ca[u] + (i32)(pbase(u) + lane)) : 0u];
#pragma unroll
      for (u32 u = 0; u < QU; ++u) v[u] = (int)lane < lim(u) ? v[u] : hi32;
      // the first pin >= hi of each stretch: a lane whose pin is >= hi while
      // the lane before holds a pin < hi of the same stretch does not qualify
      // (one lane per stretch and wave block; the block's first position
      // counts as a stretch start)
#pragma unroll
      for (u32 u = 0; u < QU; ++u) {
        const u64 B = __builtin_amdgcn_ballot_w64(v[u] >= hi32);
        const u64 st = ((u64)(u32)__builtin_amdgcn_readlane((u32)(sb_l >> 32), u) << 32 |
                        (u32)__builtin_amdgcn_readlane((u32)sb_l, u)) | 1ull;
        const u64 first = B & ~((B << 1) & ~st);
        if (__builtin_amdgcn_inverse_ballot_w64(first))
          atomicMin(&S.cnext[kk[u]], pbase(u) + lane);
      }
      u32 qv[QU];
#pragma unroll
      for (u32 u = 0; u < QU; ++u) qv[u] = S.cq[kk[u]];
      const u32 span = hi32 - lo32;
      if (direct) {
        // (the largest bin is found by the candidate pass)
#pragma unroll
        for (u32 u = 0; u < QU; ++u) {
          const u32 r = v[u] - lo32;
          if (r < span && v[u] != n) atomicAdd(&S.t.bin[r >> 1], qv[u] << ((r & 1u) << 4));
        }
      } else if (sk) {
#pragma unroll
        for (u32 u = 0; u < QU; ++u) {
          const u32 x = v[u];
          if (x - lo32 < span && x != n) atomicAdd(&S.t.bin[qsketch(x)], qv[u]);
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
            const u32 q = qv[u];
            const u32 o = atomicAdd(&S.t.h.bin[sl2], q) + q;
            vmax = o > vmax ? o : vmax;
          }
        }
      }
      if (!om && !sk && !direct) {
        u32 wv = vmax;
#pragma unroll
        for (int d = WAVE / 2; d > 0; d >>= 1) {
          const u32 o = __shfl_xor(wv, d, WAVE);
          wv = o > wv ? o : wv;
        }
        if (lane == 0) S.wvmax[wid] = wv;
      }
      __syncthreads();
    }
    if (sk) {
      // the sketch: a slot whose sum, as an upper bound for every id in it,
      // can reach the best lower bound makes the window a hash window (from
      // the same cursors); every slot is read and left empty
      lstar = umax64(lstar, q_fold(S.wbl[par ^ 1], umax64));
      // (a slot at or above the real-valued bound counts as hot: at worst a
      // window more is hashed)
      u32 hot = 0;
      const u32 vthr = q_vthr(lstar, s, qmin, errunit, ub);
      const u32 vt = vthr ? vthr - 1 : 0;  // a non-empty slot of at least vthr: above vt
#pragma unroll
      for (u32 j = 0; j < QD / (4 * QB); ++j) {
        const uint4 x = q_take4(S.t.bin, 4 * (tid + j * QB));
        hot |= (x.x > vt) | (x.y > vt) | (x.z > vt) | (x.w > vt);
      }
      hot = q_reduce<false>(hot, S.red32, [](u32 a, u32 b) { return a | b; });
      redo = hot != 0;
      if (!redo) {
        if (tid < deg) {
#pragma unroll
          for (u32 j = 0; j < 2; ++j) S.rcur[2 * tid + j] = L[j] ? cur[j] + (S.cnext[ko[j]] - po[j]) : cur[j];
        }
        last_hi = hi;  // (the cursors found above are exact in any case)
        lo = hi;
      }
      continue;
    }
    redo = false;
    // next cursors: exact first pin >= hi of every run
    if (tid < deg) {
#pragma unroll
      for (u32 j = 0; j < 2; ++j) S.rcur[2 * tid + j] = L[j] ? cur[j] + (S.cnext[ko[j]] - po[j]) : cur[j];
    }
    const u32 fmin = rfl(S.fail_min);
    // candidates of the window: the largest valid bin, then the valid bins
    // that can still reach it; every slot is read and left empty
    // the best lower bound of the windows before (their per-wave maxima were
    // published by the barriers since)
    lstar = umax64(lstar, q_fold(S.wbl[par ^ 1], umax64));
    // candidates: the largest valid bin bounds the winner's eta + noise from
    // below; the valid bins that can still reach that bound are judged.  Every
    // slot is read and left empty.
    u32 vstar = 0;
    u64 bl = 0;
    if (om) {
      // Omega can reject neighbours: the largest valid bin needs a pass of its own
      if (direct) {
        for (u32 j = 0; j < QD / QB; ++j) {
          const u32 w = S.t.bin[tid + j * QB];
          const u32 m = lo32 + 2 * (tid + j * QB);
          const u32 V0 = w & 0xFFFFu, V1 = w >> 16;
          if (V0 && size_n + A.n_size[m] <= A.omega) vstar = V0 > vstar ? V0 : vstar;
          if (V1 && size_n + A.n_size[m + 1] <= A.omega) vstar = V1 > vstar ? V1 : vstar;
        }
      } else {
        for (u32 j = 0; j < QHS / QB; ++j) {
          const u32 key = S.t.h.key[tid + j * QB];
          const u32 V = S.t.h.bin[tid + j * QB];
          if (key != 0 && key - 1 < fmin && V && size_n + A.n_size[key - 1] <= A.omega)
            vstar = V > vstar ? V : vstar;
        }
      }
      vstar = q_reduce<false>(vstar, S.red32, [](u32 a, u32 b) { return a > b ? a : b; });
    } else if (direct) {
      // every neighbour is valid: the largest 16-bit bin, a pass of its own
      q_u16x2 m2 = {0, 0};
#pragma unroll
      for (u32 j = 0; j < QD / (4 * QB); ++j) {
        const uint4 x = *reinterpret_cast<const uint4 *>(&S.t.bin[4 * (tid + j * QB)]);
        m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(q_u16x2, x.x));
        m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(q_u16x2, x.y));
        m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(q_u16x2, x.z));
        m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(q_u16x2, x.w));
      }
      vstar = q_reduce<false>(m2[0] > m2[1] ? (u32)m2[0] : (u32)m2[1], S.red32,
                              [](u32 a, u32 b) { return a > b ? a : b; });
    } else {
      // every neighbour is valid; the visits' returned sums gave the largest
      // bin (a key dropped by a full hash window holds a partial sum, still a
      // lower bound of a valid neighbour's eta)
      vstar = q_fold(S.wvmax, [](u32 a, u32 b) { return a > b ? a : b; });
    }
    const u64 T2 = umax64((u64)vstar << s, lstar);
    const u32 vthr = q_vthr(T2, s, qmin, errunit, ub);
    // (four slots per thread and step; a slot is looked at only when its
    // value, or one of its two 16-bit bins, is non-zero and reaches vthr)
    const u32 vt = vthr ? vthr - 1 : 0;
    if (direct) {
      const u32 vt16 = vt < 0xFFFFu ? vt : 0xFFFFu;
#pragma unroll 1
      for (u32 j = 0; j < QD / (4 * QB); ++j) {
        const u32 w0 = 4 * (tid + j * QB);
        const uint4 x = q_take4(S.t.bin, w0);
        const u32 xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (u32 e = 0; e < 4; ++e) {
          if (!q_half_above(xs[e], vt16)) continue;
#pragma unroll
          for (u32 b = 0; b < 2; ++b) {
            const u32 V = (xs[e] >> (16 * b)) & 0xFFFFu;
            const u32 m = lo32 + 2 * (w0 + e) + b;
            if (V > vt && (!om || size_n + A.n_size[m] <= A.omega))
              q_judge(A, S, n, m, V, s, qmin, errunit, ub, T2, dmod, magic, bl);
          }
        }
      }
    } else {
#pragma unroll 1
      for (u32 j = 0; j < QHS / (4 * QB); ++j) {
        const u32 w0 = 4 * (tid + j * QB);
        const uint4 kx = q_take4(S.t.h.key, w0), bx = q_take4(S.t.h.bin, w0);
        const u32 ks[4] = {kx.x, kx.y, kx.z, kx.w}, vs[4] = {bx.x, bx.y, bx.z, bx.w};
#pragma unroll
        for (u32 e = 0; e < 4; ++e) {
          const u32 m = ks[e] - 1;  // (a key of 0: no id, m = 0xFFFFFFFF >= fmin)
          if (m < fmin && vs[e] > vt && (!om || size_n + A.n_size[m] <= A.omega))
            q_judge(A, S, n, m, vs[e], s, qmin, errunit, ub, T2, dmod, magic, bl);
        }
      }
    }
    // this window's best lower bound, per wave (read after the next barrier)
#pragma unroll
    for (int d = WAVE / 2; d > 0; d >>= 1) bl = umax64(bl, __shfl_xor(bl, d, WAVE));
    if (lane == 0) S.wbl[par][wid] = bl;
    par ^= 1;
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
    // the next window's scan barriers order the slot clears before its
    // visits, and the reads of fail_min, wvmax and wbl before their reuse
  }
  __syncthreads();
  lstar = umax64(lstar, q_fold(S.wbl[par ^ 1], umax64));
  const u32 nc = rfl(S.ncont);
  if (nc > QCONT) return false;
  // -- exact eta of the contenders still in reach: t(e) summed over the
  // hyperedges of I(m) that are in I(n); the best by (eta + noise, -id).
  // I(n) is hashed into the bins (empty after the windows, and left empty)
  u64 be = 0;
  u32 bi = NONE32;
  if (nc) {
    u32 mine = QFAIL;
    if (tid < deg) mine = q_einsert(S, S.eid[tid], S.tx[tid]);
    __syncthreads();
    for (u32 j = wid; j < nc; j += QW) {
      const u32 m = S.cid[j];
      if (S.cub[j] < lstar) continue;
      const i64 a = A.n_off[m], b = A.n_off[m + 1];
      u64 sum = 0;
      for (i64 p0 = a; p0 < b; p0 += 4 * WAVE) {
        u32 e4[4];  // (four loads in flight per lane)
#pragma unroll
        for (u32 i = 0; i < 4; ++i) {
          const i64 p = p0 + i * WAVE + lane;
          e4[i] = p < b ? A.n_inc[p] : 0xFFFFFFFFu;
        }
#pragma unroll
        for (u32 i = 0; i < 4; ++i)
          if (e4[i] != 0xFFFFFFFFu) sum += q_efind(S, e4[i]);
      }
#pragma unroll
      for (int d = WAVE / 2; d > 0; d >>= 1) sum += __shfl_xor(sum, d, WAVE);
      const u64 key = sum + (A.noise_on ? pair_noise(A.seed, n, m, dmod, magic) : 0);
      if (better(key, m, be, bi)) be = key, bi = m;
    }
    __syncthreads();
    if (mine != QFAIL) *reinterpret_cast<uint4 *>(&S.t.bin[4 * mine]) = make_uint4(0u, 0u, 0u, 0u);
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
                                                  NodeRec *spill, u32 *spill_cnt,
                                                  const i64 *samp_off, const u32 *samp) {
  __shared__ QSmem S;
  const u32 tid = threadIdx.x;
  const u64 cap = A.capinfo[0], dmod = A.capinfo[1], magic = A.capinfo[2];
  const u32 max_size = gmax[0], max_nin = gmax[1];
  const u32 total = *cnt;
  for (u32 i = tid; i < QD; i += QB) S.t.bin[i] = 0;
  // the start bits are left clear by their readers from here on
  for (u32 i = tid; i < 2 * QNBLK; i += QB) S.sbits[i / QNBLK][i % QNBLK] = 0;
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
    const bool done =
        rate_node_q(A, S, h, max_size, max_nin, hcap, cap, dmod, magic, samp_off, samp);
    if (!done && tid == 0) spill[atomicAdd(spill_cnt, 1u)] = recs[w];
    __syncthreads();
  }
}

// Entries of hyperedge e in the sample array: every 2^QSG-th pin of its
// source run, then of its destination run.
__global__ void k_samples_count(u32 E, const i64 *e_off, const u32 *e_nsrc, u32 *cnt) {
  const u32 e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  const u32 len = (u32)(e_off[e + 1] - e_off[e]), ns = e_nsrc[e];
  cnt[e] = ((ns + (1u << QSG) - 1) >> QSG) + ((len - ns + (1u << QSG) - 1) >> QSG);
}

// A wave per hyperedge, a lane per entry.
__global__ __launch_bounds__(256) void k_samples_fill(u32 E, const i64 *e_off, const u32 *e_nsrc,
                                                      const u32 *pins, const i64 *samp_off,
                                                      u32 *samp) {
  const u32 nwaves = gridDim.x * (blockDim.x / WAVE);
  const u32 l = lane_id();
  for (u32 e = blockIdx.x * (blockDim.x / WAVE) + wave_id(); e < E; e += nwaves) {
    const i64 a = e_off[e], o = samp_off[e];
    const u32 ns = e_nsrc[e];
    const u32 c0 = (ns + (1u << QSG) - 1) >> QSG, c = (u32)(samp_off[e + 1] - o);
    for (u32 j = l; j < c; j += WAVE)
      samp[o + j] = pins[a + (j < c0 ? (i64)j << QSG : (i64)ns + ((i64)(j - c0) << QSG))];
  }
}

}  // namespace

void launch_samples(chp_ctx *c, u32 E, const i64 *e_off, const u32 *e_nsrc, const u32 *pins,
                    u32 *cnt, i64 *samp_off, i64 *tmp, u32 *samp) {
  if (E == 0) return;
  CHP_LAUNCH(c, "samples_count", k_samples_count, grid_for(E, 256), 256, 0, E, e_off, e_nsrc,
             cnt);
  scan_u32_to_i64(c, cnt, samp_off, E, tmp);
  CHP_LAUNCH(c, "samples_fill", k_samples_fill, waves_grid(E), 256, 0, E, e_off, e_nsrc, pins,
             samp_off, samp);
}

u64 samples_bound(u32 E, u64 P) { return (P >> QSG) + 2ull * E; }

void launch_rate_incq(chp_ctx *c, const RateArgs &a, const NodeRec *recs, const u32 *cnt,
                      const u32 *gmax, u32 *work, u32 host_count, u32 hash_keys, NodeRec *spill,
                      u32 *spill_cnt, const i64 *samp_off, const u32 *samp) {
  if (!host_count) return;
  const u32 g = host_count < c->n_cu ? host_count : c->n_cu;
  const u32 hcap = hash_keys && hash_keys < QCAP ? hash_keys : QCAP;
  CHP_LAUNCH(c, "rate_incq", k_rate_incq, g, QB, 0, a, recs, cnt, gmax, work, hcap, spill,
             spill_cnt, samp_off, samp);
}
