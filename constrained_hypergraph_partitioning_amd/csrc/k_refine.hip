// One refinement pass over proposed moves ("Hypergraph Partitioning on GPU
// with Distinct Incident Hyperedges and Size Constraints", Sec. VI-A, VI-C,
// VI-D, Eqs. 14-15).
//
// Sequence.  By gain alone: the moves in (gain desc, id asc) order, sorted as
// u64 keys (2^31 - 1 - gain) << 32 | n.  As chains (Sec. VI-C, Fig. 5): the
// moves sorted by (source partition, gain rank) give every partition a run of
// the moves leaving it.  In each round every move without a successor scans
// the first 256 of the run leaving its destination for moves still without a
// predecessor and picks the largest grade (gain - 1e-6 |size diff| - 1e-7
// ||in| diff|, held exactly as 10^7 times that; ties to the smaller node); a
// move picked by several goes to the largest grade, then the largest picker
// (two atomic maxima).  The links form paths and cycles: pointer jumping
// finds each cycle's smallest node, the cycle is cut there, and a second
// jumping gives every move its chain head and position.  Chains are ranked
// by (total gain desc, first node asc) and laid out by a scan.
//
// In-sequence gains and inbound transitions (per hyperedge).  Hyperedge e
// holds one base event per pin, (rho(v), pin index), and two per moving pin
// v of sequence rank r: leave (rho(v), r) and enter (move(v), r).  Sorted by
// (partition, base before moves, rank), a segmented scan over each
// partition's events gives, at every move event, the pins (and destination
// pins) of e in that partition with the earlier moves applied:
//   leave with 1 pin left before it:  the move frees e of its partition, +w(e)
//   enter with 0 pins before it:      the move adds a partition to e,   -w(e)
// and a destination pin leaving its partition's last (entering an empty)
// destination slot takes e out of (puts e into) that partition's inbound set.
// The base events also give the starting inbound count of every partition.
//
// Validity (per partition).  A move changes size and inbound count of its
// two partitions only, so it yields two events (p, r) carrying both deltas.
// Sorted by (p, r) and prefix summed per partition they give each partition's
// state after each of its moves; where validity flips, the move's violation
// count changes by one.  The prefix applied is the one of largest cumulative
// gain with no violation (ties to the shorter; none when no prefix gains).
#include "dev.h"
#include "kernels.h"

namespace {

constexpr int RB = 256;
constexpr u32 MOVE_BIT = 0x80000000u;
constexpr u32 RANK_MASK = (1u << 29) - 1;

// ---- sequence -------------------------------------------------------------------
__global__ void k_seq_keys(u32 N, u32 k, const u32 *rho, const u32 *move, const i64 *gain,
                           u64 *keys, u32 *cnt, u32 *flags) {
  const u32 n = blockIdx.x * blockDim.x + threadIdx.x;
  bool take = false;
  u64 key = 0;
  if (n < N) {
    const u32 p = rho[n], d = move[n];
    if (p >= k || (d != NONE32 && (d >= k || d == p))) atomicOr(flags, FLAG_EINVAL);
    else if (d != NONE32) {
      const i64 g = gain[n];
      if (g < -(i64)0x80000000ll || g > (i64)0x7FFFFFFFll) atomicOr(flags, FLAG_EOVERFLOW);
      key = ((u64)((i64)0x7FFFFFFFll - g) << 32) | n;
      take = true;
    }
  }
  const u32 s = wave_append(cnt, take);
  if (take) keys[s] = key;
}

__global__ void k_seq_rank(u32 M, const u64 *keys, u32 *seq, u32 *rank) {
  const u32 i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= M) return;
  const u32 n = (u32)keys[i];
  seq[i] = n;
  rank[n] = i;
}

// ---- chains -----------------------------------------------------------------------
constexpr u32 CHAIN_WINDOW = 256;

struct ChainPos {  // per position of the (source partition, gain rank) order
  u32 *node, *size, *nin, *dest;
  i64 *gain;
  u32 *pred, *succ;  // positions
};

__global__ void k_chain_keys(u32 M, const u32 *seq, const u32 *rho, u64 *keys) {
  const u32 r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= M) return;
  keys[r] = ((u64)rho[seq[r]] << 32) | r;
}

__global__ void k_chain_setup(u32 M, const u64 *keys, const u32 *seq, const u32 *move,
                              const u32 *n_size, const u32 *n_nin, const i64 *gain, ChainPos C,
                              u32 *posn) {
  const u32 t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= M) return;
  const u32 n = seq[(u32)keys[t]];
  C.node[t] = n;
  C.size[t] = n_size[n];
  C.nin[t] = n_nin[n];
  C.dest[t] = move[n];
  C.gain[t] = gain[n];
  C.pred[t] = NONE32;
  C.succ[t] = NONE32;
  posn[n] = t;
}

__device__ __forceinline__ u32 lower_bound_u64(const u64 *a, u32 n, u64 v) {
  u32 lo = 0, hi = n;
  while (lo < hi) {
    const u32 mid = (lo + hi) >> 1;
    if (a[mid] < v) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}


// first position of every source partition's run (k + 1 entries)
__global__ void k_chain_pstart(u32 M, u32 k, const u64 *keys, u32 *pstart) {
  const u32 t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= M) return;
  const u32 p = (u32)(keys[t] >> 32);
  const u32 q0 = t ? (u32)(keys[t - 1] >> 32) + 1 : 0;
  for (u32 q = q0; q <= p; ++q) pstart[q] = t;
  if (t == M - 1)
    for (u32 q = p + 1; q <= k; ++q) pstart[q] = M;
}

// One wave per free end: its window's candidates a lane each, then the
// largest grade (smallest node on ties) by shuffles.  A window with no
// candidate left stays so (predecessors are never removed): the picker is
// marked exhausted and skipped in later rounds.
constexpr int CPB = 256;
__global__ __launch_bounds__(CPB) void k_chain_pick(u32 M, const u32 *pstart, ChainPos C,
                                                    u32 *done, u32 *pick, i64 *pgr, i64 *wgr) {
  const u32 l = lane_id();
  const u32 nw = gridDim.x * (CPB / WAVE);
  for (u32 t = blockIdx.x * (CPB / WAVE) + wave_id(); t < M; t += nw) {
    if (C.succ[t] != NONE32 || done[t]) {
      if (l == 0) pick[t] = NONE32;
      continue;
    }
    const u32 d = C.dest[t];
    const u32 a = pstart[d], e = pstart[d + 1];
    const u32 b = e - a > CHAIN_WINDOW ? a + CHAIN_WINDOW : e;
    const u32 ts = C.size[t], tn = C.nin[t];
    i64 bg = 0;
    u32 bu = NONE32, bn = NONE32;
    for (u32 u = a + l; u < b; u += WAVE) {
      if (C.pred[u] != NONE32) continue;
      const u32 us = C.size[u], un = C.nin[u], node = C.node[u];
      const i64 ds = ts > us ? (i64)ts - us : (i64)us - ts;
      const i64 di = tn > un ? (i64)tn - un : (i64)un - tn;
      const i64 g = 10000000ll * C.gain[u] - 10 * ds - di;
      if (bu == NONE32 || g > bg || (g == bg && node < bn)) {
        bg = g;
        bu = u;
        bn = node;
      }
    }
#pragma unroll
    for (int s = WAVE / 2; s > 0; s >>= 1) {
      const i64 og = __shfl_xor(bg, s, WAVE);
      const u32 ou = __shfl_xor(bu, s, WAVE), on = __shfl_xor(bn, s, WAVE);
      if (ou != NONE32 && (bu == NONE32 || og > bg || (og == bg && on < bn))) {
        bg = og;
        bu = ou;
        bn = on;
      }
    }
    if (l == 0) {
      pick[t] = bu;
      if (bu != NONE32) {
        pgr[t] = bg;
        atomicMax((long long *)(wgr + bu), (long long)bg);
      } else {
        done[t] = 1;
      }
    }
  }
}

__global__ void k_chain_claim(u32 M, const u32 *pick, const i64 *pgr, const i64 *wgr,
                              const u32 *node, u32 *wid) {
  const u32 t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= M) return;
  const u32 u = pick[t];
  if (u != NONE32 && pgr[t] == wgr[u]) atomicMax(wid + u, node[t] + 1);
}

__global__ void k_chain_link(u32 M, const u32 *pick, const u32 *wid, ChainPos C, u32 *links) {
  const u32 t = blockIdx.x * blockDim.x + threadIdx.x;
  bool won = false;
  if (t < M) {
    const u32 u = pick[t];
    if (u != NONE32 && wid[u] == C.node[t] + 1) {
      C.succ[t] = u;
      C.pred[u] = t;
      won = true;
    }
  }
  const u64 b = __ballot(won);
  if (lane_id() == 0 && b) atomicAdd(links, (u32)__popcll(b));
}

// jumping over predecessors: ancestor, and the smallest node on the way
__global__ void k_cj_init(u32 M, const u32 *pred, const u32 *node, u32 *anc, u32 *mn) {
  const u32 t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= M) return;
  anc[t] = pred[t] == NONE32 ? t : pred[t];
  mn[t] = node[t];
}

__global__ void k_cj_jump_min(u32 M, const u32 *anc, const u32 *mn, u32 *anc2, u32 *mn2) {
  const u32 t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= M) return;
  const u32 a = anc[t];
  anc2[t] = anc[a];
  mn2[t] = mn[a] < mn[t] ? mn[a] : mn[t];
}

// cut every cycle before its smallest node; then ancestors and distances
__global__ void k_cj_cut(u32 M, const u32 *pred, const u32 *node, const u32 *anc, const u32 *mn,
                         u32 *cut, u32 *anc2, u32 *dist) {
  const u32 t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= M) return;
  u32 p = pred[t];
  const bool in_cycle = pred[anc[t]] != NONE32;
  if (in_cycle && mn[t] == node[t]) p = NONE32;
  cut[t] = p;
  anc2[t] = p == NONE32 ? t : p;
  dist[t] = p == NONE32 ? 0 : 1;
}

__global__ void k_cj_jump_dist(u32 M, const u32 *anc, const u32 *dist, u32 *anc2, u32 *dist2) {
  const u32 t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= M) return;
  const u32 a = anc[t];
  anc2[t] = anc[a];
  dist2[t] = dist[t] + dist[a];
}

__global__ void k_chain_totals(u32 M, const u32 *anc, const i64 *gain, i64 *ctot, u32 *clen) {
  const u32 t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= M) return;
  const u32 h = anc[t];
  atomicAdd((unsigned long long *)(ctot + h), (unsigned long long)gain[t]);
  atomicAdd(clen + h, 1u);
}

__device__ __forceinline__ u64 desc_key(i64 v) { return (u64)(-v) ^ (1ull << 63); }

__global__ void k_chain_heads(u32 M, const u32 *cut, const i64 *ctot, u32 *heads, u64 *hk,
                              u32 *cnt) {
  const u32 t = blockIdx.x * blockDim.x + threadIdx.x;
  const bool h = t < M && cut[t] == NONE32;
  const u32 s = wave_append(cnt, h);
  if (h) {
    heads[s] = t;
    hk[s] = desc_key(ctot[t]);
  }
}

// (rank of the total among the sorted totals) << 32 | first node: distinct
__global__ void k_chain_rank_keys(u32 H, const u32 *heads, const i64 *ctot, const u64 *sorted,
                                  const u32 *node, u64 *keys) {
  const u32 i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= H) return;
  const u32 t = heads[i];
  keys[i] = ((u64)lower_bound_u64(sorted, H, desc_key(ctot[t])) << 32) | node[t];
}

__global__ void k_chain_lens(u32 H, const u64 *keys, const u32 *posn, const u32 *clen,
                             u32 *lens) {
  const u32 c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= H) return;
  lens[c] = clen[posn[(u32)keys[c]]];
}

__global__ void k_chain_starts(u32 H, const u64 *keys, const u32 *posn, const i64 *coff,
                               u32 *cstart) {
  const u32 c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= H) return;
  cstart[posn[(u32)keys[c]]] = (u32)coff[c];
}

__global__ void k_chain_place(u32 M, const u32 *anc, const u32 *dist, const u32 *cstart,
                              const u32 *node, u32 *seq, u32 *rank) {
  const u32 t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= M) return;
  const u32 p = cstart[anc[t]] + dist[t];
  seq[p] = node[t];
  rank[node[t]] = p;
}

// ---- hyperedge events -------------------------------------------------------------
struct EvArgs {
  const i64 *e_off;
  const u32 *e_nsrc, *pins, *e_w, *rho, *move, *rank;
  i64 *ingain;   // [M] in-sequence gain by rank
  u32 *dleave;   // [M] inbound sets the move's source partition loses
  u32 *denter;   // [M] inbound sets the move's destination partition gains
  u32 *inb0;     // [k] starting inbound counts
};

// hyperedge classes by |e|: events <= 3 |e| fit 256 (class 0) or 8192 (class 1)
constexpr u32 EV_C0 = 85, EV_C1 = 2730;

__global__ void k_ev_classify(u32 E, const i64 *e_off, u32 *lists, u32 *cnt) {
  const u32 e = blockIdx.x * blockDim.x + threadIdx.x;
  u32 len = 0;
  if (e < E) len = (u32)(e_off[e + 1] - e_off[e]);
  const int c = e >= E ? -1 : (len <= EV_C0 ? 0 : (len <= EV_C1 ? 1 : 2));
  for (int k = 0; k < 3; ++k) {
    const u32 s = wave_append(cnt + k, c == k);
    if (c == k) lists[(u64)k * E + s] = e;
  }
  if (c == 2) atomicMax(cnt + 3, len);
}

// The events of e into s[0, ...); returns their count (all threads).
__device__ __forceinline__ u32 ev_build(const EvArgs &A, u32 e, u64 *s, u32 *s_n) {
  const i64 a = A.e_off[e];
  const u32 len = (u32)(A.e_off[e + 1] - a), ns = A.e_nsrc[e];
  if (threadIdx.x == 0) *s_n = len;
  __syncthreads();
  for (u32 j = threadIdx.x; j < len; j += blockDim.x) {
    const u32 v = A.pins[a + j];
    const u32 isd = j >= ns ? 1u : 0u;
    const u32 p = A.rho[v];
    s[j] = ((u64)p << 32) | (j << 1) | isd;
    const u32 r = A.rank[v];
    if (r != NONE32) {
      const u32 slot = atomicAdd(s_n, 2u);
      const u32 lo = MOVE_BIT | (r << 2) | (isd << 1);
      s[slot] = ((u64)p << 32) | lo;
      s[slot + 1] = ((u64)A.move[v] << 32) | lo | 1u;
    }
  }
  __syncthreads();
  return *s_n;
}

template <int BLOCK>
struct SegLds {
  int wf[BLOCK / WAVE], wa[BLOCK / WAVE], wb[BLOCK / WAVE];
  int ca, cb;
};

// Walk the sorted events s[0, m) of e: segmented (by partition) exclusive
// counts of all pins and of destination pins before each event.
template <int BLOCK>
__device__ void ev_scan_emit(const EvArgs &A, const u64 *s, u32 m, u32 w, SegLds<BLOCK> &L) {
  const u32 l = lane_id(), wv = wave_id();
  int ca = 0, cb = 0;
  for (u32 c0 = 0; c0 < m; c0 += BLOCK) {
    const u32 i = c0 + threadIdx.x;
    const bool in = i < m;
    const u64 key = in ? s[i] : 0;
    const u32 p = (u32)(key >> 32), lo = (u32)key;
    const bool head = in && (i == 0 || (u32)(s[i - 1] >> 32) != p);
    const bool mv = (lo & MOVE_BIT) != 0;
    const bool isd = mv ? ((lo >> 1) & 1u) != 0 : (lo & 1u) != 0;
    const bool ent = mv && (lo & 1u);
    const int da = !in ? 0 : (!mv || ent ? 1 : -1);
    const int db = isd ? da : 0;
    int f = head ? 1 : 0, xa = da, xb = db;
#pragma unroll
    for (int d = 1; d < WAVE; d <<= 1) {
      const int fu = __shfl_up(f, d, WAVE), au = __shfl_up(xa, d, WAVE),
                bu = __shfl_up(xb, d, WAVE);
      if ((int)l >= d && !f) {
        xa += au;
        xb += bu;
        f = fu;
      }
    }
    if (l == WAVE - 1) {
      L.wf[wv] = f;
      L.wa[wv] = xa;
      L.wb[wv] = xb;
    }
    __syncthreads();
    if (!f) {  // no head at or before this lane in its wave: add what came before
      int ya = ca, yb = cb;
      for (u32 v = 0; v < wv; ++v) {
        if (L.wf[v]) {
          ya = L.wa[v];
          yb = L.wb[v];
        } else {
          ya += L.wa[v];
          yb += L.wb[v];
        }
      }
      xa += ya;
      xb += yb;
    }
    const int ea = xa - da, eb = xb - db;  // before this event, within its partition
    if (in && mv) {
      const u32 r = (lo >> 2) & RANK_MASK;
      if (!ent) {
        if (ea == 1) atomicAdd((unsigned long long *)(A.ingain + r), (unsigned long long)w);
        if (isd && eb == 1) atomicAdd(A.dleave + r, 1u);
      } else {
        if (ea == 0)
          atomicAdd((unsigned long long *)(A.ingain + r), (unsigned long long)(-(i64)w));
        if (isd && eb == 0) atomicAdd(A.denter + r, 1u);
      }
    } else if (in && isd && eb == 0) {
      atomicAdd(A.inb0 + p, 1u);  // e's first destination pin in p: e is inbound to p
    }
    __syncthreads();
    if (threadIdx.x == BLOCK - 1) {
      L.ca = xa;
      L.cb = xb;
    }
    __syncthreads();
    ca = L.ca;
    cb = L.cb;
  }
}

template <int BLOCK, int CAP>
__global__ __launch_bounds__(BLOCK) void k_ev_lds(EvArgs A, const u32 *list, const u32 *cnt) {
  __shared__ u64 s[CAP];
  __shared__ u32 s_n;
  __shared__ SegLds<BLOCK> L;
  const u32 total = *cnt;
  for (u32 w = blockIdx.x; w < total; w += gridDim.x) {
    const u32 e = list[w];
    const u32 m = ev_build(A, e, s, &s_n);
    const u32 pm = next_pow2(m);
    for (u32 i = m + threadIdx.x; i < pm; i += BLOCK) s[i] = ~0ull;
    __syncthreads();
    lds_bitonic<BLOCK>(s, pm);
    ev_scan_emit<BLOCK>(A, s, m, A.e_w[e], L);
    __syncthreads();
  }
}

template <int BLOCK, int CAP>
__global__ __launch_bounds__(BLOCK) void k_ev_global(EvArgs A, const u32 *list, const u32 *cnt,
                                                     u64 *scratch, u64 per_wg) {
  __shared__ u64 s[CAP];
  __shared__ u32 s_n;
  __shared__ SegLds<BLOCK> L;
  const u32 total = *cnt;
  u64 *X = scratch + (u64)blockIdx.x * per_wg;
  u64 *Y = X + per_wg / 2;
  for (u32 w = blockIdx.x; w < total; w += gridDim.x) {
    const u32 e = list[w];
    const u32 m = ev_build(A, e, X, &s_n);
    const u64 *res = wg_sort_global<BLOCK, CAP>(X, Y, m, s);
    ev_scan_emit<BLOCK>(A, res, m, A.e_w[e], L);
    __syncthreads();
  }
}

// ---- partition events ---------------------------------------------------------------
__global__ void k_pev_keys(u32 M, const u32 *seq, const u32 *rho, const u32 *move, u64 *keys) {
  const u32 r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= M) return;
  const u32 n = seq[r];
  keys[2 * (u64)r] = ((u64)rho[n] << 32) | ((u64)r << 1);
  keys[2 * (u64)r + 1] = ((u64)move[n] << 32) | ((u64)r << 1) | 1u;
}

__global__ void k_pev_vals(u64 Q, const u64 *keys, const u32 *seq, const u32 *n_size,
                           const u32 *dleave, const u32 *denter, i64 *vs, i64 *vi) {
  const u64 i = (u64)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= Q) return;
  const u64 key = keys[i];
  const u32 r = (u32)key >> 1;
  const bool ent = key & 1u;
  const i64 sz = n_size[seq[r]];
  vs[i] = ent ? sz : -sz;
  vi[i] = ent ? (i64)denter[r] : -(i64)dleave[r];
}

__device__ __forceinline__ u64 first_of(const u64 *keys, u64 Q, u32 p) {
  const u64 want = (u64)p << 32;
  u64 lo = 0, hi = Q;
  while (lo < hi) {
    const u64 mid = (lo + hi) >> 1;
    if (keys[mid] < want) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

__device__ __forceinline__ bool part_valid(u64 size0, u32 inb0, i64 ds, i64 di, u64 omega,
                                           u32 delta) {
  return (i64)size0 + ds <= (i64)omega && (i64)inb0 + di <= (i64)delta;
}

// validity flips of each partition along its own moves
__global__ void k_pev_flips(u64 Q, const u64 *keys, const i64 *vs, const i64 *vi,
                            const i64 *Ps, const i64 *Pi, const u64 *size0, const u32 *inb0,
                            u64 omega, u32 delta, i64 *vdelta) {
  const u64 i = (u64)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= Q) return;
  const u64 key = keys[i];
  const u32 p = (u32)(key >> 32), r = (u32)key >> 1;
  const u64 h = first_of(keys, Q, p);
  const i64 bs = Ps[i] - Ps[h], bi = Pi[i] - Pi[h];
  const bool before = part_valid(size0[p], inb0[p], bs, bi, omega, delta);
  const bool after = part_valid(size0[p], inb0[p], bs + vs[i], bi + vi[i], omega, delta);
  if (before != after)
    atomicAdd((unsigned long long *)(vdelta + r), (unsigned long long)(before ? 1ll : -1ll));
}

__global__ void k_viol0(u32 k, const u64 *size0, const u32 *inb0, u64 omega, u32 delta,
                        u32 *v0) {
  const u32 p = blockIdx.x * blockDim.x + threadIdx.x;
  const bool bad = p < k && !part_valid(size0[p], inb0[p], 0, 0, omega, delta);
  const u64 b = __ballot(bad);
  if (lane_id() == 0 && b) atomicAdd(v0, (u32)__popcll(b));
}

// per rank: cumulative gain and violations; the largest valid positive gain
__global__ void k_prefix_best(u32 M, const i64 *ingain, const i64 *Pg, const i64 *vdelta,
                              const i64 *Pv, const u32 *v0, i64 *seq_gain, u32 *seq_viol,
                              u64 *best) {
  const u32 r = blockIdx.x * blockDim.x + threadIdx.x;
  u64 cand = 0;
  if (r < M) {
    const i64 G = Pg[r] + ingain[r];
    const i64 V = (i64)*v0 + Pv[r] + vdelta[r];
    if (seq_gain) seq_gain[r] = ingain[r];
    if (seq_viol) seq_viol[r] = (u32)V;
    if (V == 0 && G > 0) cand = (u64)G;
  }
#pragma unroll
  for (int d = WAVE / 2; d > 0; d >>= 1) {
    const u64 o = __shfl_xor(cand, d, WAVE);
    cand = o > cand ? o : cand;
  }
  if (lane_id() == 0 && cand) atomicMax((unsigned long long *)best, (unsigned long long)cand);
}

__global__ void k_prefix_pick(u32 M, const i64 *ingain, const i64 *Pg, const i64 *vdelta,
                              const i64 *Pv, const u32 *v0, const u64 *best, u32 *best_len) {
  const u32 r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= M) return;
  const u64 b = *best;
  if (b == 0) return;
  const i64 G = Pg[r] + ingain[r];
  const i64 V = (i64)*v0 + Pv[r] + vdelta[r];
  if (V == 0 && G > 0 && (u64)G == b) atomicMin(best_len, r + 1);
}

__global__ void k_apply(u32 M, const u32 *seq, const u32 *move, const u32 *best_len, u32 *rho) {
  const u32 r = blockIdx.x * blockDim.x + threadIdx.x;
  const u32 L = *best_len;
  if (r >= M || L == NONE32 || r >= L) return;
  const u32 n = seq[r];
  rho[n] = move[n];
}

}  // namespace

void launch_seq_keys(chp_ctx *c, u32 N, u32 k, const u32 *rho, const u32 *move, const i64 *gain,
                     u64 *keys, u32 *cnt) {
  CHP_LAUNCH(c, "seq_keys", k_seq_keys, grid_for(N, RB), RB, 0, N, k, rho, move, gain, keys, cnt,
             c->flags);
}

void launch_seq_rank(chp_ctx *c, u32 M, const u64 *keys, u32 *seq, u32 *rank) {
  CHP_LAUNCH(c, "seq_rank", k_seq_rank, grid_for(M, RB), RB, 0, M, keys, seq, rank);
}

void launch_ev_classify(chp_ctx *c, u32 E, const i64 *e_off, u32 *lists, u32 *cnt) {
  CHP_LAUNCH(c, "ev_classify", k_ev_classify, grid_for(E, RB), RB, 0, E, e_off, lists, cnt);
}

u64 ev_global_words(u32 max_len) { return 2ull * 3ull * max_len; }

void launch_ev_edges(chp_ctx *c, u32 E, const i64 *e_off, const u32 *e_nsrc, const u32 *pins,
                     const u32 *e_w, const u32 *rho, const u32 *move, const u32 *rank,
                     i64 *ingain, u32 *dleave, u32 *denter, u32 *inb0, const u32 *lists,
                     const u32 *cnt, const u32 *host_cnt, u64 *scratch, u32 grid_global) {
  EvArgs A;
  A.e_off = e_off;
  A.e_nsrc = e_nsrc;
  A.pins = pins;
  A.e_w = e_w;
  A.rho = rho;
  A.move = move;
  A.rank = rank;
  A.ingain = ingain;
  A.dleave = dleave;
  A.denter = denter;
  A.inb0 = inb0;
  const u32 per_cu0 = 16, per_cu1 = 2;
  if (host_cnt[0]) {
    const u32 g = host_cnt[0] < per_cu0 * c->n_cu ? host_cnt[0] : per_cu0 * c->n_cu;
    CHP_LAUNCH(c, "ev_small", (k_ev_lds<64, 256>), g, 64, 0, A, lists, cnt + 0);
  }
  if (host_cnt[1]) {
    const u32 g = host_cnt[1] < per_cu1 * c->n_cu ? host_cnt[1] : per_cu1 * c->n_cu;
    CHP_LAUNCH(c, "ev_mid", (k_ev_lds<256, 8192>), g, 256, 0, A, lists + E, cnt + 1);
  }
  if (host_cnt[2])
    CHP_LAUNCH(c, "ev_large", (k_ev_global<256, 4096>), grid_global, 256, 0, A, lists + 2ull * E,
               cnt + 2, scratch, ev_global_words(host_cnt[3]));
}

void launch_pev(chp_ctx *c, u32 M, const u32 *seq, const u32 *rho, const u32 *move, u64 *keys) {
  CHP_LAUNCH(c, "pev_keys", k_pev_keys, grid_for(M, RB), RB, 0, M, seq, rho, move, keys);
}

void launch_pev_vals(chp_ctx *c, u64 Q, const u64 *keys, const u32 *seq, const u32 *n_size,
                     const u32 *dleave, const u32 *denter, i64 *vs, i64 *vi) {
  CHP_LAUNCH(c, "pev_vals", k_pev_vals, grid_for(Q, RB), RB, 0, Q, keys, seq, n_size, dleave,
             denter, vs, vi);
}

void launch_pev_flips(chp_ctx *c, u64 Q, const u64 *keys, const i64 *vs, const i64 *vi,
                      const i64 *Ps, const i64 *Pi, const u64 *size0, const u32 *inb0,
                      u64 omega, u32 delta, i64 *vdelta) {
  CHP_LAUNCH(c, "pev_flips", k_pev_flips, grid_for(Q, RB), RB, 0, Q, keys, vs, vi, Ps, Pi, size0,
             inb0, omega, delta, vdelta);
}

void launch_viol0(chp_ctx *c, u32 k, const u64 *size0, const u32 *inb0, u64 omega, u32 delta,
                  u32 *v0) {
  CHP_LAUNCH(c, "viol0", k_viol0, grid_for(k, RB), RB, 0, k, size0, inb0, omega, delta, v0);
}

void launch_prefix(chp_ctx *c, u32 M, const i64 *ingain, const i64 *Pg, const i64 *vdelta,
                   const i64 *Pv, const u32 *v0, i64 *seq_gain, u32 *seq_viol, u64 *best,
                   u32 *best_len, const u32 *seq, const u32 *move, u32 *rho) {
  const u32 g = grid_for(M, RB);
  CHP_LAUNCH(c, "prefix_best", k_prefix_best, g, RB, 0, M, ingain, Pg, vdelta, Pv, v0, seq_gain,
             seq_viol, best);
  CHP_LAUNCH(c, "prefix_pick", k_prefix_pick, g, RB, 0, M, ingain, Pg, vdelta, Pv, v0,
             (const u64 *)best, best_len);
  CHP_LAUNCH(c, "apply_moves", k_apply, g, RB, 0, M, seq, move, (const u32 *)best_len, rho);
}

// ---- chain launchers -----------------------------------------------------------------
void launch_chain_setup(chp_ctx *c, u32 M, u32 k, const u32 *seq, const u32 *rho,
                        const u32 *move, const u32 *n_size, const u32 *n_nin, const i64 *gain,
                        u64 *keys, u64 *ktmp, ChainBufs &B, const u64 **sorted) {
  CHP_LAUNCH(c, "chain_keys", k_chain_keys, grid_for(M, RB), RB, 0, M, seq, rho, keys);
  const u64 *sk = sort_keys_u64(c, keys, ktmp, M);
  *sorted = sk;
  ChainPos C{B.node, B.size, B.nin, B.dest, B.gain, B.pred, B.succ};
  CHP_LAUNCH(c, "chain_setup", k_chain_setup, grid_for(M, RB), RB, 0, M, sk, seq, move, n_size,
             n_nin, gain, C, B.posn);
  CHP_LAUNCH(c, "chain_pstart", k_chain_pstart, grid_for(M, RB), RB, 0, M, k, sk, B.pstart);
}

void launch_chain_round(chp_ctx *c, u32 M, ChainBufs &B, u32 *links) {
  ChainPos C{B.node, B.size, B.nin, B.dest, B.gain, B.pred, B.succ};
  const u32 g = grid_for(M, RB);
  launch_fills(c, {{B.wgr, M, 0x8000000000000000ull, true}, {B.wid, M, 0, false}});
  const u32 waves = M < 64u * c->n_cu * (CPB / WAVE) ? M : 64u * c->n_cu * (CPB / WAVE);
  CHP_LAUNCH(c, "chain_pick", k_chain_pick, (waves + CPB / WAVE - 1) / (CPB / WAVE), CPB, 0, M,
             (const u32 *)B.pstart, C, B.done, B.pick, B.pgr, B.wgr);
  CHP_LAUNCH(c, "chain_claim", k_chain_claim, g, RB, 0, M, (const u32 *)B.pick,
             (const i64 *)B.pgr, (const i64 *)B.wgr, (const u32 *)B.node, B.wid);
  CHP_LAUNCH(c, "chain_link", k_chain_link, g, RB, 0, M, (const u32 *)B.pick,
             (const u32 *)B.wid, C, links);
}

void launch_chain_walk(chp_ctx *c, u32 M, ChainBufs &B) {
  const u32 g = grid_for(M, RB);
  u32 rounds = 1;
  while ((1ull << rounds) < (u64)M + 1) ++rounds;
  CHP_LAUNCH(c, "cj_init", k_cj_init, g, RB, 0, M, (const u32 *)B.pred, (const u32 *)B.node,
             B.anc, B.mn);
  for (u32 r = 0; r < rounds; ++r) {
    CHP_LAUNCH(c, "cj_jump_min", k_cj_jump_min, g, RB, 0, M, (const u32 *)B.anc,
               (const u32 *)B.mn, B.anc2, B.mn2);
    std::swap(B.anc, B.anc2);
    std::swap(B.mn, B.mn2);
  }
  CHP_LAUNCH(c, "cj_cut", k_cj_cut, g, RB, 0, M, (const u32 *)B.pred, (const u32 *)B.node,
             (const u32 *)B.anc, (const u32 *)B.mn, B.cut, B.anc2, B.dist);
  std::swap(B.anc, B.anc2);
  for (u32 r = 0; r < rounds; ++r) {
    CHP_LAUNCH(c, "cj_jump_dist", k_cj_jump_dist, g, RB, 0, M, (const u32 *)B.anc,
               (const u32 *)B.dist, B.anc2, B.mn2);
    std::swap(B.anc, B.anc2);
    std::swap(B.dist, B.mn2);
  }
  CHP_LAUNCH(c, "chain_totals", k_chain_totals, g, RB, 0, M, (const u32 *)B.anc,
             (const i64 *)B.gain, B.ctot, B.clen);
}

void launch_chain_heads(chp_ctx *c, u32 M, ChainBufs &B, u32 *heads, u64 *hk, u32 *cnt) {
  CHP_LAUNCH(c, "chain_heads", k_chain_heads, grid_for(M, RB), RB, 0, M, (const u32 *)B.cut,
             (const i64 *)B.ctot, heads, hk, cnt);
}

void launch_chain_rank_keys(chp_ctx *c, u32 H, const u32 *heads, ChainBufs &B,
                            const u64 *sorted_totals, u64 *keys) {
  CHP_LAUNCH(c, "chain_rank_keys", k_chain_rank_keys, grid_for(H, RB), RB, 0, H, heads,
             (const i64 *)B.ctot, sorted_totals, (const u32 *)B.node, keys);
}

void launch_chain_lens(chp_ctx *c, u32 H, const u64 *keys, ChainBufs &B, u32 *lens) {
  CHP_LAUNCH(c, "chain_lens", k_chain_lens, grid_for(H, RB), RB, 0, H, keys,
             (const u32 *)B.posn, (const u32 *)B.clen, lens);
}

void launch_chain_place(chp_ctx *c, u32 M, u32 H, const u64 *keys, const i64 *coff,
                        ChainBufs &B, u32 *seq, u32 *rank) {
  CHP_LAUNCH(c, "chain_starts", k_chain_starts, grid_for(H, RB), RB, 0, H, keys,
             (const u32 *)B.posn, coff, B.cstart);
  CHP_LAUNCH(c, "chain_place", k_chain_place, grid_for(M, RB), RB, 0, M, (const u32 *)B.anc,
             (const u32 *)B.dist, (const u32 *)B.cstart, (const u32 *)B.node, seq, rank);
}
