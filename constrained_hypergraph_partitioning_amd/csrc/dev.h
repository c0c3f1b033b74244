// Device-side building blocks for wave64 / workgroup cooperation on gfx950:
// scans and reductions built from cross-lane shuffles, LDS bitonic sorting,
// a merge-path merge of sorted runs in global memory, and the rating noise.
#pragma once
#include "common.h"

#define WAVE 64

__device__ __forceinline__ u32 lane_id() { return __lane_id(); }
__device__ __forceinline__ u32 wave_id() { return threadIdx.x / WAVE; }

// Inclusive prefix sum across the 64 lanes of a wave.
template <typename T>
__device__ __forceinline__ T wave_incl_scan(T v) {
  const u32 l = lane_id();
#pragma unroll
  for (int d = 1; d < WAVE; d <<= 1) {
    T o = __shfl_up(v, d, WAVE);
    if (l >= (u32)d) v += o;
  }
  return v;
}

// LDS writes of this wave become visible to its other lanes
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int d = WAVE / 2; d > 0; d >>= 1) v += __shfl_xor(v, d, WAVE);
  return v;
}

// Exclusive scan across a workgroup of BLOCK threads.  `lds` holds at least
// BLOCK/64 + 1 elements.  Returns this thread's exclusive prefix; *total gets
// the workgroup total.  Contains barriers: call from every thread.
template <int BLOCK, typename T>
__device__ __forceinline__ T wg_excl_scan(T v, T *lds, T *total) {
  constexpr int NW = BLOCK / WAVE;
  T inc = wave_incl_scan(v);
  if (NW == 1) {
    T tot = __shfl(inc, WAVE - 1, WAVE);
    *total = tot;
    return inc - v;
  }
  if (lane_id() == WAVE - 1) lds[wave_id()] = inc;
  __syncthreads();
  T off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    T s = lds[w];
    if (w < (int)wave_id()) off += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return off + inc - v;
}

template <int BLOCK, typename T>
__device__ __forceinline__ T wg_sum(T v, T *lds) {
  constexpr int NW = BLOCK / WAVE;
  v = wave_sum(v);
  if (NW == 1) return v;
  if (lane_id() == 0) lds[wave_id()] = v;
  __syncthreads();
  T tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) tot += lds[w];
  __syncthreads();
  return tot;
}

__device__ __forceinline__ u64 sat_add(u64 a, u64 b) {
  u64 s = a + b;
  return s < a ? ~0ull : s;
}

// (eta desc, id asc): is (e1,i1) strictly better than (e2,i2)?
__device__ __forceinline__ bool better(u64 e1, u32 i1, u64 e2, u32 i2) {
  return e1 > e2 || (e1 == e2 && i1 < i2);
}

// The MP best (eta, id) seen by one thread, sorted by `better`; an empty
// entry is {0, NONE32}, which every candidate beats (eta > 0 for any node
// that shares a hyperedge).  All indices are compile-time, so the list stays
// in registers.
template <int MP>
struct TopList {
  u64 e[MP];
  u32 i[MP];
  __device__ __forceinline__ void clear() {
#pragma unroll
    for (int k = 0; k < MP; ++k) e[k] = 0, i[k] = NONE32;
  }
  // could (ev, iv) enter the list?
  __device__ __forceinline__ bool admits(u64 ev, u32 iv) const {
    return better(ev, iv, e[MP - 1], i[MP - 1]);
  }
  // insert an admitted (ev, iv); the last entry falls out
  __device__ __forceinline__ void insert(u64 ev, u32 iv) {
    bool placed = false;
#pragma unroll
    for (int k = MP - 1; k > 0; --k) {
      if (!placed) {
        if (better(ev, iv, e[k - 1], i[k - 1])) {
          e[k] = e[k - 1], i[k] = i[k - 1];
        } else {
          e[k] = ev, i[k] = iv;
          placed = true;
        }
      }
    }
    if (!placed) e[0] = ev, i[0] = iv;
  }
  // drop the head
  __device__ __forceinline__ void pop() {
#pragma unroll
    for (int k = 0; k + 1 < MP; ++k) e[k] = e[k + 1], i[k] = i[k + 1];
    e[MP - 1] = 0, i[MP - 1] = NONE32;
  }
};

// Workgroup argmax of (eta, id) under `better`; result broadcast to all.
template <int BLOCK>
__device__ __forceinline__ void wg_best(u64 &eta, u32 &id, u64 *lds_e, u32 *lds_i) {
  constexpr int NW = BLOCK / WAVE;
#pragma unroll
  for (int d = WAVE / 2; d > 0; d >>= 1) {
    u64 oe = __shfl_xor(eta, d, WAVE);
    u32 oi = __shfl_xor(id, d, WAVE);
    if (better(oe, oi, eta, id)) eta = oe, id = oi;
  }
  if (NW == 1) return;
  if (lane_id() == 0) lds_e[wave_id()] = eta, lds_i[wave_id()] = id;
  __syncthreads();
  eta = lds_e[0];
  id = lds_i[0];
#pragma unroll
  for (int w = 1; w < NW; ++w)
    if (better(lds_e[w], lds_i[w], eta, id)) eta = lds_e[w], id = lds_i[w];
  __syncthreads();
}

// The pi (<= MP) best entries over every thread's list, in order: one
// workgroup argmax of the heads per row, after which the thread holding the
// winner drops it (a node's neighbours sit in one bin each, so ids are
// distinct across threads).  `lead` writes row r of target/score at node n
// (rows of stride N); rows past the candidates get NONE32 and 0.
template <int BLOCK, int MP>
__device__ __forceinline__ void emit_top(TopList<MP> &b, u32 pi, u64 *lds_e, u32 *lds_i,
                                         bool lead, u32 *target, u64 *score, u64 N, u32 n) {
  for (u32 r = 0; r < pi; ++r) {
    u64 e = b.e[0];
    u32 id = b.i[0];
    wg_best<BLOCK>(e, id, lds_e, lds_i);
    if (id != NONE32 && b.i[0] == id) b.pop();
    if (lead) {
      target[r * N + n] = id;
      score[r * N + n] = id == NONE32 ? 0 : e;
    }
  }
}

// ---- binary searches -----------------------------------------------------
// first index in a[lo,hi) with a[i] >= v
template <typename P>
__device__ __forceinline__ i64 lower_bound_i(const P *a, i64 lo, i64 hi, u32 v) {
  while (lo < hi) {
    i64 mid = lo + ((hi - lo) >> 1);
    if (a[mid] < v) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}
// first index in a[lo,hi) with a[i] > v
template <typename P>
__device__ __forceinline__ i64 upper_bound_i(const P *a, i64 lo, i64 hi, u32 v) {
  while (lo < hi) {
    i64 mid = lo + ((hi - lo) >> 1);
    if (a[mid] <= v) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}
// index of the last entry of the non-decreasing u32 array pre[0..n] that is <= v
// (pre[0] == 0 <= v is assumed); this is the run holding flat index v.
__device__ __forceinline__ u32 run_of(const u32 *pre, u32 n, u32 v) {
  u32 lo = 0, hi = n;  // answer in [0, n-1]
  while (hi - lo > 1) {
    u32 mid = (lo + hi) >> 1;
    if (pre[mid] <= v) lo = mid;
    else hi = mid;
  }
  return lo;
}

__device__ __forceinline__ u32 next_pow2(u32 x) {
  u32 p = 2;
  while (p < x) p <<= 1;
  return p;
}

// ---- LDS bitonic sort ----------------------------------------------------
// Sorts s[0..m) ascending, m a power of two >= 2, all BLOCK threads taking
// part.  Entries beyond the data must already be padded with the max key.
template <int BLOCK, typename K>
__device__ void lds_bitonic(K *s, u32 m) {
  for (u32 k = 2; k <= m; k <<= 1) {
    for (u32 j = k >> 1; j > 0; j >>= 1) {
      for (u32 i = threadIdx.x; i < (m >> 1); i += BLOCK) {
        u32 lo = ((i & ~(j - 1)) << 1) | (i & (j - 1));
        u32 hi = lo + j;
        K a = s[lo], b = s[hi];
        bool up = (lo & k) == 0;
        if ((a > b) == up) {
          s[lo] = b;
          s[hi] = a;
        }
      }
      __syncthreads();
    }
  }
}

template <typename K>
__device__ __forceinline__ K key_max();
template <>
__device__ __forceinline__ u32 key_max<u32>() { return 0xFFFFFFFFu; }
template <>
__device__ __forceinline__ u64 key_max<u64>() { return ~0ull; }

// Merge sorted A[0,na) and B[0,nb) into C (merge path; ties take A first).
template <int BLOCK, typename K>
__device__ void wg_merge(const K *A, u64 na, const K *B, u64 nb, K *C) {
  constexpr int ITEMS = 8;
  const u64 total = na + nb;
  for (u64 base = 0; base < total; base += (u64)BLOCK * ITEMS) {
    u64 d = base + (u64)threadIdx.x * ITEMS;
    if (d >= total) continue;
    u64 lo = d > nb ? d - nb : 0, hi = d < na ? d : na;
    while (lo < hi) {
      u64 mid = (lo + hi) >> 1;
      if (A[mid] <= B[d - 1 - mid]) lo = mid + 1;
      else hi = mid;
    }
    u64 i = lo, j = d - lo;
    for (int k = 0; k < ITEMS && d + k < total; ++k) {
      bool takeA = j >= nb || (i < na && A[i] <= B[j]);
      C[d + k] = takeA ? A[i++] : B[j++];
    }
  }
}

// Sort a[0,n) (global memory) with b[0,n) as scratch.  Chunks of CAP keys
// are sorted in LDS (lds holds CAP keys), then merged pairwise.  Returns the
// array holding the sorted result (a or b).  All threads must call.
template <int BLOCK, int CAP, typename K>
__device__ K *wg_sort_global(K *a, K *b, u64 n, K *lds) {
  for (u64 c0 = 0; c0 < n; c0 += CAP) {
    u32 cnt = (u32)((n - c0) < CAP ? (n - c0) : CAP);
    for (u32 i = threadIdx.x; i < CAP; i += BLOCK) lds[i] = i < cnt ? a[c0 + i] : key_max<K>();
    __syncthreads();
    lds_bitonic<BLOCK>(lds, (u32)CAP);
    for (u32 i = threadIdx.x; i < cnt; i += BLOCK) a[c0 + i] = lds[i];
    __syncthreads();
  }
  K *src = a, *dst = b;
  for (u64 w = CAP; w < n; w <<= 1) {
    for (u64 s = 0; s < n; s += 2 * w) {
      u64 na = (n - s) < w ? (n - s) : w;
      u64 rest = n - s - na;
      u64 nb = rest < w ? rest : w;
      wg_merge<BLOCK>(src + s, na, src + s + na, nb, dst + s);
    }
    __syncthreads();
    K *t = src;
    src = dst;
    dst = t;
  }
  __syncthreads();
  return src;
}

// Append the lanes of a wave whose `pred` holds to a device list: one atomic
// per wave on the shared counter; returns each such lane's slot.
__device__ __forceinline__ u32 wave_append(u32 *counter, bool pred) {
  const u64 m = __ballot(pred);
  if (m == 0) return 0;
  const u32 leader = (u32)__ffsll((unsigned long long)m) - 1;
  u32 base = 0;
  if (lane_id() == leader) base = atomicAdd(counter, (u32)__popcll(m));
  base = __shfl(base, leader, WAVE);
  return base + (u32)__popcll(m & ((1ull << lane_id()) - 1));
}

// Workgroup-aggregated append into NC class lists: a thread of class cls
// (0 <= cls < NC; any other value appends nothing) gets a slot unique within
// its class.  One atomic per class per workgroup (shared counters serialise
// their atomics, so per-wave appends cost ~1 ms per million items); every
// thread of the workgroup must call it.  lds holds NC * (BLOCK / WAVE) + NC
// words.
template <int BLOCK, int NC>
__device__ __forceinline__ u32 block_append(u32 *counters, int cls, u32 *lds) {
  constexpr int NW = BLOCK / WAVE;
  const u32 w = wave_id(), l = lane_id();
  u32 rank = 0;
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const u64 m = __ballot(cls == k);
    if (cls == k) rank = (u32)__popcll(m & ((1ull << l) - 1));
    if (l == 0) lds[k * NW + w] = (u32)__popcll(m);
  }
  __syncthreads();
  if ((int)threadIdx.x < NC) {
    const int k = threadIdx.x;
    u32 tot = 0;
    for (int i = 0; i < NW; ++i) {
      const u32 c = lds[k * NW + i];
      lds[k * NW + i] = tot;
      tot += c;
    }
    lds[NC * NW + k] = tot ? atomicAdd(&counters[k], tot) : 0u;
  }
  __syncthreads();
  const u32 slot = (cls >= 0 && cls < NC) ? lds[NC * NW + cls] + lds[cls * NW + w] + rank : 0u;
  __syncthreads();
  return slot;
}

// Bitonic sort of one key per lane across a wave (ascending by lane).
template <typename K>
__device__ __forceinline__ K wave_sort64(K v) {
  const u32 l = lane_id();
#pragma unroll
  for (u32 k = 2; k <= 64; k <<= 1) {
#pragma unroll
    for (u32 j = k >> 1; j > 0; j >>= 1) {
      K w = __shfl_xor(v, j, WAVE);
      bool up = (l & k) == 0;
      bool lower = (l & j) == 0;
      v = (lower == up) ? (v < w ? v : w) : (v < w ? w : v);
    }
  }
  return v;
}

// Compare-exchange: x takes the smaller key, y the larger.
__device__ __forceinline__ void cswap(u64 &x, u64 &y) {
  const u64 lo = x < y ? x : y, hi = x < y ? y : x;
  x = lo;
  y = hi;
}

// Bitonic sort of 64 PER keys across a wave, PER a lane (afterwards lane l
// holds sorted positions PER l .. PER l + PER - 1, ascending; where each key
// starts does not matter): the compare-exchanges at distances below PER stay
// within a lane, the others pair lanes l and l ^ (j / PER).
template <typename K, int PER>
__device__ __forceinline__ void wave_sort_regs(K (&v)[PER]) {
  const u32 l = lane_id();
#pragma unroll
  for (u32 k = 2; k <= 64 * PER; k <<= 1) {
#pragma unroll
    for (u32 j = k >> 1; j > 0; j >>= 1) {
      if (j >= (u32)PER) {
#pragma unroll
        for (u32 r = 0; r < (u32)PER; ++r) {
          const u32 i = PER * l + r;
          const K w = __shfl_xor(v[r], (int)(j / PER), WAVE);
          const bool up = (i & k) == 0, lower = (i & j) == 0;
          v[r] = (lower == up) ? (v[r] < w ? v[r] : w) : (v[r] < w ? w : v[r]);
        }
      } else {
#pragma unroll
        for (u32 r = 0; r < (u32)PER; ++r) {
          if (r & j) continue;
          const bool up = ((PER * l + r) & k) == 0;
          const K a = v[r], b = v[r | j];
          const bool sw = up ? b < a : a < b;
          v[r] = sw ? b : a;
          v[r | j] = sw ? a : b;
        }
      }
    }
  }
}

// wave_group_split_emit for m sorted keys held PER a lane as wave_sort_regs
// leaves them (value << 1 | tag, 32 or 64 bits; a group of equal value is
// represented by its first key): the values of the groups whose first tag is
// FIRST_TAG go to out[0, n_first), the others to out[n_first, n_total), each
// in order.
template <u32 FIRST_TAG, int PER, typename K>
__device__ __forceinline__ void wave_group_split_emit_regs(const K (&v)[PER], u32 m, u32 *out,
                                                           u32 &n_first, u32 &n_total) {
  const u32 l = lane_id();
  const K prev_last = __shfl_up(v[PER - 1], 1, WAVE);
  u32 fmask = 0, omask = 0;
#pragma unroll
  for (u32 r = 0; r < (u32)PER; ++r) {
    const u32 i = PER * l + r;
    const K pk = r ? v[r - 1] : prev_last;
    const bool f = i < m && (i == 0 || (pk >> 1) != (v[r] >> 1));
    const bool ff = f && (u32)(v[r] & 1) == FIRST_TAG;
    fmask |= (ff ? 1u : 0u) << r;
    omask |= (f && !ff ? 1u : 0u) << r;
  }
  const u32 cf = (u32)__builtin_popcount(fmask), co = (u32)__builtin_popcount(omask);
  const u32 incf = wave_incl_scan(cf), inco = wave_incl_scan(co);
  const u32 nf = __shfl(incf, WAVE - 1, WAVE), no = __shfl(inco, WAVE - 1, WAVE);
  u32 pf = incf - cf, po = nf + inco - co;
#pragma unroll
  for (u32 r = 0; r < (u32)PER; ++r) {
    if ((fmask >> r) & 1) out[pf++] = (u32)(v[r] >> 1);
    else if ((omask >> r) & 1) out[po++] = (u32)(v[r] >> 1);
  }
  n_first = nf;
  n_total = nf + no;
}

// Sorted keys s[0,m) of the form (value << 1 | tag); each group of equal
// value is represented by its first key, whose tag is the group's smallest.
// Writes the distinct values of the groups whose first tag is FIRST_TAG to
// out[0, n_first), then the others to out[n_first, n_total).  Works on LDS or
// global keys; every thread of the workgroup calls it.
template <int BLOCK, u32 FIRST_TAG>
__device__ void group_split_emit(const u64 *s, u32 m, u32 *out, u32 &n_first, u32 &n_total,
                                 u32 *s_red) {
  u32 nf = 0, no = 0;
  for (u32 c0 = 0; c0 < m; c0 += BLOCK) {
    const u32 i = c0 + threadIdx.x;
    const u64 k = i < m ? s[i] : 0;
    const bool f = i < m && (i == 0 || (s[i - 1] >> 1) != (k >> 1));
    nf += wg_sum<BLOCK>((u32)(f && (u32)(k & 1) == FIRST_TAG), s_red);
    no += wg_sum<BLOCK>((u32)(f && (u32)(k & 1) != FIRST_TAG), s_red);
  }
  u32 rf = 0, ro = 0;
  for (u32 c0 = 0; c0 < m; c0 += BLOCK) {
    const u32 i = c0 + threadIdx.x;
    const u64 k = i < m ? s[i] : 0;
    const bool f = i < m && (i == 0 || (s[i - 1] >> 1) != (k >> 1));
    const bool ff = f && (u32)(k & 1) == FIRST_TAG, fo = f && (u32)(k & 1) != FIRST_TAG;
    u32 tf, to;
    const u32 of = wg_excl_scan<BLOCK>((u32)ff, s_red, &tf);
    const u32 oo = wg_excl_scan<BLOCK>((u32)fo, s_red, &to);
    if (ff) out[rf + of] = (u32)(k >> 1);
    if (fo) out[nf + ro + oo] = (u32)(k >> 1);
    rf += tf;
    ro += to;
  }
  n_first = nf;
  n_total = nf + no;
}

// The same for one wave holding one key per lane (sorted across lanes, keys
// of lanes >= m are the maximum key).
template <u32 FIRST_TAG>
__device__ __forceinline__ void wave_group_split_emit(u64 key, u32 m, u32 *out, u32 &n_first,
                                                      u32 &n_total) {
  const u32 l = lane_id();
  const u64 prev = __shfl_up(key, 1, WAVE);
  const bool f = l < m && (l == 0 || (prev >> 1) != (key >> 1));
  const bool ff = f && (u32)(key & 1) == FIRST_TAG;
  const u64 fm = __ballot(ff), om = __ballot(f && !ff);
  const u64 lt = (1ull << l) - 1;
  const u32 nf = (u32)__popcll(fm);
  if (f) out[ff ? (u32)__popcll(fm & lt) : nf + (u32)__popcll(om & lt)] = (u32)(key >> 1);
  n_first = nf;
  n_total = nf + (u32)__popcll(om);
}

// Write the unique keys of sorted src[0,m) other than `skip` to out; returns
// the count (all threads).
template <int BLOCK>
__device__ u32 unique_out(const u32 *src, u64 m, u32 skip, u32 *out, u32 *s_red) {
  u32 run = 0;
  for (u64 c0 = 0; c0 < m; c0 += BLOCK) {
    u64 i = c0 + threadIdx.x;
    bool keep = false;
    u32 v = 0;
    if (i < m) {
      v = src[i];
      keep = v != skip && v != NONE32 && (i == 0 || src[i - 1] != v);
    }
    u32 tot;
    u32 off = wg_excl_scan<BLOCK>((u32)keep, s_red, &tot);
    if (keep) out[run + off] = v;
    run += tot;
  }
  return run;
}

// ---- rating noise ---------------------------------------------------------
// One output of splitmix64 (Steele, Lea & Flood, OOPSLA 2014) from `state`.
__device__ __forceinline__ u64 splitmix64_out(u64 state) {
  u64 z = state + 0x9e3779b97f4a7c15ull;
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}

// x mod d for d >= 2 given magic = floor((2^64-1)/d): the quotient estimate
// mulhi(x, magic) is at most 2 below floor(x/d) (division by invariant
// integers, Granlund & Montgomery, PLDI 1994), fixed by two subtractions.
__device__ __forceinline__ u64 mod_magic(u64 x, u64 d, u64 magic) {
  u64 q = __umul64hi(x, magic);
  u64 r = x - q * d;
  if (r >= d) r -= d;
  if (r >= d) r -= d;
  return r;
}

// Symmetric noise of the pair {n, m} in [0, cap]; d = cap + 1.
__device__ __forceinline__ u64 pair_noise(u64 seed, u32 n, u32 m, u64 d, u64 magic) {
  if (d <= 1) return 0;
  u32 a = n < m ? n : m, b = n < m ? m : n;
  u64 x = splitmix64_out(seed ^ (((u64)a << 32) | b));
  return mod_magic(x, d, magic);
}
