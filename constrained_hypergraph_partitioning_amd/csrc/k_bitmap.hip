// Sorted distinct neighbour lists through an LDS bitmap over the id span.
//
// A neighbourhood N(n) ("Hypergraph Partitioning on GPU with Distinct
// Incident Hyperedges and Size Constraints", Sec. II-A, materialised as in
// Sec. V-B) is the set of distinct ids among a multiset of values: the pins
// of n's incident hyperedges at the first level, gamma of the members'
// neighbour lists on a coarse level (Sec. V-E).  Instead of sorting the
// multiset, each value sets one bit of an LDS bitmap covering [lo, hi] of
// the values' span (in windows of BMW * 32 ids when the span is larger), and
// the set bits are read back in id order: word popcounts, a workgroup scan
// for the output positions, then each thread writes the ids of its words.
// Work is O(values + span / 32) and the output comes out sorted.
#include "dev.h"
#include "kernels.h"

namespace {

constexpr int BB = 256;       // threads per workgroup
// 33 KB of LDS per workgroup, four workgroups per CU (two of twice the size
// were 4% slower on the ring, 7% on the netlist)
constexpr u32 BMW = 4096;      // bitmap words (131,072 ids per window)
constexpr u32 STG = 4096;      // values staged in LDS (larger sets are read twice)
constexpr u32 NB_WG_PER_CU = 4;

constexpr u32 NHB = 64;       // buckets of the id histogram (level 0, wide spans)

struct BitmapSmem {
  u32 bm[BMW];
  u32 stg[STG];
  i64 start[BB];
  u32 pre[BB + 1];
  u32 red[BB / WAVE + 1];
  u32 redx[BB / WAVE + 1];
  u32 hist[NHB];
  u32 lcnt, wlo;
};

// Emit the set bits of bm[0, nw) as ids lo + bit, ascending, to out; the
// bitmap is cleared on the way.  Returns the count (all threads).
__device__ u32 bitmap_emit(u32 *bm, u32 nw, u32 lo, u32 *out, u32 *s_red) {
  const u32 per = (nw + BB - 1) / BB;
  const u32 w0 = threadIdx.x * per < nw ? threadIdx.x * per : nw;
  const u32 w1 = w0 + per < nw ? w0 + per : nw;
  u32 c = 0;
  for (u32 w = w0; w < w1; ++w) c += (u32)__popc(bm[w]);
  u32 tot;
  u32 off = wg_excl_scan<BB>(c, s_red, &tot);
  for (u32 w = w0; w < w1; ++w) {
    u32 bits = bm[w];
    if (!bits) continue;
    bm[w] = 0;
    const u32 base = lo + w * 32;
    while (bits) {
      const u32 j = (u32)__ffs(bits) - 1;
      bits &= bits - 1;
      out[off++] = base + j;
    }
  }
  __syncthreads();
  return tot;
}

__device__ __forceinline__ u32 wg_min_u32(u32 v, u32 *lds) {
#pragma unroll
  for (int d = WAVE / 2; d > 0; d >>= 1) {
    const u32 o = __shfl_xor(v, d, WAVE);
    v = o < v ? o : v;
  }
  if (lane_id() == 0) lds[wave_id()] = v;
  __syncthreads();
  u32 m = lds[0];
#pragma unroll
  for (int w = 1; w < BB / WAVE; ++w) m = lds[w] < m ? lds[w] : m;
  __syncthreads();
  return m;
}

__device__ __forceinline__ u32 wg_max_u32(u32 v, u32 *lds) {
#pragma unroll
  for (int d = WAVE / 2; d > 0; d >>= 1) {
    const u32 o = __shfl_xor(v, d, WAVE);
    v = o > v ? o : v;
  }
  if (lane_id() == 0) lds[wave_id()] = v;
  __syncthreads();
  u32 m = lds[0];
#pragma unroll
  for (int w = 1; w < BB / WAVE; ++w) m = lds[w] > m ? lds[w] : m;
  __syncthreads();
  return m;
}

// Call f(pin) for every pin of the hyperedges n_inc[a, b): hyperedges are
// taken BB at a time, a scan lays their segments end to end and each thread
// finds its segment by binary search over the prefix.
template <typename F>
__device__ void for_each_pin(const i64 *e_off, const u32 *pins, const u32 *n_inc, i64 a, i64 b,
                             BitmapSmem &S, F f) {
  for (i64 c0 = a; c0 < b; c0 += BB) {
    const u32 ne = (u32)((b - c0) < BB ? (b - c0) : BB);
    u32 len = 0;
    if (threadIdx.x < ne) {
      const u32 e = n_inc[c0 + threadIdx.x];
      const i64 s = e_off[e];
      len = (u32)(e_off[e + 1] - s);
      S.start[threadIdx.x] = s;
    }
    u32 tot;
    const u32 off = wg_excl_scan<BB>(len, S.red, &tot);
    if (threadIdx.x < ne) S.pre[threadIdx.x] = off;
    if (threadIdx.x == 0) S.pre[ne] = tot;
    __syncthreads();
    for (u32 i = threadIdx.x; i < tot; i += BB) {
      const u32 r = run_of(S.pre, ne + 1, i);
      f(pins[S.start[r] + (i - S.pre[r])]);
    }
    __syncthreads();
  }
}

// Bits of the values in [lo, lo + 32 nw) other than skip, then emit.
template <typename G>
__device__ u32 window_pass(BitmapSmem &S, u32 lo, u32 nw, u32 skip, u32 *out, G for_values) {
  const u32 span = nw * 32;
  for_values([&](u32 v) {
    const u32 d = v - lo;
    if (v != skip && d < span) atomicOr(&S.bm[d >> 5], 1u << (d & 31));
  });
  __syncthreads();
  return bitmap_emit(S.bm, nw, lo, out, S.red);
}

// All windows over [mn, mx]; returns the number of distinct values.
template <typename G>
__device__ u32 bitmap_distinct(BitmapSmem &S, u32 mn, u32 mx, u32 skip, u32 *out,
                               G for_values) {
  u32 cnt = 0;
  if (mn > mx) return 0;
  for (u64 lo = mn; lo <= mx; lo += (u64)BMW * 32) {
    const u64 hi = (lo + (u64)BMW * 32 - 1) < mx ? (lo + (u64)BMW * 32 - 1) : mx;
    const u32 nw = (u32)((hi - lo) / 32 + 1);
    cnt += window_pass(S, (u32)lo, nw, skip, out + cnt, for_values);
  }
  return cnt;
}

// The same over keys value << 1 | flag: a value is kept iff none of its
// copies is flagged (its bit is set by every copy, then cleared by the
// flagged ones).
template <typename G>
__device__ u32 bitmap_distinct_unflagged(BitmapSmem &S, u32 mn, u32 mx, u32 skip, u32 *out,
                                         G for_keys) {
  u32 cnt = 0;
  if (mn > mx) return 0;
  for (u64 lo = mn; lo <= mx; lo += (u64)BMW * 32) {
    const u64 hi = (lo + (u64)BMW * 32 - 1) < mx ? (lo + (u64)BMW * 32 - 1) : mx;
    const u32 nw = (u32)((hi - lo) / 32 + 1);
    const u32 span = nw * 32, l0 = (u32)lo;
    for_keys([&](u32 k) {
      const u32 v = k >> 1, d = v - l0;
      if (v != skip && d < span) atomicOr(&S.bm[d >> 5], 1u << (d & 31));
    });
    __syncthreads();
    for_keys([&](u32 k) {
      const u32 d = (k >> 1) - l0;
      if ((k & 1) && d < span) atomicAnd(&S.bm[d >> 5], ~(1u << (d & 31)));
    });
    __syncthreads();
    cnt += bitmap_emit(S.bm, nw, l0, out + cnt, S.red);
  }
  return cnt;
}

// Level 0 for a node whose values are not staged and whose id span exceeds
// one window: the histogram (NHB buckets of 2^hshift ids) picks the window
// with the most values; those set bits, the others go to a list in LDS
// (stg), which is sorted and made unique.  Output: list values below the
// window, the window's ids, list values above it.  Returns false (bitmap
// clean) if the list overflows, the caller then takes every window in turn.
__device__ bool hybrid_distinct(BitmapSmem &S, const i64 *e_off, const u32 *pins,
                                const u32 *n_inc, i64 a, i64 b, u32 n, u32 mn, u32 mx,
                                u32 hshift, u32 *out, u32 *count_out) {
  const u32 span = BMW * 32;
  const u32 wb = (span >> hshift) > 0 ? (span >> hshift) : 1;  // buckets per window
  if (threadIdx.x == 0) {
    u32 best = 0, bs = 0;
    for (u32 s0 = 0; s0 < NHB; ++s0) {
      u32 t = 0;
      for (u32 k = s0; k < s0 + wb && k < NHB; ++k) t += S.hist[k];
      if (t > best) best = t, bs = s0;
    }
    const u64 lo = (u64)bs << hshift;
    S.wlo = lo < mn ? mn : (u32)lo;
    S.lcnt = 0;
  }
  __syncthreads();
  const u32 wlo = S.wlo;
  const u32 whi = (u64)wlo + span - 1 < mx ? wlo + span - 1 : mx;
  for_each_pin(e_off, pins, n_inc, a, b, S, [&](u32 v) {
    if (v == n) return;
    if (v >= wlo && v <= whi) {
      const u32 d = v - wlo;
      atomicOr(&S.bm[d >> 5], 1u << (d & 31));
    } else {
      const u32 i = atomicAdd(&S.lcnt, 1u);
      if (i < STG) S.stg[i] = v;
    }
  });
  __syncthreads();
  const u32 lc = S.lcnt;
  const u32 nw = (whi - wlo) / 32 + 1;
  if (lc > STG) {
    for (u32 i = threadIdx.x; i < nw; i += BB) S.bm[i] = 0;
    __syncthreads();
    return false;
  }
  // sort the list, then its distinct values get their ranks
  if (lc > 1) {
    const u32 p = next_pow2(lc);
    for (u32 i = lc + threadIdx.x; i < p; i += BB) S.stg[i] = NONE32;
    __syncthreads();
    lds_bitonic<BB>(S.stg, p);
  }
  __syncthreads();
  u32 below = 0;
  for (u32 i = threadIdx.x; i < lc; i += BB) {
    const u32 v = S.stg[i];
    if (v < wlo && (i == 0 || S.stg[i - 1] != v)) ++below;
  }
  below = wg_sum<BB>(below, S.red);
  const u32 nbm = bitmap_emit(S.bm, nw, wlo, out + below, S.red);
  u32 run = 0;
  for (u32 c0 = 0; c0 < lc; c0 += BB) {
    const u32 i = c0 + threadIdx.x;
    u32 v = 0;
    bool keep = false;
    if (i < lc) {
      v = S.stg[i];
      keep = i == 0 || S.stg[i - 1] != v;
    }
    u32 tot;
    const u32 off = wg_excl_scan<BB>((u32)keep, S.red, &tot);
    if (keep) out[run + off + (v < wlo ? 0 : nbm)] = v;
    run += tot;
  }
  if (threadIdx.x == 0) *count_out = nbm + run;
  __syncthreads();
  return true;
}

// Level 0: N(n) = distinct pins of I(n) other than n.  W_n = bound[n] + |I(n)|.
__global__ __launch_bounds__(BB) void k_nb_bitmap(const i64 *e_off, const u32 *pins,
                                                  const i64 *n_off, const u32 *n_inc,
                                                  const u32 *bound, const i64 *ooff, u32 *obuf,
                                                  u32 *count, const u32 *list, const u32 *cnt,
                                                  u32 hshift) {
  __shared__ BitmapSmem S;
  for (u32 i = threadIdx.x; i < BMW; i += BB) S.bm[i] = 0;
  __syncthreads();
  const u32 total = *cnt;
  for (u32 w = blockIdx.x; w < total; w += gridDim.x) {
    const u32 n = list[w];
    const i64 a = n_off[n], b = n_off[n + 1];
    const u64 W = (u64)bound[n] + (u64)(b - a);
    const bool staged = W <= STG;
    if (!staged)
      for (u32 i = threadIdx.x; i < NHB; i += BB) S.hist[i] = 0;
    __syncthreads();
    u32 mn = NONE32, mx = 0;
    // stage (when small) and take the span; unstaged, also the histogram
    u32 base = 0;
    for (i64 c0 = a; c0 < b; c0 += BB) {
      const u32 ne = (u32)((b - c0) < BB ? (b - c0) : BB);
      u32 len = 0;
      if (threadIdx.x < ne) {
        const u32 e = n_inc[c0 + threadIdx.x];
        const i64 s = e_off[e];
        len = (u32)(e_off[e + 1] - s);
        S.start[threadIdx.x] = s;
      }
      u32 tot;
      const u32 off = wg_excl_scan<BB>(len, S.red, &tot);
      if (threadIdx.x < ne) S.pre[threadIdx.x] = off;
      if (threadIdx.x == 0) S.pre[ne] = tot;
      __syncthreads();
      for (u32 i = threadIdx.x; i < tot; i += BB) {
        const u32 r = run_of(S.pre, ne + 1, i);
        const u32 v = pins[S.start[r] + (i - S.pre[r])];
        if (staged) S.stg[base + i] = v;
        if (v != n) {
          mn = v < mn ? v : mn;
          mx = v > mx ? v : mx;
          if (!staged) atomicAdd(&S.hist[v >> hshift], 1u);
        }
      }
      base += tot;
      __syncthreads();
    }
    mn = wg_min_u32(mn, S.redx);
    mx = wg_max_u32(mx, S.redx);
    if (staged) {
      const u32 m = (u32)W;
      const u32 c = bitmap_distinct(S, mn, mx, n, obuf + ooff[n], [&](auto f) {
        for (u32 i = threadIdx.x; i < m; i += BB) f(S.stg[i]);
      });
      if (threadIdx.x == 0) count[n] = c;
    } else if (mn > mx || (u64)(mx - mn) < (u64)BMW * 32 ||
               !hybrid_distinct(S, e_off, pins, n_inc, a, b, n, mn, mx, hshift, obuf + ooff[n],
                                count + n)) {
      const u32 c = bitmap_distinct(S, mn, mx, n, obuf + ooff[n], [&](auto f) {
        for_each_pin(e_off, pins, n_inc, a, b, S, f);
      });
      if (threadIdx.x == 0) count[n] = c;
    }
    __syncthreads();
  }
}

// Coarse level: N'(c) = distinct gamma(N(a) u N(b)) other than c; with the
// invalid-neighbour flags fl, also without the images of flagged entries.
__global__ __launch_bounds__(BB) void k_nbm_bitmap(const i64 *nb_off, const u32 *nb,
                                                   const uint8_t *fl, const u32 *gamma,
                                                   const u32 *match, const u32 *rep_of,
                                                   const i64 *ooff, u32 *obuf, u32 *count,
                                                   const u32 *list, const u32 *cnt) {
  __shared__ BitmapSmem S;
  for (u32 i = threadIdx.x; i < BMW; i += BB) S.bm[i] = 0;
  __syncthreads();
  const u32 total = *cnt;
  for (u32 w = blockIdx.x; w < total; w += gridDim.x) {
    const u32 c = list[w];
    const u32 a = rep_of[c], b = match[a];
    const i64 a0 = nb_off[a];
    const u32 ka = (u32)(nb_off[a + 1] - a0);
    i64 b0 = 0;
    u32 kb = 0;
    if (b != a) {
      b0 = nb_off[b];
      kb = (u32)(nb_off[b + 1] - b0);
    }
    const u32 m = ka + kb;
    const bool staged = m <= STG;
    // a key is gamma, or gamma << 1 | flag with flags
    auto key_at = [&](u32 i) {
      const i64 j = i < ka ? a0 + i : b0 + (i - ka);
      const u32 g = gamma[nb[j]];
      return fl ? (g << 1) | (u32)fl[j] : g;
    };
    u32 mn = NONE32, mx = 0;
    // KU keys per thread per pass, their loads issued together
    constexpr u32 KU = 4;
    for (u32 i0 = threadIdx.x; i0 < m; i0 += BB * KU) {
      u32 kv[KU];
#pragma unroll
      for (u32 u = 0; u < KU; ++u) {
        const u32 i = i0 + u * BB;
        kv[u] = key_at(i < m ? i : 0);
      }
#pragma unroll
      for (u32 u = 0; u < KU; ++u) {
        const u32 i = i0 + u * BB;
        if (i >= m) continue;
        if (staged) S.stg[i] = kv[u];
        const u32 v = fl ? kv[u] >> 1 : kv[u];
        if (v != c) {
          mn = v < mn ? v : mn;
          mx = v > mx ? v : mx;
        }
      }
    }
    mn = wg_min_u32(mn, S.redx);
    mx = wg_max_u32(mx, S.redx);
    u32 k;
    if (fl) {
      if (staged)
        k = bitmap_distinct_unflagged(S, mn, mx, c, obuf + ooff[c], [&](auto f) {
          for (u32 i = threadIdx.x; i < m; i += BB) f(S.stg[i]);
        });
      else
        k = bitmap_distinct_unflagged(S, mn, mx, c, obuf + ooff[c], [&](auto f) {
          for (u32 i = threadIdx.x; i < m; i += BB) f(key_at(i));
        });
    } else if (staged) {
      k = bitmap_distinct(S, mn, mx, c, obuf + ooff[c], [&](auto f) {
        for (u32 i = threadIdx.x; i < m; i += BB) f(S.stg[i]);
      });
    } else {
      k = bitmap_distinct(S, mn, mx, c, obuf + ooff[c], [&](auto f) {
        for (u32 i = threadIdx.x; i < m; i += BB) f(key_at(i));
      });
    }
    if (threadIdx.x == 0) count[c] = k;
    __syncthreads();
  }
}

}  // namespace

void launch_nb_bitmap(chp_ctx *c, u32 N, const i64 *e_off, const u32 *pins, const i64 *n_off,
                      const u32 *n_inc, const u32 *bound, const i64 *ooff, u32 *obuf, u32 *count,
                      const u32 *list, const u32 *cnt, u32 host_count) {
  if (!host_count) return;
  u32 hshift = 0;  // NHB buckets of 2^hshift ids cover [0, N)
  while (((u64)(N ? N - 1 : 0) >> hshift) >= NHB) ++hshift;
  const u32 g = NB_WG_PER_CU * c->n_cu;
  CHP_LAUNCH(c, "nb_bitmap", k_nb_bitmap, host_count < g ? host_count : g,
             BB, 0, e_off, pins, n_off, n_inc, bound, ooff, obuf, count, list, cnt, hshift);
}

void launch_nbm_bitmap(chp_ctx *c, const i64 *nb_off, const u32 *nb, const uint8_t *fl,
                       const u32 *gamma, const u32 *match, const u32 *rep_of, const i64 *ooff,
                       u32 *obuf, u32 *count, const u32 *list, const u32 *cnt, u32 host_count) {
  if (!host_count) return;
  const u32 g = NB_WG_PER_CU * c->n_cu;
  CHP_LAUNCH(c, "nbm_bitmap", k_nbm_bitmap, host_count < g ? host_count : g,
             BB, 0, nb_off, nb, fl, gamma, match, rep_of, ooff, obuf, count, list, cnt);
}
