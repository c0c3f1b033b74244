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
constexpr u32 BMW = 8192;     // bitmap words (262,144 ids per window)
constexpr u32 STG = 8192;     // values staged in LDS (larger sets are read twice)

struct BitmapSmem {
  u32 bm[BMW];
  u32 stg[STG];
  i64 start[BB];
  u32 pre[BB + 1];
  u32 red[BB / WAVE + 1];
  u32 redx[BB / WAVE + 1];
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

// Level 0: N(n) = distinct pins of I(n) other than n.  W_n = bound[n] + |I(n)|.
__global__ __launch_bounds__(BB) void k_nb_bitmap(const i64 *e_off, const u32 *pins,
                                                  const i64 *n_off, const u32 *n_inc,
                                                  const u32 *bound, const i64 *ooff, u32 *obuf,
                                                  u32 *count, const u32 *list, const u32 *cnt) {
  __shared__ BitmapSmem S;
  for (u32 i = threadIdx.x; i < BMW; i += BB) S.bm[i] = 0;
  __syncthreads();
  const u32 total = *cnt;
  for (u32 w = blockIdx.x; w < total; w += gridDim.x) {
    const u32 n = list[w];
    const i64 a = n_off[n], b = n_off[n + 1];
    const u64 W = (u64)bound[n] + (u64)(b - a);
    const bool staged = W <= STG;
    u32 mn = NONE32, mx = 0;
    // stage (when small) and take the span
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
        }
      }
      base += tot;
      __syncthreads();
    }
    mn = wg_min_u32(mn, S.redx);
    mx = wg_max_u32(mx, S.redx);
    u32 c;
    if (staged) {
      const u32 m = (u32)W;
      c = bitmap_distinct(S, mn, mx, n, obuf + ooff[n], [&](auto f) {
        for (u32 i = threadIdx.x; i < m; i += BB) f(S.stg[i]);
      });
    } else {
      c = bitmap_distinct(S, mn, mx, n, obuf + ooff[n], [&](auto f) {
        for_each_pin(e_off, pins, n_inc, a, b, S, f);
      });
    }
    if (threadIdx.x == 0) count[n] = c;
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
    for (u32 i = threadIdx.x; i < m; i += BB) {
      const u32 k = key_at(i);
      if (staged) S.stg[i] = k;
      const u32 v = fl ? k >> 1 : k;
      if (v != c) {
        mn = v < mn ? v : mn;
        mx = v > mx ? v : mx;
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

void launch_nb_bitmap(chp_ctx *c, const i64 *e_off, const u32 *pins, const i64 *n_off,
                      const u32 *n_inc, const u32 *bound, const i64 *ooff, u32 *obuf, u32 *count,
                      const u32 *list, const u32 *cnt, u32 host_count) {
  if (!host_count) return;
  CHP_LAUNCH(c, "nb_bitmap", k_nb_bitmap, host_count < 2 * c->n_cu ? host_count : 2 * c->n_cu,
             BB, 0, e_off, pins, n_off, n_inc, bound, ooff, obuf, count, list, cnt);
}

void launch_nbm_bitmap(chp_ctx *c, const i64 *nb_off, const u32 *nb, const uint8_t *fl,
                       const u32 *gamma, const u32 *match, const u32 *rep_of, const i64 *ooff,
                       u32 *obuf, u32 *count, const u32 *list, const u32 *cnt, u32 host_count) {
  if (!host_count) return;
  CHP_LAUNCH(c, "nbm_bitmap", k_nbm_bitmap, host_count < 2 * c->n_cu ? host_count : 2 * c->n_cu,
             BB, 0, nb_off, nb, fl, gamma, match, rep_of, ooff, obuf, count, list, cnt);
}
