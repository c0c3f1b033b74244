// Coarse incidence and coarse neighbourhoods, built from the members' lists
// ("Hypergraph Partitioning on GPU with Distinct Incident Hyperedges and Size
// Constraints", Sec. V-E: incidence and neighbour sets of a cluster are unions
// of its members' sets).
//
// A coarse hyperedge keeps the id of its fine one and gamma(dst) is its
// destination set, so for the cluster c = {a, b}
//   in'(c)  = in(a) u in(b),
//   out'(c) = (out(a) u out(b)) \ in'(c),
//   N'(c)   = (gamma(N(a)) u gamma(N(b))) \ {c}.
// All three equal the definitions on the coarse graph.  A singleton keeps
// its incidence unchanged (a copy).  gamma is strictly increasing on
// cluster representatives (the rank of the smallest member), so gamma(N(a))
// restricted to representatives is already sorted: only the entries that are
// second members of a pair need sorting before the lists are merged.
#include "dev.h"
#include "kernels.h"

namespace {

// ---------------------------------------------------------------------------
// coarse incidence
//
// Per cluster: singletons get their final counts at once and are copied in
// the compaction pass; a pair gets the bound |I(a)| + |I(b)| in the oversize
// buffer and is merged by one sort of 64-bit keys (edge << 1 | is_out): in
// each group of equal edge the first key tells whether it is inbound.
// Classes by that bound: one wave (<= 64 keys in one register a lane,
// <= CINC_SMALL in up to 16), a workgroup with an LDS table of LDS_CAP_U64
// keys, global.
constexpr u32 CINC_SMALL = 1024;
__global__ __launch_bounds__(256) void k_cinc_classify(u32 Nc, const u32 *rep_of,
                                                       const u32 *match, const i64 *n_off,
                                                       const u32 *n_nin, u32 *bound,
                                                       u32 *cnt_in, u32 *cnt_tot, EdgeLists el) {
  __shared__ u32 s_app[4 * (256 / WAVE) + 4];
  const u32 c = blockIdx.x * blockDim.x + threadIdx.x;
  int cls = 4;
  u64 w = 0;
  if (c < Nc) {
    const u32 a = rep_of[c], b = match[a];
    const u64 da = (u64)(n_off[a + 1] - n_off[a]);
    if (b == a) {
      cnt_in[c] = n_nin[a];
      cnt_tot[c] = (u32)da;
      bound[c] = 0;
    } else {
      w = da + (u64)(n_off[b + 1] - n_off[b]);
      bound[c] = (u32)w;
      cls = w <= 64 ? 0 : w <= CINC_SMALL ? 1 : w <= LDS_CAP_U64 ? 3 : 2;
    }
  }
  const u32 slot = block_append<256, 4>(el.cnt, cls, s_app);
  if (cls < 4) el.list[cls][slot] = c;
  if (cls == 2) atomicMax(&el.cnt[4], (u32)w);
}

__device__ __forceinline__ u64 inc_key(const i64 *n_off, const u32 *n_nin, const u32 *n_inc,
                                       u32 a, u32 b, u32 i) {
  const i64 a0 = n_off[a];
  const u32 da = (u32)(n_off[a + 1] - a0);
  u32 node = a, j = i;
  i64 base = a0;
  if (i >= da) {
    node = b;
    j = i - da;
    base = n_off[b];
  }
  return ((u64)n_inc[base + j] << 1) | (j >= n_nin[node] ? 1u : 0u);
}

__global__ __launch_bounds__(256) void k_cinc_wave(const i64 *n_off, const u32 *n_nin,
                                                   const u32 *n_inc, const u32 *rep_of,
                                                   const u32 *match, const i64 *ooff, u32 *obuf,
                                                   u32 *cnt_in, u32 *cnt_tot, const u32 *list,
                                                   const u32 *cnt) {
  const u32 total = *cnt;
  const u32 nwaves = gridDim.x * (blockDim.x / WAVE);
  const u32 l = lane_id();
  for (u32 w = blockIdx.x * (blockDim.x / WAVE) + wave_id(); w < total; w += nwaves) {
    const u32 c = list[w];
    const u32 a = rep_of[c], b = match[a];
    const u32 m = (u32)(n_off[a + 1] - n_off[a] + n_off[b + 1] - n_off[b]);
    u64 key = ~0ull;
    if (l < m) key = inc_key(n_off, n_nin, n_inc, a, b, l);
    key = wave_sort64(key);
    u32 nin, ntot;
    wave_group_split_emit<0>(key, m, obuf + ooff[c], nin, ntot);
    if (l == 0) {
      cnt_in[c] = nin;
      cnt_tot[c] = ntot;
    }
  }
}

// Pairs with a bound of 65 .. CINC_SMALL: a wave each, the keys sorted in
// registers (4, 8 or 16 a lane, by the bound), inbound hyperedges first.
// K = u32 when every hyperedge id is below 2^31 - 1 (the key e << 1 | is_out
// then fits 32 bits, below the padding ~0), u64 otherwise.
template <typename K, int PER>
__device__ __forceinline__ void cinc_regs(const i64 *n_off, const u32 *n_nin, const u32 *n_inc,
                                          u32 a, u32 b, u32 m, u32 *out, u32 &nin, u32 &ntot) {
  const u32 l = lane_id();
  K v[PER];
#pragma unroll
  for (u32 q = 0; q < (u32)PER; ++q) {
    const u32 i = q * WAVE + l;
    v[q] = i < m ? (K)inc_key(n_off, n_nin, n_inc, a, b, i) : ~(K)0;
  }
  wave_sort_regs<K, PER>(v);
  wave_group_split_emit_regs<0, PER>(v, m, out, nin, ntot);
}

template <typename K>
__global__ __launch_bounds__(256) void k_cinc_wreg(const i64 *n_off, const u32 *n_nin,
                                                   const u32 *n_inc, const u32 *rep_of,
                                                   const u32 *match, const i64 *ooff, u32 *obuf,
                                                   u32 *cnt_in, u32 *cnt_tot, const u32 *list,
                                                   const u32 *cnt) {
  const u32 total = *cnt;
  const u32 nwaves = gridDim.x * (blockDim.x / WAVE);
  for (u32 w = blockIdx.x * (blockDim.x / WAVE) + wave_id(); w < total; w += nwaves) {
    const u32 c = list[w];
    const u32 a = rep_of[c], b = match[a];
    const u32 m = (u32)(n_off[a + 1] - n_off[a] + n_off[b + 1] - n_off[b]);
    u32 nin, ntot;
    u32 *out = obuf + ooff[c];
    if (m <= 4 * WAVE) cinc_regs<K, 4>(n_off, n_nin, n_inc, a, b, m, out, nin, ntot);
    else if (m <= 8 * WAVE) cinc_regs<K, 8>(n_off, n_nin, n_inc, a, b, m, out, nin, ntot);
    else cinc_regs<K, 16>(n_off, n_nin, n_inc, a, b, m, out, nin, ntot);
    if (lane_id() == 0) {
      cnt_in[c] = nin;
      cnt_tot[c] = ntot;
    }
  }
}

template <int BLOCK, int CAP>
__global__ __launch_bounds__(BLOCK) void k_cinc_lds(const i64 *n_off, const u32 *n_nin,
                                                    const u32 *n_inc, const u32 *rep_of,
                                                    const u32 *match, const i64 *ooff, u32 *obuf,
                                                    u32 *cnt_in, u32 *cnt_tot, const u32 *list,
                                                    const u32 *cnt) {
  __shared__ u64 s[CAP];
  __shared__ u32 s_red[BLOCK / WAVE + 1];
  const u32 total = *cnt;
  for (u32 w = blockIdx.x; w < total; w += gridDim.x) {
    const u32 c = list[w];
    const u32 a = rep_of[c], b = match[a];
    const u32 m = (u32)(n_off[a + 1] - n_off[a] + n_off[b + 1] - n_off[b]);
    const u32 p = next_pow2(m);
    for (u32 i = threadIdx.x; i < p; i += BLOCK)
      s[i] = i < m ? inc_key(n_off, n_nin, n_inc, a, b, i) : ~0ull;
    __syncthreads();
    lds_bitonic<BLOCK>(s, p);
    u32 nin, ntot;
    group_split_emit<BLOCK, 0>(s, m, obuf + ooff[c], nin, ntot, s_red);
    if (threadIdx.x == 0) {
      cnt_in[c] = nin;
      cnt_tot[c] = ntot;
    }
    __syncthreads();
  }
}

template <int BLOCK, int CAP>
__global__ __launch_bounds__(BLOCK) void k_cinc_global(const i64 *n_off, const u32 *n_nin,
                                                       const u32 *n_inc, const u32 *rep_of,
                                                       const u32 *match, const i64 *ooff,
                                                       u32 *obuf, u32 *cnt_in, u32 *cnt_tot,
                                                       const u32 *list, const u32 *cnt,
                                                       u64 *scratch, u64 per_wg) {
  __shared__ u64 s[CAP];
  __shared__ u32 s_red[BLOCK / WAVE + 1];
  const u32 total = *cnt;
  u64 *A = scratch + (u64)blockIdx.x * per_wg;
  u64 *B = A + per_wg / 2;
  for (u32 w = blockIdx.x; w < total; w += gridDim.x) {
    const u32 c = list[w];
    const u32 a = rep_of[c], b = match[a];
    const u32 m = (u32)(n_off[a + 1] - n_off[a] + n_off[b + 1] - n_off[b]);
    for (u32 i = threadIdx.x; i < m; i += BLOCK) A[i] = inc_key(n_off, n_nin, n_inc, a, b, i);
    __syncthreads();
    const u64 *res = wg_sort_global<BLOCK, CAP>(A, B, m, s);
    u32 nin, ntot;
    group_split_emit<BLOCK, 0>(res, m, obuf + ooff[c], nin, ntot, s_red);
    if (threadIdx.x == 0) {
      cnt_in[c] = nin;
      cnt_tot[c] = ntot;
    }
    __syncthreads();
  }
}

// final coarse incidence: singletons copied from the fine graph, pairs from
// the oversize buffer
__global__ __launch_bounds__(256) void k_cinc_compact(u32 Nc, const u32 *rep_of, const u32 *match,
                                                      const i64 *n_off, const u32 *n_inc,
                                                      const i64 *ooff, const u32 *obuf,
                                                      const i64 *c_off, u32 *c_inc) {
  const u32 nwaves = gridDim.x * (blockDim.x / WAVE);
  const u32 l = lane_id();
  for (u32 c = blockIdx.x * (blockDim.x / WAVE) + wave_id(); c < Nc; c += nwaves) {
    const u32 a = rep_of[c];
    const u32 *src = match[a] == a ? n_inc + n_off[a] : obuf + ooff[c];
    const i64 d = c_off[c];
    const u32 k = (u32)(c_off[c + 1] - d);
    for (u32 i = l; i < k; i += WAVE) c_inc[d + i] = src[i];
  }
}

// ---------------------------------------------------------------------------
// coarse neighbourhoods
__global__ __launch_bounds__(256) void k_nbm_classify(u32 Nc, const u32 *rep_of,
                                                      const u32 *match, const i64 *nb_off,
                                                      u32 *bound, NbLists nl) {
  __shared__ u32 s_app[4 * (256 / WAVE) + 4];
  const u32 c = blockIdx.x * blockDim.x + threadIdx.x;
  u64 w = 0;
  if (c < Nc) {
    const u32 a = rep_of[c], b = match[a];
    w = (u64)(nb_off[a + 1] - nb_off[a]);
    if (b != a) w += (u64)(nb_off[b + 1] - nb_off[b]);
    if (w > 0xFFFFFFFFull) {
      atomicOr(nl.cnt + 7, 1u);
      w = 0;
    }
    bound[c] = (u32)w;
  }
  // classes: one wave in registers (<= 64); a one-wave merge with tables of
  // 256 (class 3: few registers, many waves per CU) or 1024 ids; the LDS
  // bitmap (larger)
  const int cls = (c >= Nc || w == 0) ? 4 : w <= 64 ? 0 : w <= 256 ? 3 : w <= 1024 ? 1 : 2;
  const u32 slot = block_append<256, 4>(nl.cnt, cls, s_app);
  if (cls < 4) nl.list[cls][slot] = c;
}

// bound <= 64: one wave, keys in registers.  With flags (fl, the invalid-
// neighbour flags of the fine lists) a key is gamma << 1 | flag: in a sorted
// run of one coarse id the flagged copies come last, so the id is kept iff
// the run's last key is unflagged.
__global__ __launch_bounds__(256) void k_nbm_wave(const i64 *nb_off, const u32 *nb,
                                                  const uint8_t *fl, const u32 *gamma,
                                                  const u32 *match, const u32 *rep_of,
                                                  const i64 *ooff, u32 *obuf, u32 *count,
                                                  const u32 *list, const u32 *cnt) {
  const u32 total = *cnt;
  const u32 nwaves = gridDim.x * (blockDim.x / WAVE);
  const u32 l = lane_id();
  for (u32 w = blockIdx.x * (blockDim.x / WAVE) + wave_id(); w < total; w += nwaves) {
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
    u32 v = NONE32;
    if (l < ka + kb) {
      const i64 j = l < ka ? a0 + l : b0 + (l - ka);
      v = gamma[nb[j]];
      if (fl) v = (v << 1) | (u32)fl[j];
    }
    v = wave_sort64(v);
    bool keep;
    u32 out;
    if (!fl) {
      const u32 prev = __shfl_up(v, 1, WAVE);
      keep = v != NONE32 && v != c && (l == 0 || prev != v);
      out = v;
    } else {
      const u32 next = __shfl_down(v, 1, WAVE);
      const bool last = l == WAVE - 1 || (next >> 1) != (v >> 1);
      keep = v != NONE32 && last && !(v & 1) && (v >> 1) != c;
      out = v >> 1;
    }
    const u64 mask = __ballot(keep);
    const u32 pos = (u32)__popcll(mask & ((1ull << l) - 1));
    if (keep) obuf[ooff[c] + pos] = out;
    if (l == 0) count[c] = (u32)__popcll(mask);
  }
}

// Split gamma(L) (L sorted, k ids) into the representatives' images, which
// stay sorted (appended to R at *r), and the second members' images
// (appended to Q at *q).  With flags (F, L's flags) the images are keys
// gamma << 1 | flag, in the same order.  Ids are taken U per thread at a
// time: all their loads and gathers are issued before the first scan, so a
// batch costs one chain of memory round trips, not U of them.
template <int BLOCK, int U>
__device__ void split_reps(const u32 *L, const uint8_t *F, u32 k, const u32 *gamma,
                           const u32 *match, u32 *R, u32 &r, u32 *Q, u32 &q, u32 *s_red) {
  for (u32 base = 0; base < k; base += BLOCK * U) {
    u32 m[U], g[U], pm[U], fv[U];
#pragma unroll
    for (u32 j = 0; j < U; ++j) {  // branch-free: past the end reads entry 0
      const u32 i = base + j * BLOCK + threadIdx.x;
      m[j] = L[i < k ? i : 0];
      fv[j] = F ? (u32)F[i < k ? i : 0] : 0u;
    }
#pragma unroll
    for (u32 j = 0; j < U; ++j) {
      g[j] = gamma[m[j]];
      pm[j] = match[m[j]];
    }
#pragma unroll
    for (u32 j = 0; j < U; ++j) {
      const u32 i = base + j * BLOCK + threadIdx.x;
      const bool valid = i < k;
      const u32 key = F ? (g[j] << 1) | fv[j] : g[j];
      const bool rep = pm[j] >= m[j];
      u32 tr, tq;
      const u32 orr = wg_excl_scan<BLOCK>((u32)(valid && rep), s_red, &tr);
      const u32 oq = wg_excl_scan<BLOCK>((u32)(valid && !rep), s_red, &tq);
      if (valid && rep) R[r + orr] = key;
      if (valid && !rep) Q[q + oq] = key;
      r += tr;
      q += tq;
    }
  }
}

// The distinct coarse ids of the sorted keys src[0, m) (gamma << 1 | flag)
// other than skip, an id kept iff the last key of its run is unflagged;
// written to out in order, the count returned (all threads).
template <int BLOCK>
__device__ u32 unique_unflagged(const u32 *src, u32 m, u32 skip, u32 *out, u32 *s_red) {
  u32 run = 0;
  for (u32 c0 = 0; c0 < m; c0 += BLOCK) {
    const u32 i = c0 + threadIdx.x;
    bool keep = false;
    u32 v = 0;
    if (i < m) {
      const u32 k = src[i];
      v = k >> 1;
      keep = k != NONE32 && !(k & 1) && v != skip && (i + 1 == m || (src[i + 1] >> 1) != v);
    }
    u32 tot;
    const u32 off = wg_excl_scan<BLOCK>((u32)keep, s_red, &tot);
    if (keep) out[run + off] = v;
    run += tot;
  }
  return run;
}

// N'(c) by split, sort of the second members' images, and two merges.  X, Y
// hold CAP ids each; Z holds the second members' images (sorted in place).
// With flags the same on keys gamma << 1 | flag (see k_nbm_wave).
template <int BLOCK, int CAP>
__global__ __launch_bounds__(BLOCK) void k_nbm_merge(const i64 *nb_off, const u32 *nb,
                                                     const uint8_t *fl, const u32 *gamma,
                                                     const u32 *match, const u32 *rep_of,
                                                     const i64 *ooff, u32 *obuf, u32 *count,
                                                     const u32 *list, const u32 *cnt) {
  __shared__ u32 X[CAP], Y[CAP], Z[CAP];
  __shared__ u32 s_red[BLOCK / WAVE + 1];
  const u32 total = *cnt;
  for (u32 w = blockIdx.x; w < total; w += gridDim.x) {
    const u32 c = list[w];
    const u32 a = rep_of[c], b = match[a];
    u32 r1 = 0, r2 = 0, q = 0;
    const i64 a0 = nb_off[a];
    split_reps<BLOCK, CAP / BLOCK>(nb + a0, fl ? fl + a0 : nullptr, (u32)(nb_off[a + 1] - a0),
                                   gamma, match, X, r1, Z, q, s_red);
    if (b != a) {
      const i64 b0 = nb_off[b];
      split_reps<BLOCK, CAP / BLOCK>(nb + b0, fl ? fl + b0 : nullptr, (u32)(nb_off[b + 1] - b0),
                                     gamma, match, X + r1, r2, Z, q, s_red);
    }
    if (q > 1) {
      const u32 p = next_pow2(q);
      for (u32 i = q + threadIdx.x; i < p; i += BLOCK) Z[i] = NONE32;
      __syncthreads();
      lds_bitonic<BLOCK>(Z, p);
    }
    __syncthreads();
    const u32 *R = X;
    if (r2) {
      wg_merge<BLOCK>(X, r1, X + r1, r2, Y);
      __syncthreads();
      R = Y;
    }
    u32 *F = R == X ? Y : X;
    wg_merge<BLOCK>(R, r1 + r2, Z, q, F);
    __syncthreads();
    const u32 k = fl ? unique_unflagged<BLOCK>(F, r1 + r2 + q, c, obuf + ooff[c], s_red)
                     : unique_out<BLOCK>(F, r1 + r2 + q, c, obuf + ooff[c], s_red);
    if (threadIdx.x == 0) count[c] = k;
    __syncthreads();
  }
}

}  // namespace

void launch_cinc_classify(chp_ctx *c, u32 Nc, const u32 *rep_of, const u32 *match,
                          const i64 *n_off, const u32 *n_nin, u32 *bound, u32 *cnt_in,
                          u32 *cnt_tot, EdgeLists el) {
  if (Nc == 0) return;
  CHP_LAUNCH(c, "cinc_classify", k_cinc_classify, grid_for(Nc, 256), 256, 0, Nc, rep_of, match,
             n_off, n_nin, bound, cnt_in, cnt_tot, el);
}

void launch_cinc_build(chp_ctx *c, const i64 *n_off, const u32 *n_nin, const u32 *n_inc,
                       const u32 *rep_of, const u32 *match, const i64 *ooff, u32 *obuf,
                       u32 *cnt_in, u32 *cnt_tot, EdgeLists el, const u32 *host_cnt,
                       u64 *scratch, u64 per_wg, u32 grid_big, bool narrow) {
  if (host_cnt[0])
    CHP_LAUNCH(c, "cinc_wave", k_cinc_wave, waves_grid(host_cnt[0]), 256, 0, n_off, n_nin, n_inc,
               rep_of, match, ooff, obuf, cnt_in, cnt_tot, (const u32 *)el.list[0],
               (const u32 *)el.cnt + 0);
  if (host_cnt[1]) {
    const u32 gw = (host_cnt[1] + 3) / 4, gc = gw < 32 * c->n_cu ? gw : 32 * c->n_cu;
    if (narrow)
      CHP_LAUNCH(c, "cinc_wreg", k_cinc_wreg<u32>, gc, 256, 0, n_off, n_nin, n_inc, rep_of, match,
                 ooff, obuf, cnt_in, cnt_tot, (const u32 *)el.list[1], (const u32 *)el.cnt + 1);
    else
      CHP_LAUNCH(c, "cinc_wreg", k_cinc_wreg<u64>, gc, 256, 0, n_off, n_nin, n_inc, rep_of, match,
                 ooff, obuf, cnt_in, cnt_tot, (const u32 *)el.list[1], (const u32 *)el.cnt + 1);
  }
  if (host_cnt[3])
    CHP_LAUNCH(c, "cinc_lds", (k_cinc_lds<256, LDS_CAP_U64>),
               host_cnt[3] > 8192 ? 8192 : host_cnt[3], 256, 0, n_off, n_nin, n_inc, rep_of,
               match, ooff, obuf, cnt_in, cnt_tot, (const u32 *)el.list[3],
               (const u32 *)el.cnt + 3);
  if (host_cnt[2])
    CHP_LAUNCH(c, "cinc_global", (k_cinc_global<256, LDS_CAP_U64>), grid_big, 256, 0, n_off,
               n_nin, n_inc, rep_of, match, ooff, obuf, cnt_in, cnt_tot,
               (const u32 *)el.list[2], (const u32 *)el.cnt + 2, scratch, per_wg);
}

void launch_cinc_compact(chp_ctx *c, u32 Nc, const u32 *rep_of, const u32 *match,
                         const i64 *n_off, const u32 *n_inc, const i64 *ooff, const u32 *obuf,
                         const i64 *c_off, u32 *c_inc) {
  if (Nc == 0) return;
  CHP_LAUNCH(c, "cinc_compact", k_cinc_compact, waves_grid(Nc), 256, 0, Nc, rep_of, match, n_off,
             n_inc, ooff, obuf, c_off, c_inc);
}

void launch_nbm_classify(chp_ctx *c, u32 Nc, const u32 *rep_of, const u32 *match,
                         const i64 *nb_off, u32 *bound, NbLists nl) {
  if (Nc == 0) return;
  CHP_LAUNCH(c, "nbm_classify", k_nbm_classify, grid_for(Nc, 256), 256, 0, Nc, rep_of, match,
             nb_off, bound, nl);
}

void launch_nbm_build(chp_ctx *c, const i64 *nb_off, const u32 *nb, const uint8_t *fl,
                      const u32 *gamma, const u32 *match, const u32 *rep_of, const i64 *ooff,
                      u32 *obuf, u32 *count, NbLists nl, const u32 *host_cnt) {
  if (host_cnt[0])
    CHP_LAUNCH(c, "nbm_wave", k_nbm_wave, waves_grid(host_cnt[0]), 256, 0, nb_off, nb, fl, gamma,
               match, rep_of, ooff, obuf, count, (const u32 *)nl.list[0],
               (const u32 *)nl.cnt + 0);
  if (host_cnt[3])
    CHP_LAUNCH(c, "nbm_merge", (k_nbm_merge<64, 256>),
               host_cnt[3] > 65536 ? 65536 : host_cnt[3], 64, 0, nb_off, nb, fl, gamma, match,
               rep_of, ooff, obuf, count, (const u32 *)nl.list[3], (const u32 *)nl.cnt + 3);
  if (host_cnt[1])
    CHP_LAUNCH(c, "nbm_merge", (k_nbm_merge<64, 1024>),
               host_cnt[1] > 65536 ? 65536 : host_cnt[1], 64, 0, nb_off, nb, fl, gamma, match,
               rep_of, ooff, obuf, count, (const u32 *)nl.list[1], (const u32 *)nl.cnt + 1);
  launch_nbm_bitmap(c, nb_off, nb, fl, gamma, match, rep_of, ooff, obuf, count, nl.list[2],
                    nl.cnt + 2, host_cnt[2]);
}
