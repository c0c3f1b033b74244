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

// cap = floor(sum t / (10 |E|)), d = cap + 1, magic = floor((2^64-1)/d)
__global__ void k_cap(u32 nparts, const u64 *partials, u32 E, u64 *capinfo) {
  if (threadIdx.x != 0) return;
  u64 lo = 0, hi = 0;
  for (u32 i = 0; i < nparts; ++i) {
    u64 r = lo + partials[2 * i];
    hi += partials[2 * i + 1] + (r < lo ? 1 : 0);
    lo = r;
  }
  u64 cap = 0;
  if (E) {
    const u64 dv = 10ull * E;
    u64 rem = 0, q = 0;
    for (int bit = 127; bit >= 0; --bit) {
      u64 b = bit >= 64 ? (hi >> (bit - 64)) & 1 : (lo >> bit) & 1;
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
  u32 n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= N) return;
  u64 K = (u64)(nb_off[n + 1] - nb_off[n]);
  if (K == 0) {
    target[n] = NONE32;
    score[n] = 0;
    return;
  }
  int c = K <= small_cap ? 0 : 1;
  u32 slot = atomicAdd(&nl.cnt[c], 1u);
  nl.list[c][slot] = n;
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

// One workgroup per node.  N(n) is taken in slices of at most CAP ids
// (sorted, so each slice covers an id interval); the slice's eta and inter
// accumulators live in LDS.  Incident hyperedges are taken ECH at a time:
// each contributes a source run and a destination run (clipped to the
// slice's id interval when N(n) needs several slices), and the pins of all
// runs are spread evenly over the workgroup.  Each pin m finds its bin by a
// binary search of the slice and adds t(e) to eta(n,m); a destination pin of
// an inbound hyperedge also increments inter(n,m).
template <int BLOCK, int CAP, int ECH>
__global__ __launch_bounds__(BLOCK) void k_rate(RateArgs A, const u32 *list, const u32 *cnt) {
  __shared__ u32 s_id[CAP];
  __shared__ u64 s_eta[CAP];
  __shared__ u32 s_int[CAP];
  __shared__ u64 s_rs[2 * ECH];
  __shared__ u64 s_rt[2 * ECH];
  __shared__ u32 s_pre[2 * ECH + 1];
  __shared__ u32 s_red32[BLOCK / WAVE + 1];
  __shared__ u64 s_red64[BLOCK / WAVE + 1];
  __shared__ u32 s_redi[BLOCK / WAVE + 1];
  static_assert(ECH <= BLOCK, "one thread per hyperedge of a chunk");
  constexpr u64 INB = 1ull << 63;
  const u32 total = *cnt;
  const u32 tid = threadIdx.x;
  const u64 cap = A.capinfo[0], dmod = A.capinfo[1], magic = A.capinfo[2];
  const u64 ub_add = A.noise_on ? cap : 0;
  for (u32 w = blockIdx.x; w < total; w += gridDim.x) {
    const u32 n = list[w];
    const i64 nb0 = A.nb_off[n];
    const u32 K = (u32)(A.nb_off[n + 1] - nb0);
    const i64 i0 = A.n_off[n], i1 = A.n_off[n + 1];
    const u32 nin = A.n_nin[n];
    const u64 size_n = A.n_size[n];
    u64 best_e = 0;
    u32 best_i = NONE32;
    u64 tsum = 0;
    for (u32 s0 = 0; s0 < K; s0 += CAP) {
      const u32 cw = (K - s0) < (u32)CAP ? (K - s0) : (u32)CAP;
      for (u32 i = tid; i < cw; i += BLOCK) {
        s_id[i] = A.nb[nb0 + s0 + i];
        s_eta[i] = 0;
        s_int[i] = 0;
      }
      __syncthreads();
      const u32 lo_id = s_id[0], hi_id = s_id[cw - 1];
      const bool clip = K > (u32)CAP;
      for (i64 c0 = i0; c0 < i1; c0 += ECH) {
        const u32 ne = (u32)((i1 - c0) < ECH ? (i1 - c0) : ECH);
        u32 ls = 0, ld = 0;
        if (tid < ne) {
          const u32 e = A.n_inc[c0 + tid];
          const bool isin = (u64)(c0 + tid - i0) < (u64)nin;
          const i64 a = A.e_off[e], b = A.e_off[e + 1];
          const i64 dm = a + A.e_nsrc[e];
          const u64 te = A.t[e];
          if (s0 == 0 && b - a >= 2) tsum = sat_add(tsum, te);
          i64 sa = a, sb = dm, da = dm, db = b;
          if (clip) {
            sa = lower_bound_i(A.e_pins, a, dm, lo_id);
            sb = upper_bound_i(A.e_pins, sa, dm, hi_id);
            da = lower_bound_i(A.e_pins, dm, b, lo_id);
            db = upper_bound_i(A.e_pins, da, b, hi_id);
          }
          s_rs[2 * tid] = (u64)sa;
          s_rs[2 * tid + 1] = (u64)da | (isin ? INB : 0);
          s_rt[2 * tid] = te;
          s_rt[2 * tid + 1] = te;
          ls = (u32)(sb - sa);
          ld = (u32)(db - da);
        }
        u32 tot;
        const u32 off = wg_excl_scan<BLOCK>(ls + ld, s_red32, &tot);
        if (tid < ne) {
          s_pre[2 * tid] = off;
          s_pre[2 * tid + 1] = off + ls;
        }
        if (tid == 0) s_pre[2 * ne] = tot;
        __syncthreads();
        for (u32 idx = tid; idx < tot; idx += BLOCK) {
          const u32 r = run_of(s_pre, 2 * ne + 1, idx);
          const u64 rs = s_rs[r];
          const u32 m = A.e_pins[(i64)(rs & ~INB) + (idx - s_pre[r])];
          if (m == n) continue;
          const u32 pos = (u32)lower_bound_i(s_id, 0, cw, m);
          if (pos >= cw || s_id[pos] != m) continue;  // cannot happen for a valid N(n)
          atomicAdd(&s_eta[pos], s_rt[r]);
          if (rs & INB) atomicAdd(&s_int[pos], 1u);
        }
        __syncthreads();
      }
      // candidates of this slice: keep the best valid (eta, -id); a bin whose
      // upper bound eta + cap cannot beat the current best is skipped before
      // its noise and limits are evaluated
      for (u32 i = tid; i < cw; i += BLOCK) {
        const u32 m = s_id[i];
        const u64 v = s_eta[i];
        if (!better(v + ub_add, m, best_e, best_i)) continue;
        const u64 tv = A.noise_on ? v + pair_noise(A.seed, n, m, dmod, magic) : v;
        if (!better(tv, m, best_e, best_i)) continue;
        if (size_n + A.n_size[m] > A.omega) continue;
        if ((u64)nin + A.n_nin[m] - s_int[i] > (u64)A.delta) continue;
        best_e = tv;
        best_i = m;
      }
      __syncthreads();
    }
    tsum = wg_sat_sum<BLOCK>(tsum, s_red64);
    wg_best<BLOCK>(best_e, best_i, s_red64, s_redi);
    if (tid == 0) {
      if (sat_add(tsum, cap) >= (1ull << 63)) atomicOr(A.flags, FLAG_EOVERFLOW);
      A.target[n] = best_i;
      A.score[n] = best_i == NONE32 ? 0 : best_e;
    }
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
  CHP_LAUNCH(c, "cap", k_cap, 1, 64, 0, E ? nparts : 0u, (const u64 *)partials, E, capinfo);
}

void launch_rate_classify(chp_ctx *c, u32 N, const i64 *nb_off, NbLists nl, u32 *target,
                          u64 *score) {
  if (N == 0) return;
  CHP_LAUNCH(c, "rate_classify", k_rate_classify, grid_for(N, 256), 256, 0, N, nb_off, nl, target,
             score, RATE_SMALL_CAP);
}

void launch_rate(chp_ctx *c, const RateArgs &a, NbLists nl, const u32 *host_cnt) {
  if (host_cnt[0])
    CHP_LAUNCH(c, "rate_small", (k_rate<64, RATE_SMALL_CAP, 32>),
               host_cnt[0] > 65536 ? 65536 : host_cnt[0], 64, 0, a, (const u32 *)nl.list[0],
               (const u32 *)nl.cnt + 0);
  if (host_cnt[1])
    CHP_LAUNCH(c, "rate_large", (k_rate<256, 2048, 128>),
               host_cnt[1] > 16384 ? 16384 : host_cnt[1], 256, 0, a, (const u32 *)nl.list[1],
               (const u32 *)nl.cnt + 1);
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
