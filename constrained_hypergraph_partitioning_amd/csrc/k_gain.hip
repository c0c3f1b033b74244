// Refinement move proposal ("Hypergraph Partitioning on GPU with Distinct
// Incident Hyperedges and Size Constraints", Sec. VI-A/B, Eq. 13):
//   pins(p, e) = pins of e in partition p,
//   saving(n)  = w of n's hyperedges where n is its partition's only pin,
//   loss(n, p) = w of n's hyperedges with no pin in p,
//   move(n)    = argmax over p != rho(n) of saving(n) - loss(n, p), ties to
//                the smallest p; with Omega enforced only partitions with
//                part_size(p) + size(n) <= Omega.
// pins(., e) is held per hyperedge as its sorted distinct partitions with
// their counts, packed (p << 32 | count), in the hyperedge's own pin range
// (e_off[e] .. e_off[e] + lambda(e)): sparse, where the pages keep a dense
// |P| x |E| matrix.  A partition p touched by n's hyperedges has
// loss(n, p) = W(n) - conn(n, p), with W the total weight of I(n) and conn the
// weight of those with a pin in p; every untouched one loses W(n).  So the
// best move is the touched admissible p of largest conn, else the smallest
// admissible untouched p.  A light node (at most 384 list entries over its
// hyperedges) takes a wave and an LDS hash over the partitions it touches;
// a heavy one a workgroup and a larger hash (up to 3072 list entries), or,
// beyond that, direct-mapped windows of 4096 partition ids.
#include "dev.h"
#include "kernels.h"

namespace {

__device__ __forceinline__ u32 part_of(const u32 *rho, u32 k, u32 pin, u32 *flags) {
  const u32 p = rho[pin];
  if (p >= k) {
    atomicOr(flags, FLAG_EINVAL);
    return 0;
  }
  return p;
}

// ---- pins(., e) lists --------------------------------------------------------
__global__ __launch_bounds__(256) void k_pins_wave(const i64 *e_off, const u32 *pins,
                                                   const u32 *rho, u32 k, u64 *pl, u32 *lam,
                                                   const u32 *list, const u32 *cnt, u32 *flags) {
  const u32 total = *cnt;
  const u32 nwaves = gridDim.x * (blockDim.x / WAVE);
  const u32 l = lane_id();
  for (u32 w = blockIdx.x * (blockDim.x / WAVE) + wave_id(); w < total; w += nwaves) {
    const u32 e = list[w];
    const i64 a = e_off[e];
    const u32 len = (u32)(e_off[e + 1] - a);
    u64 key = ~0ull;
    if (l < len) key = part_of(rho, k, pins[a + l], flags);
    key = wave_sort64(key);
    const u64 prev = __shfl_up(key, 1, WAVE);
    const bool head = l < len && (l == 0 || prev != key);
    const u64 hm = __ballot(head);
    if (head) {
      const u64 above = l + 1 < WAVE ? hm >> (l + 1) : 0;
      const u32 next = above ? l + 1 + (u32)__builtin_ctzll(above) : len;
      const u32 r = (u32)__popcll(hm & ((1ull << l) - 1));
      pl[a + r] = (key << 32) | (next - l);
    }
    if (l == 0) lam[e] = (u32)__popcll(hm);
  }
}

// groups of the sorted keys s[0, m) into out[0, lambda); returns lambda
template <int BLOCK>
__device__ u32 pins_groups(const u64 *s, u32 m, u64 *out, u32 *s_red) {
  u32 base = 0;
  for (u32 c0 = 0; c0 < m; c0 += BLOCK) {  // head positions, by rank
    const u32 i = c0 + threadIdx.x;
    const bool head = i < m && (i == 0 || s[i - 1] != s[i]);
    u32 tot;
    const u32 r = wg_excl_scan<BLOCK>(head ? 1u : 0u, s_red, &tot);
    if (head) out[base + r] = i;
    base += tot;
  }
  __syncthreads();
  for (u32 r0 = 0; r0 < base; r0 += BLOCK) {  // counts from the next head
    const u32 r = r0 + threadIdx.x;
    u64 v = 0;
    if (r < base) {
      const u32 h = (u32)out[r];
      const u32 nx = r + 1 < base ? (u32)out[r + 1] : m;
      v = (s[h] << 32) | (nx - h);
    }
    __syncthreads();
    if (r < base) out[r] = v;
    __syncthreads();
  }
  return base;
}

template <int BLOCK, int CAP>
__global__ __launch_bounds__(BLOCK) void k_pins_lds(const i64 *e_off, const u32 *pins,
                                                    const u32 *rho, u32 k, u64 *pl, u32 *lam,
                                                    const u32 *list, const u32 *cnt,
                                                    u32 *flags) {
  __shared__ u64 s[CAP];
  __shared__ u32 s_red[BLOCK / WAVE + 1];
  const u32 total = *cnt;
  for (u32 w = blockIdx.x; w < total; w += gridDim.x) {
    const u32 e = list[w];
    const i64 a = e_off[e];
    const u32 len = (u32)(e_off[e + 1] - a);
    const u32 p = next_pow2(len);
    for (u32 i = threadIdx.x; i < p; i += BLOCK)
      s[i] = i < len ? (u64)part_of(rho, k, pins[a + i], flags) : ~0ull;
    __syncthreads();
    lds_bitonic<BLOCK>(s, p);
    const u32 lm = pins_groups<BLOCK>(s, len, pl + a, s_red);
    if (threadIdx.x == 0) lam[e] = lm;
    __syncthreads();
  }
}

template <int BLOCK, int CAP>
__global__ __launch_bounds__(BLOCK) void k_pins_global(const i64 *e_off, const u32 *pins,
                                                       const u32 *rho, u32 k, u64 *pl, u32 *lam,
                                                       const u32 *list, const u32 *cnt,
                                                       u32 *flags, u64 *scratch, u64 per_wg) {
  __shared__ u64 s[CAP];
  __shared__ u32 s_red[BLOCK / WAVE + 1];
  const u32 total = *cnt;
  u64 *A = scratch + (u64)blockIdx.x * per_wg;
  u64 *B = A + per_wg / 2;
  for (u32 w = blockIdx.x; w < total; w += gridDim.x) {
    const u32 e = list[w];
    const i64 a = e_off[e];
    const u32 len = (u32)(e_off[e + 1] - a);
    for (u32 i = threadIdx.x; i < len; i += BLOCK) A[i] = part_of(rho, k, pins[a + i], flags);
    __syncthreads();
    const u64 *res = wg_sort_global<BLOCK, CAP>(A, B, len, s);
    const u32 lm = pins_groups<BLOCK>(res, len, pl + a, s_red);
    if (threadIdx.x == 0) lam[e] = lm;
    __syncthreads();
  }
}

// ---- admissible partitions: a max-tree over the free capacity -----------------
// leaves K2 .. 2 K2 - 1 hold Omega - part_size(p) (0 when full or p >= k)
__global__ void k_free_leaves(u32 k, u32 K2, const u64 *part_size, u64 omega, u64 *tree) {
  const u32 p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= K2) return;
  u64 f = 0;
  if (p < k) f = part_size[p] < omega ? omega - part_size[p] : 0;
  tree[K2 + p] = f;
}

__global__ void k_free_level(u32 lo, u32 cnt, u64 *tree) {
  const u32 i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= cnt) return;
  const u32 v = lo + i;
  const u64 a = tree[2 * v], b = tree[2 * v + 1];
  tree[v] = a > b ? a : b;
}

// first p >= x with free(p) >= s, or NONE
__device__ u32 first_free(const u64 *tree, u32 K2, u32 x, u64 s) {
  if (x >= K2) return NONE32;
  u32 i = K2 + x;
  if (tree[i] >= s) return x;
  for (;;) {
    if (!(i & 1) && tree[i + 1] >= s) {
      ++i;
      break;
    }
    i >>= 1;
    if (i <= 1) return NONE32;
  }
  while (i < K2) {
    i <<= 1;
    if (tree[i] < s) ++i;
  }
  return i - K2;
}

// ---- per-node proposal ------------------------------------------------------------
struct GainArgs {
  u32 N, k, K2, enforce;
  u64 omega;
  const i64 *e_off;
  const u32 *e_w;
  const u64 *pl;
  const u32 *lam;
  const i64 *n_off;
  const u32 *n_inc;
  const u32 *n_size;
  const u32 *rho;
  const u64 *part_size;
  const u64 *tree;
  u32 *move;
  i64 *gain;
};

__device__ __forceinline__ bool admissible(const GainArgs &G, u32 p, u64 size_n) {
  return !G.enforce || G.part_size[p] + size_n <= G.omega;
}

// pins(p, e) by binary search in e's list
__device__ u32 pins_in(const GainArgs &G, u32 e, u32 p) {
  const i64 a = G.e_off[e];
  u32 lo = 0, hi = G.lam[e];
  while (lo < hi) {
    const u32 mid = (lo + hi) >> 1;
    if ((u32)(G.pl[a + mid] >> 32) < p) lo = mid + 1;
    else hi = mid;
  }
  return lo < G.lam[e] && (u32)(G.pl[a + lo] >> 32) == p ? (u32)G.pl[a + lo] : 0;
}

// classes: light (sum of lambda over I(n) <= GL_CAP) or heavy
constexpr u32 GL_T = 512, GL_CAP = 384;
constexpr int GW_ECH = 64;  // hyperedges per chunk, light path

__global__ void k_gain_classify(GainArgs G, u32 *lists, u32 *cnt) {
  const u32 n = blockIdx.x * blockDim.x + threadIdx.x;
  int c = 2;
  if (n < G.N) {
    u64 t = 0;
    for (i64 j = G.n_off[n]; j < G.n_off[n + 1]; ++j) t += G.lam[G.n_inc[j]];
    c = t <= GL_CAP ? 0 : 1;
  }
  const u32 s0 = wave_append(cnt + 0, c == 0);
  if (c == 0) lists[s0] = n;
  const u32 s1 = wave_append(cnt + 1, c == 1);
  if (c == 1) lists[G.N - 1 - s1] = n;  // heavy nodes from the back
}

struct GainWave {
  u32 key[GL_T];  // p + 1, 0 = empty
  u64 conn[GL_T];
  u32 rb[GW_ECH];    // each hyperedge's first list entry (within e_off)
  u32 rw[GW_ECH];
  u32 pre[GW_ECH + 1];
  u64 ra[GW_ECH];
};

__device__ __forceinline__ u32 gw_slot(u32 p) { return (p * 0x9E3779B1u) >> 23; }

__device__ __forceinline__ void gw_add(GainWave &S, u32 p, u64 w) {
  u32 s = gw_slot(p);
  for (;;) {
    const u32 cur = S.key[s];
    if (cur == p + 1) break;
    if (cur == 0) {
      const u32 old = atomicCAS(&S.key[s], 0u, p + 1);
      if (old == 0 || old == p + 1) break;
    }
    s = (s + 1) & (GL_T - 1);
  }
  atomicAdd((unsigned long long *)&S.conn[s], (unsigned long long)w);
}

__device__ __forceinline__ bool gw_has(const GainWave &S, u32 p) {
  u32 s = gw_slot(p);
  for (;;) {
    const u32 cur = S.key[s];
    if (cur == p + 1) return true;
    if (cur == 0) return false;
    s = (s + 1) & (GL_T - 1);
  }
}

__device__ void gain_light(const GainArgs &G, GainWave &S, u32 n) {
  const u32 l = lane_id();
  const u32 pn = G.rho[n];
  const u64 size_n = G.n_size[n];
  const i64 i0 = G.n_off[n], i1 = G.n_off[n + 1];
  u64 W = 0, saving = 0;
  for (i64 c0 = i0; c0 < i1; c0 += GW_ECH) {
    const u32 ne = (u32)((i1 - c0) < GW_ECH ? (i1 - c0) : GW_ECH);
    u32 len = 0;
    if (l < ne) {
      const u32 e = G.n_inc[c0 + l];
      len = G.lam[e];
      S.ra[l] = (u64)G.e_off[e];
      S.rw[l] = G.e_w[e];
      W += G.e_w[e];
    }
    const u32 inc = wave_incl_scan(len);
    const u32 tot = __shfl(inc, WAVE - 1, WAVE);
    if (l < ne) S.pre[l] = inc - len;
    if (l == 0) S.pre[ne] = tot;
    wave_sync();
    for (u32 t = l; t < tot; t += WAVE) {
      const u32 r = run_of(S.pre, ne, t);
      const u64 x = G.pl[S.ra[r] + (t - S.pre[r])];
      const u32 p = (u32)(x >> 32), c = (u32)x;
      if (p == pn) {
        if (c == 1) saving += S.rw[r];
      } else {
        gw_add(S, p, S.rw[r]);
      }
    }
    wave_sync();
  }
  W = wave_sum(W);
  saving = wave_sum(saving);
  // best touched admissible partition by (conn desc, id asc)
  u64 be = 0;
  u32 bp = NONE32;
  for (u32 s = l; s < GL_T; s += WAVE) {
    const u32 key = S.key[s];
    if (key && admissible(G, key - 1, size_n) && better(S.conn[s], key - 1, be, bp)) {
      be = S.conn[s];
      bp = key - 1;
    }
  }
#pragma unroll
  for (int d = WAVE / 2; d > 0; d >>= 1) {
    const u64 oe = __shfl_xor(be, d, WAVE);
    const u32 oi = __shfl_xor(bp, d, WAVE);
    if (better(oe, oi, be, bp)) be = oe, bp = oi;
  }
  u32 mv = bp;
  i64 gn = bp != NONE32 ? (i64)saving - (i64)W + (i64)be : 0;
  if (bp == NONE32) {
    // the smallest admissible partition that no hyperedge of n touches
    u32 x = 0;
    for (;;) {
      if (G.enforce) x = first_free(G.tree, G.K2, x, size_n);
      if (x == NONE32 || x >= G.k) break;
      const u32 p = x + l;
      const bool ok = p < G.k && p != pn && admissible(G, p, size_n) && !gw_has(S, p);
      const u64 b = __ballot(ok);
      if (b) {
        mv = x + (u32)__builtin_ctzll(b);
        gn = (i64)saving - (i64)W;
        break;
      }
      if (x > 0xFFFFFFFFu - WAVE) break;
      x += WAVE;
    }
  }
  // empty the table for the next node
  for (u32 s = l; s < GL_T; s += WAVE) {
    S.key[s] = 0;
    S.conn[s] = 0;
  }
  if (l == 0) {
    G.move[n] = mv;
    G.gain[n] = mv == NONE32 ? 0 : gn;
  }
  wave_sync();
}

constexpr int GB = 256;
constexpr u32 GD = 4096;    // partition ids per direct window, largest nodes
constexpr u32 GM_T = 4096;  // hash slots, heavy nodes
constexpr u32 GM_CAP = 3072;  // list entries a heavy node may bring to the hash

__device__ __forceinline__ u32 gm_slot(u32 p) { return (p * 0x9E3779B1u) >> 20; }

struct GainWg {
  u64 conn[GM_T];  // the hash's counters, or a direct window over GD ids
  u32 key[GM_T];   // p + 1, 0 = empty (hash only)
  u64 red64[GB / WAVE];
  u64 rede[GB / WAVE];
  u32 redi[GB / WAVE];
  u32 ans, item;
};
constexpr u32 GH_PER_CU = 3;  // workgroups of k_gain_heavy that fit a CU's LDS
static_assert(GH_PER_CU * sizeof(GainWg) <= 160 * 1024, "LDS");
static_assert(GD <= GM_T, "direct window in the hash's counters");

__device__ __forceinline__ void gm_add(GainWg &S, u32 p, u64 w) {
  u32 s = gm_slot(p);
  for (;;) {
    const u32 cur = S.key[s];
    if (cur == p + 1) break;
    if (cur == 0) {
      const u32 old = atomicCAS(&S.key[s], 0u, p + 1);
      if (old == 0 || old == p + 1) break;
    }
    s = (s + 1) & (GM_T - 1);
  }
  atomicAdd((unsigned long long *)&S.conn[s], (unsigned long long)w);
}

__device__ __forceinline__ bool gm_has(const GainWg &S, u32 p) {
  u32 s = gm_slot(p);
  for (;;) {
    const u32 cur = S.key[s];
    if (cur == p + 1) return true;
    if (cur == 0) return false;
    s = (s + 1) & (GM_T - 1);
  }
}

__device__ __forceinline__ void wg_best_reduce(GainWg &S, u64 &be, u32 &bp) {
#pragma unroll
  for (int d = WAVE / 2; d > 0; d >>= 1) {
    const u64 oe = __shfl_xor(be, d, WAVE);
    const u32 oi = __shfl_xor(bp, d, WAVE);
    if (better(oe, oi, be, bp)) be = oe, bp = oi;
  }
  if (lane_id() == 0) {
    S.rede[wave_id()] = be;
    S.redi[wave_id()] = bp;
  }
  __syncthreads();
  be = S.rede[0];
  bp = S.redi[0];
  for (int v = 1; v < GB / WAVE; ++v)
    if (better(S.rede[v], S.redi[v], be, bp)) be = S.rede[v], bp = S.redi[v];
  __syncthreads();
}

__global__ __launch_bounds__(GB) void k_gain_light(GainArgs G, const u32 *lists,
                                                    const u32 *cnt) {
  __shared__ GainWave sm[GB / WAVE];
  GainWave &S = sm[wave_id()];
  for (u32 s = lane_id(); s < GL_T; s += WAVE) {
    S.key[s] = 0;
    S.conn[s] = 0;
  }
  wave_sync();
  const u32 total = cnt[0];
  const u32 nw = gridDim.x * (GB / WAVE);
  for (u32 w = blockIdx.x * (GB / WAVE) + wave_id(); w < total; w += nw)
    gain_light(G, S, lists[w]);
}

// A workgroup per node: list entries into the LDS hash when they number at
// most GM_CAP (then the untouched fallback as on the light path, by wave 0),
// otherwise direct windows of GD partition ids over [0, k), each scanned in
// full (touched or not).
// Nodes are taken from a counter (their costs vary widely); the item is a
// scalar and the loop body ends with a barrier.
__global__ __launch_bounds__(GB) void k_gain_heavy(GainArgs G, const u32 *lists,
                                                    const u32 *cnt, u32 *work) {
  __shared__ GainWg S;
  const u32 tid = threadIdx.x;
  const u32 total = cnt[1];
  for (u32 s = tid; s < GM_T; s += GB) {
    S.key[s] = 0;
    S.conn[s] = 0;
  }
  for (;;) {
    if (tid == 0) S.item = atomicAdd(work, 1u);
    __syncthreads();
    const u32 w = __builtin_amdgcn_readfirstlane(S.item);
    if (w >= total) break;
    const u32 n = lists[G.N - 1 - w];
    const u32 pn = G.rho[n];
    const u64 size_n = G.n_size[n];
    const i64 i0 = G.n_off[n], i1 = G.n_off[n + 1];
    u64 W = 0, saving = 0, ent = 0;
    for (i64 j = i0 + tid; j < i1; j += GB) {
      const u32 e = G.n_inc[j];
      W += G.e_w[e];
      ent += G.lam[e];
      if (pins_in(G, e, pn) == 1) saving += G.e_w[e];
    }
    W = wg_sum<GB>(W, S.red64);
    saving = wg_sum<GB>(saving, S.red64);
    ent = wg_sum<GB>(ent, S.red64);
    u64 be = 0;
    u32 bp = NONE32;
    if (ent <= GM_CAP) {
      for (i64 j = i0 + wave_id(); j < i1; j += GB / WAVE) {
        const u32 e = G.n_inc[j];
        const i64 a = G.e_off[e];
        const u32 lm = G.lam[e];
        const u64 we = G.e_w[e];
        for (u32 t = lane_id(); t < lm; t += WAVE) {
          const u32 p = (u32)(G.pl[a + t] >> 32);
          if (p != pn) gm_add(S, p, we);
        }
      }
      __syncthreads();
      for (u32 s = tid; s < GM_T; s += GB) {
        const u32 key = S.key[s];
        if (key && admissible(G, key - 1, size_n) && better(S.conn[s], key - 1, be, bp)) {
          be = S.conn[s];
          bp = key - 1;
        }
      }
      wg_best_reduce(S, be, bp);
      if (bp == NONE32 && wave_id() == 0) {
        // the smallest admissible partition no hyperedge of n touches
        const u32 l = lane_id();
        u32 found = NONE32, x = 0;
        for (;;) {
          if (G.enforce) x = first_free(G.tree, G.K2, x, size_n);
          if (x == NONE32 || x >= G.k) break;
          const u32 p = x + l;
          const bool ok = p < G.k && p != pn && admissible(G, p, size_n) && !gm_has(S, p);
          const u64 b = __ballot(ok);
          if (b) {
            found = x + (u32)__builtin_ctzll(b);
            break;
          }
          if (x > 0xFFFFFFFFu - WAVE) break;
          x += WAVE;
        }
        if (l == 0) S.ans = found;
      }
      __syncthreads();
      for (u32 s = tid; s < GM_T; s += GB) {
        S.key[s] = 0;
        S.conn[s] = 0;
      }
      if (bp == NONE32) {
        bp = S.ans;
        be = 0;
      }
    } else {
      for (u32 lo = 0; lo < G.k; lo += GD) {
        const u32 hi = G.k - lo < GD ? G.k : lo + GD;
        // every list entry of every incident hyperedge, a wave per hyperedge
        for (i64 j = i0 + wave_id(); j < i1; j += GB / WAVE) {
          const u32 e = G.n_inc[j];
          const i64 a = G.e_off[e];
          const u32 lm = G.lam[e];
          const u64 we = G.e_w[e];
          for (u32 t = lane_id(); t < lm; t += WAVE) {
            const u32 p = (u32)(G.pl[a + t] >> 32);
            if (p >= lo && p < hi && p != pn)
              atomicAdd((unsigned long long *)&S.conn[p - lo], (unsigned long long)we);
          }
        }
        __syncthreads();
        // every partition of the window, touched or not; the window is left empty
        for (u32 p = lo + tid; p < lo + GD; p += GB) {
          const u64 cv = S.conn[p - lo];
          S.conn[p - lo] = 0;
          if (p < hi && p != pn && admissible(G, p, size_n) && better(cv, p, be, bp)) {
            be = cv;
            bp = p;
          }
        }
        __syncthreads();
      }
      wg_best_reduce(S, be, bp);
    }
    if (tid == 0) {
      G.move[n] = bp;
      G.gain[n] = bp == NONE32 ? 0 : (i64)saving - (i64)W + (i64)be;
    }
    __syncthreads();
  }
}

}  // namespace

void launch_pins_lists(chp_ctx *c, const i64 *e_off, const u32 *pins, const u32 *rho, u32 k,
                       u64 *pl, u32 *lam, EdgeLists el, const u32 *host_cnt, u64 *scratch,
                       u64 per_wg, u32 grid_big) {
  if (host_cnt[0])
    CHP_LAUNCH(c, "pins_wave", k_pins_wave, waves_grid(host_cnt[0]), 256, 0, e_off, pins, rho, k,
               pl, lam, (const u32 *)el.list[0], (const u32 *)el.cnt + 0, c->flags);
  if (host_cnt[1])
    CHP_LAUNCH(c, "pins_lds", (k_pins_lds<256, LDS_CAP_U64>),
               host_cnt[1] > 8192 ? 8192 : host_cnt[1], 256, 0, e_off, pins, rho, k, pl, lam,
               (const u32 *)el.list[1], (const u32 *)el.cnt + 1, c->flags);
  if (host_cnt[2])
    CHP_LAUNCH(c, "pins_global", (k_pins_global<256, LDS_CAP_U64>), grid_big, 256, 0, e_off,
               pins, rho, k, pl, lam, (const u32 *)el.list[2], (const u32 *)el.cnt + 2, c->flags,
               scratch, per_wg);
}

void launch_free_tree(chp_ctx *c, u32 k, u32 K2, const u64 *part_size, u64 omega, u64 *tree) {
  CHP_LAUNCH(c, "free_leaves", k_free_leaves, grid_for(K2, 256), 256, 0, k, K2, part_size, omega,
             tree);
  for (u32 cnt = K2 / 2; cnt >= 1; cnt /= 2)
    CHP_LAUNCH(c, "free_level", k_free_level, grid_for(cnt, 256), 256, 0, cnt, cnt, tree);
}

void launch_gains(chp_ctx *c, u32 N, u32 k, u32 K2, int enforce, u64 omega, const i64 *e_off,
                  const u32 *e_w, const u64 *pl, const u32 *lam, const i64 *n_off,
                  const u32 *n_inc, const u32 *n_size, const u32 *rho, const u64 *part_size,
                  const u64 *tree, u32 *move, i64 *gain, u32 *lists, u32 *cnt,
                  const u32 *host_cnt) {
  GainArgs G;
  G.N = N;
  G.k = k;
  G.K2 = K2;
  G.enforce = enforce ? 1u : 0u;
  G.omega = omega;
  G.e_off = e_off;
  G.e_w = e_w;
  G.pl = pl;
  G.lam = lam;
  G.n_off = n_off;
  G.n_inc = n_inc;
  G.n_size = n_size;
  G.rho = rho;
  G.part_size = part_size;
  G.tree = tree;
  G.move = move;
  G.gain = gain;
  if (host_cnt == nullptr) {
    CHP_LAUNCH(c, "gain_classify", k_gain_classify, grid_for(N, 256), 256, 0, G, lists, cnt);
    return;
  }
  if (host_cnt[0])
    CHP_LAUNCH(c, "gain_light", k_gain_light, waves_grid(host_cnt[0]), GB, 0, G,
               (const u32 *)lists, (const u32 *)cnt);
  if (host_cnt[1])
    CHP_LAUNCH(c, "gain_heavy", k_gain_heavy,
               host_cnt[1] < GH_PER_CU * c->n_cu ? host_cnt[1] : GH_PER_CU * c->n_cu, GB, 0, G,
               (const u32 *)lists, (const u32 *)cnt, cnt + 2);
}
