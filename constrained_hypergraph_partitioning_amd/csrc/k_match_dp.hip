// Exact maximum-weight matching on the proposal pseudo-forest ("Hypergraph
// Partitioning on GPU with Distinct Incident Hyperedges and Size
// Constraints", Sec. V-D, Eqs. 7-12).  The proposal edge of n is
// {n, target(n)} with weight score(n); two-cycles are the roots of their
// trees, a node without target tops its own.  Bottom up, per node:
//   A(n) = sum of ss0 over its children, best(n) = max of ss1 - ss0 over
//   them (smallest id on ties), ss0(n) = A(n) + max(0, best(n)),
//   ss1(n) = score(n) + A(n);
// top down, a two-cycle pairs when score + A(n) + A(t) > ss0(n) + ss0(t),
// a node taken by its target pairs with it, and any other node takes its best
// child when best > 0.
//
// Work is level-synchronous over depth: the depth of every node comes from
// pointer jumping, nodes are bucketed by depth, and each depth is one launch
// up (children add ss0 into the parent, raise its best difference, then the
// children holding it lower the best id) and one launch down.  Sums and the
// (value, id) choices do not depend on the order of the atomics.
#include "dev.h"
#include "kernels.h"

namespace {

constexpr int DB = 256;

__global__ void k_dp_init(u32 N, const u32 *target, u32 *par, u32 *anc, u32 *dist, u32 *match,
                          u64 *A, u64 *bestv, u32 *bestc, u32 *flags) {
  const u32 n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= N) return;
  const u32 t = target[n];
  if (t != NONE32 && (t >= N || t == n)) {
    atomicOr(flags, FLAG_EINVAL);
    par[n] = NONE32;
  } else {
    const bool inR = t != NONE32 && target[t] == n;
    par[n] = inR ? NONE32 : t;
  }
  anc[n] = par[n] == NONE32 ? n : par[n];
  dist[n] = par[n] == NONE32 ? 0 : 1;
  match[n] = n;
  A[n] = 0;
  bestv[n] = 0;
  bestc[n] = NONE32;
}

__global__ void k_dp_jump(u32 N, const u32 *anc, const u32 *dist, u32 *anc2, u32 *dist2) {
  const u32 n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= N) return;
  const u32 a = anc[n];
  anc2[n] = anc[a];
  const u32 d = dist[n] + dist[a];
  dist2[n] = d < dist[n] ? 0xFFFFFFFFu : d;
}

// after the jumps every node must reach a root; depth histogram
__global__ void k_dp_depths(u32 N, const u32 *par, const u32 *anc, const u32 *dist, u32 *maxd,
                            u32 *flags) {
  const u32 n = blockIdx.x * blockDim.x + threadIdx.x;
  u32 d = 0;
  if (n < N) {
    if (par[anc[n]] != NONE32) atomicOr(flags, FLAG_ECYCLE);
    d = dist[n];
  }
#pragma unroll
  for (int s = WAVE / 2; s > 0; s >>= 1) {
    const u32 o = __shfl_xor(d, s, WAVE);
    d = o > d ? o : d;
  }
  if (lane_id() == 0) atomicMax(maxd, d);
}

// One atomic per distinct bucket of the wave (most nodes share a few depths):
// returns this lane's slot in bucket `key` of `ctr` (active lanes only).
__device__ u32 wave_bucket_append(u32 *ctr, u32 key, bool active) {
  const u32 l = lane_id();
  u32 slot = 0;
  u64 left = __ballot(active);
  while (left) {
    const u32 leader = (u32)__builtin_ctzll(left);
    const u32 k = __shfl(key, leader, WAVE);
    const u64 same = __ballot(active && key == k);
    u32 base = 0;
    if (l == leader) base = atomicAdd(ctr + k, (u32)__popcll(same));
    base = __shfl(base, leader, WAVE);
    if (active && key == k) slot = base + (u32)__popcll(same & ((1ull << l) - 1));
    left &= ~same;
  }
  return slot;
}

__global__ void k_dp_count(u32 N, const u32 *dist, u32 *cntd) {
  const u32 n = blockIdx.x * blockDim.x + threadIdx.x;
  const bool ok = n < N;
  wave_bucket_append(cntd, ok ? dist[n] : 0, ok);
}

__global__ void k_dp_scatter(u32 N, const u32 *dist, u32 *cur, u32 *byd) {
  const u32 n = blockIdx.x * blockDim.x + threadIdx.x;
  const bool ok = n < N;
  const u32 slot = wave_bucket_append(cur, ok ? dist[n] : 0, ok);
  if (ok) byd[slot] = n;
}

__device__ __forceinline__ void add_ovf(u64 *p, u64 v, u32 *flags) {
  const u64 old = atomicAdd((unsigned long long *)p, (unsigned long long)v);
  if (old + v < old) atomicOr(flags, FLAG_EOVERFLOW);
}

// nodes at one depth: ss0, ss1 from their children's sums, then their own
// contribution to the parent
__global__ void k_dp_up(const u32 *nodes, u32 cnt, const u32 *target, const u64 *score,
                        const u32 *par, u64 *A, u64 *bestv, const u32 *bestc, u64 *ss0,
                        u64 *diff, u32 *flags) {
  const u32 i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= cnt) return;
  const u32 n = nodes[i];
  const u64 a = A[n];
  const u64 b = bestc[n] != NONE32 ? bestv[n] : 0;
  const u64 s0 = a + b;
  if (s0 < a) atomicOr(flags, FLAG_EOVERFLOW);
  ss0[n] = s0;
  u64 df = 0;
  if (target[n] != NONE32) {
    const u64 s1 = score[n] + a;
    if (s1 < a) atomicOr(flags, FLAG_EOVERFLOW);
    df = s1 >= s0 ? s1 - s0 : 0;
  }
  diff[n] = df;
  const u32 p = par[n];
  if (p != NONE32) {
    add_ovf(A + p, s0, flags);
    if (df) atomicMax((unsigned long long *)(bestv + p), (unsigned long long)df);
  }
}

// the children holding their parent's best difference lower its best id
__global__ void k_dp_up_ids(const u32 *nodes, u32 cnt, const u32 *par, const u64 *bestv,
                            const u64 *diff, u32 *bestc) {
  const u32 i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= cnt) return;
  const u32 n = nodes[i];
  const u32 p = par[n];
  if (p != NONE32 && diff[n] && diff[n] == bestv[p]) atomicMin(bestc + p, n);
}

// depth 0: two-cycles and free tops decide
__global__ void k_dp_roots(const u32 *nodes, u32 cnt, const u32 *target, const u64 *score,
                           const u64 *A, const u64 *ss0, const u64 *bestv, const u32 *bestc,
                           u32 *match, u32 *flags) {
  const u32 i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= cnt) return;
  const u32 n = nodes[i];
  const u32 t = target[n];
  if (t != NONE32) {  // a two-cycle, decided by its smaller node
    if (n > t) return;
    const u64 pair = score[n] + A[n];
    const u64 pair2 = pair + A[t];
    const u64 apart = ss0[n] + ss0[t];
    if (pair < A[n] || pair2 < pair || apart < ss0[n]) atomicOr(flags, FLAG_EOVERFLOW);
    if (pair2 > apart) {
      match[n] = t;
      match[t] = n;
      return;
    }
    if (bestc[t] != NONE32 && bestv[t] > 0) {
      match[t] = bestc[t];
      match[bestc[t]] = t;
    }
  }
  if (bestc[n] != NONE32 && bestv[n] > 0) {
    match[n] = bestc[n];
    match[bestc[n]] = n;
  }
}

// depth d > 0: taken by the target, or take the best child
__global__ void k_dp_down(const u32 *nodes, u32 cnt, const u32 *par, const u64 *bestv,
                          const u32 *bestc, u32 *match) {
  const u32 i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= cnt) return;
  const u32 n = nodes[i];
  if (match[par[n]] == n) return;
  if (bestc[n] != NONE32 && bestv[n] > 0) {
    match[n] = bestc[n];
    match[bestc[n]] = n;
  }
}

__global__ void k_dp_pairs(u32 N, const u32 *match, u32 *npairs) {
  const u32 n = blockIdx.x * blockDim.x + threadIdx.x;
  const bool p = n < N && match[n] > n;
  const u64 b = __ballot(p);
  if (lane_id() == 0 && b) atomicAdd(npairs, (u32)__popcll(b));
}

}  // namespace

void launch_dp_prepare(chp_ctx *c, u32 N, const u32 *target, DpScratch &d, u32 *match) {
  const u32 g = grid_for(N, DB);
  CHP_LAUNCH(c, "dp_init", k_dp_init, g, DB, 0, N, target, d.par, d.anc, d.dist, match, d.A,
             d.bestv, d.bestc, c->flags);
  u32 rounds = 1;
  while ((1ull << rounds) < (u64)N + 1) ++rounds;
  for (u32 r = 0; r < rounds; ++r) {
    CHP_LAUNCH(c, "dp_jump", k_dp_jump, g, DB, 0, N, (const u32 *)d.anc, (const u32 *)d.dist,
               d.anc2, d.dist2);
    u32 *t = d.anc;
    d.anc = d.anc2;
    d.anc2 = t;
    t = d.dist;
    d.dist = d.dist2;
    d.dist2 = t;
  }
  CHP_LAUNCH(c, "dp_depths", k_dp_depths, g, DB, 0, N, (const u32 *)d.par, (const u32 *)d.anc,
             (const u32 *)d.dist, d.small, c->flags);
}

void launch_dp_levels(chp_ctx *c, u32 N, const u32 *target, const u64 *score, DpScratch &d,
                      u32 D, u32 *cursor, const u32 *offd, u32 *match, u32 *npairs) {
  const u32 g = grid_for(N, DB);
  CHP_LAUNCH(c, "dp_scatter", k_dp_scatter, g, DB, 0, N, (const u32 *)d.dist, cursor, d.byd);
  for (u32 lv = D + 1; lv-- > 0;) {
    const u32 cnt = offd[lv + 1] - offd[lv];
    if (!cnt) continue;
    const u32 *nodes = d.byd + offd[lv];
    CHP_LAUNCH(c, "dp_up", k_dp_up, grid_for(cnt, DB), DB, 0, nodes, cnt, target, score,
               (const u32 *)d.par, d.A, d.bestv, (const u32 *)d.bestc, d.ss0, d.diff, c->flags);
    if (lv > 0)
      CHP_LAUNCH(c, "dp_up_ids", k_dp_up_ids, grid_for(cnt, DB), DB, 0, nodes, cnt,
                 (const u32 *)d.par, (const u64 *)d.bestv, (const u64 *)d.diff, d.bestc);
  }
  for (u32 lv = 0; lv <= D; ++lv) {
    const u32 cnt = offd[lv + 1] - offd[lv];
    if (!cnt) continue;
    const u32 *nodes = d.byd + offd[lv];
    if (lv == 0)
      CHP_LAUNCH(c, "dp_roots", k_dp_roots, grid_for(cnt, DB), DB, 0, nodes, cnt, target, score,
                 (const u64 *)d.A, (const u64 *)d.ss0, (const u64 *)d.bestv,
                 (const u32 *)d.bestc, match, c->flags);
    else
      CHP_LAUNCH(c, "dp_down", k_dp_down, grid_for(cnt, DB), DB, 0, nodes, cnt,
                 (const u32 *)d.par, (const u64 *)d.bestv, (const u32 *)d.bestc, match);
  }
  CHP_LAUNCH(c, "dp_pairs", k_dp_pairs, g, DB, 0, N, (const u32 *)match, npairs);
}

void launch_dp_count(chp_ctx *c, u32 N, const u32 *dist, u32 *cntd) {
  CHP_LAUNCH(c, "dp_count", k_dp_count, grid_for(N, DB), DB, 0, N, dist, cntd);
}
