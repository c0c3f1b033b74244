// Best-effort pairing of the nodes left without a partner ("Hypergraph
// Partitioning on GPU with Distinct Incident Hyperedges and Size
// Constraints", Sec. V-C, last mechanism): the unmatched nodes without a
// target are gathered and sorted by (size, id); each finds, by binary search,
// the last position whose size fits its Omega slack and takes the first node
// within LEFT_WINDOW positions below it whose inbound count, added to its
// own, stays within Delta (the union overestimated by the sum).  A node
// claimed by several goes to the smallest id (an atomic min), and a claimer
// pairs with its choice when it won it and nobody claimed the claimer.
#include "dev.h"
#include "kernels.h"

namespace {

constexpr int LB = 256;

// keys (size << 32 | n) of the unmatched nodes without a target; cnt[2] and
// cnt[3] (filled with NONE32 before) get their smallest size and smallest
// inbound count: when twice either exceeds its limit, no two of them can pair
__global__ __launch_bounds__(LB) void k_left_gather(u32 N, const u32 *target, const u32 *match,
                                                    const u32 *n_size, const u32 *n_nin,
                                                    u64 *keys, u32 *cnt) {
  __shared__ u32 s_app[LB / WAVE + 1];
  const u32 n = blockIdx.x * blockDim.x + threadIdx.x;
  const bool take = n < N && target[n] == NONE32 && match[n] == n;
  const u32 s = block_append<LB, 1>(cnt, take ? 0 : 1, s_app);
  u32 sz = NONE32, ni = NONE32;
  if (take) {
    sz = n_size[n];
    ni = n_nin[n];
    keys[s] = ((u64)sz << 32) | n;
  }
#pragma unroll
  for (int d = WAVE / 2; d > 0; d >>= 1) {
    const u32 o1 = __shfl_xor(sz, d, WAVE), o2 = __shfl_xor(ni, d, WAVE);
    sz = o1 < sz ? o1 : sz;
    ni = o2 < ni ? o2 : ni;
  }
  if (lane_id() == 0 && sz != NONE32) {
    atomicMin(cnt + 2, sz);
    atomicMin(cnt + 3, ni);
  }
}

__global__ void k_left_choose(u32 nl, const u64 *keys, const u32 *n_nin, u64 omega, u32 delta,
                              u32 window, u32 *choice, u32 *claim) {
  const u32 i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nl) return;
  const u64 key = keys[i];
  const u32 n = (u32)key, size = (u32)(key >> 32);
  u32 got = NONE32;
  if ((u64)size <= omega) {
    const u64 slack = omega - size;
    u32 lo = 0, hi = nl;  // positions whose size is <= slack: [0, lo)
    while (lo < hi) {
      const u32 mid = lo + (hi - lo) / 2;
      if ((keys[mid] >> 32) <= slack) lo = mid + 1;
      else hi = mid;
    }
    const u64 nin_n = n_nin[n];
    for (u32 s = 0; s < window && s < lo; ++s) {
      const u32 j = lo - 1 - s;
      if (j == i) continue;
      const u32 m = (u32)keys[j];
      if (nin_n + n_nin[m] <= (u64)delta) {
        got = m;
        break;
      }
    }
  }
  choice[i] = got;
  if (got != NONE32) atomicMin(claim + got, n);
}

__global__ void k_left_pair(u32 nl, const u64 *keys, const u32 *choice, const u32 *claim,
                            u32 *match, u32 *npairs) {
  const u32 i = blockIdx.x * blockDim.x + threadIdx.x;
  bool paired = false;
  if (i < nl) {
    const u32 n = (u32)keys[i], m = choice[i];
    if (m != NONE32 && claim[m] == n && claim[n] == NONE32) {
      match[n] = m;  // the only writer of both: m is claimed, so it pairs with no one else
      match[m] = n;
      paired = true;
    }
  }
  const u64 b = __ballot(paired);
  if (lane_id() == 0 && b) atomicAdd(npairs, (u32)__popcll(b));
}

}  // namespace

void launch_left_gather(chp_ctx *c, u32 N, const u32 *target, const u32 *match,
                        const u32 *n_size, const u32 *n_nin, u64 *keys, u32 *cnt) {
  if (N == 0) return;
  CHP_LAUNCH(c, "left_gather", k_left_gather, grid_for(N, LB), LB, 0, N, target, match, n_size,
             n_nin, keys, cnt);
}

void launch_left_pair(chp_ctx *c, u32 nl, const u64 *keys, const u32 *n_nin, u64 omega,
                      u32 delta, u32 window, u32 *choice, u32 *claim, u32 *match, u32 *npairs) {
  if (nl == 0) return;
  CHP_LAUNCH(c, "left_choose", k_left_choose, grid_for(nl, LB), LB, 0, nl, keys, n_nin, omega,
             delta, window, choice, claim);
  CHP_LAUNCH(c, "left_pair", k_left_pair, grid_for(nl, LB), LB, 0, nl, keys,
             (const u32 *)choice, (const u32 *)claim, match, npairs);
}
