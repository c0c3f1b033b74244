// Device-wide sort of distinct u64 keys: each workgroup sorts a tile of
// STILE keys in LDS (bitonic network), then merge passes double the sorted
// run length; in a pass every thread finds its own merge-path split of the
// pair of runs it writes into and emits MPT consecutive outputs.
#include "dev.h"
#include "kernels.h"

namespace {

constexpr int SB = 256;         // threads per workgroup
constexpr u32 STILE = 4096;     // keys per LDS tile
constexpr u32 MPT = 8;          // outputs per thread in a merge pass

// tiles of m keys (m a power of two <= STILE; fewer keys are padded)
__global__ __launch_bounds__(SB) void k_sort_tiles(u64 *a, u64 n, u32 m) {
  __shared__ u64 s[STILE];
  const u64 t0 = (u64)blockIdx.x * m;
  const u32 cnt = (u32)(n - t0 < m ? n - t0 : m);
  for (u32 i = threadIdx.x; i < m; i += SB) s[i] = i < cnt ? a[t0 + i] : ~0ull;
  __syncthreads();
  lds_bitonic<SB>(s, m);
  for (u32 i = threadIdx.x; i < cnt; i += SB) a[t0 + i] = s[i];
}

// Runs of length w in src (the last one shorter) merged pairwise into dst.
__global__ __launch_bounds__(SB) void k_merge_runs(const u64 *src, u64 *dst, u64 n, u64 w) {
  const u64 d = ((u64)blockIdx.x * SB + threadIdx.x) * MPT;
  if (d >= n) return;
  const u64 a0 = d / (2 * w) * (2 * w);
  const u64 na = n - a0 < w ? n - a0 : w;
  const u64 b0 = a0 + na;
  const u64 nb = n - b0 < w ? n - b0 : w;
  const u64 *A = src + a0, *B = src + b0;
  const u64 k = d - a0;  // diagonal inside this pair
  u64 lo = k > nb ? k - nb : 0, hi = k < na ? k : na;
  while (lo < hi) {  // first i with A[i] > B[k - 1 - i]
    const u64 mid = (lo + hi) >> 1;
    if (A[mid] < B[k - 1 - mid]) lo = mid + 1;
    else hi = mid;
  }
  u64 i = lo, j = k - lo;
  const u64 end = d + MPT < a0 + na + nb ? d + MPT : a0 + na + nb;
  for (u64 o = d; o < end; ++o) {
    const bool ta = j >= nb || (i < na && A[i] < B[j]);
    dst[o] = ta ? A[i++] : B[j++];
  }
}

}  // namespace

u64 *sort_keys_u64(chp_ctx *c, u64 *a, u64 *tmp, u64 n) {
  if (n <= 1) return a;
  u32 m = STILE;  // a short input takes one tile of its own size
  if (n < STILE) {
    m = 2;
    while (m < n) m <<= 1;
  }
  CHP_LAUNCH(c, "sort_tiles", k_sort_tiles, grid_for(n, m), SB, 0, a, n, m);
  u64 *src = a, *dst = tmp;
  for (u64 w = STILE; w < n; w <<= 1) {
    CHP_LAUNCH(c, "merge_runs", k_merge_runs, grid_for(n, (u64)SB * MPT), SB, 0,
               (const u64 *)src, dst, n, w);
    u64 *t = src;
    src = dst;
    dst = t;
  }
  return src;
}
