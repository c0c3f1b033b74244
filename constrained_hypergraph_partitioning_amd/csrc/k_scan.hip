// Device-wide exclusive prefix sums.  Output has n+1 entries, the last one the
// grand total, which is how every CSR offset array here is built.
//
// Up to 4096 tiles of 4096 elements: tile totals, then each workgroup adds up
// the totals of the tiles before its own (at most 4095 reads, from L2) and
// scans its tile: two launches, one when the array fits one tile.  Larger
// arrays take three phases over 1024-element tiles: per-tile scan, scan of
// the tile totals by one workgroup, add-back.
#include "dev.h"

namespace {

constexpr int SB = 256;     // threads per tile
constexpr int SI = 4;       // items per thread
constexpr int TILE = SB * SI;

template <typename In>
__global__ __launch_bounds__(SB) void k_scan_tiles(const In *in, i64 *out, u64 n, i64 *tile_sums) {
  __shared__ i64 lds[SB / WAVE + 1];
  u64 base = (u64)blockIdx.x * TILE + (u64)threadIdx.x * SI;
  i64 v[SI];
  i64 s = 0;
#pragma unroll
  for (int k = 0; k < SI; ++k) {
    v[k] = (base + k < n) ? (i64)in[base + k] : 0;
    s += v[k];
  }
  i64 tot;
  i64 off = wg_excl_scan<SB>(s, lds, &tot);
#pragma unroll
  for (int k = 0; k < SI; ++k) {
    if (base + k < n) out[base + k] = off;
    off += v[k];
  }
  if (threadIdx.x == 0) tile_sums[blockIdx.x] = tot;
}

// one workgroup scans the tile totals in place (exclusive), any count
__global__ __launch_bounds__(SB) void k_scan_sums(i64 *tile_sums, u64 ntiles, i64 *out, u64 n) {
  __shared__ i64 lds[SB / WAVE + 1];
  i64 carry = 0;
  for (u64 b = 0; b < ntiles; b += SB) {
    u64 i = b + threadIdx.x;
    i64 v = i < ntiles ? tile_sums[i] : 0;
    i64 tot;
    i64 off = wg_excl_scan<SB>(v, lds, &tot);
    if (i < ntiles) tile_sums[i] = carry + off;
    carry += tot;
  }
  if (threadIdx.x == 0) out[n] = carry;
}

__global__ __launch_bounds__(SB) void k_scan_add(i64 *out, u64 n, const i64 *tile_sums) {
  u64 base = (u64)blockIdx.x * TILE;
  i64 add = tile_sums[blockIdx.x];
  for (u64 i = base + threadIdx.x; i < base + TILE && i < n; i += SB) out[i] += add;
}

constexpr int BI = 16;  // items per thread, two-launch scan
constexpr u64 BTILE = (u64)SB * BI;
constexpr u64 BMAX_TILES = 4096;

template <typename In>
__global__ __launch_bounds__(SB) void k_scan_totals(const In *in, u64 n, i64 *tile_sums) {
  __shared__ i64 lds[SB / WAVE + 1];
  const u64 base = (u64)blockIdx.x * BTILE;
  i64 s = 0;
#pragma unroll
  for (int k = 0; k < BI; ++k) {
    const u64 i = base + (u64)k * SB + threadIdx.x;
    s += i < n ? (i64)in[i] : 0;
  }
  s = wg_sum<SB>(s, lds);
  if (threadIdx.x == 0) tile_sums[blockIdx.x] = s;
}

// Tile b: the sum of the totals of tiles [0, b), then the scan of its own
// elements; the last tile also writes the grand total out[n].
template <typename In>
__global__ __launch_bounds__(SB) void k_scan_down(const In *in, i64 *out, u64 n,
                                                  const i64 *tile_sums) {
  __shared__ i64 lds[SB / WAVE + 1];
  const u32 b = blockIdx.x;
  i64 pre = 0;
  for (u32 j = threadIdx.x; j < b; j += SB) pre += tile_sums[j];
  pre = wg_sum<SB>(pre, lds);
  const u64 base = (u64)b * BTILE + (u64)threadIdx.x * BI;
  i64 v[BI];
  i64 s = 0;
#pragma unroll
  for (int k = 0; k < BI; ++k) {
    v[k] = (base + k < n) ? (i64)in[base + k] : 0;
    s += v[k];
  }
  i64 tot;
  i64 off = pre + wg_excl_scan<SB>(s, lds, &tot);
#pragma unroll
  for (int k = 0; k < BI; ++k) {
    if (base + k < n) out[base + k] = off;
    off += v[k];
  }
  if (b + 1 == gridDim.x && threadIdx.x == 0) out[n] = pre + tot;
}

template <typename In>
void scan_impl(chp_ctx *c, const In *in, i64 *out, u64 n, i64 *tmp) {
  const u64 bt = (n + BTILE - 1) / BTILE;
  if (bt <= BMAX_TILES) {
    const u32 nt = bt ? (u32)bt : 1u;
    if (nt > 1) CHP_LAUNCH(c, "scan_totals", k_scan_totals<In>, nt, SB, 0, in, n, tmp);
    CHP_LAUNCH(c, "scan_down", k_scan_down<In>, nt, SB, 0, in, out, n, (const i64 *)tmp);
    return;
  }
  u64 ntiles = (n + TILE - 1) / TILE;
  CHP_LAUNCH(c, "scan_tiles", k_scan_tiles<In>, (u32)ntiles, SB, 0, in, out, n, tmp);
  CHP_LAUNCH(c, "scan_sums", k_scan_sums, 1, SB, 0, tmp, ntiles, out, n);
  CHP_LAUNCH(c, "scan_add", k_scan_add, (u32)ntiles, SB, 0, out, n, (const i64 *)tmp);
}

}  // namespace

size_t scan_tmp_words(u64 n) { return (size_t)((n + TILE - 1) / TILE + 1); }
void scan_u32_to_i64(chp_ctx *c, const u32 *in, i64 *out, u64 n, i64 *tmp) {
  scan_impl<u32>(c, in, out, n, tmp);
}
void scan_i64(chp_ctx *c, const i64 *in, i64 *out, u64 n, i64 *tmp) {
  scan_impl<i64>(c, in, out, n, tmp);
}
