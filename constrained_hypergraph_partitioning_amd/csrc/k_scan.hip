// Device-wide exclusive prefix sums (three phases: per-tile scan, scan of the
// tile totals by one workgroup, add-back).  Output has n+1 entries, the last
// one the grand total, which is how every CSR offset array here is built.
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

template <typename In>
void scan_impl(chp_ctx *c, const In *in, i64 *out, u64 n, i64 *tmp) {
  u64 ntiles = (n + TILE - 1) / TILE;
  if (ntiles == 0) ntiles = 1;
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
