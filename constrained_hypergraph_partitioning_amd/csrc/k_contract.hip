// Contraction of one level ("Hypergraph Partitioning on GPU with Distinct
// Incident Hyperedges and Size Constraints", Sec. III and V-E).
//
// gamma(n) is the rank of min(n, match(n)) among cluster representatives
// (an exclusive scan of "match(n) >= n").  A coarse hyperedge keeps the id and
// weight of its fine hyperedge; its destinations are the distinct gamma(dst)
// and its sources the distinct gamma(src) that are not destinations (Sec. V-E
// drops such duplicates from the sources).  Per hyperedge this is one sort of
// 64-bit keys (gamma << 1 | is_source): in each group of equal gamma the
// first key tells whether some destination maps there.
#include "dev.h"
#include "kernels.h"

namespace {

__global__ void k_rep(u32 N, const u32 *match, u32 *is_rep, u32 *flags) {
  u32 n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= N) return;
  u32 m = match[n];
  bool ok = m < N && match[m] == n;
  if (!ok) atomicOr(flags, FLAG_EINVAL);
  is_rep[n] = (ok && m >= n) ? 1u : 0u;
}

__global__ void k_gamma(u32 N, const u32 *match, const i64 *rank, const u32 *n_size, u32 *gamma,
                        u32 *c_size, u32 *rep_of) {
  u32 n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= N) return;
  u32 m = match[n];
  u32 r = m < n ? m : n;
  u32 g = (u32)rank[r];
  gamma[n] = g;
  if (r == n) {
    c_size[g] = n_size[n] + (m != n ? n_size[m] : 0u);
    rep_of[g] = n;
  }
}

__global__ __launch_bounds__(256) void k_edge_classify(u32 E, const i64 *e_off, EdgeLists el) {
  __shared__ u32 s_app[3 * (256 / WAVE) + 3];
  const u32 e = blockIdx.x * blockDim.x + threadIdx.x;
  u64 len = 0;
  if (e < E) len = (u64)(e_off[e + 1] - e_off[e]);
  const int c = e >= E ? 3 : (len <= 64 ? 0 : (len <= LDS_CAP_U64 ? 1 : 2));
  const u32 slot = block_append<256, 3>(el.cnt, c, s_app);
  if (c < 3) el.list[c][slot] = e;
  if (c == 2) atomicMax(&el.cnt[3], (u32)len);
}

// Hyperedges of at most TINY pins (most nets of a netlist): one thread each,
// the keys (gamma << 1 | is_source) sorted in registers by a 19-comparator
// sorting network, then the groups written as the wave kernel writes them
// (distinct sources first, then the distinct destinations).  The other
// hyperedges of the wave class are passed on: those of at most 32 pins in
// rest[0, rest_cnt[0]) to k_econ_half, the others in rest[T, T + rest_cnt[1])
// to k_econ_wave, with T = *cnt; rest holds 2 T entries and rest_cnt[0..1]
// are zeroed before.  One thread per entry of list[0, *cnt).
constexpr u32 TINY = 8;
__global__ __launch_bounds__(256) void k_econ_tiny(const i64 *e_off, const u32 *e_nsrc,
                                                   const u32 *pins, const u32 *gamma, u32 *opins,
                                                   u32 *olen, u32 *onsrc, const u32 *list,
                                                   const u32 *cnt, u32 *rest, u32 *rest_cnt) {
  __shared__ u32 s_app[2 * (256 / WAVE) + 2];
  const u32 total = *cnt;
  const u32 i = blockIdx.x * blockDim.x + threadIdx.x;
  u32 e = 0, len = 0, ns = 0;
  i64 a = 0;
  if (i < total) {
    e = list[i];
    a = e_off[e];
    len = (u32)(e_off[e + 1] - a);
    ns = e_nsrc[e];
  }
  const bool tiny = i < total && len <= TINY;
  const int cls = (i >= total || tiny) ? 2 : len <= 32 ? 0 : 1;
  const u32 slot = block_append<256, 2>(rest_cnt, cls, s_app);
  if (cls == 0) rest[slot] = e;
  if (cls == 1) rest[total + slot] = e;
  if (!tiny) return;
  u64 k[TINY];
#pragma unroll
  for (u32 j = 0; j < TINY; ++j)
    k[j] = j < len ? ((u64)gamma[pins[a + j]] << 1) | (j < ns ? 1u : 0u) : ~0ull;
  cswap(k[0], k[1]), cswap(k[2], k[3]), cswap(k[4], k[5]), cswap(k[6], k[7]);
  cswap(k[0], k[2]), cswap(k[1], k[3]), cswap(k[4], k[6]), cswap(k[5], k[7]);
  cswap(k[1], k[2]), cswap(k[5], k[6]), cswap(k[0], k[4]), cswap(k[3], k[7]);
  cswap(k[1], k[5]), cswap(k[2], k[6]);
  cswap(k[1], k[4]), cswap(k[3], k[6]);
  cswap(k[2], k[4]), cswap(k[3], k[5]);
  cswap(k[3], k[4]);
  // a group of equal gamma is a source' iff its first (smallest) key is a source
  u32 nsp = 0, ntot = 0;
#pragma unroll
  for (u32 j = 0; j < TINY; ++j) {
    const bool first = k[j] != ~0ull && (j == 0 || (k[j - 1] >> 1) != (k[j] >> 1));
    ntot += first ? 1u : 0u;
    nsp += (first && (k[j] & 1)) ? 1u : 0u;
  }
  u32 *out = opins + a;
  u32 ps = 0, pd = nsp;
#pragma unroll
  for (u32 j = 0; j < TINY; ++j) {
    const bool first = k[j] != ~0ull && (j == 0 || (k[j - 1] >> 1) != (k[j] >> 1));
    if (first) {
      if (k[j] & 1) out[ps++] = (u32)(k[j] >> 1);
      else out[pd++] = (u32)(k[j] >> 1);
    }
  }
  olen[e] = ntot;
  onsrc[e] = nsp;
}

// The LDS class (65 .. LDS_CAP_U64 pins) split by size: those of at most
// ECON_SMALL pins go to small[0, small_cnt[0]) for a wave each (keys in
// registers), the others to big[0, small_cnt[1]) for a workgroup with a
// 64 KB LDS table (two per CU).  small_cnt[0..1] zeroed before; one thread per list entry.
constexpr u32 ECON_SMALL = 1024;
__global__ __launch_bounds__(256) void k_econ_split(const i64 *e_off, const u32 *list,
                                                    const u32 *cnt, u32 *small, u32 *big,
                                                    u32 *small_cnt) {
  __shared__ u32 s_app[2 * (256 / WAVE) + 2];
  const u32 total = *cnt;
  const u32 i = blockIdx.x * blockDim.x + threadIdx.x;
  u32 e = 0;
  int cls = 2;
  if (i < total) {
    e = list[i];
    cls = (u64)(e_off[e + 1] - e_off[e]) <= ECON_SMALL ? 0 : 1;
  }
  const u32 slot = block_append<256, 2>(small_cnt, cls, s_app);
  if (cls == 0) small[slot] = e;
  if (cls == 1) big[slot] = e;
}

// Hyperedges of 9 to 32 pins: two per wave, one per half, each sorted by the
// bitonic network over its 32 lanes and emitted within its half.
__global__ __launch_bounds__(256) void k_econ_half(const i64 *e_off, const u32 *e_nsrc,
                                                   const u32 *pins, const u32 *gamma, u32 *opins,
                                                   u32 *olen, u32 *onsrc, const u32 *list,
                                                   const u32 *cnt) {
  const u32 total = *cnt;
  const u32 nwaves = gridDim.x * (blockDim.x / WAVE);
  const u32 l = lane_id(), h = l >> 5, hl = l & 31;
  const u64 half = 0xFFFFFFFFull << (32 * h);
  const u64 lt = (1ull << l) - 1;
  for (u32 w0 = 2 * (blockIdx.x * (blockDim.x / WAVE) + wave_id()); w0 < total;
       w0 += 2 * nwaves) {
    const u32 w = w0 + h;
    u32 e = 0, len = 0, ns = 0;
    i64 a = 0;
    if (w < total) {
      e = list[w];
      a = e_off[e];
      len = (u32)(e_off[e + 1] - a);
      ns = e_nsrc[e];
    }
    u64 key = ~0ull;
    if (hl < len) key = ((u64)gamma[pins[a + hl]] << 1) | (hl < ns ? 1u : 0u);
    // bitonic sort within each 32-lane half, both halves ascending
#pragma unroll
    for (u32 k = 2; k <= 32; k <<= 1) {
#pragma unroll
      for (u32 j = k >> 1; j > 0; j >>= 1) {
        const u64 o = __shfl_xor(key, j, WAVE);
        const bool up = k == 32 || (hl & k) == 0;
        const bool lower = (hl & j) == 0;
        key = (lower == up) ? (key < o ? key : o) : (key < o ? o : key);
      }
    }
    // groups within the half: sources first, then destinations
    const u64 prev = __shfl_up(key, 1, WAVE);
    const bool f = hl < len && (hl == 0 || (prev >> 1) != (key >> 1));
    const bool ff = f && (key & 1);
    const u64 fm = __ballot(ff) & half, om = __ballot(f && !ff) & half;
    const u32 nf = (u32)__popcll(fm);
    if (f)
      opins[a + (ff ? (u32)__popcll(fm & lt) : nf + (u32)__popcll(om & lt))] = (u32)(key >> 1);
    if (hl == 0 && w < total) {
      olen[e] = nf + (u32)__popcll(om);
      onsrc[e] = nf;
    }
  }
}

// small hyperedges: one wave each, keys in registers
__global__ __launch_bounds__(256) void k_econ_wave(const i64 *e_off, const u32 *e_nsrc,
                                                   const u32 *pins, const u32 *gamma, u32 *opins,
                                                   u32 *olen, u32 *onsrc, const u32 *list,
                                                   const u32 *cnt) {
  const u32 total = *cnt;
  const u32 nwaves = gridDim.x * (blockDim.x / WAVE);
  const u32 l = lane_id();
  const u64 lt = (1ull << l) - 1;
  for (u32 w = blockIdx.x * (blockDim.x / WAVE) + wave_id(); w < total; w += nwaves) {
    const u32 e = list[w];
    const i64 a = e_off[e];
    const u32 len = (u32)(e_off[e + 1] - a), ns = e_nsrc[e];
    u64 key = ~0ull;
    if (l < len) key = ((u64)gamma[pins[a + l]] << 1) | (l < ns ? 1u : 0u);
    key = wave_sort64(key);
    u32 nsp, ntot;
    wave_group_split_emit<1>(key, len, opins + a, nsp, ntot);
    if (l == 0) {
      olen[e] = ntot;
      onsrc[e] = nsp;
    }
  }
}

// Hyperedges of 65 .. ECON_SMALL pins: a wave each, the keys sorted in
// registers (4, 8 or 16 a lane, by |e|), distinct sources first.  K = u32
// when every coarse id is below 2^31 - 1 (the key gamma << 1 | tag then
// fits 32 bits, below the padding ~0), u64 otherwise.
template <typename K, int PER>
__device__ __forceinline__ void econ_regs(const u32 *pins, i64 a, u32 len, u32 ns,
                                          const u32 *gamma, u32 *out, u32 &nsp, u32 &ntot) {
  const u32 l = lane_id();
  K v[PER];
#pragma unroll
  for (u32 q = 0; q < (u32)PER; ++q) {
    const u32 i = q * WAVE + l;
    v[q] = i < len ? ((K)gamma[pins[a + i]] << 1) | (i < ns ? 1u : 0u) : ~(K)0;
  }
  wave_sort_regs<K, PER>(v);
  wave_group_split_emit_regs<1, PER>(v, len, out, nsp, ntot);
}

template <typename K>
__global__ __launch_bounds__(256) void k_econ_wreg(const i64 *e_off, const u32 *e_nsrc,
                                                   const u32 *pins, const u32 *gamma, u32 *opins,
                                                   u32 *olen, u32 *onsrc, const u32 *list,
                                                   const u32 *cnt) {
  const u32 total = *cnt;
  const u32 nwaves = gridDim.x * (blockDim.x / WAVE);
  for (u32 w = blockIdx.x * (blockDim.x / WAVE) + wave_id(); w < total; w += nwaves) {
    const u32 e = list[w];
    const i64 a = e_off[e];
    const u32 len = (u32)(e_off[e + 1] - a), ns = e_nsrc[e];
    u32 nsp, ntot;
    if (len <= 4 * WAVE) econ_regs<K, 4>(pins, a, len, ns, gamma, opins + a, nsp, ntot);
    else if (len <= 8 * WAVE) econ_regs<K, 8>(pins, a, len, ns, gamma, opins + a, nsp, ntot);
    else econ_regs<K, 16>(pins, a, len, ns, gamma, opins + a, nsp, ntot);
    if (lane_id() == 0) {
      olen[e] = ntot;
      onsrc[e] = nsp;
    }
  }
}

// distinct sources first (tag 1), then the distinct destinations
template <int BLOCK>
__device__ void econ_emit(const u64 *s, u32 m, u32 *out, u32 *olen, u32 *onsrc, u32 e,
                          u32 *s_red) {
  u32 nsrc, ntot;
  group_split_emit<BLOCK, 1>(s, m, out, nsrc, ntot, s_red);
  if (threadIdx.x == 0) {
    olen[e] = ntot;
    onsrc[e] = nsrc;
  }
}

template <int BLOCK, int CAP>
__global__ __launch_bounds__(BLOCK) void k_econ_lds(const i64 *e_off, const u32 *e_nsrc,
                                                    const u32 *pins, const u32 *gamma, u32 *opins,
                                                    u32 *olen, u32 *onsrc, const u32 *list,
                                                    const u32 *cnt) {
  __shared__ u64 s[CAP];
  __shared__ u32 s_red[BLOCK / WAVE + 1];
  const u32 total = *cnt;
  for (u32 w = blockIdx.x; w < total; w += gridDim.x) {
    const u32 e = list[w];
    const i64 a = e_off[e];
    const u32 len = (u32)(e_off[e + 1] - a), ns = e_nsrc[e];
    const u32 p = next_pow2(len);
    for (u32 i = threadIdx.x; i < p; i += BLOCK)
      s[i] = i < len ? (((u64)gamma[pins[a + i]] << 1) | (i < ns ? 1u : 0u)) : ~0ull;
    __syncthreads();
    lds_bitonic<BLOCK>(s, p);
    econ_emit<BLOCK>(s, len, opins + a, olen, onsrc, e, s_red);
    __syncthreads();
  }
}

template <int BLOCK, int CAP>
__global__ __launch_bounds__(BLOCK) void k_econ_global(const i64 *e_off, const u32 *e_nsrc,
                                                       const u32 *pins, const u32 *gamma,
                                                       u32 *opins, u32 *olen, u32 *onsrc,
                                                       const u32 *list, const u32 *cnt,
                                                       u64 *scratch, u64 per_wg) {
  __shared__ u64 s[CAP];
  __shared__ u32 s_red[BLOCK / WAVE + 1];
  const u32 total = *cnt;
  u64 *A = scratch + (u64)blockIdx.x * per_wg;
  u64 *B = A + per_wg / 2;
  for (u32 w = blockIdx.x; w < total; w += gridDim.x) {
    const u32 e = list[w];
    const i64 a = e_off[e];
    const u32 len = (u32)(e_off[e + 1] - a), ns = e_nsrc[e];
    for (u32 i = threadIdx.x; i < len; i += BLOCK)
      A[i] = ((u64)gamma[pins[a + i]] << 1) | (i < ns ? 1u : 0u);
    __syncthreads();
    u64 *res = wg_sort_global<BLOCK, CAP>(A, B, len, s);
    econ_emit<BLOCK>(res, len, opins + a, olen, onsrc, e, s_red);
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void k_pins_compact(u32 E, const i64 *src_off,
                                                      const u32 *src, const i64 *dst_off,
                                                      u32 *dst) {
  const u32 nwaves = gridDim.x * (blockDim.x / WAVE);
  const u32 l = lane_id();
  for (u32 e = blockIdx.x * (blockDim.x / WAVE) + wave_id(); e < E; e += nwaves) {
    i64 s = src_off[e], d = dst_off[e];
    u32 c = (u32)(dst_off[e + 1] - d);
    for (u32 i = l; i < c; i += WAVE) dst[d + i] = src[s + i];
  }
}


}  // namespace

void launch_rep(chp_ctx *c, u32 N, const u32 *match, u32 *is_rep) {
  if (N == 0) return;
  CHP_LAUNCH(c, "rep", k_rep, grid_for(N, 256), 256, 0, N, match, is_rep, c->flags);
}

void launch_gamma(chp_ctx *c, u32 N, const u32 *match, const i64 *rank, const u32 *n_size,
                  u32 *gamma, u32 *c_size, u32 *rep_of) {
  if (N == 0) return;
  CHP_LAUNCH(c, "gamma", k_gamma, grid_for(N, 256), 256, 0, N, match, rank, n_size, gamma,
             c_size, rep_of);
}

void launch_edge_classify(chp_ctx *c, u32 E, const i64 *e_off, EdgeLists el) {
  if (E == 0) return;
  CHP_LAUNCH(c, "edge_classify", k_edge_classify, grid_for(E, 256), 256, 0, E, e_off, el);
}

void launch_edge_contract(chp_ctx *c, const i64 *e_off, const u32 *e_nsrc, const u32 *pins,
                          const u32 *gamma, u32 *opins, u32 *olen, u32 *onsrc, EdgeLists el,
                          const u32 *host_cnt, u64 *scratch, u64 per_wg, u32 grid_big,
                          u32 *rest, bool narrow) {
  if (host_cnt[0]) {
    // el.cnt[4] and el.cnt[5] count the wave-class hyperedges of 9..32 and
    // 33..64 pins (zeroed by the classification's fill)
    CHP_LAUNCH(c, "econ_tiny", k_econ_tiny, grid_for(host_cnt[0], 256), 256, 0, e_off, e_nsrc,
               pins, gamma, opins, olen, onsrc, (const u32 *)el.list[0],
               (const u32 *)el.cnt + 0, rest, el.cnt + 4);
    CHP_LAUNCH(c, "econ_half", k_econ_half, waves_grid((host_cnt[0] + 1) / 2), 256, 0, e_off,
               e_nsrc, pins, gamma, opins, olen, onsrc, (const u32 *)rest,
               (const u32 *)el.cnt + 4);
    CHP_LAUNCH(c, "econ_wave", k_econ_wave, waves_grid(host_cnt[0]), 256, 0, e_off, e_nsrc, pins,
               gamma, opins, olen, onsrc, (const u32 *)(rest + host_cnt[0]),
               (const u32 *)el.cnt + 5);
  }
  if (host_cnt[1]) {
    // el.cnt[6] and el.cnt[7] count the LDS-class hyperedges of at most
    // ECON_SMALL pins and the larger ones (zeroed by the classification's fill)
    u32 *small = rest + 2ull * host_cnt[0], *big = small + host_cnt[1];
    CHP_LAUNCH(c, "econ_split", k_econ_split, grid_for(host_cnt[1], 256), 256, 0, e_off,
               (const u32 *)el.list[1], (const u32 *)el.cnt + 1, small, big, el.cnt + 6);
    const u32 gw = (host_cnt[1] + 3) / 4, ge = gw < 32 * c->n_cu ? gw : 32 * c->n_cu;
    if (narrow)
      CHP_LAUNCH(c, "econ_wreg", k_econ_wreg<u32>, ge, 256, 0, e_off, e_nsrc, pins, gamma, opins,
                 olen, onsrc, (const u32 *)small, (const u32 *)el.cnt + 6);
    else
      CHP_LAUNCH(c, "econ_wreg", k_econ_wreg<u64>, ge, 256, 0, e_off, e_nsrc, pins, gamma, opins,
                 olen, onsrc, (const u32 *)small, (const u32 *)el.cnt + 6);
    CHP_LAUNCH(c, "econ_lds", (k_econ_lds<256, LDS_CAP_U64>),
               host_cnt[1] > 8192 ? 8192 : host_cnt[1], 256, 0, e_off, e_nsrc, pins, gamma, opins,
               olen, onsrc, (const u32 *)big, (const u32 *)el.cnt + 7);
  }
  if (host_cnt[2])
    CHP_LAUNCH(c, "econ_global", (k_econ_global<256, LDS_CAP_U64>), grid_big, 256, 0, e_off,
               e_nsrc, pins, gamma, opins, olen, onsrc, (const u32 *)el.list[2],
               (const u32 *)el.cnt + 2, scratch, per_wg);
}

void launch_pins_compact(chp_ctx *c, u32 E, const i64 *src_off, const u32 *src,
                         const i64 *dst_off, u32 *dst) {
  if (E == 0) return;
  CHP_LAUNCH(c, "pins_compact", k_pins_compact, waves_grid(E), 256, 0, E, src_off, src, dst_off,
             dst);
}
