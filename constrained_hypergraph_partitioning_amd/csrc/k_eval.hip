// Partition evaluation ("Hypergraph Partitioning on GPU with Distinct
// Incident Hyperedges and Size Constraints": connectivity, Eq. 1; cut-net,
// Eq. 16; the per-partition size and distinct-inbound counts of Sec. II-B).
//
// Per hyperedge the distinct partitions of its pins: lambda(e) is their
// number, and each one holding a destination pin is a partition that e
// enters (e counts once towards that partition's inbound set).  Hyperedges of
// at most 64 pins and those above 512 sort 64-bit keys (rho << 1 | is_source:
// a group of equal rho whose first key is a destination is entered), those
// of at most 8 in one lane's registers; the others insert rho into a hash
// table per wave, destinations first.
#include "dev.h"
#include "kernels.h"

namespace {

__global__ void k_eval_nodes(u32 N, const u32 *rho, u32 k, const u32 *n_size, u64 *part_size,
                             u32 *part_cnt, u32 *flags) {
  u32 n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= N) return;
  u32 p = rho[n];
  if (p >= k) {
    atomicOr(flags, FLAG_EINVAL);
    return;
  }
  atomicAdd((unsigned long long *)&part_size[p], (unsigned long long)n_size[n]);
  atomicAdd(&part_cnt[p], 1u);
}

__device__ __forceinline__ u64 eval_key(const u32 *rho, u32 k, u32 pin, bool src, u32 *flags) {
  u32 p = rho[pin];
  if (p >= k) {
    atomicOr(flags, FLAG_EINVAL);
    p = 0;
  }
  return ((u64)p << 1) | (src ? 1u : 0u);
}


__device__ __forceinline__ void flush_sums(u64 conn, u64 cut, u64 lam, u64 *summary) {
  if (conn) atomicAdd((unsigned long long *)&summary[0], (unsigned long long)conn);
  if (cut) atomicAdd((unsigned long long *)&summary[1], (unsigned long long)cut);
  if (lam) atomicAdd((unsigned long long *)&summary[7], (unsigned long long)lam);
}

// Hyperedges of at most 64 pins.  A wave takes 64 consecutive entries of the
// list, a lane each: a hyperedge of at most 8 pins (most nets of a netlist)
// is done by its own lane, its keys sorted in registers by a 19-comparator
// network; the others one after the other by the whole wave (a key per lane,
// a wave bitonic sort).  The sums are gathered per workgroup and flushed by
// one thread (three atomics per workgroup: the grid is a few workgroups per
// CU, so the shared summary words see few atomics).
__global__ __launch_bounds__(256) void k_eval_wave(const i64 *e_off, const u32 *e_nsrc,
                                                   const u32 *pins, const u32 *e_w,
                                                   const u32 *rho, u32 k, u32 *part_inb,
                                                   u64 *summary, const u32 *list, const u32 *cnt,
                                                   u32 *flags) {
  __shared__ u64 s_sum[3][256 / WAVE];
  const u32 total = *cnt;
  const u32 nwaves = gridDim.x * (blockDim.x / WAVE);
  const u32 l = lane_id();
  u64 conn = 0, cut = 0, lams = 0;
  for (u32 w0 = (blockIdx.x * (blockDim.x / WAVE) + wave_id()) * WAVE; w0 < total;
       w0 += nwaves * WAVE) {
    const u32 w = w0 + l;
    u32 e = 0, len = 0, ns = 0;
    i64 a = 0;
    if (w < total) {
      e = list[w];
      a = e_off[e];
      len = (u32)(e_off[e + 1] - a);
      ns = e_nsrc[e];
    }
    const bool tiny = w < total && len <= 8;
    if (tiny) {
      u64 key[8];
#pragma unroll
      for (u32 j = 0; j < 8; ++j)
        key[j] = j < len ? eval_key(rho, k, pins[a + j], j < ns, flags) : ~0ull;
      cswap(key[0], key[2]), cswap(key[1], key[3]), cswap(key[4], key[6]), cswap(key[5], key[7]);
      cswap(key[0], key[4]), cswap(key[1], key[5]), cswap(key[2], key[6]), cswap(key[3], key[7]);
      cswap(key[0], key[1]), cswap(key[2], key[3]), cswap(key[4], key[5]), cswap(key[6], key[7]);
      cswap(key[2], key[4]), cswap(key[3], key[5]);
      cswap(key[1], key[4]), cswap(key[3], key[6]);
      cswap(key[1], key[2]), cswap(key[3], key[4]), cswap(key[5], key[6]);
      u64 lam = 0;
#pragma unroll
      for (u32 j = 0; j < 8; ++j) {
        if (j < len && (j == 0 || (key[j - 1] >> 1) != (key[j] >> 1))) {
          ++lam;
          if (!(key[j] & 1)) atomicAdd(&part_inb[key[j] >> 1], 1u);
        }
      }
      const u64 we = e_w[e];
      conn += we * (lam - 1);
      cut += lam > 1 ? we : 0;
      lams += lam;
    }
    u64 rest = __ballot(w < total && !tiny);
    while (rest) {
      const u32 i = (u32)__builtin_ctzll(rest);
      rest &= rest - 1;
      const u32 ei = (u32)__builtin_amdgcn_readlane((int)e, (int)i);
      const u32 li = (u32)__builtin_amdgcn_readlane((int)len, (int)i);
      const u32 nsi = (u32)__builtin_amdgcn_readlane((int)ns, (int)i);
      const i64 ai = (i64)((u64)(u32)__builtin_amdgcn_readlane((int)(u32)((u64)a >> 32), (int)i)
                               << 32 |
                           (u32)__builtin_amdgcn_readlane((int)(u32)(u64)a, (int)i));
      u64 key = ~0ull;
      if (l < li) key = eval_key(rho, k, pins[ai + l], l < nsi, flags);
      key = wave_sort64(key);
      const u64 prev = __shfl_up(key, 1, WAVE);
      const bool first = l < li && (l == 0 || (prev >> 1) != (key >> 1));
      if (first && !(key & 1)) atomicAdd(&part_inb[key >> 1], 1u);
      const u64 lam = (u64)__popcll(__ballot(first));
      if (l == 0) {
        const u64 we = e_w[ei];
        conn += we * (lam - 1);
        cut += lam > 1 ? we : 0;
        lams += lam;
      }
    }
  }
  conn = wave_sum(conn);
  cut = wave_sum(cut);
  lams = wave_sum(lams);
  if (l == 0) {
    s_sum[0][wave_id()] = conn;
    s_sum[1][wave_id()] = cut;
    s_sum[2][wave_id()] = lams;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 256 / WAVE; ++w) {
      conn += s_sum[0][w];
      cut += s_sum[1][w];
      lams += s_sum[2][w];
    }
    flush_sums(conn, cut, lams, summary);
  }
}

// lambda and inbound marks from sorted keys s[0,m); returns lambda (all threads)
template <int BLOCK>
__device__ u32 eval_groups(const u64 *s, u32 m, u32 *part_inb, u32 *s_red) {
  u32 lam = 0;
  for (u32 c0 = 0; c0 < m; c0 += BLOCK) {
    u32 i = c0 + threadIdx.x;
    bool f = false;
    if (i < m) {
      u64 key = s[i];
      f = i == 0 || (s[i - 1] >> 1) != (key >> 1);
      if (f && !(key & 1)) atomicAdd(&part_inb[key >> 1], 1u);
    }
    lam += wg_sum<BLOCK>((u32)f, s_red);
  }
  return lam;
}

// Hyperedges of 65 .. EH_MAX pins, a wave each, without a sort: the
// partitions of the pins go into the wave's own LDS table (open addressing,
// key p + 1, 0 = empty, at most half full).  The destinations go in first, so
// every partition holding a destination pin is claimed by one (the claiming
// lane counts e towards that partition's inbound set), then the sources;
// lambda(e) is the number of claims.  Each lane gathers all its pins' rho
// before its first insert.
//
// A workgroup takes a chunk of consecutive hyperedges (by id, not from the
// class list, whose order is that of the workgroups that filled it; at most
// EV_CHUNK, fewer where the graph would not fill the GPU), its waves the
// ones of this class among them.  Its inbound counts for the
// partitions in a window of EV_IDS ids (centred on the median of the
// partitions of 64 destinations sampled from the chunk) gather in LDS
// (16-bit counts, two a word: a chunk adds at most EV_CHUNK to a partition)
// and are flushed with one atomic per touched partition; where hyperedges
// are local and the partition ids follow the node ids (as after a
// contraction, whose coarse ids rise with the members' ids) most of them fall
// in it.  The others count in global memory directly.
constexpr u32 EH_MAX = 512;           // pins of the largest hyperedge hashed per wave
constexpr u32 EH_SLOTS = 2 * EH_MAX;  // table slots per wave
constexpr u32 EH_PER = EH_MAX / WAVE;
constexpr u32 EV_BLOCK = 1024;  // threads per workgroup
constexpr u32 EV_CHUNK = 2048;  // most hyperedges in a chunk
constexpr u32 EV_IDS = 45056;   // partition ids of the LDS window

__global__ __launch_bounds__(EV_BLOCK) void k_eval_hash(u32 E, u32 epc, const i64 *e_off,
                                                        const u32 *e_nsrc, const u32 *pins,
                                                        const u32 *e_w, const u32 *rho, u32 k,
                                                        u32 *part_inb, u64 *summary,
                                                        u32 *flags) {
  __shared__ u32 tab[EV_BLOCK / WAVE][EH_SLOTS];
  __shared__ u32 h[EV_IDS / 2];
  __shared__ u64 s_sum[3][EV_BLOCK / WAVE];
  __shared__ u32 s_wb;
  const u32 nch = (E + epc - 1) / epc;
  const u32 l = lane_id();
  u32 *t = tab[wave_id()];
  for (u32 i = l; i < EH_SLOTS; i += WAVE) t[i] = 0;
  u64 conn = 0, cut = 0, lams = 0;
  for (u32 ch = blockIdx.x; ch < nch; ch += gridDim.x) {
    const u32 w0 = ch * epc, w1 = E - w0 < epc ? E : w0 + epc;
    for (u32 i = threadIdx.x; i < EV_IDS / 2; i += EV_BLOCK) h[i] = 0;
    if (wave_id() == 0) {
      // the window: the partition of the middle destination (of a sorted
      // run: the smallest ones are the far ones where the others are local;
      // the first pin where all are sources) of 64 hyperedges spread over
      // the chunk
      const u32 e = w0 + (u32)((u64)(w1 - w0) * l / WAVE);
      const i64 ea = e_off[e];
      const u32 elen = (u32)(e_off[e + 1] - ea), ens = e_nsrc[e];
      u32 p = elen ? rho[pins[ea + (ens < elen ? ens + (elen - ens) / 2 : 0)]] : 0u;
      p = p < k ? p : 0;
      const u64 key = wave_sort64((u64)p);
      const u32 med = (u32)__shfl(key, WAVE / 2, WAVE);
      if (l == 0) s_wb = med > EV_IDS / 2 ? med - EV_IDS / 2 : 0u;
    }
    __syncthreads();
    const u32 wb = s_wb;
    // a wave screens 64 consecutive hyperedges at a time, a lane each, and
    // takes those of this class one after the other
    for (u32 eb = w0 + wave_id() * WAVE; eb < w1; eb += EV_BLOCK) {
      i64 al = 0;
      u32 lenl = 0, nsl = 0;
      if (eb + l < w1) {
        al = e_off[eb + l];
        lenl = (u32)(e_off[eb + l + 1] - al);
        nsl = e_nsrc[eb + l];
      }
      u64 todo = __ballot(eb + l < w1 && lenl > WAVE && lenl <= EH_MAX);
      while (todo) {
        const u32 li = (u32)__builtin_ctzll(todo);
        todo &= todo - 1;
        const u32 e = eb + li;
        const u32 ahi = (u32)__builtin_amdgcn_readlane((int)(u32)((u64)al >> 32), (int)li);
        const u32 alo = (u32)__builtin_amdgcn_readlane((int)(u32)(u64)al, (int)li);
        const i64 a = (i64)((u64)ahi << 32 | alo);
        const u32 len = (u32)__builtin_amdgcn_readlane((int)lenl, (int)li);
        const u32 ns = (u32)__builtin_amdgcn_readlane((int)nsl, (int)li);
        const u32 hs = next_pow2(2 * len);
        const u32 sh = 32 - (31 - __builtin_clz(hs));
        u32 p[EH_PER];
#pragma unroll
        for (u32 j = 0; j < EH_PER; ++j) {
          const u32 i = l + j * WAVE;
          p[j] = i < len ? pins[a + i] : 0;
        }
#pragma unroll
        for (u32 j = 0; j < EH_PER; ++j) {
          const u32 i = l + j * WAVE;
          if (i < len) {
            p[j] = rho[p[j]];
            if (p[j] >= k) {
              atomicOr(flags, FLAG_EINVAL);
              p[j] = 0;
            }
          }
        }
        u32 claims = 0;
#pragma unroll
        for (u32 pass = 0; pass < 2; ++pass) {
          // pass 0: destinations (pins ns .. len - 1); pass 1: sources
#pragma unroll
          for (u32 j = 0; j < EH_PER; ++j) {
            const u32 i = l + j * WAVE;
            if (i < len && (pass ? i < ns : i >= ns)) {
              const u32 key = p[j] + 1;
              u32 s = (p[j] * 0x9E3779B1u) >> sh;
              for (;;) {
                const u32 o = atomicCAS(&t[s], 0u, key);
                if (o == 0) {
                  ++claims;
                  if (!pass) {
                    const u32 r = p[j] - wb;
                    if (r < EV_IDS) atomicAdd(&h[r >> 1], 1u << ((r & 1) << 4));
                    else atomicAdd(&part_inb[p[j]], 1u);
                  }
                  break;
                }
                if (o == key) break;
                s = (s + 1) & (hs - 1);
              }
            }
          }
        }
        const u64 lam = wave_sum(claims);
        for (u32 i = l; i < hs; i += WAVE) t[i] = 0;
        if (l == 0) {
          const u64 we = e_w[e];
          conn += we * (lam - 1);
          cut += lam > 1 ? we : 0;
          lams += lam;
        }
      }
    }
    __syncthreads();
    for (u32 i = threadIdx.x; i < EV_IDS / 2; i += EV_BLOCK) {
      const u32 x = h[i];
      if (x & 0xFFFFu) atomicAdd(&part_inb[wb + 2 * i], x & 0xFFFFu);
      if (x >> 16) atomicAdd(&part_inb[wb + 2 * i + 1], x >> 16);
    }
    __syncthreads();
  }
  if (l == 0) {
    s_sum[0][wave_id()] = conn;
    s_sum[1][wave_id()] = cut;
    s_sum[2][wave_id()] = lams;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < EV_BLOCK / WAVE; ++w) {
      conn += s_sum[0][w];
      cut += s_sum[1][w];
      lams += s_sum[2][w];
    }
    flush_sums(conn, cut, lams, summary);
  }
}

// The hyperedges of EH_MAX + 1 .. CAP pins: a workgroup sort of the keys.
// The workgroup reads BLOCK entries of the list at a time and sorts the long
// ones among them, one after the other.
template <int BLOCK, int CAP>
__global__ __launch_bounds__(BLOCK) void k_eval_lds(const i64 *e_off, const u32 *e_nsrc,
                                                    const u32 *pins, const u32 *e_w,
                                                    const u32 *rho, u32 k, u32 *part_inb,
                                                    u64 *summary, const u32 *list, const u32 *cnt,
                                                    u32 *flags) {
  __shared__ u64 s[CAP];
  __shared__ u32 s_red[BLOCK / WAVE + 1];
  __shared__ u32 s_long[BLOCK];
  __shared__ u32 s_nlong;
  const u32 total = *cnt;
  u64 conn = 0, cut = 0, lams = 0;
  for (u32 base = blockIdx.x * BLOCK; base < total; base += gridDim.x * BLOCK) {
    if (threadIdx.x == 0) s_nlong = 0;
    __syncthreads();
    const u32 w = base + threadIdx.x;
    if (w < total) {
      const u32 e = list[w];
      if (e_off[e + 1] - e_off[e] > (i64)EH_MAX) s_long[atomicAdd(&s_nlong, 1u)] = e;
    }
    __syncthreads();
    const u32 nl = s_nlong;
    for (u32 j = 0; j < nl; ++j) {
      const u32 e = s_long[j];
      const i64 a = e_off[e];
      const u32 len = (u32)(e_off[e + 1] - a), ns = e_nsrc[e];
      const u32 p = next_pow2(len);
      for (u32 i = threadIdx.x; i < p; i += BLOCK)
        s[i] = i < len ? eval_key(rho, k, pins[a + i], i < ns, flags) : ~0ull;
      __syncthreads();
      lds_bitonic<BLOCK>(s, p);
      const u64 lam = eval_groups<BLOCK>(s, len, part_inb, s_red);
      const u64 we = e_w[e];
      conn += we * (lam - 1);
      cut += lam > 1 ? we : 0;
      lams += lam;
      __syncthreads();
    }
  }
  if (threadIdx.x == 0) flush_sums(conn, cut, lams, summary);
}

template <int BLOCK, int CAP>
__global__ __launch_bounds__(BLOCK) void k_eval_global(const i64 *e_off, const u32 *e_nsrc,
                                                       const u32 *pins, const u32 *e_w,
                                                       const u32 *rho, u32 k, u32 *part_inb,
                                                       u64 *summary, const u32 *list,
                                                       const u32 *cnt, u32 *flags, u64 *scratch,
                                                       u64 per_wg) {
  __shared__ u64 s[CAP];
  __shared__ u32 s_red[BLOCK / WAVE + 1];
  const u32 total = *cnt;
  u64 *A = scratch + (u64)blockIdx.x * per_wg;
  u64 *B = A + per_wg / 2;
  u64 conn = 0, cut = 0, lams = 0;
  for (u32 w = blockIdx.x; w < total; w += gridDim.x) {
    const u32 e = list[w];
    const i64 a = e_off[e];
    const u32 len = (u32)(e_off[e + 1] - a), ns = e_nsrc[e];
    for (u32 i = threadIdx.x; i < len; i += BLOCK)
      A[i] = eval_key(rho, k, pins[a + i], i < ns, flags);
    __syncthreads();
    u64 *res = wg_sort_global<BLOCK, CAP>(A, B, len, s);
    const u64 lam = eval_groups<BLOCK>(res, len, part_inb, s_red);
    const u64 we = e_w[e];
    conn += we * (lam - 1);
    cut += lam > 1 ? we : 0;
    lams += lam;
    __syncthreads();
  }
  if (threadIdx.x == 0) flush_sums(conn, cut, lams, summary);
}

// Violations, empty partitions and maxima, reduced per wave before the
// atomics on the shared summary words.
__global__ void k_eval_parts(u32 k, const u64 *part_size, const u32 *part_inb,
                             const u32 *part_cnt, u64 omega, u32 delta, u64 *summary) {
  const u32 p = blockIdx.x * blockDim.x + threadIdx.x;
  u64 s = 0;
  u32 in = 0, ov = 0, dv = 0, em = 0;
  if (p < k) {
    s = part_size[p];
    in = part_inb[p];
    ov = s > omega ? 1 : 0;
    dv = in > delta ? 1 : 0;
    em = part_cnt[p] == 0 ? 1 : 0;
  }
  const u64 bov = __ballot(ov), bdv = __ballot(dv), bem = __ballot(em);
#pragma unroll
  for (int d = WAVE / 2; d > 0; d >>= 1) {
    const u64 os = __shfl_xor(s, d, WAVE);
    const u32 oi = __shfl_xor(in, d, WAVE);
    s = os > s ? os : s;
    in = oi > in ? oi : in;
  }
  if (lane_id() != 0) return;
  if (bov) atomicAdd((unsigned long long *)&summary[2], (unsigned long long)__popcll(bov));
  if (bdv) atomicAdd((unsigned long long *)&summary[3], (unsigned long long)__popcll(bdv));
  if (bem) atomicAdd((unsigned long long *)&summary[4], (unsigned long long)__popcll(bem));
  atomicMax((unsigned long long *)&summary[5], (unsigned long long)s);
  atomicMax((unsigned long long *)&summary[6], (unsigned long long)in);
}


}  // namespace

void launch_eval_nodes(chp_ctx *c, u32 N, const u32 *rho, u32 k, const u32 *n_size,
                       u64 *part_size, u32 *part_cnt) {
  if (N == 0) return;
  CHP_LAUNCH(c, "eval_nodes", k_eval_nodes, grid_for(N, 256), 256, 0, N, rho, k, n_size,
             part_size, part_cnt, c->flags);
}

void launch_eval_edges(chp_ctx *c, const i64 *e_off, const u32 *e_nsrc, const u32 *pins,
                       const u32 *e_w, const u32 *rho, u32 k, u32 *part_inb, u64 *summary,
                       EdgeLists el, const u32 *host_cnt, u64 *scratch, u64 per_wg,
                       u32 grid_big) {
  if (host_cnt[0]) {
    const u32 gw = (host_cnt[0] + 4 * WAVE - 1) / (4 * WAVE);  // 64 entries a wave
    CHP_LAUNCH(c, "eval_wave", k_eval_wave, gw < 8 * c->n_cu ? gw : 8 * c->n_cu, 256, 0, e_off,
               e_nsrc, pins, e_w, rho, k, part_inb, summary, (const u32 *)el.list[0],
               (const u32 *)el.cnt + 0, c->flags);
  }
  if (host_cnt[1]) {
    // chunks of consecutive hyperedges, four per CU (from 64 to EV_CHUNK)
    const u32 E = host_cnt[0] + host_cnt[1] + host_cnt[2];
    const u32 per = E / (4 * c->n_cu);
    const u32 epc = per < 64 ? 64 : per > EV_CHUNK ? EV_CHUNK : per;
    CHP_LAUNCH(c, "eval_hash", k_eval_hash, (E + epc - 1) / epc, EV_BLOCK, 0, E, epc, e_off,
               e_nsrc, pins, e_w, rho, k, part_inb, summary, c->flags);
    const u32 gl = (host_cnt[1] + 255) / 256;
    CHP_LAUNCH(c, "eval_lds", (k_eval_lds<256, LDS_CAP_U64>), gl < 8192 ? gl : 8192, 256, 0,
               e_off, e_nsrc, pins, e_w, rho, k, part_inb, summary, (const u32 *)el.list[1],
               (const u32 *)el.cnt + 1, c->flags);
  }
  if (host_cnt[2])
    CHP_LAUNCH(c, "eval_global", (k_eval_global<256, LDS_CAP_U64>), grid_big, 256, 0, e_off,
               e_nsrc, pins, e_w, rho, k, part_inb, summary, (const u32 *)el.list[2],
               (const u32 *)el.cnt + 2, c->flags, scratch, per_wg);
}

void launch_eval_parts(chp_ctx *c, u32 k, const u64 *part_size, const u32 *part_inb,
                       const u32 *part_cnt, u64 omega, u32 delta, u64 *summary) {
  if (k == 0) return;
  CHP_LAUNCH(c, "eval_parts", k_eval_parts, grid_for(k, 256), 256, 0, k, part_size, part_inb,
             part_cnt, omega, delta, summary);
}
