// Canonical hyperedge CSR, incidence CSR and unique neighbourhoods.
//
// Data layout follows the compressed-sparse h-graph of "Hypergraph
// Partitioning on GPU with Distinct Incident Hyperedges and Size Constraints"
// (Sec. IV-B, Fig. 2): one segment per hyperedge with sources first, one
// segment per node with inbound hyperedges first.  Neighbourhoods N(n)
// (Sec. II-A, materialised as in Sec. V-B) are the sorted union of the pins of
// n's incident hyperedges without n.
#include "dev.h"
#include "kernels.h"

namespace {

// ---------------------------------------------------------------------------
// validation of offsets, weights and sizes (before any pin is read)
__global__ void k_check_edges(u32 N, u32 E, u64 P, const i64 *e_off, const u32 *e_nsrc,
                              const u32 *e_w, const u32 *n_size, u32 *flags) {
  u64 i = (u64)blockIdx.x * blockDim.x + threadIdx.x;
  u32 f = 0;
  if (i < E) {
    i64 a = e_off[i], b = e_off[i + 1];
    if (i == 0 && a != 0) f |= FLAG_EINVAL;
    if (b <= a || a < 0 || (u64)b > P) f |= FLAG_EINVAL;
    if (i + 1 == E && (u64)b != P) f |= FLAG_EINVAL;
    if (b > a && (i64)e_nsrc[i] > b - a) f |= FLAG_EINVAL;
    u32 w = e_w[i];
    if (w == 0) f |= FLAG_EINVAL;
    if (w >= (1u << 24)) f |= FLAG_EOVERFLOW;
  }
  if (E == 0 && i == 0 && (e_off[0] != 0 || P != 0)) f |= FLAG_EINVAL;
  if (i < N && n_size[i] == 0) f |= FLAG_EINVAL;
  if (f) atomicOr(flags, f);
}

// Queue a run for sorting (runs shorter than 2 need none).  Every lane of
// the wave must call it; appends are aggregated per wave.
__device__ __forceinline__ void push_run(RunLists rl, i64 start, u32 len) {
  const int c = len < 2 ? 3 : (len <= 64 ? 0 : (len <= LDS_CAP_U32 ? 1 : 2));
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const u32 slot = wave_append(&rl.cnt[k], c == k);
    if (c == k) {
      rl.start[k][slot] = start;
      rl.len[k][slot] = len;
    }
  }
  if (c == 2) atomicMax(&rl.cnt[3], len);
}

// One wave per hyperedge: copy pins, range check, detect unsorted runs.  A
// hyperedge whose runs are strictly ascending is also checked for src/dst
// overlap here; the others are queued for sorting and checked afterwards.
__global__ __launch_bounds__(256) void k_edges_canon(u32 N, u32 E, const i64 *e_off,
                                                     const u32 *e_nsrc, const u32 *pins_in,
                                                     u32 *pins_out, u32 *bad_edges, RunLists rl,
                                                     u32 *flags) {
  const u32 nwaves = gridDim.x * (blockDim.x / WAVE);
  const u32 l = lane_id();
  for (u32 e = blockIdx.x * (blockDim.x / WAVE) + wave_id(); e < E; e += nwaves) {
    i64 a = e_off[e], b = e_off[e + 1];
    u32 ns = e_nsrc[e];
    u32 len = (u32)(b - a);
    bool unsorted = false, badpin = false;
    for (u32 i = l; i < len; i += WAVE) {
      u32 v = pins_in[a + i];
      pins_out[a + i] = v;
      if (v >= N) badpin = true;
      if (i != 0 && i != ns && pins_in[a + i - 1] >= v) unsorted = true;
    }
    badpin = __any(badpin);
    unsorted = __any(unsorted);
    if (badpin) {
      if (l == 0) atomicOr(flags, FLAG_EINVAL);
      continue;
    }
    if (unsorted) {
      if (l == 0) {
        u32 slot = atomicAdd(&rl.cnt[4], 1u);
        bad_edges[slot] = e;
        push_run(rl, a, ns);
        push_run(rl, a + ns, len - ns);
      }
      continue;
    }
    bool overlap = false;
    for (u32 i = l; i < ns; i += WAVE) {
      u32 v = pins_in[a + i];
      i64 p = lower_bound_i(pins_in, a + ns, b, v);
      if (p < b && pins_in[p] == v) overlap = true;
    }
    if (__any(overlap) && l == 0) atomicOr(flags, FLAG_EINVAL);
  }
}

// Re-check queued hyperedges after sorting: duplicates and src/dst overlap.
__global__ __launch_bounds__(256) void k_edges_check(const i64 *e_off, const u32 *e_nsrc,
                                                     const u32 *pins, const u32 *list, u32 count,
                                                     u32 *flags) {
  const u32 nwaves = gridDim.x * (blockDim.x / WAVE);
  const u32 l = lane_id();
  for (u32 w = blockIdx.x * (blockDim.x / WAVE) + wave_id(); w < count; w += nwaves) {
    u32 e = list[w];
    i64 a = e_off[e], b = e_off[e + 1];
    u32 ns = e_nsrc[e];
    u32 len = (u32)(b - a);
    bool bad = false;
    for (u32 i = l; i < len; i += WAVE) {
      u32 v = pins[a + i];
      if (i != 0 && i != ns && pins[a + i - 1] == v) bad = true;
      if (i < ns) {
        i64 p = lower_bound_i(pins, a + ns, b, v);
        if (p < b && pins[p] == v) bad = true;
      }
    }
    if (__any(bad) && l == 0) atomicOr(flags, FLAG_EINVAL);
  }
}

// ---------------------------------------------------------------------------
// in-place run sorting, three length classes

__global__ __launch_bounds__(256) void k_runs_wave(u32 *data, const i64 *start, const u32 *len,
                                                   const u32 *cnt) {
  const u32 n = *cnt;
  const u32 nwaves = gridDim.x * (blockDim.x / WAVE);
  const u32 l = lane_id();
  for (u32 r = blockIdx.x * (blockDim.x / WAVE) + wave_id(); r < n; r += nwaves) {
    i64 s = start[r];
    u32 m = len[r];
    u32 v = l < m ? data[s + l] : NONE32;
    v = wave_sort64(v);
    if (l < m) data[s + l] = v;
  }
}

// Runs of 65 .. RUN_W ids: a wave each, sorted in registers (4, 8 or 16
// ids a lane, by the run's length).
constexpr u32 RUN_W = 1024;
template <int PER>
__device__ __forceinline__ void sort_run_regs(u32 *data, i64 s, u32 m) {
  const u32 l = lane_id();
  u32 v[PER];
#pragma unroll
  for (u32 q = 0; q < (u32)PER; ++q) v[q] = q * WAVE + l < m ? data[s + q * WAVE + l] : NONE32;
  wave_sort_regs<u32, PER>(v);
#pragma unroll
  for (u32 q = 0; q < (u32)PER; ++q)
    if (PER * l + q < m) data[s + PER * l + q] = v[q];
}

__global__ __launch_bounds__(256) void k_runs_wreg(u32 *data, const i64 *start, const u32 *len,
                                                   const u32 *cnt) {
  const u32 n = *cnt;
  const u32 nwaves = gridDim.x * (blockDim.x / WAVE);
  for (u32 r = blockIdx.x * (blockDim.x / WAVE) + wave_id(); r < n; r += nwaves) {
    const u32 m = len[r];
    if (m > RUN_W) continue;  // (the workgroup sort's)
    const i64 s = start[r];
    if (m <= 4 * WAVE) sort_run_regs<4>(data, s, m);
    else if (m <= 8 * WAVE) sort_run_regs<8>(data, s, m);
    else sort_run_regs<16>(data, s, m);
  }
}

// Runs of RUN_W + 1 .. CAP ids: a workgroup bitonic sort in LDS.  The
// workgroup reads BLOCK entries of the list at a time and sorts the long ones
// among them, one after the other.
template <int BLOCK, int CAP>
__global__ __launch_bounds__(BLOCK) void k_runs_lds(u32 *data, const i64 *start, const u32 *len,
                                                    const u32 *cnt) {
  __shared__ u32 s[CAP];
  __shared__ u32 s_long[BLOCK];
  __shared__ u32 s_nlong;
  const u32 n = *cnt;
  for (u32 base = blockIdx.x * BLOCK; base < n; base += gridDim.x * BLOCK) {
    if (threadIdx.x == 0) s_nlong = 0;
    __syncthreads();
    const u32 w = base + threadIdx.x;
    if (w < n && len[w] > RUN_W) s_long[atomicAdd(&s_nlong, 1u)] = w;
    __syncthreads();
    const u32 nl = s_nlong;
    for (u32 j = 0; j < nl; ++j) {
      const u32 r = s_long[j];
      const i64 st = start[r];
      const u32 m = len[r];
      const u32 p = next_pow2(m);
      for (u32 i = threadIdx.x; i < p; i += BLOCK) s[i] = i < m ? data[st + i] : NONE32;
      __syncthreads();
      lds_bitonic<BLOCK>(s, p);
      for (u32 i = threadIdx.x; i < m; i += BLOCK) data[st + i] = s[i];
      __syncthreads();
    }
  }
}

template <int BLOCK, int CAP>
__global__ __launch_bounds__(BLOCK) void k_runs_global(u32 *data, const i64 *start,
                                                       const u32 *len, const u32 *cnt,
                                                       u32 *scratch, u64 per_wg) {
  __shared__ u32 s[CAP];
  const u32 n = *cnt;
  u32 *tmp = scratch + (u64)blockIdx.x * per_wg;
  for (u32 r = blockIdx.x; r < n; r += gridDim.x) {
    i64 st = start[r];
    u32 m = len[r];
    u32 *res = wg_sort_global<BLOCK, CAP>(data + st, tmp, (u64)m, s);
    if (res != data + st)
      for (u32 i = threadIdx.x; i < m; i += BLOCK) data[st + i] = res[i];
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// incidence: degrees, feasibility, scatter, per-node runs
// Degrees and the scatter take the hyperedges in chunks of epc consecutive
// ones (at most DW_EDGES, fewer where the graph would not fill the GPU), a
// workgroup of DW_BLOCK threads each (a wave per hyperedge, the lanes over
// its pins).  A destination whose id falls in the chunk's window of DW_IDS
// ids counts in LDS (16-bit counts, two a word); where hyperedges are local
// to their sources (nodes of a ring, a block, a grid) most do, and a chunk
// then costs one global atomic per id of the window it touched instead of
// one per pin.  The window is centred on the median of 64 pins sampled
// evenly from the chunk.  A chunk adds at most epc <= DW_EDGES to an id's
// count (an id is a destination of a valid hyperedge at most once).
// Sources, and destinations outside the window, count in global memory
// directly.
constexpr u32 DW_EDGES = 2048, DW_IDS = 65536, DW_BLOCK = 1024;

// The low end of the chunk's window into *s_wb (wave 0; the caller waits).
__device__ __forceinline__ void chunk_window(const u32 *pins, i64 a0, i64 a1, u32 *s_wb) {
  if (wave_id() != 0) return;
  const u32 l = lane_id();
  const u64 span = (u64)(a1 - a0);
  u64 key = ~0ull;
  if (span) key = pins[a0 + (i64)(span * l / WAVE)];
  key = wave_sort64(key);
  const u32 med = (u32)__shfl(key, WAVE / 2, WAVE);
  if (l == 0) *s_wb = span == 0 ? 0u : (med > DW_IDS / 2 ? med - DW_IDS / 2 : 0u);
}

__global__ __launch_bounds__(DW_BLOCK) void k_degrees(u32 E, u32 epc, const i64 *e_off,
                                                      const u32 *e_nsrc, const u32 *pins,
                                                      u32 *indeg, u32 *outdeg) {
  __shared__ u32 h[DW_IDS / 2];
  __shared__ u32 s_wb;
  const u32 nch = (E + epc - 1) / epc;
  const u32 l = lane_id();
  for (u32 ch = blockIdx.x; ch < nch; ch += gridDim.x) {
    const u32 e0 = ch * epc, e1 = E - e0 < epc ? E : e0 + epc;
    for (u32 i = threadIdx.x; i < DW_IDS / 2; i += DW_BLOCK) h[i] = 0;
    chunk_window(pins, e_off[e0], e_off[e1], &s_wb);
    __syncthreads();
    const u32 wb = s_wb;
    for (u32 e = e0 + wave_id(); e < e1; e += DW_BLOCK / WAVE) {
      const i64 a = e_off[e], b = e_off[e + 1];
      const u32 ns = e_nsrc[e];
      for (u32 i = l; i < (u32)(b - a); i += WAVE) {
        const u32 v = pins[a + i];
        const u32 r = v - wb;
        if (i < ns) atomicAdd(&outdeg[v], 1u);
        else if (r < DW_IDS) atomicAdd(&h[r >> 1], 1u << ((r & 1) << 4));
        else atomicAdd(&indeg[v], 1u);
      }
    }
    __syncthreads();
    for (u32 i = threadIdx.x; i < DW_IDS / 2; i += DW_BLOCK) {
      const u32 x = h[i];
      if (x & 0xFFFFu) atomicAdd(&indeg[wb + 2 * i], x & 0xFFFFu);
      if (x >> 16) atomicAdd(&indeg[wb + 2 * i + 1], x >> 16);
    }
    __syncthreads();
  }
}

__global__ void k_node_feas(u32 N, const u32 *indeg, const u32 *outdeg, const u32 *n_size,
                            u64 omega, u32 delta, u32 *deg, u32 *n_nin, u32 *flags) {
  u32 n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= N) return;
  u32 di = indeg[n], dout = outdeg[n];
  deg[n] = di + dout;
  n_nin[n] = di;
  if ((u64)n_size[n] > omega || di > delta) atomicOr(flags, FLAG_EINFEASIBLE);
}

// The scatter in two passes over a chunk: the destinations in the window
// are counted in LDS; then each id of the window with a count reserves its
// places in one atomic on its cursor and the LDS word takes the first one,
// which the second pass hands out (an LDS atomic per pin).  An id whose
// in-degree may not fit 16 bits (n_nin >= 0xFFFF) is marked 0xFFFF and its
// pins take the global cursor one by one, as outside the window.
__global__ __launch_bounds__(DW_BLOCK) void k_scatter(u32 E, u32 epc, const i64 *e_off,
                                                      const u32 *e_nsrc, const u32 *pins,
                                                      const i64 *n_off, const u32 *n_nin,
                                                      u32 *cur_in, u32 *cur_out, u32 *n_inc) {
  __shared__ u32 h[DW_IDS / 2];
  __shared__ u32 s_wb;
  const u32 nch = (E + epc - 1) / epc;
  const u32 l = lane_id();
  for (u32 ch = blockIdx.x; ch < nch; ch += gridDim.x) {
    const u32 e0 = ch * epc, e1 = E - e0 < epc ? E : e0 + epc;
    for (u32 i = threadIdx.x; i < DW_IDS / 2; i += DW_BLOCK) h[i] = 0;
    chunk_window(pins, e_off[e0], e_off[e1], &s_wb);
    __syncthreads();
    const u32 wb = s_wb;
    for (u32 e = e0 + wave_id(); e < e1; e += DW_BLOCK / WAVE) {
      const i64 a = e_off[e], b = e_off[e + 1];
      const u32 ns = e_nsrc[e];
      for (u32 i = ns + l; i < (u32)(b - a); i += WAVE) {
        const u32 r = pins[a + i] - wb;
        if (r < DW_IDS) atomicAdd(&h[r >> 1], 1u << ((r & 1) << 4));
      }
    }
    __syncthreads();
    for (u32 i = threadIdx.x; i < DW_IDS / 2; i += DW_BLOCK) {
      const u32 x = h[i];
      if (!x) continue;
      u32 y = 0;
#pragma unroll
      for (u32 j = 0; j < 2; ++j) {
        const u32 cnt = (x >> (16 * j)) & 0xFFFFu;
        if (!cnt) continue;
        const u32 v = wb + 2 * i + j;
        const u32 first = n_nin[v] < 0xFFFFu ? atomicAdd(&cur_in[v], cnt) : 0xFFFFu;
        y |= first << (16 * j);
      }
      h[i] = y;
    }
    __syncthreads();
    for (u32 e = e0 + wave_id(); e < e1; e += DW_BLOCK / WAVE) {
      const i64 a = e_off[e], b = e_off[e + 1];
      const u32 ns = e_nsrc[e];
      for (u32 i = l; i < (u32)(b - a); i += WAVE) {
        const u32 v = pins[a + i];
        const u32 r = v - wb;
        i64 pos;
        if (i < ns) {
          pos = n_off[v] + n_nin[v] + atomicAdd(&cur_out[v], 1u);
        } else {
          const u32 sh = (r & 1) << 4;
          if (r < DW_IDS && ((h[r >> 1] >> sh) & 0xFFFFu) != 0xFFFFu)
            pos = n_off[v] + ((atomicAdd(&h[r >> 1], 1u << sh) >> sh) & 0xFFFFu);
          else
            pos = n_off[v] + atomicAdd(&cur_in[v], 1u);
        }
        n_inc[pos] = e;
      }
    }
    __syncthreads();
  }
}

__global__ void k_node_runs(u32 N, const i64 *n_off, const u32 *n_nin, RunLists rl) {
  const u32 n = blockIdx.x * blockDim.x + threadIdx.x;
  i64 a = 0, b = 0;
  u32 ni = 0;
  if (n < N) {
    a = n_off[n];
    b = n_off[n + 1];
    ni = n_nin[n];
  }
  push_run(rl, a, ni);
  push_run(rl, a + ni, (u32)(b - a - ni));
}

// ---------------------------------------------------------------------------
// neighbourhoods: W_n = sum_{e in I(n)} |e| decides the class; the oversize
// bound of |N(n)| is W_n - |I(n)| (n is a pin of each of its hyperedges).
// Nodes lo .. lo + N - 1; a node marked in skip gets bound 0 and no class.
// Classes: one wave (W_n <= 64); a workgroup sort (W_n <= NB_SORT_CAP and
// the pins' id span needs more bitmap words than there are pins: the bitmap
// would mostly scan empty words); the LDS bitmap (the rest).  The span comes
// from the ends of each hyperedge's two sorted runs.
constexpr u32 NB_SORT_CAP = 1024;
__global__ __launch_bounds__(256) void k_nb_classify(u32 lo, u32 N, const i64 *e_off,
                                                     const u32 *e_nsrc, const u32 *pins,
                                                     const i64 *n_off, const u32 *n_inc,
                                                     u32 *bound, NbLists nl,
                                                     const uint8_t *skip) {
  __shared__ u32 s_app[3 * (256 / WAVE) + 3];
  const u32 t = blockIdx.x * blockDim.x + threadIdx.x;
  const u32 n = lo + t;
  u64 w = 0, bnd = 0;
  if (t < N && skip && skip[n]) {
    bound[n] = 0;  // rated without a list: none is built
  } else if (t < N) {
    const i64 a = n_off[n], b = n_off[n + 1];
    for (i64 j = a; j < b; ++j) {
      const u32 e = n_inc[j];
      w += (u64)(e_off[e + 1] - e_off[e]);
    }
    bnd = w - (u64)(b - a);
    if (w > 0xFFFFFFFFull) {  // per-node work must fit 32 bits
      atomicOr(nl.cnt + 7, 1u);
      bnd = 0;
    }
    bound[n] = (u32)bnd;
  }
  bool sparse = false;
  if (bnd != 0 && w > 64 && w <= NB_SORT_CAP) {
    const i64 a = n_off[n], b = n_off[n + 1];
    u32 mn = NONE32, mx = 0;
    for (i64 j = a; j < b; ++j) {
      const u32 e = n_inc[j];
      const i64 s0 = e_off[e], s1 = e_off[e + 1], d0 = s0 + e_nsrc[e];
      if (d0 > s0) {  // source run
        mn = pins[s0] < mn ? pins[s0] : mn;
        mx = pins[d0 - 1] > mx ? pins[d0 - 1] : mx;
      }
      if (s1 > d0) {  // destination run
        mn = pins[d0] < mn ? pins[d0] : mn;
        mx = pins[s1 - 1] > mx ? pins[s1 - 1] : mx;
      }
    }
    sparse = (u64)(mx - mn) / 32 + 1 > w;
  }
  // isolated nodes (bnd 0) have an empty N(n) and join no class
  const int c = bnd == 0 ? 3 : (w <= 64 ? 0 : sparse ? 2 : 1);
  const u32 slot = block_append<256, 3>(nl.cnt, c, s_app);
  if (c < 3) nl.list[c][slot] = n;
}

// wave per node, W_n <= 64: gather into lanes, sort, unique, drop n
__global__ __launch_bounds__(256) void k_nb_wave(const i64 *e_off, const u32 *pins,
                                                 const i64 *n_off, const u32 *n_inc,
                                                 const i64 *ooff, u32 *obuf, u32 *count,
                                                 const u32 *list, const u32 *cnt) {
  const u32 total = *cnt;
  const u32 nwaves = gridDim.x * (blockDim.x / WAVE);
  const u32 l = lane_id();
  for (u32 w = blockIdx.x * (blockDim.x / WAVE) + wave_id(); w < total; w += nwaves) {
    u32 n = list[w];
    i64 a = n_off[n], b = n_off[n + 1];
    u32 deg = (u32)(b - a);
    // lane j < deg holds hyperedge j's segment
    i64 es = 0;
    u32 elen = 0;
    if (l < deg) {
      u32 e = n_inc[a + l];
      es = e_off[e];
      elen = (u32)(e_off[e + 1] - es);
    }
    u32 pre = wave_incl_scan(elen) - elen;
    u32 v = NONE32;
    for (u32 j = 0; j < deg; ++j) {
      u32 pj = __shfl(pre, j, WAVE);
      u32 lj = __shfl(elen, j, WAVE);
      i64 sj = __shfl(es, j, WAVE);
      if (l >= pj && l < pj + lj) v = pins[sj + (l - pj)];
    }
    v = wave_sort64(v);
    u32 prev = __shfl_up(v, 1, WAVE);
    bool keep = v != NONE32 && v != n && (l == 0 || prev != v);
    u64 mask = __ballot(keep);
    u32 pos = __popcll(mask & ((1ull << l) - 1));
    if (keep) obuf[ooff[n] + pos] = v;
    if (l == 0) count[n] = (u32)__popcll(mask);
  }
}

// A workgroup per node of the sort class: the pins of I(n) (at most CAP) are
// gathered into LDS hyperedge by hyperedge (a scan lays the segments end to
// end), sorted (bitonic) and written without repeats and without n.
template <int BLOCK, int CAP>
__global__ __launch_bounds__(BLOCK) void k_nb_sort(const i64 *e_off, const u32 *pins,
                                                   const i64 *n_off, const u32 *n_inc,
                                                   const i64 *ooff, u32 *obuf, u32 *count,
                                                   const u32 *list, const u32 *cnt) {
  __shared__ u32 s[CAP];
  __shared__ i64 st[BLOCK];
  __shared__ u32 pre[BLOCK + 1];
  __shared__ u32 s_red[BLOCK / WAVE + 1];
  const u32 total = *cnt;
  for (u32 w = blockIdx.x; w < total; w += gridDim.x) {
    const u32 n = list[w];
    const i64 a = n_off[n], b = n_off[n + 1];
    u32 fill = 0;
    for (i64 c0 = a; c0 < b; c0 += BLOCK) {
      const u32 ne = (u32)((b - c0) < BLOCK ? (b - c0) : BLOCK);
      u32 len = 0;
      if (threadIdx.x < ne) {
        const u32 e = n_inc[c0 + threadIdx.x];
        const i64 e0 = e_off[e];
        len = (u32)(e_off[e + 1] - e0);
        st[threadIdx.x] = e0;
      }
      u32 tot;
      const u32 off = wg_excl_scan<BLOCK>(len, s_red, &tot);
      if (threadIdx.x < ne) pre[threadIdx.x] = off;
      if (threadIdx.x == 0) pre[ne] = tot;
      __syncthreads();
      for (u32 i = threadIdx.x; i < tot; i += BLOCK) {
        const u32 r = run_of(pre, ne + 1, i);
        s[fill + i] = pins[st[r] + (i - pre[r])];
      }
      fill += tot;
      __syncthreads();
    }
    const u32 p = next_pow2(fill);
    for (u32 i = fill + threadIdx.x; i < p; i += BLOCK) s[i] = NONE32;
    __syncthreads();
    lds_bitonic<BLOCK>(s, p);
    const u32 k = unique_out<BLOCK>(s, fill, n, obuf + ooff[n], s_red);
    if (threadIdx.x == 0) count[n] = k;
    __syncthreads();
  }
}

// copy each node's unique list from the oversize buffer to its final place
__global__ __launch_bounds__(256) void k_nb_compact(u32 N, const i64 *ooff, const u32 *obuf,
                                                    const i64 *nb_off, u32 *nb) {
  const u32 nwaves = gridDim.x * (blockDim.x / WAVE);
  const u32 l = lane_id();
  for (u32 n = blockIdx.x * (blockDim.x / WAVE) + wave_id(); n < N; n += nwaves) {
    i64 s = ooff[n], d = nb_off[n];
    u32 c = (u32)(nb_off[n + 1] - d);
    for (u32 i = l; i < c; i += WAVE) nb[d + i] = obuf[s + i];
  }
}


}  // namespace

void launch_check_edges(chp_ctx *c, u32 N, u32 E, u64 P, const i64 *e_off, const u32 *e_nsrc,
                        const u32 *e_w, const u32 *n_size) {
  u64 n = E > N ? E : N;
  CHP_LAUNCH(c, "check_edges", k_check_edges, grid_for(n ? n : 1, 256), 256, 0, N, E, P, e_off,
             e_nsrc, e_w, n_size, c->flags);
}

void launch_edges_canon(chp_ctx *c, u32 N, u32 E, const i64 *e_off, const u32 *e_nsrc,
                        const u32 *pins_in, u32 *pins_out, u32 *bad_edges, RunLists rl) {
  if (E == 0) return;
  CHP_LAUNCH(c, "edges_canon", k_edges_canon, waves_grid(E), 256, 0, N, E, e_off, e_nsrc, pins_in,
             pins_out, bad_edges, rl, c->flags);
}

void launch_sort_runs(chp_ctx *c, u32 *data, RunLists rl, const u32 *host_cnt, u32 *scratch,
                      u64 scratch_per_wg, u32 grid_big) {
  if (host_cnt[0])
    CHP_LAUNCH(c, "runs_wave", k_runs_wave, waves_grid(host_cnt[0]), 256, 0, data, rl.start[0],
               rl.len[0], rl.cnt + 0);
  if (host_cnt[1]) {
    const u32 gw = (host_cnt[1] + 3) / 4;
    CHP_LAUNCH(c, "runs_wreg", k_runs_wreg, gw < 32 * c->n_cu ? gw : 32 * c->n_cu, 256, 0, data,
               rl.start[1], rl.len[1], rl.cnt + 1);
    const u32 gl = (host_cnt[1] + 255) / 256;
    CHP_LAUNCH(c, "runs_lds", (k_runs_lds<256, LDS_CAP_U32>), gl < 8192 ? gl : 8192, 256, 0,
               data, rl.start[1], rl.len[1], rl.cnt + 1);
  }
  if (host_cnt[2])
    CHP_LAUNCH(c, "runs_global", (k_runs_global<256, LDS_CAP_U32>), grid_big, 256, 0, data,
               rl.start[2], rl.len[2], rl.cnt + 2, scratch, scratch_per_wg);
}

void launch_edges_check(chp_ctx *c, const i64 *e_off, const u32 *e_nsrc, const u32 *pins,
                        const u32 *list, u32 count) {
  if (!count) return;
  CHP_LAUNCH(c, "edges_check", k_edges_check, waves_grid(count), 256, 0, e_off, e_nsrc, pins,
             list, count, c->flags);
}

// Hyperedges per chunk of the degree and scatter kernels: four chunks per CU,
// from 64 to DW_EDGES.
static u32 chunk_edges(const chp_ctx *c, u32 E) {
  const u32 per = E / (4 * c->n_cu);
  return per < 64 ? 64 : per > DW_EDGES ? DW_EDGES : per;
}

void launch_degrees(chp_ctx *c, u32 E, const i64 *e_off, const u32 *e_nsrc, const u32 *pins,
                    u32 *indeg, u32 *outdeg) {
  if (E == 0) return;
  const u32 epc = chunk_edges(c, E);
  CHP_LAUNCH(c, "degrees", k_degrees, (E + epc - 1) / epc, DW_BLOCK, 0, E, epc, e_off, e_nsrc,
             pins, indeg, outdeg);
}

void launch_node_feas(chp_ctx *c, u32 N, const u32 *indeg, const u32 *outdeg, const u32 *n_size,
                      u64 omega, u32 delta, u32 *deg, u32 *n_nin) {
  if (N == 0) return;
  CHP_LAUNCH(c, "node_feas", k_node_feas, grid_for(N, 256), 256, 0, N, indeg, outdeg, n_size,
             omega, delta, deg, n_nin, c->flags);
}

void launch_scatter(chp_ctx *c, u32 E, const i64 *e_off, const u32 *e_nsrc, const u32 *pins,
                    const i64 *n_off, const u32 *n_nin, u32 *cur_in, u32 *cur_out, u32 *n_inc) {
  if (E == 0) return;
  const u32 epc = chunk_edges(c, E);
  CHP_LAUNCH(c, "scatter", k_scatter, (E + epc - 1) / epc, DW_BLOCK, 0, E, epc, e_off, e_nsrc,
             pins, n_off, n_nin, cur_in, cur_out, n_inc);
}

void launch_node_runs(chp_ctx *c, u32 N, const i64 *n_off, const u32 *n_nin, RunLists rl) {
  if (N == 0) return;
  CHP_LAUNCH(c, "node_runs", k_node_runs, grid_for(N, 256), 256, 0, N, n_off, n_nin, rl);
}

void launch_nb_classify(chp_ctx *c, u32 lo, u32 N, const i64 *e_off, const u32 *e_nsrc,
                        const u32 *pins, const i64 *n_off, const u32 *n_inc, u32 *bound,
                        NbLists nl, const uint8_t *skip) {
  if (N == 0) return;
  CHP_LAUNCH(c, "nb_classify", k_nb_classify, grid_for(N, 256), 256, 0, lo, N, e_off, e_nsrc,
             pins, n_off, n_inc, bound, nl, skip);
}

void launch_nb_build(chp_ctx *c, u32 N, const i64 *e_off, const u32 *pins, const i64 *n_off,
                     const u32 *n_inc, const u32 *bound, const i64 *ooff, u32 *obuf, u32 *count,
                     NbLists nl, const u32 *host_cnt) {
  if (host_cnt[0])
    CHP_LAUNCH(c, "nb_wave", k_nb_wave, waves_grid(host_cnt[0]), 256, 0, e_off, pins, n_off,
               n_inc, ooff, obuf, count, nl.list[0], nl.cnt + 0);
  if (host_cnt[2])
    CHP_LAUNCH(c, "nb_sort", (k_nb_sort<256, NB_SORT_CAP>),
               host_cnt[2] < 8 * c->n_cu ? host_cnt[2] : 8 * c->n_cu, 256, 0, e_off, pins, n_off,
               n_inc, ooff, obuf, count, (const u32 *)nl.list[2], (const u32 *)nl.cnt + 2);
  launch_nb_bitmap(c, N, e_off, pins, n_off, n_inc, bound, ooff, obuf, count, nl.list[1],
                   nl.cnt + 1, host_cnt[1]);
}

void launch_nb_compact(chp_ctx *c, u32 N, const i64 *ooff, const u32 *obuf, const i64 *nb_off,
                       u32 *nb) {
  if (N == 0) return;
  CHP_LAUNCH(c, "nb_compact", k_nb_compact, waves_grid(N), 256, 0, N, ooff, obuf, nb_off, nb);
}
