// C ABI: context, allocation, timing, and the host-side sequencing of the
// kernels of each entry point.  Every kernel runs on the context stream; the
// host synchronises only where a count must size an allocation or a value
// is returned to the caller.
#include <algorithm>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <mutex>

#include <vector>

#include "kernels.h"

// ---------------------------------------------------------------------------
// allocation and error plumbing

void *ctx_alloc(chp_ctx *c, size_t bytes) {
  if (bytes == 0) bytes = 256;
  void *p = nullptr;
  if (c->alloc) {
    p = c->alloc(bytes, c->user);
  } else if (hipMalloc(&p, bytes) != hipSuccess) {
    (void)hipGetLastError();
    p = nullptr;
  }
  return p;
}

void ctx_free(chp_ctx *c, void *p) {
  if (!p) return;
  if (c->free_fn) c->free_fn(p, c->user);
  else (void)hipFree(p);
}

namespace {

struct Fail {
  int code;
};

void set_err(chp_ctx *c, const char *fmt, const char *a = "", long long b = 0) {
  char buf[512];
  snprintf(buf, sizeof buf, fmt, a, b);
  c->err = buf;
}

void hip_check(chp_ctx *c, hipError_t e, const char *what) {
  if (e != hipSuccess) {
    set_err(c, "%s: HIP error %lld", what, (long long)e);
    c->err += std::string(" (") + hipGetErrorString(e) + ")";
    throw Fail{CHP_EDEVICE};
  }
}

void launch_check(chp_ctx *c, const char *what) { hip_check(c, hipPeekAtLastError(), what); }

// Scratch memory of one call.  Requests up to ARENA_SMALL bytes are carved
// from the context's arena (a device block reused by every call: all work is
// on one stream, so a later call's kernels run after the earlier ones);
// larger ones, and small ones that overflow the arena, are allocated on their
// own and freed when the call returns.  An overflow grows the arena for the
// next call.
constexpr size_t ARENA_SMALL = 16u << 20;
constexpr size_t ARENA_MAX = 512u << 20;

struct Scratch {
  chp_ctx *c;
  size_t mark;
  size_t need;
  std::vector<void *> own;
  // fixed mode: every request is carved from [fixed, fixed + fixed_cap) and
  // nothing is ever allocated; a request that does not fit is an error
  char *fixed = nullptr;
  size_t fixed_cap = 0, fixed_top = 0;
  explicit Scratch(chp_ctx *cc) : c(cc), mark(cc->arena_top), need(cc->arena_top) {}
  Scratch(chp_ctx *cc, char *base, size_t cap)
      : c(cc), mark(cc->arena_top), need(cc->arena_top), fixed(base), fixed_cap(cap) {}
  ~Scratch() {
    if (fixed) return;
    for (void *p : own) ctx_free(c, p);
    c->arena_top = mark;
    if (need > c->arena_cap && mark == 0) {
      size_t cap = need + need / 4;
      if (cap > ARENA_MAX) cap = ARENA_MAX;
      if (cap > c->arena_cap) {
        ctx_free(c, c->arena);
        c->arena = (char *)ctx_alloc(c, cap);
        c->arena_cap = c->arena ? cap : 0;
      }
    }
  }
  template <typename T>
  T *get(u64 n) {
    const size_t bytes = (((size_t)(n ? n : 1) * sizeof(T)) + 255) & ~(size_t)255;
    if (fixed) {
      if (bytes > fixed_cap - fixed_top) {
        set_err(c, "%sthe call needs more than the %lld bytes of its fixed scratch", "",
                (long long)fixed_cap);
        throw Fail{CHP_EINVAL};
      }
      void *p = fixed + fixed_top;
      fixed_top += bytes;
      return (T *)p;
    }
    if (bytes <= ARENA_SMALL) {
      need += bytes;
      if (c->arena && c->arena_top + bytes <= c->arena_cap) {
        void *p = c->arena + c->arena_top;
        c->arena_top += bytes;
        return (T *)p;
      }
    }
    void *p = ctx_alloc(c, bytes);
    if (!p) {
      set_err(c, "device allocation of %s%lld bytes failed", "", (long long)bytes);
      throw Fail{CHP_ENOMEM};
    }
    own.push_back(p);
    return (T *)p;
  }
  // return a large buffer early (arena pieces are reclaimed at the end)
  void release(void *p) {
    auto it = std::find(own.begin(), own.end(), p);
    if (it != own.end()) {
      ctx_free(c, p);
      own.erase(it);
    }
  }
};

// Arrays that become part of a published chp_hgraph: freed on failure only.
struct Owned {
  chp_ctx *c;
  std::vector<void *> v;
  bool keep = false;
  explicit Owned(chp_ctx *cc) : c(cc) {}
  ~Owned() {
    if (!keep)
      for (void *p : v) ctx_free(c, p);
  }
  template <typename T>
  T *get(u64 n) {
    void *p = ctx_alloc(c, (size_t)(n ? n : 1) * sizeof(T));
    if (!p) {
      set_err(c, "device allocation of %s%lld bytes failed", "", (long long)(n * sizeof(T)));
      throw Fail{CHP_ENOMEM};
    }
    v.push_back(p);
    return (T *)p;
  }
};

__global__ void k_fill_u32(u32 *p, u64 n, u32 v) {
  for (u64 i = (u64)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (u64)gridDim.x * blockDim.x)
    p[i] = v;
}
__global__ void k_fill_u64(u64 *p, u64 n, u64 v) {
  for (u64 i = (u64)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (u64)gridDim.x * blockDim.x)
    p[i] = v;
}

// rho_fine[n] = rho_coarse[gamma[n]]; a coarse id out of range raises EINVAL
__global__ void k_project(u32 n_fine, const u32 *gamma, u32 n_coarse, const u32 *rho_coarse,
                          u32 *rho_fine, u32 *flags) {
  const u32 n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= n_fine) return;
  const u32 c = gamma[n];
  if (c >= n_coarse) {
    atomicOr(flags, FLAG_EINVAL);
    rho_fine[n] = 0;
    return;
  }
  rho_fine[n] = rho_coarse[c];
}

// Small device->host reads.  One kernel gathers the words of every item into
// the context's pinned host buffer (mapped into the device address space),
// then the stream is synchronised: one launch and no copy engine per call.
constexpr u32 PUB_MAX = 12;
struct PubDesc {
  const u32 *src[PUB_MAX];
  u32 off[PUB_MAX + 1];  // word offset of item k in the buffer; off[n] = total words
  u32 n;
};
__global__ void k_publish(PubDesc d, u32 *dst) {
  const u32 i = threadIdx.x;
  if (i >= d.off[d.n]) return;
  u32 k = 0;
  while (i >= d.off[k + 1]) ++k;
  dst[i] = d.src[k][i - d.off[k]];
}

struct HostRead {
  void *host;
  const void *dev;
  size_t n;  // a multiple of 4 bytes, the item 4-byte aligned
};
void read_many(chp_ctx *c, std::initializer_list<HostRead> items) {
  PubDesc d;
  d.n = 0;
  d.off[0] = 0;
  for (const HostRead &it : items) {
    if (d.n == PUB_MAX || (it.n & 3) || ((uintptr_t)it.dev & 3)) {
      set_err(c, "%sinternal: unsupported readback");
      throw Fail{CHP_EDEVICE};
    }
    d.src[d.n] = (const u32 *)it.dev;
    d.off[d.n + 1] = d.off[d.n] + (u32)(((it.n + 7) & ~(size_t)7) / 4);
    ++d.n;
  }
  if (d.off[d.n] > 64 * 2) {
    set_err(c, "%sinternal: readback too large");
    throw Fail{CHP_EDEVICE};
  }
  CHP_LAUNCH(c, "publish", k_publish, 1, 128, 0, d, c->pinned_dev);
  hip_check(c, hipStreamSynchronize(c->stream), "stream synchronize");
  u32 k = 0;
  for (const HostRead &it : items) memcpy(it.host, (const char *)c->pinned + 4 * d.off[k++], it.n);
}

void read_back(chp_ctx *c, void *host, const void *dev, size_t n) {
  read_many(c, {{host, dev, n}});
}

void d2d(chp_ctx *c, void *dst, const void *src, size_t n) {
  if (n) hip_check(c, hipMemcpyAsync(dst, src, n, hipMemcpyDeviceToDevice, c->stream), "copy");
}

u32 read_flags(chp_ctx *c) {
  u32 f;
  read_back(c, &f, c->flags, sizeof f);
  return f;
}

int flags_code(u32 f) {
  if (f & FLAG_EINVAL) return CHP_EINVAL;
  if (f & FLAG_EOVERFLOW) return CHP_EOVERFLOW;
  if (f & FLAG_EINFEASIBLE) return CHP_EINFEASIBLE;
  if (f & FLAG_ECYCLE) return CHP_ECYCLE;
  return CHP_OK;
}

void fail_flags(chp_ctx *c, u32 f, const char *what) {
  int code = flags_code(f);
  if (code == CHP_OK) return;
  const char *kind = code == CHP_EINVAL      ? "invalid input"
                     : code == CHP_EOVERFLOW ? "value out of the supported range"
                     : code == CHP_EINFEASIBLE
                         ? "a single node exceeds omega or delta"
                         : "proposal graph has a cycle longer than two";
  set_err(c, "%s", what);
  c->err += std::string(": ") + kind;
  throw Fail{code};
}

void clear_flags(chp_ctx *c) { launch_fill_u32(c, c->flags, 64, 0); }

u32 grid_big_for(u32 count) { return count < 256 ? (count ? count : 1) : 256; }

// ---------------------------------------------------------------------------
// shared steps

// Sort every run listed in rl (counts already on the device).
void sort_listed_runs(chp_ctx *c, Scratch &s, u32 *data, RunLists rl) {
  u32 hc[8];
  read_back(c, hc, rl.cnt, sizeof hc);
  u32 *scr = nullptr;
  u64 per_wg = 0;
  u32 gb = grid_big_for(hc[2]);
  if (hc[2]) {
    per_wg = (u64)hc[3];
    scr = s.get<u32>(per_wg * gb);
  }
  launch_sort_runs(c, data, rl, hc, scr, per_wg, gb);
  launch_check(c, "sort runs");
}

RunLists make_runlists(Scratch &s, u64 cap) {
  RunLists rl;
  for (int k = 0; k < 3; ++k) {
    rl.start[k] = s.get<i64>(cap);
    rl.len[k] = s.get<u32>(cap);
  }
  rl.cnt = s.get<u32>(8);
  return rl;
}

// incidence CSR of a canonical, validated hyperedge CSR (g->e_* set);
// allocates g->n_off, n_nin, n_inc into `own`.
void build_incidence_core(chp_ctx *c, Scratch &s, Owned &own, chp_hgraph *g, u64 omega,
                          u32 delta) {
  const u32 N = g->n_nodes, E = g->n_edges;
  const u64 P = g->n_pins;
  g->n_off = own.get<i64>((u64)N + 1);
  g->n_nin = own.get<u32>(N);
  g->n_inc = own.get<u32>(P);
  u32 *indeg = s.get<u32>(N), *outdeg = s.get<u32>(N), *deg = s.get<u32>(N);
  launch_fill_u32(c, indeg, N, 0);
  launch_fill_u32(c, outdeg, N, 0);
  launch_degrees(c, E, g->e_off, g->e_nsrc, g->e_pins, indeg, outdeg);
  launch_node_feas(c, N, indeg, outdeg, g->n_size, omega, delta, deg, g->n_nin);
  i64 *tmp = s.get<i64>(scan_tmp_words(N));
  scan_u32_to_i64(c, deg, g->n_off, N, tmp);
  launch_fill_u32(c, indeg, N, 0);
  launch_fill_u32(c, outdeg, N, 0);
  launch_scatter(c, E, g->e_off, g->e_nsrc, g->e_pins, g->n_off, g->n_nin, indeg, outdeg,
                 g->n_inc);
  launch_check(c, "incidence");
  s.release(deg);
  s.release(tmp);
  RunLists rl = make_runlists(s, 2ull * N);
  launch_fill_u32(c, rl.cnt, 8, 0);
  launch_node_runs(c, N, g->n_off, g->n_nin, rl);
  sort_listed_runs(c, s, g->n_inc, rl);
}

// neighbourhood CSR of g (incidence already built)
void build_neighbors_core(chp_ctx *c, Scratch &s, Owned &own, chp_hgraph *g) {
  const u32 N = g->n_nodes;
  g->nb_off = own.get<i64>((u64)N + 1);
  u32 *bound = s.get<u32>(N);
  NbLists nl;
  for (int k = 0; k < 3; ++k) nl.list[k] = s.get<u32>(N);
  nl.list[3] = nl.list[4] = nullptr;
  nl.cnt = s.get<u32>(8);
  launch_fill_u32(c, nl.cnt, 8, 0);
  launch_nb_classify(c, 0, N, g->e_off, g->e_nsrc, g->e_pins, g->n_off, g->n_inc, bound, nl);
  i64 *ooff = s.get<i64>((u64)N + 1);
  i64 *tmp = s.get<i64>(scan_tmp_words(N));
  scan_u32_to_i64(c, bound, ooff, N, tmp);
  launch_check(c, "neighbour classes");
  i64 obuf_total;
  u32 hc[8];
  read_many(c, {{&obuf_total, ooff + N, sizeof obuf_total}, {hc, nl.cnt, sizeof hc}});
  if (hc[7]) {
    set_err(c, "%sa node's incident pins exceed 2^32");
    throw Fail{CHP_EOVERFLOW};
  }
  u32 *obuf = s.get<u32>((u64)obuf_total);
  u32 *count = s.get<u32>(N);
  launch_fill_u32(c, count, N, 0);
  launch_nb_build(c, N, g->e_off, g->e_pins, g->n_off, g->n_inc, bound, ooff, obuf, count, nl,
                  hc);
  scan_u32_to_i64(c, count, g->nb_off, N, tmp);
  launch_check(c, "neighbours");
  i64 total;
  read_back(c, &total, g->nb_off + N, sizeof total);
  g->nb = own.get<u32>((u64)total);
  g->nb_total = (u64)total;
  launch_nb_compact(c, N, ooff, obuf, g->nb_off, g->nb);
  launch_check(c, "neighbour compaction");
}

EdgeLists make_edge_lists(chp_ctx *c, Scratch &s, u32 E, const i64 *e_off, u32 hc[8]) {
  EdgeLists el;
  for (int k = 0; k < 3; ++k) el.list[k] = s.get<u32>(E);
  el.list[3] = nullptr;
  el.cnt = s.get<u32>(8);
  launch_fill_u32(c, el.cnt, 8, 0);
  launch_edge_classify(c, E, e_off, el);
  launch_check(c, "edge classes");
  read_back(c, hc, el.cnt, 8 * sizeof(u32));
  return el;
}

template <typename F>
int guarded(chp_ctx *c, F &&f) {
  if (!c) return CHP_EINVAL;
  c->err.clear();
  try {
    int dev;
    hip_check(c, hipGetDevice(&dev), "hipGetDevice");
    if (dev != c->device) hip_check(c, hipSetDevice(c->device), "hipSetDevice");
    f();
    return CHP_OK;
  } catch (const Fail &x) {
    return x.code;
  }
}

}  // namespace

__global__ void k_fills(FillDesc d) {
  const u64 g = (u64)blockIdx.x * blockDim.x + threadIdx.x, st = (u64)gridDim.x * blockDim.x;
  for (u32 k = 0; k < d.cnt; ++k) {
    if (d.wide[k])
      for (u64 i = g; i < d.n[k]; i += st) ((u64 *)d.p[k])[i] = d.v[k];
    else
      for (u64 i = g; i < d.n[k]; i += st) ((u32 *)d.p[k])[i] = (u32)d.v[k];
  }
}

void launch_fills(chp_ctx *c, std::initializer_list<FillItem> items) {
  FillDesc d;
  d.cnt = 0;
  u64 most = 0;
  for (const FillItem &it : items) {
    if (!it.n) continue;
    if (d.cnt == 8) {
      set_err(c, "%sinternal: too many fills in one launch");
      throw Fail{CHP_EDEVICE};
    }
    d.p[d.cnt] = it.p;
    d.n[d.cnt] = it.n;
    d.v[d.cnt] = it.v;
    d.wide[d.cnt] = it.wide ? 1u : 0u;
    most = it.n > most ? it.n : most;
    ++d.cnt;
  }
  if (!d.cnt) return;
  u32 g = grid_for(most, 256);
  if (g > 4096) g = 4096;
  CHP_LAUNCH(c, "fill", k_fills, g, 256, 0, d);
}

void launch_fill_u32(chp_ctx *c, u32 *p, u64 n, u32 v) {
  if (!n) return;
  u32 g = grid_for(n, 256);
  if (g > 4096) g = 4096;
  CHP_LAUNCH(c, "fill", k_fill_u32, g, 256, 0, p, n, v);
}

void launch_fill_u64(chp_ctx *c, u64 *p, u64 n, u64 v) {
  if (!n) return;
  u32 g = grid_for(n, 256);
  if (g > 4096) g = 4096;
  CHP_LAUNCH(c, "fill", k_fill_u64, g, 256, 0, p, n, v);
}

// ---------------------------------------------------------------------------
// timing

void timing_begin(chp_ctx *c, const char *name, hipEvent_t *a, hipEvent_t *b) {
  (void)name;
  for (hipEvent_t *e : {a, b}) {
    if (!c->free_events.empty()) {
      *e = c->free_events.back();
      c->free_events.pop_back();
    } else if (hipEventCreate(e) != hipSuccess) {
      *e = nullptr;
    }
  }
  if (*a) (void)hipEventRecord(*a, c->stream);
}

static void resolve_timings(chp_ctx *c) {
  if (c->pending.empty()) return;
  (void)hipStreamSynchronize(c->stream);
  for (auto &r : c->pending) {
    float ms = 0.f;
    if (r.a && r.b) (void)hipEventElapsedTime(&ms, r.a, r.b);
    TimingSum *hit = nullptr;
    for (auto &s : c->sums)
      if (s.name == r.name || strcmp(s.name, r.name) == 0) {
        hit = &s;
        break;
      }
    if (!hit) {
      c->sums.push_back(TimingSum{r.name, 0, 0.0});
      hit = &c->sums.back();
    }
    hit->launches += 1;
    hit->total_ms += ms;
    if (r.a) c->free_events.push_back(r.a);
    if (r.b) c->free_events.push_back(r.b);
  }
  c->pending.clear();
}

void timing_end(chp_ctx *c, const char *name, hipEvent_t a, hipEvent_t b) {
  if (b) (void)hipEventRecord(b, c->stream);
  c->pending.push_back(TimingRec{name, a, b});
  if (c->pending.size() >= 4096) resolve_timings(c);
}

// ---------------------------------------------------------------------------
// Fixed scratch of the entry points that allocate nothing
// (chp_evaluate_partition_noalloc).  Every GPU the library runs on holds its
// own copy for the life of the process.  In host code the array's name is not
// a device address: its address on each device is taken once, with that
// device current, when the first context on that device is created, and only
// that address is ever handed to kernels.
constexpr size_t FIXED_SCRATCH_BYTES = 64u << 20;
static __device__ __align__(256) char scratch[FIXED_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
char *g_scratch_ptr[MAX_DEVICES] = {};

// this device's address of scratch (the device current); nullptr on error
char *fixed_scratch_of(int dev) {
  if (dev < 0 || dev >= MAX_DEVICES) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_ptr[dev] = (char *)ptr;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

// ---------------------------------------------------------------------------
// C ABI

extern "C" {

int chp_create(chp_ctx **out, void *hip_stream, chp_alloc_fn alloc, chp_free_fn free_fn,
               void *user) {
  if (!out) return CHP_EINVAL;
  *out = nullptr;
  if ((alloc == nullptr) != (free_fn == nullptr)) return CHP_EINVAL;
  chp_ctx *c = new chp_ctx();
  c->stream = (hipStream_t)hip_stream;
  c->alloc = alloc;
  c->free_fn = free_fn;
  c->user = user;
  int ncu = 0;
  if (hipGetDevice(&c->device) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, c->device) !=
          hipSuccess ||
      hipHostMalloc((void **)&c->pinned, 64 * sizeof(u64), hipHostMallocMapped) != hipSuccess ||
      hipHostGetDevicePointer((void **)&c->pinned_dev, c->pinned, 0) != hipSuccess ||
      !(c->fixed_scratch = fixed_scratch_of(c->device))) {
    (void)hipGetLastError();
    if (c->pinned) (void)hipHostFree(c->pinned);
    delete c;
    return CHP_EDEVICE;
  }
  c->n_cu = ncu > 0 ? (u32)ncu : 256;
  c->flags = (u32 *)ctx_alloc(c, 64 * sizeof(u32));
  if (!c->flags) {
    (void)hipHostFree(c->pinned);
    delete c;
    return CHP_ENOMEM;
  }
  *out = c;
  return CHP_OK;
}

void chp_destroy(chp_ctx *c) {
  if (!c) return;
  (void)hipStreamSynchronize(c->stream);
  resolve_timings(c);
  ctx_free(c, c->arena);
  for (hipEvent_t e : c->free_events) (void)hipEventDestroy(e);
  ctx_free(c, c->flags);
  (void)hipHostFree(c->pinned);
  delete c;
}

const char *chp_last_error(const chp_ctx *c) { return c ? c->err.c_str() : "null context"; }

int chp_set_batch_entries(chp_ctx *c, uint64_t entries) {
  if (!c) return CHP_EINVAL;
  c->batch_entries = entries;
  return CHP_OK;
}

int chp_last_rate_stats(const chp_ctx *c, uint64_t *nb_entries, uint32_t *batches,
                        uint32_t *inc_nodes) {
  if (!c) return CHP_EINVAL;
  if (nb_entries) *nb_entries = c->last_nb_built;
  if (batches) *batches = c->last_batches;
  if (inc_nodes) *inc_nodes = c->last_inc_nodes;
  return CHP_OK;
}

int chp_set_matching(chp_ctx *c, int mode) {
  if (!c || (mode != CHP_MATCH_HANDSHAKE && mode != CHP_MATCH_OPTIMAL)) return CHP_EINVAL;
  c->matching = (u32)mode;
  return CHP_OK;
}

int chp_set_move_order(chp_ctx *c, int order) {
  if (!c || (order != CHP_ORDER_CHAINS && order != CHP_ORDER_GAIN)) return CHP_EINVAL;
  c->move_order = (u32)order;
  return CHP_OK;
}

int chp_set_incidence_rating(chp_ctx *c, uint64_t min_visits, uint32_t hash_keys) {
  if (!c) return CHP_EINVAL;
  c->inc_min_visits = min_visits;
  c->inc_hash_keys = hash_keys;
  return CHP_OK;
}

int chp_set_incidence_bins(chp_ctx *c, int bins) {
  if (!c || (bins != CHP_INC_BINS_32 && bins != CHP_INC_BINS_64)) return CHP_EINVAL;
  c->inc_bins = (u32)bins;
  return CHP_OK;
}

int chp_set_timing_filter(chp_ctx *c, const char *prefix) {
  if (!c) return CHP_EINVAL;
  c->timing_prefix = prefix ? prefix : "";
  return CHP_OK;
}

int chp_set_timing(chp_ctx *c, int on) {
  if (!c) return CHP_EINVAL;
  c->timing = on ? 1 : 0;
  return CHP_OK;
}

int chp_get_timings(chp_ctx *c, chp_timing *out, int max) {
  if (!c) return CHP_EINVAL;
  resolve_timings(c);
  int n = (int)c->sums.size();
  for (int i = 0; i < n && i < max && out; ++i)
    out[i] = chp_timing{c->sums[i].name, c->sums[i].launches, c->sums[i].total_ms};
  return n;
}

void chp_reset_timings(chp_ctx *c) {
  if (!c) return;
  resolve_timings(c);
  c->sums.clear();
}

void chp_hgraph_free(chp_ctx *c, chp_hgraph *g) {
  if (!c || !g) return;
  void *ps[] = {g->e_off, g->e_nsrc, g->e_pins, g->e_w, g->n_size,
                g->n_off, g->n_nin,  g->n_inc,  g->nb_off, g->nb};
  for (void *p : ps) ctx_free(c, p);
  memset(g, 0, sizeof *g);
}

int chp_build_incidence(chp_ctx *c, const chp_edges *in, const chp_params *prm,
                        int build_neighbors, chp_hgraph *out) {
  return guarded(c, [&] {
    if (!in || !prm || !out) {
      set_err(c, "%snull argument");
      throw Fail{CHP_EINVAL};
    }
    const u32 N = in->n_nodes, E = in->n_edges;
    const u64 P = in->n_pins;
    if (!in->e_off || (E && (!in->e_nsrc || !in->e_w)) || (P && !in->e_pins) ||
        (N && !in->n_size)) {
      set_err(c, "%snull array in chp_edges");
      throw Fail{CHP_EINVAL};
    }
    if (N == NONE32 || E == NONE32) {
      set_err(c, "%sids must stay below 2^32-1");
      throw Fail{CHP_EOVERFLOW};
    }
    Scratch s(c);
    Owned own(c);
    clear_flags(c);
    launch_check_edges(c, N, E, P, in->e_off, in->e_nsrc, in->e_w, in->n_size);
    launch_check(c, "check edges");
    u32 f = read_flags(c);
    if (f & FLAG_EINVAL) fail_flags(c, FLAG_EINVAL, "offsets, weights or sizes");
    chp_hgraph g;
    memset(&g, 0, sizeof g);
    g.n_nodes = N;
    g.n_edges = E;
    g.n_pins = P;
    g.e_off = own.get<i64>((u64)E + 1);
    g.e_nsrc = own.get<u32>(E);
    g.e_pins = own.get<u32>(P);
    g.e_w = own.get<u32>(E);
    g.n_size = own.get<u32>(N);
    d2d(c, g.e_off, in->e_off, sizeof(i64) * ((size_t)E + 1));
    d2d(c, g.e_nsrc, in->e_nsrc, sizeof(u32) * (size_t)E);
    d2d(c, g.e_w, in->e_w, sizeof(u32) * (size_t)E);
    d2d(c, g.n_size, in->n_size, sizeof(u32) * (size_t)N);
    // canonical pins: copy, range check, queue unsorted runs
    RunLists rl = make_runlists(s, 2ull * E + 2);
    u32 *bad = s.get<u32>(E);
    launch_fill_u32(c, rl.cnt, 8, 0);
    launch_edges_canon(c, N, E, in->e_off, in->e_nsrc, in->e_pins, g.e_pins, bad, rl);
    launch_check(c, "canonical edges");
    u32 hc[8];
    read_many(c, {{hc, rl.cnt, sizeof hc}, {&f, c->flags, sizeof f}});
    if (f & FLAG_EINVAL) fail_flags(c, FLAG_EINVAL, "pins");
    if (hc[4]) {
      sort_listed_runs(c, s, g.e_pins, rl);
      launch_edges_check(c, g.e_off, g.e_nsrc, g.e_pins, bad, hc[4]);
      launch_check(c, "edge check");
      f = read_flags(c);
      if (f & FLAG_EINVAL) fail_flags(c, FLAG_EINVAL, "pins");
    }
    if (f & FLAG_EOVERFLOW) fail_flags(c, FLAG_EOVERFLOW, "hyperedge weight");
    s.release(bad);
    build_incidence_core(c, s, own, &g, prm->omega, prm->delta);
    f = read_flags(c);
    if (f) fail_flags(c, f, "node limits");
    if (build_neighbors) build_neighbors_core(c, s, own, &g);
    hip_check(c, hipStreamSynchronize(c->stream), "build_incidence");
    own.keep = true;
    *out = g;
  });
}

namespace {

// Exact matching on the proposal pseudo-forest: depths, a host scan of the
// per-depth counts, then one launch per depth up and one down.
void match_optimal(chp_ctx *c, Scratch &s, u32 N, const u32 *target, const u64 *score,
                   u32 *match, u32 *npairs, u32 *n_pairs_host) {
  DpScratch d;
  d.par = s.get<u32>(N);
  d.anc = s.get<u32>(N);
  d.dist = s.get<u32>(N);
  d.anc2 = s.get<u32>(N);
  d.dist2 = s.get<u32>(N);
  d.byd = s.get<u32>(N);
  d.bestc = s.get<u32>(N);
  d.small = s.get<u32>(4);
  d.A = s.get<u64>(N);
  d.bestv = s.get<u64>(N);
  d.ss0 = s.get<u64>(N);
  d.diff = s.get<u64>(N);
  launch_fill_u32(c, d.small, 4, 0);
  launch_dp_prepare(c, N, target, d, match);
  launch_check(c, "matching depths");
  u32 D = 0, f = 0;
  read_many(c, {{&D, d.small, sizeof D}, {&f, c->flags, sizeof f}});
  if (f & (FLAG_EINVAL | FLAG_EOVERFLOW)) fail_flags(c, f, "rating");
  if (f & FLAG_ECYCLE) fail_flags(c, FLAG_ECYCLE, "matching");
  u32 *cntd = s.get<u32>((u64)D + 1);
  u32 *cursor = s.get<u32>((u64)D + 1);
  launch_fill_u32(c, cntd, (u64)D + 1, 0);
  launch_dp_count(c, N, d.dist, cntd);
  launch_check(c, "matching depth counts");
  std::vector<u32> off((size_t)D + 2);
  hip_check(c, hipMemcpyAsync(off.data() + 1, cntd, sizeof(u32) * ((size_t)D + 1),
                              hipMemcpyDeviceToHost, c->stream),
            "readback");
  hip_check(c, hipStreamSynchronize(c->stream), "stream synchronize");
  off[0] = 0;
  for (size_t i = 1; i < off.size(); ++i) off[i] += off[i - 1];
  hip_check(c, hipMemcpyAsync(cursor, off.data(), sizeof(u32) * ((size_t)D + 1),
                              hipMemcpyHostToDevice, c->stream),
            "copy");
  launch_dp_levels(c, N, target, score, d, D, cursor, off.data(), match, npairs);
  launch_check(c, "matching levels");
  read_many(c, {{&f, c->flags, sizeof f}, {n_pairs_host, npairs, sizeof(u32)}});
  if (f & FLAG_EOVERFLOW) fail_flags(c, FLAG_EOVERFLOW, "matching");
}

// Neighbour entries one batch may hold (oversize buffer and packed lists).
constexpr u64 BATCH_ENTRIES = 3ull << 30;
// Positions a leftover node scans below its slack position.
constexpr u32 LEFT_WINDOW = 64;
// Incident pins from which a node of such a graph is rated straight from the
// incidence rather than through a neighbour list.
constexpr u64 INC_MIN_VISITS = 16384;

// Rating of a graph built without neighbourhoods (too many to hold at once;
// [HP] Sec. VII-C runs the coarsening kernels over batches of nodes, keeping
// only a few nodes' neighbourhoods in device memory).  Nodes with many
// incident pins (c->inc_min_visits, or INC_MIN_VISITS) are rated straight from
// the incidence, their N(n) held in LDS one id window at a time.  For the
// others, node ranges [lo, hi) whose level-0 neighbour bounds fit the batch
// limit (c->batch_entries, or BATCH_ENTRIES) get their N(n) built as by
// chp_build_incidence, into batch buffers, and are rated from them; the
// rating reads nb_off through a pointer shifted by lo.
void rate_batched(chp_ctx *c, Scratch &s, const chp_hgraph *g, const RateArgs &a, NbLists nl,
                  NodeRec *recs, NodeRec *big, u32 *work) {
  const u32 N = g->n_nodes;
  u32 *bound = s.get<u32>(N);
  NbLists bl;
  bl.list[0] = s.get<u32>(N);
  bl.list[1] = s.get<u32>(N);
  bl.list[2] = s.get<u32>(N);
  bl.list[3] = bl.list[4] = nullptr;
  bl.cnt = s.get<u32>(8);
  // nodes with many incident pins are rated straight from the incidence
  // (after the batches); the others through per-batch neighbour lists
  const u64 fmin = c->inc_min_visits ? c->inc_min_visits : INC_MIN_VISITS;
  uint8_t *skip = nullptr;
  NodeRec *frecs = nullptr;
  u32 *fc = s.get<u32>(4);  // count, max size, max |in|, work counter
  if (fmin != ~0ull) {
    skip = s.get<uint8_t>(N);
    frecs = s.get<NodeRec>(N);
  }
  launch_fills(c, {{bl.cnt, 8, 0, false}, {fc, 4, 0, false}});
  if (skip) launch_inc_classify(c, a, fmin, skip, frecs, fc, fc + 1);
  launch_nb_classify(c, 0, N, g->e_off, g->e_nsrc, g->e_pins, g->n_off, g->n_inc, bound, bl,
                     skip);
  i64 *ooff = s.get<i64>((u64)N + 1);
  i64 *tmp = s.get<i64>(scan_tmp_words(N));
  scan_u32_to_i64(c, bound, ooff, N, tmp);
  launch_check(c, "neighbour bounds");
  u32 hc[8], nf = 0;
  read_many(c, {{hc, bl.cnt, sizeof hc}, {&nf, fc, sizeof nf}});
  c->last_inc_nodes = nf;
  if (hc[7]) {
    set_err(c, "%sa node's incident pins exceed 2^32");
    throw Fail{CHP_EOVERFLOW};
  }
  std::vector<i64> hoff((size_t)N + 1);
  hip_check(c, hipMemcpyAsync(hoff.data(), ooff, sizeof(i64) * ((size_t)N + 1),
                              hipMemcpyDeviceToHost, c->stream),
            "readback");
  hip_check(c, hipStreamSynchronize(c->stream), "stream synchronize");
  u64 most = 0;
  for (u32 n = 0; n < N; ++n) {
    const u64 b = (u64)(hoff[n + 1] - hoff[n]);
    most = b > most ? b : most;
  }
  const u64 limit = c->batch_entries ? c->batch_entries : BATCH_ENTRIES;
  const u64 budget = most > limit ? most : limit;
  const u64 room = (u64)hoff[N] < budget ? (u64)hoff[N] : budget;
  u32 *obuf = s.get<u32>(room ? room : 1);
  u32 *nbb = s.get<u32>(room ? room : 1);
  u32 *count = s.get<u32>(N);
  i64 *nboff = s.get<i64>((u64)N + 1);
  u32 prev = 0;  // node count of the previous batch, whose list total is read next
  i64 built = 0;
  for (u32 lo = 0; lo < N;) {
    u32 hi = lo + 1;
    while (hi < N && (u64)(hoff[hi + 1] - hoff[lo]) <= budget) ++hi;
    const u32 cnt = hi - lo;
    // N(n) of the batch (bounds recomputed for the range, same values)
    launch_fills(c, {{bl.cnt, 8, 0, false}, {count + lo, cnt, 0, false}});
    launch_nb_classify(c, lo, cnt, g->e_off, g->e_nsrc, g->e_pins, g->n_off, g->n_inc, bound,
                       bl, skip);
    launch_check(c, "batch neighbour classes");
    i64 last = 0;
    if (prev)
      read_many(c, {{hc, bl.cnt, sizeof hc}, {&last, nboff + prev, sizeof last}});
    else
      read_many(c, {{hc, bl.cnt, sizeof hc}});
    built += last;
    u32 *obs = obuf - hoff[lo];  // indexed by the whole graph's oversize offsets
    launch_nb_build(c, N, g->e_off, g->e_pins, g->n_off, g->n_inc, bound, ooff, obs, count, bl,
                    hc);
    scan_u32_to_i64(c, count + lo, nboff, cnt, tmp);
    launch_nb_compact(c, cnt, ooff + lo, obs, nboff, nbb);
    launch_check(c, "batch neighbours");
    // rate the batch
    RateArgs ab = a;
    ab.nb_off = nboff - lo;
    ab.nb = nbb;
    launch_fills(c, {{nl.cnt, 8, 0, false}, {work, 3, 0, false}});
    launch_rate_classify(c, ab, lo, hi, nl, recs, big);
    launch_rate(c, ab, nl, recs, cnt, big, work);
    launch_check(c, "batch rate");
    ++c->last_batches;
    prev = cnt;
    lo = hi;
  }
  i64 last = 0;
  if (prev) read_many(c, {{&last, nboff + prev, sizeof last}});
  c->last_nb_built = (u64)(built + last);
  if (nf && a.pi == 1 && c->inc_bins == CHP_INC_BINS_32 && g->n_pins < (1ull << 31)) {
    // quantised bins first (their stretch addresses take 32 bits); the nodes
    // they cannot rate go to the 64-bit kernel
    NodeRec *spill = s.get<NodeRec>(nf);
    u32 *sc = s.get<u32>(2);  // spill count, work counter of the second launch
    launch_fill_u32(c, sc, 2, 0);
    // every 16th pin of each run, for the nodes' samples (their offsets are
    // held in 32 bits)
    const u32 E = g->n_edges;
    i64 *soff = nullptr;
    u32 *samp = nullptr;
    if (samples_bound(E, g->n_pins) < (1ull << 31)) {
      u32 *scnt = s.get<u32>(E);
      soff = s.get<i64>((u64)E + 1);
      i64 *stmp = s.get<i64>(scan_tmp_words(E));
      samp = s.get<u32>(samples_bound(E, g->n_pins));
      launch_samples(c, E, g->e_off, g->e_nsrc, g->e_pins, scnt, soff, stmp, samp);
    }
    launch_rate_incq(c, a, frecs, fc, fc + 1, fc + 3, nf, c->inc_hash_keys, spill, sc, soff,
                     samp);
    launch_rate_inc(c, a, spill, sc, fc + 1, sc + 1, c->n_cu, c->inc_hash_keys);
  } else {
    launch_rate_inc(c, a, frecs, fc, fc + 1, fc + 3, nf, c->inc_hash_keys);
  }
  launch_check(c, "rate from the incidence");
}

// One matching of the proposal graph (tr, sr) into mr, by the context's
// mode; *np gets its pair count.  Fails on the flags the rating or the
// matching raised.
void match_proposals(chp_ctx *c, Scratch &s, u32 N, const u32 *tr, const u64 *sr,
                     MatchScratch ms, u32 *npairs, u32 *mr, u32 *np) {
  if (c->matching == CHP_MATCH_OPTIMAL) {
    launch_fill_u32(c, npairs, 1, 0);
    match_optimal(c, s, N, tr, sr, mr, npairs, np);
    return;
  }
  launch_fills(c, {{ms.bscore, N, 0, true}, {ms.bid, N, NONE32, false}, {npairs, 1, 0, false}});
  launch_match(c, N, tr, sr, ms, mr, npairs);
  launch_match_write(c, N, tr, ms, mr, npairs);
  launch_check(c, "match");
  u32 f;
  read_many(c, {{&f, c->flags, sizeof f}, {np, npairs, sizeof(u32)}});
  if (f & (FLAG_EINVAL | FLAG_EOVERFLOW)) fail_flags(c, f, "rating");
  if (f & FLAG_LONGCHAIN) {
    if (!ms.p0) {
      ms.p0 = s.get<u32>(N);
      ms.p1 = s.get<u32>(N);
      ms.x0 = s.get<uint8_t>(N);
      ms.x1 = s.get<uint8_t>(N);
    }
    launch_match_jump(c, N, tr, ms);
    launch_fill_u32(c, npairs, 1, 0);
    launch_match_write(c, N, tr, ms, mr, npairs);
    launch_check(c, "match (long chains)");
    read_many(c, {{&f, c->flags, sizeof f}, {np, npairs, sizeof(u32)}});
    if (f & FLAG_ECYCLE) fail_flags(c, FLAG_ECYCLE, "matching");
  }
}

int rate_top_and_match(chp_ctx *c, const chp_hgraph *g, const chp_params *prm, u32 pi,
                       u32 *target, u64 *score_fx, u32 *match, u32 *n_pairs_host,
                       uint8_t *nb_invalid) {
  return guarded(c, [&] {
    if (!g || !prm || !n_pairs_host || (g->n_nodes && (!target || !score_fx || !match))) {
      set_err(c, "%snull argument");
      throw Fail{CHP_EINVAL};
    }
    if (pi < 1 || pi > RATE_MAX_PI) {
      set_err(c, "%spi must be 1 .. 4");
      throw Fail{CHP_EINVAL};
    }
    const u32 N = g->n_nodes, E = g->n_edges;
    const bool batched = N && (!g->nb_off || !g->nb);
    c->last_nb_built = 0;
    c->last_batches = 0;
    c->last_inc_nodes = 0;
    if (batched && nb_invalid) {
      set_err(c, "%sinvalid-neighbour flags need the graph's neighbourhoods");
      throw Fail{CHP_EINVAL};
    }
    *n_pairs_host = 0;
    if (N == 0) return;
    Scratch s(c);
    u64 *t = s.get<u64>(E);
    const u32 np = terms_partials(E);
    u64 *partials = s.get<u64>(2ull * np);
    u64 *capinfo = s.get<u64>(4);
    launch_terms(c, E, g->e_off, g->e_w, t, partials, np, capinfo);
    RateArgs a;
    a.N = N;
    a.e_off = g->e_off;
    a.e_nsrc = g->e_nsrc;
    a.e_pins = g->e_pins;
    a.t = t;
    a.n_off = g->n_off;
    a.n_nin = g->n_nin;
    a.n_inc = g->n_inc;
    a.n_size = g->n_size;
    a.nb_off = g->nb_off;
    a.nb = g->nb;
    a.flag = nb_invalid;
    a.cur = s.get<u32>(2 * g->n_pins);
    a.capinfo = capinfo;
    a.omega = prm->omega;
    a.delta = prm->delta;
    a.noise_on = prm->noise_on ? 1u : 0u;
    a.seed = prm->noise_seed;
    a.target = target;
    a.score = score_fx;
    a.pi = pi;
    a.flags = c->flags;
    NbLists nl;
    nl.list[0] = s.get<u32>(N);
    nl.list[1] = nl.list[2] = nl.list[3] = nl.list[4] = nullptr;
    nl.cnt = s.get<u32>(8);
    NodeRec *recs = s.get<NodeRec>(N);
    NodeRec *big = s.get<NodeRec>(N);
    u32 *work = s.get<u32>(3);
    MatchScratch ms;
    ms.bscore = s.get<u64>(N);
    ms.bid = s.get<u32>(N);
    ms.tk = s.get<uint8_t>(N);
    ms.p0 = ms.p1 = nullptr;
    ms.x0 = ms.x1 = nullptr;
    u32 *npairs = s.get<u32>(1);
    launch_fills(c, {{c->flags, 64, 0, false}, {nl.cnt, 8, 0, false}, {work, 3, 0, false}});
    if (!batched) {
      launch_rate_classify(c, a, 0, N, nl, recs, big);
      launch_check(c, "rate classes");
      launch_rate(c, a, nl, recs, N, big, work);
      launch_check(c, "rate");
    } else {
      rate_batched(c, s, g, a, nl, recs, big, work);
    }
    if (pi == 1) {
      match_proposals(c, s, N, target, score_fx, ms, npairs, match, n_pairs_host);
      return;
    }
    // pi rounds; a round that pairs nothing leaves the next one's proposals,
    // and so its matching, unchanged, so the rounds stop there
    u32 *tr = s.get<u32>(N);
    u64 *sr = s.get<u64>(N);
    u32 *mr = s.get<u32>(N);
    launch_iota(c, N, match);
    u32 total = 0;
    for (u32 r = 0; r < pi; ++r) {
      launch_round_prep(c, N, pi, target, score_fx, match, tr, sr);
      u32 round_pairs = 0;
      match_proposals(c, s, N, tr, sr, ms, npairs, mr, &round_pairs);
      if (round_pairs == 0) break;
      launch_round_merge(c, N, mr, match);
      total += round_pairs;
      launch_fill_u32(c, c->flags, 1, 0);  // a long chain of this round is not the next one's
    }
    launch_check(c, "matching rounds");
    *n_pairs_host = total;
  });
}

}  // namespace

int chp_rate_and_match(chp_ctx *c, const chp_hgraph *g, const chp_params *prm, u32 *target,
                       u64 *score_fx, u32 *match, u32 *n_pairs_host, uint8_t *nb_invalid) {
  return rate_top_and_match(c, g, prm, 1, target, score_fx, match, n_pairs_host, nb_invalid);
}

int chp_rate_top_and_match(chp_ctx *c, const chp_hgraph *g, const chp_params *prm, uint32_t pi,
                           u32 *target, u64 *score_fx, u32 *match, u32 *n_pairs_host,
                           uint8_t *nb_invalid) {
  return rate_top_and_match(c, g, prm, pi, target, score_fx, match, n_pairs_host, nb_invalid);
}

int chp_propose_moves(chp_ctx *c, const chp_hgraph *g, const u32 *rho, u32 k,
                      const chp_params *prm, int enforce_omega, u32 *move, i64 *gain) {
  return guarded(c, [&] {
    if (!g || !prm || (g->n_nodes && (!rho || !move || !gain))) {
      set_err(c, "%snull argument");
      throw Fail{CHP_EINVAL};
    }
    const u32 N = g->n_nodes, E = g->n_edges;
    if (N == 0) return;
    if (k == 0) {
      set_err(c, "%sk must be positive");
      throw Fail{CHP_EINVAL};
    }
    Scratch s(c);
    clear_flags(c);
    u64 *part_size = s.get<u64>(k);
    u32 *part_cnt = s.get<u32>(k);
    u32 *cnt = s.get<u32>(3);  // light, heavy, heavy work counter
    launch_fills(c, {{part_size, k, 0, true}, {part_cnt, k, 0, false}, {cnt, 3, 0, false}});
    launch_eval_nodes(c, N, rho, k, g->n_size, part_size, part_cnt);
    // pins(., e) of every hyperedge
    u32 hc[8];
    EdgeLists el = make_edge_lists(c, s, E, g->e_off, hc);
    u64 *pl = s.get<u64>(g->n_pins ? g->n_pins : 1);
    u32 *lam = s.get<u32>(E ? E : 1);
    u64 *scr = nullptr;
    u64 per_wg = 0;
    const u32 gb = grid_big_for(hc[2]);
    if (hc[2]) {
      per_wg = 2ull * hc[3];
      scr = s.get<u64>(per_wg * gb);
    }
    launch_pins_lists(c, g->e_off, g->e_pins, rho, k, pl, lam, el, hc, scr, per_wg, gb);
    // admissible partitions (Omega enforced)
    u32 K2 = 1;
    while (K2 < k) K2 <<= 1;
    u64 *tree = nullptr;
    if (enforce_omega) {
      tree = s.get<u64>(2ull * K2);
      launch_free_tree(c, k, K2, part_size, prm->omega, tree);
    }
    u32 *lists = s.get<u32>(N);
    launch_gains(c, N, k, K2, enforce_omega, prm->omega, g->e_off, g->e_w, pl, lam, g->n_off,
                 g->n_inc, g->n_size, rho, part_size, tree, move, gain, lists, cnt, nullptr);
    launch_check(c, "move classes");
    u32 gc[2], f;
    read_many(c, {{gc, cnt, sizeof gc}, {&f, c->flags, sizeof f}});
    if (f & FLAG_EINVAL) fail_flags(c, FLAG_EINVAL, "rho has an entry >= k");
    launch_gains(c, N, k, K2, enforce_omega, prm->omega, g->e_off, g->e_w, pl, lam, g->n_off,
                 g->n_inc, g->n_size, rho, part_size, tree, move, gain, lists, cnt, gc);
    launch_check(c, "moves");
    read_many(c, {{&f, c->flags, sizeof f}});
    if (f & FLAG_EINVAL) fail_flags(c, FLAG_EINVAL, "rho has an entry >= k");
  });
}

// Chains over the moves in gain order sq (rank = their positions): sq and
// rank are rewritten in chain order.
void build_chains(chp_ctx *c, Scratch &s, const chp_hgraph *g, u32 M, u32 k, const u32 *rho,
                  const u32 *move, const i64 *gain, u32 *sq, u32 *rank) {
  ChainBufs B;
  u32 **u32s[] = {&B.node, &B.size, &B.nin, &B.dest, &B.pred, &B.succ, &B.pick, &B.wid,
                  &B.anc, &B.anc2, &B.mn, &B.mn2, &B.cut, &B.dist, &B.clen, &B.cstart};
  for (u32 **p : u32s) *p = s.get<u32>(M);
  B.posn = s.get<u32>(g->n_nodes);
  B.pstart = s.get<u32>((u64)k + 1);
  B.done = s.get<u32>(M);
  B.gain = s.get<i64>(M);
  B.pgr = s.get<i64>(M);
  B.wgr = s.get<i64>(M);
  B.ctot = s.get<i64>(M);
  u64 *ck = s.get<u64>(M);
  u64 *ctmp = s.get<u64>(M);
  u32 *cc = s.get<u32>(2);  // links of a round, chain heads
  launch_fills(c, {{B.ctot, M, 0, true}, {B.clen, M, 0, false}, {cc, 2, 0, false},
                   {B.done, M, 0, false}});
  const u64 *sorted = nullptr;
  launch_chain_setup(c, M, k, sq, rho, move, g->n_size, g->n_nin, gain, ck, ctmp, B, &sorted);
  for (u32 round = 0; round < CHAIN_ROUNDS; ++round) {
    launch_fill_u32(c, cc, 1, 0);
    launch_chain_round(c, M, B, cc);
    launch_check(c, "chain round");
    u32 links = 0;
    read_many(c, {{&links, cc, sizeof links}});
    if (links == 0) break;
  }
  launch_chain_walk(c, M, B);
  u32 *heads = s.get<u32>(M);
  u64 *hk = s.get<u64>(M);
  u64 *htmp = s.get<u64>(M);
  launch_chain_heads(c, M, B, heads, hk, cc + 1);
  launch_check(c, "chain heads");
  u32 H = 0;
  read_many(c, {{&H, cc + 1, sizeof H}});
  const u64 *tot = sort_keys_u64(c, hk, htmp, H);
  u64 *rk = tot == hk ? htmp : hk;  // the array the sort left free
  launch_chain_rank_keys(c, H, heads, B, tot, ck);
  const u64 *order = sort_keys_u64(c, ck, rk, H);
  u32 *lens = B.mn;  // free after the walk
  launch_chain_lens(c, H, order, B, lens);
  i64 *coff = s.get<i64>((u64)H + 1);
  i64 *stmp = s.get<i64>(scan_tmp_words(H));
  scan_u32_to_i64(c, lens, coff, H, stmp);
  launch_chain_place(c, M, H, order, coff, B, sq, rank);
}

int chp_refine_moves(chp_ctx *c, const chp_hgraph *g, u32 *rho, u32 k, const chp_params *prm,
                     const u32 *move, const i64 *gain, u32 *seq, i64 *seq_gain, u32 *seq_viol,
                     u32 *n_seq_host, u32 *n_applied_host, i64 *gain_host) {
  return guarded(c, [&] {
    if (!g || !prm || !n_seq_host || !n_applied_host || !gain_host ||
        (g->n_nodes && (!rho || !move || !gain))) {
      set_err(c, "%snull argument");
      throw Fail{CHP_EINVAL};
    }
    *n_seq_host = 0, *n_applied_host = 0, *gain_host = 0;
    const u32 N = g->n_nodes, E = g->n_edges;
    if (N == 0) return;
    if (k == 0) {
      set_err(c, "%sk must be positive");
      throw Fail{CHP_EINVAL};
    }
    if (N >= (1u << 29)) {
      set_err(c, "%srefinement needs fewer than 2^29 nodes");
      throw Fail{CHP_EINVAL};
    }
    Scratch s(c);
    clear_flags(c);
    // -- the sequence: nodes with a move by (gain desc, id asc)
    u64 *keys = s.get<u64>(N);
    u64 *ktmp = s.get<u64>(N);
    u32 *rank = s.get<u32>(N);
    u32 *cnt = s.get<u32>(8);  // [0] moves, [1..4] hyperedge classes, [5] v0, [6] best length
    u64 *best = s.get<u64>(1);
    u64 *size0 = s.get<u64>(k);
    u32 *cnt0 = s.get<u32>(k);
    u32 *inb0 = s.get<u32>(k);
    u32 *lists = s.get<u32>(3ull * (E ? E : 1));
    launch_fills(c, {{cnt, 6, 0, false}, {cnt + 6, 2, NONE32, false}, {rank, N, NONE32, false},
                     {best, 1, 0, true}, {size0, k, 0, true}, {cnt0, k, 0, false},
                     {inb0, k, 0, false}});
    launch_seq_keys(c, N, k, rho, move, gain, keys, cnt);
    if (E) launch_ev_classify(c, E, g->e_off, lists, cnt + 1);
    launch_check(c, "move sequence keys");
    u32 hc[8], f = 0;
    read_many(c, {{hc, cnt, sizeof hc}, {&f, c->flags, sizeof f}});
    if (f & FLAG_EINVAL)
      fail_flags(c, FLAG_EINVAL, "rho or move has an entry >= k, or a move to its own partition");
    if (f & FLAG_EOVERFLOW) fail_flags(c, FLAG_EOVERFLOW, "a gain does not fit in 32 bits");
    const u32 M = hc[0];
    *n_seq_host = M;
    if (M == 0) return;
    if (hc[4] >= (1u << 30)) {
      set_err(c, "%srefinement needs hyperedges of fewer than 2^30 pins");
      throw Fail{CHP_EINVAL};
    }
    const u64 *sk = sort_keys_u64(c, keys, ktmp, M);
    u32 *sq = seq ? seq : s.get<u32>(M);
    launch_seq_rank(c, M, sk, sq, rank);
    if (c->move_order == CHP_ORDER_CHAINS) build_chains(c, s, g, M, k, rho, move, gain, sq, rank);
    // -- per hyperedge: in-sequence gains, inbound transitions, starting inbound counts
    i64 *ingain = s.get<i64>(M);
    i64 *vdelta = s.get<i64>(M);
    u32 *dleave = s.get<u32>(M);
    u32 *denter = s.get<u32>(M);
    launch_fills(c, {{ingain, M, 0, true}, {vdelta, M, 0, true}, {dleave, M, 0, false},
                     {denter, M, 0, false}});
    launch_eval_nodes(c, N, rho, k, g->n_size, size0, cnt0);
    u64 *escr = nullptr;
    u32 gg = 1;
    if (hc[3]) {
      const u64 per = ev_global_words(hc[4]);
      const u64 budget = (1ull << 31) / 8;  // words of scratch for the long hyperedges
      u64 fit = budget / per;
      gg = hc[3] < 256 ? hc[3] : 256;
      if (fit < gg) gg = fit ? (u32)fit : 1;
      escr = s.get<u64>(per * gg);
    }
    const u32 ec[4] = {hc[1], hc[2], hc[3], hc[4]};
    launch_ev_edges(c, E, g->e_off, g->e_nsrc, g->e_pins, g->e_w, rho, move, rank, ingain, dleave,
                    denter, inb0, lists, cnt + 1, ec, escr, gg);
    // -- per partition: validity flips along the sequence
    const u64 Q = 2ull * M;
    u64 *pk = s.get<u64>(Q);
    u64 *ptmp = s.get<u64>(Q);
    i64 *vs = s.get<i64>(Q);
    i64 *vi = s.get<i64>(Q);
    i64 *Ps = s.get<i64>(Q + 1);
    i64 *Pi = s.get<i64>(Q + 1);
    i64 *Pg = s.get<i64>((u64)M + 1);
    i64 *Pv = s.get<i64>((u64)M + 1);
    i64 *stmp = s.get<i64>(scan_tmp_words(Q));
    launch_pev(c, M, sq, rho, move, pk);
    const u64 *spk = sort_keys_u64(c, pk, ptmp, Q);
    launch_pev_vals(c, Q, spk, sq, g->n_size, dleave, denter, vs, vi);
    scan_i64(c, vs, Ps, Q, stmp);
    scan_i64(c, vi, Pi, Q, stmp);
    launch_pev_flips(c, Q, spk, vs, vi, Ps, Pi, size0, inb0, prm->omega, prm->delta, vdelta);
    launch_viol0(c, k, size0, inb0, prm->omega, prm->delta, cnt + 5);
    scan_i64(c, ingain, Pg, M, stmp);
    scan_i64(c, vdelta, Pv, M, stmp);
    // -- the best valid prefix, applied
    launch_prefix(c, M, ingain, Pg, vdelta, Pv, cnt + 5, seq_gain, seq_viol, best, cnt + 6, sq,
                  move, rho);
    launch_check(c, "refinement");
    u32 L = NONE32;
    u64 b = 0;
    read_many(c, {{&L, cnt + 6, sizeof L}, {&b, best, sizeof b}});
    *n_applied_host = L == NONE32 ? 0 : L;
    *gain_host = (i64)b;
  });
}

int chp_project_partition(chp_ctx *c, uint32_t n_fine, const uint32_t *gamma, uint32_t n_coarse,
                          const uint32_t *rho_coarse, uint32_t *rho_fine) {
  return guarded(c, [&] {
    if (n_fine && (!gamma || !rho_coarse || !rho_fine)) {
      set_err(c, "%snull argument");
      throw Fail{CHP_EINVAL};
    }
    if (n_fine == 0) return;
    clear_flags(c);
    CHP_LAUNCH(c, "project", k_project, grid_for(n_fine, 256), 256, 0, n_fine, gamma, n_coarse,
               rho_coarse, rho_fine, c->flags);
    launch_check(c, "project");
    if (read_flags(c) & FLAG_EINVAL) fail_flags(c, FLAG_EINVAL, "gamma has an id >= n_coarse");
  });
}

int chp_refine_level(chp_ctx *c, const chp_hgraph *g, uint32_t *rho, uint32_t k,
                     const chp_params *prm, uint32_t theta, uint32_t *n_applied_host,
                     int64_t *gain_host) {
  return guarded(c, [&] {
    if (!g || !prm || !n_applied_host || !gain_host || (g->n_nodes && !rho)) {
      set_err(c, "%snull argument");
      throw Fail{CHP_EINVAL};
    }
    *n_applied_host = 0;
    *gain_host = 0;
    const u32 N = g->n_nodes;
    if (N == 0 || theta == 0) return;
    Scratch s(c);
    u32 *move = s.get<u32>(N);
    i64 *gain = s.get<i64>(N);
    for (u32 r = 0; r < theta; ++r) {
      // the first half of the passes may propose moves that overfill a
      // partition; the second half only moves that fit (both apply valid
      // prefixes only)
      int rc = chp_propose_moves(c, g, rho, k, prm, r >= theta / 2 ? 1 : 0, move, gain);
      if (rc != CHP_OK) throw Fail{rc};
      u32 nseq = 0, na = 0;
      i64 ga = 0;
      rc = chp_refine_moves(c, g, rho, k, prm, move, gain, nullptr, nullptr, nullptr, &nseq, &na,
                            &ga);
      if (rc != CHP_OK) throw Fail{rc};
      *n_applied_host += na;
      *gain_host += ga;
    }
  });
}

int chp_pair_leftovers(chp_ctx *c, const chp_hgraph *g, const chp_params *prm,
                       const u32 *target, u32 *match, u32 *n_pairs_host) {
  return guarded(c, [&] {
    if (!g || !prm || !n_pairs_host || (g->n_nodes && (!target || !match))) {
      set_err(c, "%snull argument");
      throw Fail{CHP_EINVAL};
    }
    *n_pairs_host = 0;
    const u32 N = g->n_nodes;
    if (N < 2) return;
    Scratch s(c);
    u64 *keys = s.get<u64>(N);
    u64 *tmp = s.get<u64>(N);
    u32 *claim = s.get<u32>(N);
    u32 *choice = s.get<u32>(N);
    u32 *cnt = s.get<u32>(4);  // gathered, pairs, smallest size, smallest |in|
    launch_fills(c, {{cnt, 2, 0, false}, {cnt + 2, 2, NONE32, false}});
    launch_left_gather(c, N, target, match, g->n_size, g->n_nin, keys, cnt);
    launch_check(c, "leftover gather");
    u32 hc[4] = {0, 0, 0, 0};
    read_many(c, {{hc, cnt, sizeof hc}});
    const u32 nl = hc[0];
    // no two gathered nodes fit together: nothing to pair
    if (nl < 2 || 2 * (u64)hc[2] > prm->omega || 2 * (u64)hc[3] > (u64)prm->delta) return;
    launch_fill_u32(c, claim, N, NONE32);
    const u64 *sorted = sort_keys_u64(c, keys, tmp, nl);
    launch_left_pair(c, nl, sorted, g->n_nin, prm->omega, prm->delta, LEFT_WINDOW, choice, claim,
                     match, cnt + 1);
    launch_check(c, "leftover pairing");
    read_many(c, {{n_pairs_host, cnt + 1, sizeof(u32)}});
  });
}

int chp_contract(chp_ctx *c, const chp_hgraph *g, const u32 *match, u32 *gamma,
                 int build_neighbors, chp_hgraph *coarse, const uint8_t *nb_invalid) {
  return guarded(c, [&] {
    if (!g || !coarse || (g->n_nodes && (!match || !gamma))) {
      set_err(c, "%snull argument");
      throw Fail{CHP_EINVAL};
    }
    const u32 N = g->n_nodes, E = g->n_edges;
    const u64 P = g->n_pins;
    const bool merge_nb = build_neighbors && g->nb_off && g->nb;
    const uint8_t *purge = merge_nb ? nb_invalid : nullptr;
    if (purge && N >= 0x7FFFFFFFu) {
      set_err(c, "%sneighbour purge needs fewer than 2^31 - 1 nodes");
      throw Fail{CHP_EINVAL};
    }
    Scratch s(c);
    Owned own(c);
    // -- representatives and hyperedge classes, then the first readback
    u32 *is_rep = s.get<u32>(N);
    i64 *rank = s.get<i64>((u64)N + 1);
    i64 *tmp = s.get<i64>(scan_tmp_words(N > E ? N : E));
    EdgeLists el;
    for (int k = 0; k < 3; ++k) el.list[k] = s.get<u32>(E);
    el.list[3] = nullptr;
    el.cnt = s.get<u32>(8);
    EdgeLists il;
    il.cnt = s.get<u32>(8);
    NbLists nl;
    nl.cnt = s.get<u32>(8);
    launch_fills(c, {{c->flags, 64, 0, false},
                     {el.cnt, 8, 0, false},
                     {il.cnt, 8, 0, false},
                     {nl.cnt, 8, 0, false}});
    launch_rep(c, N, match, is_rep);
    scan_u32_to_i64(c, is_rep, rank, N, tmp);
    launch_edge_classify(c, E, g->e_off, el);
    launch_check(c, "representatives");
    i64 nc;
    u32 f, he[8];
    read_many(c, {{&nc, rank + N, sizeof nc}, {&f, c->flags, sizeof f}, {he, el.cnt, sizeof he}});
    if (f & FLAG_EINVAL) fail_flags(c, FLAG_EINVAL, "match is not a symmetric pairing");
    const u32 Nc = (u32)nc;
    chp_hgraph cg;
    memset(&cg, 0, sizeof cg);
    cg.n_nodes = Nc;
    cg.n_edges = E;
    cg.n_size = own.get<u32>(Nc);
    cg.e_w = own.get<u32>(E);
    cg.e_off = own.get<i64>((u64)E + 1);
    cg.e_nsrc = own.get<u32>(E);
    cg.n_off = own.get<i64>((u64)Nc + 1);
    cg.n_nin = own.get<u32>(Nc);
    d2d(c, cg.e_w, g->e_w, sizeof(u32) * (size_t)E);
    u32 *rep_of = s.get<u32>(Nc);
    launch_gamma(c, N, match, rank, g->n_size, gamma, cg.n_size, rep_of);
    // -- coarse hyperedges (oversize, then packed)
    u64 *escr = nullptr;
    u64 eper = 0;
    const u32 egb = grid_big_for(he[2]);
    if (he[2]) {
      eper = 2ull * he[3];
      escr = s.get<u64>(eper * egb);
    }
    u32 *opins = s.get<u32>(P);
    u32 *olen = s.get<u32>(E);
    // the wave class above the tiny size (twice its count), then the LDS class
    // split by size (twice its count)
    u32 *erest = s.get<u32>(2ull * he[0] + 2ull * he[1] + 1);
    launch_edge_contract(c, g->e_off, g->e_nsrc, g->e_pins, gamma, opins, olen, cg.e_nsrc, el, he,
                         escr, eper, egb, erest, Nc < (1u << 31) - 1);
    scan_u32_to_i64(c, olen, cg.e_off, E, tmp);
    // -- coarse incidence classes: in'(c) = in(a) u in(b), out' = (out(a) u out(b)) \ in'
    u32 *ibound = s.get<u32>(Nc), *icnt = s.get<u32>(Nc);
    for (int k = 0; k < 4; ++k) il.list[k] = s.get<u32>(Nc);
    launch_cinc_classify(c, Nc, rep_of, match, g->n_off, g->n_nin, ibound, cg.n_nin, icnt, il);
    i64 *iooff = s.get<i64>((u64)Nc + 1);
    i64 *tmp2 = s.get<i64>(scan_tmp_words(Nc));
    scan_u32_to_i64(c, ibound, iooff, Nc, tmp2);
    // -- coarse neighbour classes: N'(c) = gamma(N(a) u N(b)) \ {c}
    u32 *nbound = nullptr;
    i64 *nooff = nullptr;
    i64 *tmp3 = nullptr;
    if (merge_nb) {
      nbound = s.get<u32>(Nc);
      for (int k = 0; k < 4; ++k) nl.list[k] = s.get<u32>(Nc);
      nl.list[4] = nullptr;
      launch_nbm_classify(c, Nc, rep_of, match, g->nb_off, nbound, nl);
      nooff = s.get<i64>((u64)Nc + 1);
      tmp3 = s.get<i64>(scan_tmp_words(Nc));
      scan_u32_to_i64(c, nbound, nooff, Nc, tmp3);
    }
    launch_check(c, "coarse classes");
    i64 pc = 0, itot = 0, ntot = 0;
    u32 hi[8] = {0}, hn[8] = {0};
    if (merge_nb)
      read_many(c, {{&pc, cg.e_off + E, sizeof pc},
                    {&itot, iooff + Nc, sizeof itot},
                    {hi, il.cnt, sizeof hi},
                    {&ntot, nooff + Nc, sizeof ntot},
                    {hn, nl.cnt, sizeof hn}});
    else
      read_many(c, {{&pc, cg.e_off + E, sizeof pc},
                    {&itot, iooff + Nc, sizeof itot},
                    {hi, il.cnt, sizeof hi}});
    if (hn[7]) {
      set_err(c, "%sa cluster's neighbour lists exceed 2^32 entries");
      throw Fail{CHP_EOVERFLOW};
    }
    cg.n_pins = (u64)pc;
    cg.e_pins = own.get<u32>((u64)pc);
    launch_pins_compact(c, E, g->e_off, opins, cg.e_off, cg.e_pins);
    // -- coarse incidence
    u32 *iobuf = s.get<u32>((u64)itot);
    u64 *iscr = nullptr;
    u64 iper = 0;
    const u32 igb = grid_big_for(hi[2]);
    if (hi[2]) {
      iper = 2ull * hi[4];  // the largest bound of the global class
      iscr = s.get<u64>(iper * igb);
    }
    launch_cinc_build(c, g->n_off, g->n_nin, g->n_inc, rep_of, match, iooff, iobuf, cg.n_nin,
                      icnt, il, hi, iscr, iper, igb, E < (1u << 31) - 1);
    scan_u32_to_i64(c, icnt, cg.n_off, Nc, tmp2);
    cg.n_inc = own.get<u32>(cg.n_pins);  // |I'| summed over clusters = pins of G'
    launch_cinc_compact(c, Nc, rep_of, match, g->n_off, g->n_inc, iooff, iobuf, cg.n_off,
                        cg.n_inc);
    launch_check(c, "coarse incidence");
    // -- coarse neighbours
    if (merge_nb) {
      cg.nb_off = own.get<i64>((u64)Nc + 1);
      u32 *nobuf = s.get<u32>((u64)ntot);
      u32 *ncount = s.get<u32>(Nc);
      launch_fill_u32(c, ncount, Nc, 0);
      launch_nbm_build(c, g->nb_off, g->nb, purge, gamma, match, rep_of, nooff, nobuf, ncount, nl,
                       hn);
      scan_u32_to_i64(c, ncount, cg.nb_off, Nc, tmp3);
      launch_check(c, "coarse neighbours");
      i64 total;
      read_back(c, &total, cg.nb_off + Nc, sizeof total);
      cg.nb = own.get<u32>((u64)total);
      cg.nb_total = (u64)total;
      launch_nb_compact(c, Nc, nooff, nobuf, cg.nb_off, cg.nb);
      launch_check(c, "coarse neighbour compaction");
    } else if (build_neighbors) {
      build_neighbors_core(c, s, own, &cg);
    }
    own.keep = true;
    *coarse = cg;
  });
}

}  // extern "C"

namespace {

void check_eval_args(chp_ctx *c, const chp_hgraph *g, const u32 *rho, u32 k,
                     const chp_params *prm, u64 *part_size, u32 *part_inb, u64 *summary_host) {
  if (!g || !prm || !summary_host || (g->n_nodes && !rho) || (k && (!part_size || !part_inb))) {
    set_err(c, "%snull argument");
    throw Fail{CHP_EINVAL};
  }
  if (g->n_nodes && k == 0) {
    set_err(c, "%sk must be positive");
    throw Fail{CHP_EINVAL};
  }
}

// The evaluation with every scratch buffer taken from s.
void evaluate_with(chp_ctx *c, Scratch &s, const chp_hgraph *g, const u32 *rho, u32 k,
                   const chp_params *prm, u64 *part_size, u32 *part_inb, u64 *summary_host) {
  const u32 N = g->n_nodes, E = g->n_edges;
  clear_flags(c);
  u64 *summary = s.get<u64>(8);
  u32 *part_cnt = s.get<u32>(k);
  launch_fill_u64(c, summary, 8, 0);
  launch_fill_u64(c, part_size, k, 0);
  launch_fill_u32(c, part_inb, k, 0);
  launch_fill_u32(c, part_cnt, k, 0);
  launch_eval_nodes(c, N, rho, k, g->n_size, part_size, part_cnt);
  u32 hc[8];
  EdgeLists el = make_edge_lists(c, s, E, g->e_off, hc);
  u64 *scr = nullptr;
  u64 per_wg = 0;
  u32 gb = grid_big_for(hc[2]);
  if (hc[2]) {
    per_wg = 2ull * hc[3];
    scr = s.get<u64>(per_wg * gb);
  }
  launch_eval_edges(c, g->e_off, g->e_nsrc, g->e_pins, g->e_w, rho, k, part_inb, summary, el,
                    hc, scr, per_wg, gb);
  launch_eval_parts(c, k, part_size, part_inb, part_cnt, prm->omega, prm->delta, summary);
  launch_check(c, "evaluate");
  u64 sum[8];
  u32 f;
  read_many(c, {{sum, summary, sizeof sum}, {&f, c->flags, sizeof f}});
  if (f & FLAG_EINVAL) fail_flags(c, FLAG_EINVAL, "rho has an entry >= k");
  memcpy(summary_host, sum, sizeof sum);
}

}  // namespace

extern "C" {

int chp_evaluate_partition(chp_ctx *c, const chp_hgraph *g, const u32 *rho, u32 k,
                           const chp_params *prm, u64 *part_size, u32 *part_inb,
                           u64 summary_host[8]) {
  return guarded(c, [&] {
    check_eval_args(c, g, rho, k, prm, part_size, part_inb, summary_host);
    Scratch s(c);
    evaluate_with(c, s, g, rho, k, prm, part_size, part_inb, summary_host);
  });
}

int chp_evaluate_partition_noalloc(chp_ctx *c, const chp_hgraph *g, const u32 *rho, u32 k,
                                   const chp_params *prm, u64 *part_size, u32 *part_inb,
                                   u64 summary_host[8]) {
  if (!c) return CHP_EINVAL;
  // no timing events are recorded inside this call
  const int timing = c->timing;
  c->timing = 0;
  const int rc = guarded(c, [&] {
    check_eval_args(c, g, rho, k, prm, part_size, part_inb, summary_host);
    // everything but the long-hyperedge buffer is known before any work:
    // the summary, k counters, three hyperedge class lists and their counts
    const u64 need = 256 + (((u64)k * 4 + 255) & ~255ull) +
                     3 * (((u64)g->n_edges * 4 + 255) & ~255ull) + 256;
    if (need > FIXED_SCRATCH_BYTES) {
      set_err(c, "%sk and the hyperedge count need %lld bytes of scratch, above the fixed "
                 "67108864", "", (long long)need);
      throw Fail{CHP_EINVAL};
    }
    Scratch s(c, c->fixed_scratch, FIXED_SCRATCH_BYTES);
    evaluate_with(c, s, g, rho, k, prm, part_size, part_inb, summary_host);
  });
  c->timing = timing;
  return rc;
}

}  // extern "C"
