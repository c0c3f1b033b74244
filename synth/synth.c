/*
 * Seeded synthetic directed hypergraphs shaped like the workloads of
 * "Hypergraph Partitioning on GPU with Distinct Incident Hyperedges and Size
 * Constraints" (Ronzani & Silvano): SNN-style graphs shaped after its Table I
 * and VLSI-style netlists shaped after its Table III.
 *
 * This module only draws inputs.  It holds none of the partitioner's
 * arithmetic and is shared, as plain arrays, by the CPU oracle and by the GPU
 * library.
 *
 * Randomness is counter based: every value is a pure function of
 * (seed, stream, counter), so the output does not depend on the number of
 * OpenMP threads.  The mixing function is the splitmix64 output finaliser
 * (Steele, Lea & Flood, "Fast splittable pseudorandom number generators",
 * OOPSLA 2014), applied twice.
 *
 * Output layout (one hyperedge per CSR segment):
 *   e_off[E+1]  int64   segment starts
 *   e_nsrc[E]   uint32  number of source pins (stored first in the segment)
 *   e_pins[P]   uint32  pins: sources ascending, then destinations ascending
 *   e_w[E]      uint32  hyperedge weight
 *   n_size[N]   uint32  node weight
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define SYN_UNIFORM 1 /* src = edge id, |dst| ~ U{kmin..kmax}, dst uniform      */
#define SYN_RING 2    /* 1-D ring, |dst| ~ Poisson, local window with prob p     */
#define SYN_LAYERED 3 /* layers, |dst| ~ lognormal, dst uniform in next layer   */
#define SYN_VLSI 4    /* 2-D grid netlist, |e| ~ power law, Gaussian locality  */
#define SYN_BLOCK 5   /* |dst| ~ Poisson, dst in the src's aligned block w.p. p */

typedef struct {
  int32_t kind;
  uint32_t n_nodes;
  uint32_t n_edges;
  uint32_t kmin, kmax;  /* bounds on the drawn pin count (see kind)         */
  uint32_t wmax;        /* hyperedge weight ~ U{1..wmax}                    */
  uint32_t smax;        /* node weight ~ U{1..smax}                         */
  uint32_t window;      /* ring half-window / block size / layer count      */
  uint32_t grid_w;      /* VLSI grid width (height = n_nodes / grid_w)      */
  uint32_t pad_;
  double lam;           /* Poisson mean, lognormal median, power exponent   */
  double sigma;         /* lognormal sigma, Gaussian sigma in cells         */
  double p_local;       /* probability of a local draw                      */
  uint64_t seed;
} synth_spec;

static inline uint64_t fin64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
  return z ^ (z >> 31);
}

static inline uint64_t rnd(uint64_t seed, uint64_t stream, uint64_t ctr) {
  uint64_t s = fin64(seed + 0x9e3779b97f4a7c15ULL * (stream + 1));
  return fin64(s + 0x9e3779b97f4a7c15ULL * (ctr + 1));
}

static inline double unif01(uint64_t x) { return (double)(x >> 11) * (1.0 / 9007199254740992.0); }

/* Uniform integer in [0, n) by the multiply-high method (Lemire 2019). */
static inline uint32_t below(uint64_t x, uint32_t n) {
  return (uint32_t)(((x >> 32) * (uint64_t)n) >> 32);
}

/* streams: the edge id selects a stream; sub-streams separate the uses */
#define ST_SIZE 0x100000000ULL
#define ST_PIN 0x200000000ULL
#define ST_W 0x300000000ULL
#define ST_NODE 0x400000000ULL
#define ST_PERM 0x500000000ULL
#define ST_SRC 0x600000000ULL

/* ---- discrete distributions by inversion of a tabulated CDF -------------- */

typedef struct {
  uint32_t lo, n;
  double *cdf;
} table_dist;

static int table_poisson(table_dist *t, double lam, uint32_t kmax) {
  t->lo = 0;
  t->n = kmax + 1;
  t->cdf = (double *)malloc(sizeof(double) * t->n);
  if (!t->cdf) return -1;
  double acc = 0.0;
  for (uint32_t k = 0; k < t->n; ++k) {
    double lp = -lam + k * log(lam) - lgamma((double)k + 1.0);
    acc += exp(lp);
    t->cdf[k] = acc;
  }
  t->cdf[t->n - 1] = 2.0; /* mass above kmax folds into kmax */
  return 0;
}

static int table_power(table_dist *t, double alpha, uint32_t kmin, uint32_t kmax) {
  t->lo = kmin;
  t->n = kmax - kmin + 1;
  t->cdf = (double *)malloc(sizeof(double) * t->n);
  if (!t->cdf) return -1;
  double acc = 0.0;
  for (uint32_t i = 0; i < t->n; ++i) {
    acc += pow((double)(kmin + i), -alpha);
    t->cdf[i] = acc;
  }
  for (uint32_t i = 0; i < t->n; ++i) t->cdf[i] /= acc;
  t->cdf[t->n - 1] = 2.0;
  return 0;
}

static uint32_t table_draw(const table_dist *t, double u) {
  uint32_t lo = 0, hi = t->n - 1; /* first index with cdf > u */
  while (lo < hi) {
    uint32_t mid = (lo + hi) >> 1;
    if (t->cdf[mid] > u) hi = mid;
    else lo = mid + 1;
  }
  return t->lo + lo;
}

static double gauss(uint64_t a, uint64_t b) { /* Box-Muller, one normal */
  double u1 = unif01(a), u2 = unif01(b);
  if (u1 < 1e-300) u1 = 1e-300;
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2);
}

static uint32_t clampu(long long v, uint32_t lo, uint32_t hi) {
  if (v < (long long)lo) return lo;
  if (v > (long long)hi) return hi;
  return (uint32_t)v;
}

/* ---- per-edge shape ------------------------------------------------------- */

static uint32_t edge_src(const synth_spec *s, uint32_t e) {
  if (s->kind == SYN_VLSI) return below(rnd(s->seed, ST_SRC + e, 0), s->n_nodes);
  return e; /* one outbound hyperedge per node */
}

/* number of destination pins of edge e */
static uint32_t edge_ndst(const synth_spec *s, const table_dist *t, uint32_t e) {
  uint64_t x = rnd(s->seed, ST_SIZE + e, 0);
  switch (s->kind) {
    case SYN_UNIFORM:
      return s->kmin + below(x, s->kmax - s->kmin + 1);
    case SYN_RING:
    case SYN_BLOCK:
      return clampu(table_draw(t, unif01(x)), s->kmin, s->kmax);
    case SYN_LAYERED: {
      double z = gauss(x, rnd(s->seed, ST_SIZE + e, 1));
      double v = floor(exp(log(s->lam) + s->sigma * z));
      if (v > 4e9) v = 4e9;
      return clampu((long long)v, s->kmin, s->kmax);
    }
    case SYN_VLSI:
      return table_draw(t, unif01(x)) - 1; /* pin count includes the source */
  }
  return 0;
}

/* One candidate destination for edge e (src = src), draw number c. */
static uint32_t draw_dst(const synth_spec *s, uint32_t e, uint32_t src, uint64_t c, int *ok) {
  uint64_t x = rnd(s->seed, ST_PIN + e, 2 * c);
  uint64_t y = rnd(s->seed, ST_PIN + e, 2 * c + 1);
  uint32_t N = s->n_nodes;
  *ok = 1;
  switch (s->kind) {
    case SYN_UNIFORM:
      return below(x, N);
    case SYN_RING: {
      if (unif01(y) < s->p_local) {
        uint32_t off = 1 + below(x, s->window);
        int neg = (int)((x >> 7) & 1);
        uint64_t v = neg ? ((uint64_t)src + N - (off % N)) % N : ((uint64_t)src + off) % N;
        return (uint32_t)v;
      }
      return below(x, N);
    }
    case SYN_LAYERED: {
      uint32_t L = s->window, per = N / L;
      uint32_t layer = src / per;
      uint32_t next = (layer + 1) % L;
      return next * per + below(x, per);
    }
    case SYN_BLOCK: {
      if (unif01(y) < s->p_local) {
        uint32_t B = s->window;
        uint32_t b0 = (src / B) * B;
        uint32_t bl = (b0 + B <= N) ? B : (N - b0);
        return b0 + below(x, bl);
      }
      return below(x, N);
    }
    case SYN_VLSI: {
      uint32_t W = s->grid_w, H = N / W;
      long long sx = src % W, sy = src / W;
      long long dx = llround(s->sigma * gauss(x, y));
      long long dy = llround(s->sigma * gauss(rnd(s->seed, ST_PIN + e, 0x40000000ULL + 2 * c),
                                                 rnd(s->seed, ST_PIN + e, 0x40000000ULL + 2 * c + 1)));
      long long px = sx + dx, py = sy + dy;
      if (px < 0 || py < 0 || px >= W || py >= H) {
        *ok = 0;
        return 0;
      }
      return (uint32_t)(py * W + px);
    }
  }
  *ok = 0;
  return 0;
}

static int cmp_u32(const void *a, const void *b) {
  uint32_t x = *(const uint32_t *)a, y = *(const uint32_t *)b;
  return (x > y) - (x < y);
}

static int make_table(const synth_spec *s, table_dist *t) {
  t->cdf = NULL;
  if (s->kind == SYN_RING || s->kind == SYN_BLOCK) return table_poisson(t, s->lam, s->kmax);
  if (s->kind == SYN_VLSI) return table_power(t, s->lam, s->kmin, s->kmax);
  return 0;
}

/* Pass 1: pin count per edge (1 source + destinations). */
int synth_edge_sizes(const synth_spec *s, uint32_t *e_size) {
  table_dist t;
  if (make_table(s, &t)) return -1;
  long long E = s->n_edges;
#pragma omp parallel for schedule(static)
  for (long long e = 0; e < E; ++e) e_size[e] = 1 + edge_ndst(s, &t, (uint32_t)e);
  free(t.cdf);
  return 0;
}

/* Pass 2: fill pins (given offsets from pass 1), weights and node sizes. */
int synth_fill(const synth_spec *s, const int64_t *e_off, uint32_t *e_nsrc, uint32_t *e_pins,
               uint32_t *e_w, uint32_t *n_size) {
  table_dist t;
  if (make_table(s, &t)) return -1;
  long long E = s->n_edges;
  int bad = 0;
#pragma omp parallel
  {
    uint32_t cap = 0;
    uint32_t *hs = NULL; /* open-addressing set of accepted ids */
#pragma omp for schedule(dynamic, 256)
    for (long long ee = 0; ee < E; ++ee) {
      uint32_t e = (uint32_t)ee;
      uint32_t src = edge_src(s, e);
      uint32_t k = (uint32_t)(e_off[e + 1] - e_off[e]) - 1;
      uint32_t need = 1;
      while (need < 4 * (k + 1)) need <<= 1;
      if (need > cap) {
        free(hs);
        cap = need;
        hs = (uint32_t *)malloc(sizeof(uint32_t) * cap);
      }
      memset(hs, 0xff, sizeof(uint32_t) * need);
      uint32_t mask = need - 1;
      /* the source is never a destination */
      hs[fin64(src) & mask] = src;
      uint32_t *out = e_pins + e_off[e];
      out[0] = src;
      uint32_t got = 0;
      uint64_t c = 0, limit = 1000ULL * (k + 1) + 1000000ULL;
      while (got < k) {
        if (c > limit) {
#pragma omp atomic write
          bad = 1;
          break;
        }
        int ok;
        uint32_t v = draw_dst(s, e, src, c++, &ok);
        if (!ok) continue;
        uint32_t h = (uint32_t)(fin64(v) & mask);
        int dup = 0;
        while (hs[h] != 0xffffffffu) {
          if (hs[h] == v) {
            dup = 1;
            break;
          }
          h = (h + 1) & mask;
        }
        if (dup) continue;
        hs[h] = v;
        out[1 + got++] = v;
      }
      qsort(out + 1, k, sizeof(uint32_t), cmp_u32);
      e_nsrc[e] = 1;
      e_w[e] = 1 + below(rnd(s->seed, ST_W + e, 0), s->wmax);
    }
    free(hs);
  }
  long long N = s->n_nodes;
#pragma omp parallel for schedule(static)
  for (long long n = 0; n < N; ++n)
    n_size[n] = 1 + below(rnd(s->seed, ST_NODE + (uint64_t)n, 0), s->smax);
  free(t.cdf);
  return bad ? -2 : 0;
}

/* A seeded permutation (Fisher-Yates over the counter stream). */
void synth_permutation(uint64_t seed, uint32_t n, uint32_t *perm) {
  for (uint32_t i = 0; i < n; ++i) perm[i] = i;
  for (uint32_t i = n; i > 1; --i) {
    uint32_t j = below(rnd(seed, ST_PERM, i), i);
    uint32_t tmp = perm[i - 1];
    perm[i - 1] = perm[j];
    perm[j] = tmp;
  }
}

/* Generic seeded uniform integers in [0, bound) (for test partitions etc.). */
void synth_uniform_u32(uint64_t seed, uint64_t stream, uint64_t n, uint32_t bound, uint32_t *out) {
  long long nn = (long long)n;
#pragma omp parallel for schedule(static)
  for (long long i = 0; i < nn; ++i) out[i] = below(rnd(seed, stream, (uint64_t)i), bound);
}
