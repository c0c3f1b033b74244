/*
 * CPU ORACLE -- test infrastructure only.
 *
 * A plain, slow statement of what one constrained coarsening
 * level and the partition evaluation compute, written from the definitions in
 *   [P1] Ronzani & Silvano, "Hypergraph Partitioning on GPU with Distinct
 *        Incident Hyperedges and Size Constraints" (TPDS submission), and
 *   [P2] Ronzani & Silvano, "Incidence Constraints in Hypergraph Partitioning
 *        on GPU" (AsHES 2026 prototype).
 * Only the tests, the smoke check and the CPU-baseline leg of the benchmark
 * may load this file.  It shares no code with the GPU library.
 *
 * Every array is a plain CSR.  Ids are uint32 (0xFFFFFFFF = none), offsets
 * int64, weights and sizes uint32, fixed-point scores uint64.  Every set is
 * stored sorted ascending (the canonical form both sides compare bit-exactly).
 *
 * Readings of the pages that the text leaves open are applied here exactly as
 * stated next to each function; the same readings are listed in the design
 * notes of the repository.
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_OK 0
#define OR_EINVAL (-1)
#define OR_ENOMEM (-2)
#define OR_EOVERFLOW (-3)
#define OR_EINFEASIBLE (-4)
#define OR_ECYCLE (-5)
#define OR_EINTERNAL (-7)

#define NONE 0xFFFFFFFFu
#define FX_SHIFT 40 /* fixed-point scale of the rating: 2^40 */

typedef struct {
  uint32_t n_nodes, n_edges;
  const int64_t *e_off;   /* [E+1] */
  const uint32_t *e_nsrc; /* [E]   sources are stored first in a segment */
  const uint32_t *e_pins; /* [P]   */
  const uint32_t *e_w;    /* [E]   */
  const uint32_t *n_size; /* [N]   */
} or_edges;

void or_free(void *p) { free(p); }

static int cmp_u32(const void *a, const void *b) {
  uint32_t x = *(const uint32_t *)a, y = *(const uint32_t *)b;
  return (x > y) - (x < y);
}

/* membership in a sorted array, by plain binary search */
static int sorted_has(const uint32_t *a, int64_t n, uint32_t v) {
  int64_t lo = 0, hi = n;
  while (lo < hi) {
    int64_t mid = lo + (hi - lo) / 2;
    if (a[mid] < v) lo = mid + 1;
    else hi = mid;
  }
  return lo < n && a[lo] == v;
}

/* ------------------------------------------------------------------------ */
/* O1: canonical form and validation.                                       */
/* [P1] Sec. II-A: an h-edge is a set of pins split into src(e) and dst(e)   */
/* with src(e) and dst(e) disjoint; omega maps h-edges to weights.           */
/* [P1] Sec. II-B: |p| <= Omega and at most Delta distinct inbound h-edges   */
/* per partition, and a valid solution is assumed to exist -- so a node that */
/* alone breaks a limit is reported as infeasible.                           */
/* Precedence of errors: EINVAL, then EOVERFLOW, then EINFEASIBLE.           */
/* Writes every edge's src and dst sub-lists sorted into pins_out.           */
/* ------------------------------------------------------------------------ */
int or_canonicalize(const or_edges *g, uint64_t omega, uint32_t delta, uint32_t *pins_out) {
  uint32_t N = g->n_nodes, E = g->n_edges;
  if (N == 0xFFFFFFFFu || E == 0xFFFFFFFFu) return OR_EOVERFLOW;
  if (g->e_off[0] != 0) return OR_EINVAL;
  for (uint32_t e = 0; e < E; ++e) {
    int64_t a = g->e_off[e], b = g->e_off[e + 1];
    if (b <= a) return OR_EINVAL; /* an h-edge holds at least one pin */
    if ((int64_t)g->e_nsrc[e] > b - a) return OR_EINVAL;
    if (g->e_w[e] == 0) return OR_EINVAL;
  }
  for (uint32_t n = 0; n < N; ++n)
    if (g->n_size[n] == 0) return OR_EINVAL;
  int64_t P = g->e_off[E];
  memcpy(pins_out, g->e_pins, sizeof(uint32_t) * (size_t)P);
  for (int64_t i = 0; i < P; ++i)
    if (pins_out[i] >= N) return OR_EINVAL;
  for (uint32_t e = 0; e < E; ++e) {
    int64_t a = g->e_off[e], b = g->e_off[e + 1];
    uint32_t ns = g->e_nsrc[e];
    uint32_t *src = pins_out + a, *dst = pins_out + a + ns;
    int64_t nd = b - a - ns;
    qsort(src, ns, sizeof(uint32_t), cmp_u32);
    qsort(dst, (size_t)nd, sizeof(uint32_t), cmp_u32);
    for (uint32_t i = 1; i < ns; ++i)
      if (src[i] == src[i - 1]) return OR_EINVAL; /* duplicate pin */
    for (int64_t i = 1; i < nd; ++i)
      if (dst[i] == dst[i - 1]) return OR_EINVAL;
    for (uint32_t i = 0; i < ns; ++i)
      if (sorted_has(dst, nd, src[i])) return OR_EINVAL; /* src and dst overlap */
  }
  for (uint32_t e = 0; e < E; ++e)
    if (g->e_w[e] >= (1u << 24)) return OR_EOVERFLOW; /* omega * 2^40 must fit 64 bits */
  /* feasibility of single nodes */
  uint32_t *indeg = (uint32_t *)calloc(N ? N : 1, sizeof(uint32_t));
  if (!indeg) return OR_ENOMEM;
  for (uint32_t e = 0; e < E; ++e)
    for (int64_t i = g->e_off[e] + g->e_nsrc[e]; i < g->e_off[e + 1]; ++i) indeg[pins_out[i]]++;
  int rc = OR_OK;
  for (uint32_t n = 0; n < N; ++n)
    if ((uint64_t)g->n_size[n] > omega || indeg[n] > delta) rc = OR_EINFEASIBLE;
  free(indeg);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* O2: incidence sets.  [P1] Sec. II-A: in(n) = {e : n in dst(e)},          */
/* out(n) = {e : n in src(e)}, I(n) = in(n) u out(n).  [P1] Sec. IV-B,      */
/* Fig. 2: one segment per node, inbound ids stored first, |in(n)| kept in   */
/* a second array.  Edges are visited in ascending id, so each list is       */
/* produced sorted.                                                          */
/* ------------------------------------------------------------------------ */
int or_incidence(const or_edges *g, int64_t *n_off, uint32_t *n_nin, uint32_t *n_inc) {
  uint32_t N = g->n_nodes, E = g->n_edges;
  uint32_t *nout = (uint32_t *)calloc(N ? N : 1, sizeof(uint32_t));
  int64_t *fin = (int64_t *)malloc(sizeof(int64_t) * (N ? N : 1));
  int64_t *fout = (int64_t *)malloc(sizeof(int64_t) * (N ? N : 1));
  if (!nout || !fin || !fout) {
    free(nout), free(fin), free(fout);
    return OR_ENOMEM;
  }
  memset(n_nin, 0, sizeof(uint32_t) * N);
  for (uint32_t e = 0; e < E; ++e)
    for (int64_t i = g->e_off[e]; i < g->e_off[e + 1]; ++i) {
      uint32_t n = g->e_pins[i];
      if (i < g->e_off[e] + g->e_nsrc[e]) nout[n]++;
      else n_nin[n]++;
    }
  n_off[0] = 0;
  for (uint32_t n = 0; n < N; ++n) n_off[n + 1] = n_off[n] + n_nin[n] + nout[n];
  for (uint32_t n = 0; n < N; ++n) {
    fin[n] = n_off[n];
    fout[n] = n_off[n] + n_nin[n];
  }
  for (uint32_t e = 0; e < E; ++e)
    for (int64_t i = g->e_off[e]; i < g->e_off[e + 1]; ++i) {
      uint32_t n = g->e_pins[i];
      if (i < g->e_off[e] + g->e_nsrc[e]) n_inc[fout[n]++] = e;
      else n_inc[fin[n]++] = e;
    }
  free(nout), free(fin), free(fout);
  return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* O3: unique neighbourhoods.  [P1] Sec. II-A: N(n) = {m in e : e in I(n)}  */
/* minus {n}.  [P1] Sec. V-B materialises N(.) as one more CSR.  Output is  */
/* sorted ascending.  *nb_out is malloc'd (free with or_free).               */
/* ------------------------------------------------------------------------ */
int or_neighbors(const or_edges *g, const int64_t *n_off, const uint32_t *n_inc,
                 int64_t *nb_off, uint32_t **nb_out, uint64_t *nb_total) {
  uint32_t N = g->n_nodes;
  uint32_t *seen = (uint32_t *)malloc(sizeof(uint32_t) * (N ? N : 1));
  uint32_t *list = (uint32_t *)malloc(sizeof(uint32_t) * (N ? N : 1));
  if (!seen || !list) {
    free(seen), free(list);
    return OR_ENOMEM;
  }
  for (uint32_t n = 0; n < N; ++n) seen[n] = NONE;
  /* pass 1: sizes */
  nb_off[0] = 0;
  for (uint32_t n = 0; n < N; ++n) {
    uint32_t cnt = 0;
    for (int64_t j = n_off[n]; j < n_off[n + 1]; ++j) {
      uint32_t e = n_inc[j];
      for (int64_t i = g->e_off[e]; i < g->e_off[e + 1]; ++i) {
        uint32_t m = g->e_pins[i];
        if (m != n && seen[m] != n) {
          seen[m] = n;
          cnt++;
        }
      }
    }
    nb_off[n + 1] = nb_off[n] + cnt;
  }
  uint64_t total = (uint64_t)nb_off[N];
  uint32_t *nb = (uint32_t *)malloc(sizeof(uint32_t) * (total ? total : 1));
  if (!nb) {
    free(seen), free(list);
    return OR_ENOMEM;
  }
  for (uint32_t n = 0; n < N; ++n) seen[n] = NONE;
  /* pass 2: contents */
  for (uint32_t n = 0; n < N; ++n) {
    uint32_t cnt = 0;
    for (int64_t j = n_off[n]; j < n_off[n + 1]; ++j) {
      uint32_t e = n_inc[j];
      for (int64_t i = g->e_off[e]; i < g->e_off[e + 1]; ++i) {
        uint32_t m = g->e_pins[i];
        if (m != n && seen[m] != n) {
          seen[m] = n;
          list[cnt++] = m;
        }
      }
    }
    qsort(list, cnt, sizeof(uint32_t), cmp_u32);
    memcpy(nb + nb_off[n], list, sizeof(uint32_t) * cnt);
  }
  free(seen), free(list);
  *nb_out = nb;
  *nb_total = total;
  return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* O4: per-edge rating term and noise cap.                                   */
/* [P1] Eq. 5 adds omega(e)/|e| for every shared h-edge.  Reading: the term  */
/* is held in fixed point, t(e) = floor(omega(e) * 2^40 / |e|), so sums are  */
/* exact and eta(n,m) = eta(m,n) holds bit for bit.  |e| is the pin count of */
/* the current level.                                                        */
/* [P1] Sec. V-C caps the symmetric noise at 10% of the mean h-edge weight.  */
/* Reading: the mean of the normalised weight omega/|e| over all h-edges, so */
/* cap = floor(sum_e t(e) / (10 |E|)) (exact integer division).              */
/* ------------------------------------------------------------------------ */
int or_terms(const or_edges *g, uint64_t *t, uint64_t *cap) {
  unsigned __int128 sum = 0;
  for (uint32_t e = 0; e < g->n_edges; ++e) {
    uint64_t sz = (uint64_t)(g->e_off[e + 1] - g->e_off[e]);
    t[e] = ((uint64_t)g->e_w[e] << FX_SHIFT) / sz;
    sum += t[e];
  }
  *cap = g->n_edges ? (uint64_t)(sum / ((unsigned __int128)10 * g->n_edges)) : 0;
  return OR_OK;
}

/* The noise generator.  [P1] Sec. V-C: rng(min(n,m), max(n,m)).  Reading:   */
/* one output of Vigna's splitmix64 generator whose state is                 */
/* seed XOR (min * 2^32 + max), reduced modulo cap + 1.                      */
static uint64_t splitmix64_once(uint64_t state) {
  uint64_t z = state + 0x9e3779b97f4a7c15ULL;
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
  return z ^ (z >> 31);
}

uint64_t or_noise(uint64_t seed, uint64_t cap, uint32_t n, uint32_t m) {
  uint32_t a = n < m ? n : m, b = n < m ? m : n;
  uint64_t r = splitmix64_once(seed ^ (((uint64_t)a << 32) | b));
  return r % (cap + 1);
}

/* |A u B| for two sorted sets, by a plain merge */
static uint64_t union_size(const uint32_t *a, int64_t na, const uint32_t *b, int64_t nb) {
  int64_t i = 0, j = 0;
  uint64_t u = 0;
  while (i < na && j < nb) {
    if (a[i] < b[j]) i++;
    else if (b[j] < a[i]) j++;
    else i++, j++;
    u++;
  }
  return u + (uint64_t)(na - i) + (uint64_t)(nb - j);
}

typedef struct {
  uint64_t eta;
  uint32_t id;
} cand;

static int cmp_cand(const void *x, const void *y) { /* eta descending, id ascending */
  const cand *a = (const cand *)x, *b = (const cand *)y;
  if (a->eta != b->eta) return a->eta > b->eta ? -1 : 1;
  return (a->id > b->id) - (a->id < b->id);
}

/* ------------------------------------------------------------------------ */
/* O5: candidate proposal for nodes lo..hi-1.                                */
/* [P1] Eq. 5: eta(n,m) = sum over e in I(n) with m in e of omega(e)/|e|     */
/*   (fixed point, see O4), plus the symmetric noise of Sec. V-C once per m. */
/* [P1] Eq. 6: target(n) is the best valid m, ties to the smallest id        */
/*   (Sec. V-C: equal scores go to the lowest-id neighbour);                 */
/*   valid(n,m) <=> size(n)+size(m) <= Omega and |in(n) u in(m)| <= Delta.   */
/* The union is counted by a sorted merge of the two inbound sets ([P2]      */
/* Sec. III-B2 keeps in(.) sorted for this) and cross-checked against the    */
/* identity |in(n)| + |in(m)| - inter(n,m) of [P1] Sec. V-C.                 */
/* A node with no valid neighbour gets target NONE and score 0.              */
/* EOVERFLOW if some node's sum of terms plus cap reaches 2^63.              */
/* ------------------------------------------------------------------------ */
/* The top pi valid candidates ([P1] Sec. V-D: the top-Pi valid neighbours of
 * each histogram) go to target[r * N + n], score[r * N + n] for r < pi, in the
 * order of Eq. 6 (score desc, id asc); missing ones are NONE / 0.
 *
 * Every node is rated on its own (its accumulator is cleared per node), so the
 * node loop may be split over threads: each thread owns its accumulators and
 * takes blocks of consecutive nodes from a shared counter.  The outputs do not
 * depend on the number of threads; the error returned is that of the smallest
 * node that fails. */
typedef struct {
  const or_edges *g;
  const int64_t *n_off;
  const uint32_t *n_nin, *n_inc;
  const uint64_t *t;
  uint64_t cap, omega, seed;
  uint32_t delta, lo, hi, pi;
  int noise_on;
  uint32_t *target;
  uint64_t *score;
  uint32_t next;     /* next node to hand out (atomic) */
  uint32_t bad_node; /* smallest failing node (atomic min), NONE if none */
  int bad_rc;        /* its error (written under bad_mu) */
  pthread_mutex_t bad_mu;
} rate_job;

#define RATE_BLOCK 16 /* nodes a thread takes at a time */

/* Rate node n with the caller's accumulators (eta, inter, seen: one entry
 * per node id; cl: one per node id).  Returns OR_OK or an error. */
static int rate_node(const rate_job *J, uint32_t n, uint64_t *eta, uint32_t *inter,
                     uint32_t *seen, cand *cl) {
  const or_edges *g = J->g;
  const int64_t *n_off = J->n_off;
  const uint32_t *n_nin = J->n_nin, *n_inc = J->n_inc;
  const uint64_t *t = J->t;
  uint32_t N = g->n_nodes;
  /* overflow guard */
  unsigned __int128 bound = J->cap;
  for (int64_t j = n_off[n]; j < n_off[n + 1]; ++j) {
    uint32_t e = n_inc[j];
    if (g->e_off[e + 1] - g->e_off[e] >= 2) bound += t[e];
  }
  if (bound >= ((unsigned __int128)1 << 63)) return OR_EOVERFLOW;
  uint32_t cnt = 0;
  int64_t nin = n_nin[n];
  for (int64_t j = n_off[n]; j < n_off[n + 1]; ++j) {
    uint32_t e = n_inc[j];
    int e_is_in = (j - n_off[n]) < nin; /* e in in(n) */
    int64_t a = g->e_off[e], b = g->e_off[e + 1], d0 = a + g->e_nsrc[e];
    for (int64_t i = a; i < b; ++i) {
      uint32_t m = g->e_pins[i];
      if (m == n) continue;
      if (seen[m] != n) {
        seen[m] = n;
        eta[m] = 0;
        inter[m] = 0;
        cl[cnt++].id = m;
      }
      eta[m] += t[e];
      if (e_is_in && i >= d0) inter[m]++; /* e in in(n) and m in dst(e) */
    }
  }
  for (uint32_t c = 0; c < cnt; ++c) {
    uint32_t m = cl[c].id;
    if (J->noise_on) eta[m] += or_noise(J->seed, J->cap, n, m);
    cl[c].eta = eta[m];
  }
  qsort(cl, cnt, sizeof(cand), cmp_cand);
  for (uint32_t r = 0; r < J->pi; ++r) {
    J->target[(size_t)r * N + n] = NONE;
    J->score[(size_t)r * N + n] = 0;
  }
  const uint32_t *in_n = n_inc + n_off[n];
  uint32_t got = 0;
  for (uint32_t c = 0; c < cnt && got < J->pi; ++c) {
    uint32_t m = cl[c].id;
    if ((uint64_t)g->n_size[n] + g->n_size[m] > J->omega) continue;
    uint64_t u = union_size(in_n, nin, n_inc + n_off[m], n_nin[m]);
    if (u != (uint64_t)n_nin[n] + n_nin[m] - inter[m]) return OR_EINTERNAL;
    if (u > J->delta) continue;
    J->target[(size_t)got * N + n] = m;
    J->score[(size_t)got * N + n] = cl[c].eta;
    ++got;
  }
  return OR_OK;
}

static void *rate_worker(void *arg) {
  rate_job *J = (rate_job *)arg;
  uint32_t N = J->g->n_nodes;
  uint64_t *eta = (uint64_t *)calloc(N ? N : 1, sizeof(uint64_t));
  uint32_t *inter = (uint32_t *)calloc(N ? N : 1, sizeof(uint32_t));
  uint32_t *seen = (uint32_t *)malloc(sizeof(uint32_t) * (N ? N : 1));
  cand *cl = (cand *)malloc(sizeof(cand) * (N ? N : 1));
  if (!eta || !inter || !seen || !cl) {
    pthread_mutex_lock(&J->bad_mu);
    if (J->lo < __atomic_load_n(&J->bad_node, __ATOMIC_RELAXED) || !J->bad_rc) {
      J->bad_node = J->lo;
      J->bad_rc = OR_ENOMEM;
    }
    pthread_mutex_unlock(&J->bad_mu);
    free(eta), free(inter), free(seen), free(cl);
    return NULL;
  }
  for (uint32_t i = 0; i < N; ++i) seen[i] = NONE;
  for (;;) {
    uint32_t b = __atomic_fetch_add(&J->next, RATE_BLOCK, __ATOMIC_RELAXED);
    if (b >= J->hi || b < J->lo) break;
    uint32_t e = J->hi - b < RATE_BLOCK ? J->hi : b + RATE_BLOCK;
    for (uint32_t n = b; n < e; ++n) {
      if (n > __atomic_load_n(&J->bad_node, __ATOMIC_RELAXED)) break;
      int rc = rate_node(J, n, eta, inter, seen, cl);
      if (rc != OR_OK) {
        pthread_mutex_lock(&J->bad_mu);
        if (n < J->bad_node) {
          J->bad_node = n;
          J->bad_rc = rc;
        }
        pthread_mutex_unlock(&J->bad_mu);
        break;
      }
    }
  }
  free(eta), free(inter), free(seen), free(cl);
  return NULL;
}

static int rate_top(const or_edges *g, const int64_t *n_off, const uint32_t *n_nin,
                    const uint32_t *n_inc, const uint64_t *t, uint64_t cap, uint64_t omega,
                    uint32_t delta, int noise_on, uint64_t seed, uint32_t lo, uint32_t hi,
                    uint32_t pi, uint32_t nthreads, uint32_t *target, uint64_t *score) {
  uint32_t N = g->n_nodes;
  if (hi > N || lo > hi || nthreads == 0) return OR_EINVAL;
  rate_job J;
  memset(&J, 0, sizeof J);
  J.g = g, J.n_off = n_off, J.n_nin = n_nin, J.n_inc = n_inc, J.t = t;
  J.cap = cap, J.omega = omega, J.seed = seed, J.delta = delta;
  J.lo = lo, J.hi = hi, J.pi = pi, J.noise_on = noise_on;
  J.target = target, J.score = score;
  J.next = lo;
  J.bad_node = NONE;
  J.bad_rc = OR_OK;
  pthread_mutex_init(&J.bad_mu, NULL);
  uint32_t nt = nthreads;
  if (nt > 256) nt = 256;
  if (nt == 1) {
    rate_worker(&J);
  } else {
    pthread_t th[256];
    uint32_t started = 0;
    for (; started < nt; ++started)
      if (pthread_create(&th[started], NULL, rate_worker, &J) != 0) break;
    if (started == 0) rate_worker(&J);
    for (uint32_t i = 0; i < started; ++i) pthread_join(th[i], NULL);
  }
  pthread_mutex_destroy(&J.bad_mu);
  return J.bad_rc;
}

int or_rate(const or_edges *g, const int64_t *n_off, const uint32_t *n_nin, const uint32_t *n_inc,
            const uint64_t *t, uint64_t cap, uint64_t omega, uint32_t delta, int noise_on,
            uint64_t seed, uint32_t lo, uint32_t hi, uint32_t *target, uint64_t *score) {
  return rate_top(g, n_off, n_nin, n_inc, t, cap, omega, delta, noise_on, seed, lo, hi, 1, 1,
                  target, score);
}

int or_rate_top(const or_edges *g, const int64_t *n_off, const uint32_t *n_nin,
                const uint32_t *n_inc, const uint64_t *t, uint64_t cap, uint64_t omega,
                uint32_t delta, int noise_on, uint64_t seed, uint32_t pi, uint32_t *target,
                uint64_t *score) {
  if (pi == 0) return OR_EINVAL;
  return rate_top(g, n_off, n_nin, n_inc, t, cap, omega, delta, noise_on, seed, 0, g->n_nodes, pi,
                  1, target, score);
}

/* The same ratings with the node loop over nthreads threads, for nodes
 * lo..hi-1 (other entries untouched). */
int or_rate_top_mt(const or_edges *g, const int64_t *n_off, const uint32_t *n_nin,
                   const uint32_t *n_inc, const uint64_t *t, uint64_t cap, uint64_t omega,
                   uint32_t delta, int noise_on, uint64_t seed, uint32_t lo, uint32_t hi,
                   uint32_t pi, uint32_t nthreads, uint32_t *target, uint64_t *score) {
  if (pi == 0) return OR_EINVAL;
  return rate_top(g, n_off, n_nin, n_inc, t, cap, omega, delta, noise_on, seed, lo, hi, pi,
                  nthreads, target, score);
}

/* ------------------------------------------------------------------------ */
/* O6: deterministic handshake matching ([P2] Sec. III-A and III-B3).       */
/*  R = {n : target(target(n)) = n}: two-cycles, matched by default.         */
/*  Each other node places its score on its candidate; the best proposer of  */
/*  t, bc(t), has the highest score, ties to the smallest id.                */
/*  Walking down from the roots, n takes its candidate iff the candidate is  */
/*  still free and n is its best proposer:                                   */
/*    taken(n) = n in R  or  (target(n) != NONE and bc(target(n)) = n and    */
/*               not taken(target(n))).                                      */
/*  match(n) = target(n) if taken(n); otherwise bc(n) if n has a proposer    */
/*  (that proposer is then taken by n); otherwise n itself.                  */
/* Reading for nodes with no candidate (left open by [P2]): they are tops of */
/* their trees, never taken, and may accept their best proposer.             */
/* ECYCLE if the proposal graph has a cycle longer than two ([P1] Sec. V-A   */
/* proves there is none).                                                    */
/* ------------------------------------------------------------------------ */
int or_match(uint32_t N, const uint32_t *target, const uint64_t *score, uint32_t *match,
             uint64_t *n_pairs) {
  for (uint32_t n = 0; n < N; ++n)
    if (target[n] != NONE && (target[n] >= N || target[n] == n)) return OR_EINVAL;
  /* cycle check on the functional graph n -> target(n) */
  uint8_t *col = (uint8_t *)calloc(N ? N : 1, 1);
  uint32_t *path = (uint32_t *)malloc(sizeof(uint32_t) * (N ? N : 1));
  uint32_t *bc = (uint32_t *)malloc(sizeof(uint32_t) * (N ? N : 1));
  int8_t *tk = (int8_t *)malloc(N ? N : 1);
  if (!col || !path || !bc || !tk) {
    free(col), free(path), free(bc), free(tk);
    return OR_ENOMEM;
  }
  int rc = OR_OK;
  for (uint32_t s = 0; s < N && rc == OR_OK; ++s) {
    if (col[s]) continue;
    uint32_t len = 0, v = s;
    while (v != NONE && col[v] == 0) {
      col[v] = 1; /* on the current path */
      path[len++] = v;
      v = target[v];
    }
    if (v != NONE && col[v] == 1) { /* closed a cycle on this path */
      uint32_t cyc = 0;
      for (uint32_t i = len; i > 0; --i) {
        cyc++;
        if (path[i - 1] == v) break;
      }
      if (cyc != 2) rc = OR_ECYCLE;
    }
    for (uint32_t i = 0; i < len; ++i) col[path[i]] = 2;
  }
  if (rc != OR_OK) {
    free(col), free(path), free(bc), free(tk);
    return rc;
  }
  /* best proposer of every node, over proposers outside R */
  for (uint32_t n = 0; n < N; ++n) bc[n] = NONE;
  for (uint32_t c = 0; c < N; ++c) {
    uint32_t tg = target[c];
    if (tg == NONE || target[tg] == c) continue; /* no candidate, or c in R */
    uint32_t b = bc[tg];
    if (b == NONE || score[c] > score[b] || (score[c] == score[b] && c < b)) bc[tg] = c;
  }
  /* taken(.), resolved top-down with an explicit path */
  for (uint32_t n = 0; n < N; ++n) tk[n] = -1;
  for (uint32_t s = 0; s < N; ++s) {
    uint32_t len = 0, v = s;
    int val = 0;
    for (;;) {
      if (tk[v] >= 0) {
        val = tk[v];
        break;
      }
      uint32_t tg = target[v];
      if (tg != NONE && target[tg] == v) { /* v in R */
        tk[v] = 1;
        val = 1;
        break;
      }
      if (tg == NONE || bc[tg] != v) { /* top of a chain: not taken */
        tk[v] = 0;
        val = 0;
        break;
      }
      path[len++] = v; /* taken(v) = not taken(target(v)) */
      v = tg;
    }
    for (uint32_t i = len; i > 0; --i) {
      val = !val;
      tk[path[i - 1]] = (int8_t)val;
    }
  }
  uint64_t moved = 0;
  for (uint32_t n = 0; n < N; ++n) {
    if (tk[n]) match[n] = target[n];
    else if (bc[n] != NONE) match[n] = bc[n];
    else match[n] = n;
    moved += match[n] != n;
  }
  for (uint32_t n = 0; n < N; ++n)
    if (match[match[n]] != n) rc = OR_EINTERNAL;
  *n_pairs = moved / 2;
  free(col), free(path), free(bc), free(tk);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* O7: contraction.  [P1] Sec. III and V-E, [P2] Sec. III-B4.                */
/*  gamma(n) = {n, match(n)}; reading: coarse ids are the ranks of the       */
/*  smallest member ids.  size'(c) = sum of member sizes.                    */
/*  E' = {gamma(e)}, omega' = omega, one coarse edge per fine edge, same id  */
/*  (edges are not merged; single-pin edges are kept).  dst' = gamma(dst),   */
/*  src' = gamma(src) minus dst' (duplicates between src and dst are dropped  */
/*  from src, [P1] Sec. V-E).  All lists sorted.                             */
/*  Outputs are malloc'd (free with or_free).                                */
/* ------------------------------------------------------------------------ */
int or_contract(const or_edges *g, const uint32_t *match, uint32_t *gamma, uint32_t *n_coarse,
                uint32_t **size_out, int64_t **e_off_out, uint32_t **nsrc_out,
                uint32_t **pins_out) {
  uint32_t N = g->n_nodes, E = g->n_edges;
  for (uint32_t n = 0; n < N; ++n)
    if (match[n] >= N || match[match[n]] != n) return OR_EINVAL;
  uint32_t *rank = (uint32_t *)malloc(sizeof(uint32_t) * (N ? N : 1));
  if (!rank) return OR_ENOMEM;
  uint32_t nc = 0;
  for (uint32_t n = 0; n < N; ++n) {
    uint32_t rep = n < match[n] ? n : match[n];
    if (rep == n) rank[n] = nc++;
  }
  for (uint32_t n = 0; n < N; ++n) {
    uint32_t rep = n < match[n] ? n : match[n];
    gamma[n] = rank[rep];
  }
  free(rank);
  uint32_t *sz = (uint32_t *)calloc(nc ? nc : 1, sizeof(uint32_t));
  int64_t *off = (int64_t *)malloc(sizeof(int64_t) * ((size_t)E + 1));
  uint32_t *ns = (uint32_t *)malloc(sizeof(uint32_t) * (E ? E : 1));
  uint32_t *pins = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)(g->e_off[E] ? g->e_off[E] : 1));
  uint32_t *tmp = (uint32_t *)malloc(sizeof(uint32_t) * (N ? N : 1));
  if (!sz || !off || !ns || !pins || !tmp) {
    free(sz), free(off), free(ns), free(pins), free(tmp);
    return OR_ENOMEM;
  }
  for (uint32_t n = 0; n < N; ++n) sz[gamma[n]] += g->n_size[n];
  off[0] = 0;
  for (uint32_t e = 0; e < E; ++e) {
    int64_t a = g->e_off[e], b = g->e_off[e + 1], d0 = a + g->e_nsrc[e];
    /* dst' */
    uint32_t nd = 0;
    for (int64_t i = d0; i < b; ++i) tmp[nd++] = gamma[g->e_pins[i]];
    qsort(tmp, nd, sizeof(uint32_t), cmp_u32);
    uint32_t ud = 0;
    for (uint32_t i = 0; i < nd; ++i)
      if (i == 0 || tmp[i] != tmp[i - 1]) tmp[ud++] = tmp[i];
    /* src' */
    uint32_t *sl = (uint32_t *)malloc(sizeof(uint32_t) * (g->e_nsrc[e] ? g->e_nsrc[e] : 1));
    if (!sl) {
      free(sz), free(off), free(ns), free(pins), free(tmp);
      return OR_ENOMEM;
    }
    uint32_t nsrc = 0;
    for (int64_t i = a; i < d0; ++i) sl[nsrc++] = gamma[g->e_pins[i]];
    qsort(sl, nsrc, sizeof(uint32_t), cmp_u32);
    uint32_t us = 0;
    for (uint32_t i = 0; i < nsrc; ++i) {
      if (i > 0 && sl[i] == sl[i - 1]) continue;
      if (sorted_has(tmp, ud, sl[i])) continue;
      sl[us++] = sl[i];
    }
    int64_t o = off[e];
    memcpy(pins + o, sl, sizeof(uint32_t) * us);
    memcpy(pins + o + us, tmp, sizeof(uint32_t) * ud);
    ns[e] = us;
    off[e + 1] = o + us + ud;
    free(sl);
  }
  free(tmp);
  *n_coarse = nc;
  *size_out = sz;
  *e_off_out = off;
  *nsrc_out = ns;
  *pins_out = pins;
  return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* O10: invalid-neighbour flags and the purge of coarse neighbourhoods       */
/* ([P1] Sec. V-C, third mechanism; Sec. V-B: neighbourhoods are updated in  */
/* place from level to level).                                              */
/*  flag[i] for entry i of N(n) (i in nb_off[n]..nb_off[n+1]) is 1 iff the   */
/*  pair (n, nb[i]) is not valid by Eq. 6: size(n)+size(m) > Omega or        */
/*  |in(n) u in(m)| > Delta, the union counted by merging the two sorted     */
/*  inbound lists.                                                           */
/*  Reading: every invalid neighbour is flagged (the rating judges them all), */
/*  a flag marks every occurrence of the same coarse neighbour, and purged   */
/*  neighbours stay purged: the coarse lists are built from the members'     */
/*  current (purged) lists.  For c = gamma(a) = gamma(b):                    */
/*    N'(c) = {gamma(m) : m in N(a) u N(b)} \ {c}                            */
/*            \ {gamma(m) : m flagged in N(a) or in N(b)},                   */
/*  which on the first level equals the definition of N' on G' minus the    */
/*  flagged images.  Only invalid pairs are dropped: size and inbound set of */
/*  a cluster contain those of each member, so an invalid (a, m) stays       */
/*  invalid for (c, gamma(m)).  or_purge writes malloc'd lists.              */
/* ------------------------------------------------------------------------ */
int or_flags(const or_edges *g, const int64_t *n_off, const uint32_t *n_nin, const uint32_t *n_inc,
             const int64_t *nb_off, const uint32_t *nb, uint64_t omega, uint32_t delta,
             uint8_t *flag) {
  uint32_t N = g->n_nodes;
  for (uint32_t n = 0; n < N; ++n) {
    for (int64_t i = nb_off[n]; i < nb_off[n + 1]; ++i) {
      uint32_t m = nb[i];
      if (m >= N) return OR_EINVAL;
      int bad = (uint64_t)g->n_size[n] + g->n_size[m] > omega;
      if (!bad)
        bad = union_size(n_inc + n_off[n], n_nin[n], n_inc + n_off[m], n_nin[m]) > delta;
      flag[i] = (uint8_t)bad;
    }
  }
  return OR_OK;
}

int or_purge(uint32_t N, const int64_t *nb_off, const uint32_t *nb, const uint8_t *flag,
             const uint32_t *match, const uint32_t *gamma, uint32_t nc, int64_t *pnb_off,
             uint32_t **pnb_out, uint64_t *pnb_total) {
  uint32_t *rep_of = (uint32_t *)malloc(sizeof(uint32_t) * (nc ? nc : 1));
  /* a cluster's entries: at most |N(a)| + |N(b)| <= 2 (N - 1) */
  uint32_t *val = (uint32_t *)malloc(sizeof(uint32_t) * (2 * (size_t)N + 1));
  uint32_t *kill = (uint32_t *)malloc(sizeof(uint32_t) * (2 * (size_t)N + 1));
  uint32_t *out = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)(nb_off[N] ? nb_off[N] : 1));
  if (!rep_of || !val || !kill || !out) {
    free(rep_of), free(val), free(kill), free(out);
    return OR_ENOMEM;
  }
  for (uint32_t n = 0; n < N; ++n)
    if (match[n] >= n) rep_of[gamma[n]] = n;
  pnb_off[0] = 0;
  for (uint32_t c = 0; c < nc; ++c) {
    uint32_t a = rep_of[c], b = match[a], nv = 0, nk = 0;
    for (int k = 0; k < (b != a ? 2 : 1); ++k) {
      uint32_t x = k == 0 ? a : b;
      for (int64_t i = nb_off[x]; i < nb_off[x + 1]; ++i) {
        val[nv++] = gamma[nb[i]];
        if (flag[i]) kill[nk++] = gamma[nb[i]];
      }
    }
    qsort(val, nv, sizeof(uint32_t), cmp_u32);
    qsort(kill, nk, sizeof(uint32_t), cmp_u32);
    int64_t o = pnb_off[c];
    for (uint32_t i = 0; i < nv; ++i) {
      if (i > 0 && val[i] == val[i - 1]) continue;
      if (val[i] == c || sorted_has(kill, nk, val[i])) continue;
      out[o++] = val[i];
    }
    pnb_off[c + 1] = o;
  }
  free(rep_of), free(val), free(kill);
  *pnb_out = out;
  *pnb_total = (uint64_t)pnb_off[nc];
  return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* O8: partition evaluation.                                                 */
/*  [P1] Eq. 1: Conn = sum_e omega(e) (lambda(e) - 1), lambda(e) = number    */
/*  of distinct partitions among e's pins.  [P1] Eq. 16 (k-way section):     */
/*  cut-net = sum_e omega(e) [lambda(e) > 1].                                */
/*  [P1] Sec. II-B: size(p) = sum of node sizes in p; inbound(p) =           */
/*  |{e : pins_in(p,e) > 0}| = number of h-edges with a destination in p.    */
/*  summary = {conn, cutnet, #parts over Omega, #parts over Delta,           */
/*             #empty parts, max part size, max part inbound, sum lambda}.   */
/*  Empty parts are counted, not rejected.                                    */
/* ------------------------------------------------------------------------ */
int or_evaluate(const or_edges *g, const uint32_t *rho, uint32_t k, uint64_t omega, uint32_t delta,
                uint64_t *part_size, uint32_t *part_inb, uint64_t *summary) {
  uint32_t N = g->n_nodes, E = g->n_edges;
  if (k == 0 && N > 0) return OR_EINVAL;
  for (uint32_t n = 0; n < N; ++n)
    if (rho[n] >= k) return OR_EINVAL;
  uint32_t *cnt = (uint32_t *)calloc(k ? k : 1, sizeof(uint32_t));
  uint32_t *mark = (uint32_t *)malloc(sizeof(uint32_t) * (k ? k : 1));
  uint32_t *dmark = (uint32_t *)malloc(sizeof(uint32_t) * (k ? k : 1));
  if (!cnt || !mark || !dmark) {
    free(cnt), free(mark), free(dmark);
    return OR_ENOMEM;
  }
  for (uint32_t p = 0; p < k; ++p) {
    part_size[p] = 0;
    part_inb[p] = 0;
    mark[p] = NONE;
    dmark[p] = NONE;
  }
  for (uint32_t n = 0; n < N; ++n) {
    part_size[rho[n]] += g->n_size[n];
    cnt[rho[n]]++;
  }
  uint64_t conn = 0, cut = 0, sum_lambda = 0;
  for (uint32_t e = 0; e < E; ++e) {
    uint64_t lambda = 0;
    int64_t a = g->e_off[e], b = g->e_off[e + 1], d0 = a + g->e_nsrc[e];
    for (int64_t i = a; i < b; ++i) {
      uint32_t p = rho[g->e_pins[i]];
      if (mark[p] != e) {
        mark[p] = e;
        lambda++;
      }
      if (i >= d0 && dmark[p] != e) {
        dmark[p] = e;
        part_inb[p]++;
      }
    }
    conn += (uint64_t)g->e_w[e] * (lambda - 1);
    cut += lambda > 1 ? g->e_w[e] : 0;
    sum_lambda += lambda;
  }
  uint64_t over_o = 0, over_d = 0, empty = 0, max_s = 0, max_i = 0;
  for (uint32_t p = 0; p < k; ++p) {
    over_o += part_size[p] > omega;
    over_d += part_inb[p] > delta;
    empty += cnt[p] == 0;
    if (part_size[p] > max_s) max_s = part_size[p];
    if (part_inb[p] > max_i) max_i = part_inb[p];
  }
  summary[0] = conn;
  summary[1] = cut;
  summary[2] = over_o;
  summary[3] = over_d;
  summary[4] = empty;
  summary[5] = max_s;
  summary[6] = max_i;
  summary[7] = sum_lambda;
  free(cnt), free(mark), free(dmark);
  return OR_OK;
}

/*
 * O11 -- best-effort pairing of the nodes left without a partner
 * ([P1] Sec. V-C, last mechanism).  Reading (the pages leave the details
 * open): the nodes gathered are those still unmatched after the matching
 * whose target is undefined.  They are sorted by (size, id) ascending.  Node n
 * finds, by binary search, the last position whose size fits its slack
 * Omega - size(n), then takes the first node m != n, scanning down at most
 * `window` positions from there, whose inbound count together with n's stays
 * within Delta (the union overestimated by the sum).  A node claimed by
 * several takes the smallest id; n pairs with its choice m when it won m and
 * no node claimed n itself.  match is updated in place; returns the number
 * of new pairs in *n_pairs.
 */
typedef struct {
  uint32_t size, id;
} or_sz;

static int cmp_sz(const void *x, const void *y) {
  const or_sz *a = (const or_sz *)x, *b = (const or_sz *)y;
  if (a->size != b->size) return a->size < b->size ? -1 : 1;
  return a->id < b->id ? -1 : (a->id > b->id ? 1 : 0);
}

int or_pair_leftovers(uint32_t N, const uint32_t *target, const uint32_t *n_size,
                      const uint32_t *n_nin, uint64_t omega, uint32_t delta, uint32_t window,
                      uint32_t *match, uint64_t *n_pairs) {
  *n_pairs = 0;
  uint32_t nl = 0;
  for (uint32_t n = 0; n < N; ++n)
    if (target[n] == NONE && match[n] == n) ++nl;
  if (nl < 2) return OR_OK;
  or_sz *L = (or_sz *)malloc(sizeof(or_sz) * nl);
  uint32_t *choice = (uint32_t *)malloc(sizeof(uint32_t) * nl);
  uint32_t *claim = (uint32_t *)malloc(sizeof(uint32_t) * N);
  if (!L || !choice || !claim) {
    free(L), free(choice), free(claim);
    return OR_ENOMEM;
  }
  uint32_t k = 0;
  for (uint32_t n = 0; n < N; ++n)
    if (target[n] == NONE && match[n] == n) L[k].size = n_size[n], L[k].id = n, ++k;
  qsort(L, nl, sizeof(or_sz), cmp_sz);
  for (uint32_t n = 0; n < N; ++n) claim[n] = NONE;
  for (uint32_t i = 0; i < nl; ++i) {
    const uint32_t n = L[i].id;
    choice[i] = NONE;
    if ((uint64_t)L[i].size > omega) continue;
    const uint64_t slack = omega - L[i].size;
    /* binary search: number of positions whose size is <= slack */
    uint32_t lo = 0, hi = nl;
    while (lo < hi) {
      uint32_t mid = lo + (hi - lo) / 2;
      if ((uint64_t)L[mid].size <= slack) lo = mid + 1;
      else hi = mid;
    }
    /* scan down from position lo - 1, at most `window` positions */
    for (uint32_t s = 0; s < window && s < lo; ++s) {
      const uint32_t j = lo - 1 - s;
      if (j == i) continue;
      const uint32_t m = L[j].id;
      if ((uint64_t)n_nin[n] + n_nin[m] <= delta) {
        choice[i] = m;
        break;
      }
    }
    if (choice[i] != NONE && n < claim[choice[i]]) claim[choice[i]] = n;
  }
  for (uint32_t i = 0; i < nl; ++i) {
    const uint32_t n = L[i].id, m = choice[i];
    if (m != NONE && claim[m] == n && claim[n] == NONE) {
      match[n] = m;
      match[m] = n;
      ++*n_pairs;
    }
  }
  free(L), free(choice), free(claim);
  return OR_OK;
}

/*
 * O12 -- refinement move proposal ([P1] Sec. VI-A/B, Eq. 13).
 *   pins(p, e) = |{m in e : rho(m) = p}|,
 *   saving(n)  = sum of w(e) over e in I(n) with pins(rho(n), e) = 1,
 *   loss(n, p) = sum of w(e) over e in I(n) with pins(p, e) = 0,
 *   gain(n, p) = saving(n) - loss(n, p),
 *   move(n)    = the partition p != rho(n) of largest gain, ties to the
 *                smallest id (the reading of the pages' tie rule used for
 *                targets as well); with enforce_omega only partitions with
 *                part_size(p) + size(n) <= Omega are considered.
 * move[n] = NONE and gain[n] = 0 when no partition qualifies.  pins(p, e) is
 * held per hyperedge as its sorted distinct partitions with their counts.
 */
static int cmp_u32b(const void *a, const void *b) {
  uint32_t x = *(const uint32_t *)a, y = *(const uint32_t *)b;
  return x < y ? -1 : (x > y ? 1 : 0);
}

/* pins(p, e) by binary search in e's sorted partition list */
static uint32_t pins_of(const int64_t *poff, const uint32_t *ppart, const uint32_t *pcnt,
                        uint32_t e, uint32_t p) {
  int64_t lo = poff[e], hi = poff[e + 1];
  while (lo < hi) {
    int64_t mid = lo + (hi - lo) / 2;
    if (ppart[mid] < p) lo = mid + 1;
    else hi = mid;
  }
  return (lo < poff[e + 1] && ppart[lo] == p) ? pcnt[lo] : 0;
}

int or_moves(const or_edges *g, const int64_t *n_off, const uint32_t *n_inc, const uint32_t *rho,
             uint32_t k, uint64_t omega, int enforce_omega, uint32_t *move, int64_t *gain) {
  const uint32_t N = g->n_nodes, E = g->n_edges;
  const int64_t P = g->e_off[E];
  for (uint32_t n = 0; n < N; ++n)
    if (rho[n] >= k) return OR_EINVAL;
  int64_t *poff = (int64_t *)malloc(sizeof(int64_t) * ((size_t)E + 1));
  uint32_t *ppart = (uint32_t *)malloc(sizeof(uint32_t) * (P ? (size_t)P : 1));
  uint32_t *pcnt = (uint32_t *)malloc(sizeof(uint32_t) * (P ? (size_t)P : 1));
  uint32_t *tmp = (uint32_t *)malloc(sizeof(uint32_t) * (P ? (size_t)P : 1));
  uint64_t *psize = (uint64_t *)calloc(k ? k : 1, sizeof(uint64_t));
  if (!poff || !ppart || !pcnt || !tmp || !psize) {
    free(poff), free(ppart), free(pcnt), free(tmp), free(psize);
    return OR_ENOMEM;
  }
  /* pins(., e): sort the partitions of e's pins, count equal runs */
  int64_t w = 0;
  for (uint32_t e = 0; e < E; ++e) {
    poff[e] = w;
    const int64_t a = g->e_off[e], b = g->e_off[e + 1];
    for (int64_t i = a; i < b; ++i) tmp[i - a] = rho[g->e_pins[i]];
    qsort(tmp, (size_t)(b - a), sizeof(uint32_t), cmp_u32b);
    for (int64_t i = 0; i < b - a; ++i) {
      if (i == 0 || tmp[i] != tmp[i - 1]) {
        ppart[w] = tmp[i];
        pcnt[w] = 0;
        ++w;
      }
      pcnt[w - 1]++;
    }
  }
  poff[E] = w;
  for (uint32_t n = 0; n < N; ++n) psize[rho[n]] += g->n_size[n];
  for (uint32_t n = 0; n < N; ++n) {
    const uint32_t pn = rho[n];
    int64_t saving = 0;
    for (int64_t j = n_off[n]; j < n_off[n + 1]; ++j) {
      const uint32_t e = n_inc[j];
      if (pins_of(poff, ppart, pcnt, e, pn) == 1) saving += g->e_w[e];
    }
    uint32_t best = NONE;
    int64_t best_gain = 0;
    for (uint32_t p = 0; p < k; ++p) {
      if (p == pn) continue;
      if (enforce_omega && psize[p] + g->n_size[n] > omega) continue;
      int64_t loss = 0;
      for (int64_t j = n_off[n]; j < n_off[n + 1]; ++j) {
        const uint32_t e = n_inc[j];
        if (pins_of(poff, ppart, pcnt, e, p) == 0) loss += g->e_w[e];
      }
      const int64_t gp = saving - loss;
      if (best == NONE || gp > best_gain) best = p, best_gain = gp;
    }
    move[n] = best;
    gain[n] = best == NONE ? 0 : best_gain;
  }
  free(poff), free(ppart), free(pcnt), free(tmp), free(psize);
  return OR_OK;
}

/*
 * O13 -- exact maximum-weight matching on the proposal pseudo-forest
 * ([P1] Sec. V-D, Eqs. 7-12).  The proposal edge of n is {n, target(n)} with
 * weight score(n).  R = the nodes in two-cycles (target(target(n)) = n); the
 * parent of n not in R is target(n) (a node with no target tops its tree);
 * children(n) = {c not in R : target(c) = n}.  Bottom up:
 *   A(n)     = sum of ss0(c) over children(n),
 *   best(n)  = max over children c of ss1(c) - ss0(c), at the smallest such c,
 *   ss0(n)   = A(n) + max(0, best(n))        (n not matched to its target),
 *   ss1(n)   = score(n) + A(n)                (n matched to its target).
 * A two-cycle {n, t} matches when score(n) + A(n) + A(t) > ss0(n) + ss0(t)
 * (strictly); otherwise, and for a node with no target, a node takes its best
 * child when best > 0.  Top down, a node not in R pairs with its target when
 * the target took it, and otherwise takes its best child when best > 0.
 * Sums that do not fit 64 bits give OR_EOVERFLOW.
 */
int or_match_dp(uint32_t N, const uint32_t *target, const uint64_t *score, uint32_t *match,
                uint64_t *n_pairs) {
  *n_pairs = 0;
  for (uint32_t n = 0; n < N; ++n)
    if (target[n] != NONE && (target[n] >= N || target[n] == n)) return OR_EINVAL;
  uint8_t *inR = (uint8_t *)calloc(N ? N : 1, 1);
  uint32_t *order = (uint32_t *)malloc(sizeof(uint32_t) * (N ? N : 1));
  uint32_t *pend = (uint32_t *)calloc(N ? N : 1, sizeof(uint32_t));
  uint64_t *A = (uint64_t *)calloc(N ? N : 1, sizeof(uint64_t));
  uint64_t *ss0 = (uint64_t *)calloc(N ? N : 1, sizeof(uint64_t));
  uint64_t *ss1 = (uint64_t *)calloc(N ? N : 1, sizeof(uint64_t));
  uint64_t *bestv = (uint64_t *)calloc(N ? N : 1, sizeof(uint64_t));
  uint32_t *bestc = (uint32_t *)malloc(sizeof(uint32_t) * (N ? N : 1));
  if (!inR || !order || !pend || !A || !ss0 || !ss1 || !bestv || !bestc) {
    free(inR), free(order), free(pend), free(A), free(ss0), free(ss1), free(bestv), free(bestc);
    return OR_ENOMEM;
  }
  int rc = OR_OK;
  for (uint32_t n = 0; n < N; ++n) {
    const uint32_t t = target[n];
    inR[n] = t != NONE && target[t] == n;
    bestc[n] = NONE;
  }
  /* children counts; leaves first (a queue over nodes whose children are done) */
  for (uint32_t n = 0; n < N; ++n)
    if (!inR[n] && target[n] != NONE) pend[target[n]]++;
  uint32_t head = 0, tail = 0;
  for (uint32_t n = 0; n < N; ++n)
    if (pend[n] == 0) order[tail++] = n;
  while (head < tail) {
    const uint32_t n = order[head++];
    /* all children of n are done: A(n), best(n) are final */
    ss0[n] = A[n] + (bestc[n] != NONE && bestv[n] > 0 ? bestv[n] : 0);
    if (ss0[n] < A[n]) rc = OR_EOVERFLOW;
    if (target[n] != NONE) {
      ss1[n] = score[n] + A[n];
      if (ss1[n] < A[n]) rc = OR_EOVERFLOW;
    }
    if (!inR[n] && target[n] != NONE) {
      const uint32_t p = target[n];
      const uint64_t s = A[p] + ss0[n];
      if (s < A[p]) rc = OR_EOVERFLOW;
      A[p] = s;
      /* ss1 >= ss0 always holds for a child (its best child scores at most
         its own score), so the difference is well defined */
      const uint64_t d = ss1[n] >= ss0[n] ? ss1[n] - ss0[n] : 0;
      if (bestc[p] == NONE || d > bestv[p] || (d == bestv[p] && n < bestc[p]))
        bestv[p] = d, bestc[p] = n;
      if (--pend[p] == 0) order[tail++] = p;
    }
  }
  if (tail != N) rc = OR_ECYCLE; /* a cycle longer than two */
  if (rc == OR_OK) {
    for (uint32_t n = 0; n < N; ++n) match[n] = n;
    /* the two-cycles decide first */
    for (uint32_t n = 0; n < N; ++n) {
      const uint32_t t = target[n];
      if (!inR[n] || n > t) continue;
      const uint64_t pair = score[n] + A[n] + A[t];
      const uint64_t apart = ss0[n] + ss0[t];
      if (pair < A[n] || pair - A[n] < A[t] || apart < ss0[n]) rc = OR_EOVERFLOW;
      if (pair > apart) {
        match[n] = t, match[t] = n;
      } else {
        if (bestc[n] != NONE && bestv[n] > 0) match[n] = bestc[n], match[bestc[n]] = n;
        if (bestc[t] != NONE && bestv[t] > 0) match[t] = bestc[t], match[bestc[t]] = t;
      }
    }
    /* then top down: the order reversed visits every parent before its children */
    for (uint32_t i = N; i-- > 0;) {
      const uint32_t n = order[i];
      const uint32_t t = target[n];
      if (inR[n]) {
        /* decided above */
      } else if (t != NONE && match[t] == n) {
        /* taken by its target: already recorded */
      } else if (bestc[n] != NONE && bestv[n] > 0) {
        match[n] = bestc[n], match[bestc[n]] = n;
      }
    }
    for (uint32_t n = 0; n < N; ++n)
      if (match[n] > n) ++*n_pairs;
  }
  free(inR), free(order), free(pend), free(A), free(ss0), free(ss1), free(bestv), free(bestc);
  return rc;
}

/*
 * O14 -- one refinement pass over proposed moves ([P1] Sec. VI-A, VI-C,
 * VI-D; Eqs. 14-15).  move/gain are the in-isolation proposals of O12.
 * Readings (the pages leave these open):
 *  - the sequence holds every node with a proposed move, each move its own
 *    chain (no chaining), so chains ranked by total gain order the moves by
 *    (gain desc, id asc);
 *  - the in-sequence gain of the i-th move is the connectivity it removes
 *    with the moves before it already applied: for every hyperedge e of the
 *    node, +w(e) when the node is the last pin of e left in its partition,
 *    -w(e) when e has no pin in the destination yet (Eqs. 14-15 state the
 *    same as corrections of the in-isolation gain);
 *  - a partition is invalid while its size exceeds Omega or its inbound count
 *    (hyperedges with a destination pin in it) exceeds Delta; the violation
 *    count after a move is the number of invalid partitions then;
 *  - the prefix applied is the one of largest cumulative gain among those
 *    leaving no violation, the empty prefix (gain 0, nothing applied) always
 *    eligible, ties to the shorter prefix.
 * Outputs: seq[M] nodes in order, seq_gain[M] in-sequence gains, seq_viol[M]
 * violation counts after each move, *n_seq = M, *n_applied = moves applied,
 * *gain_applied = their summed gain, rho_out = rho with them applied.
 * A simulation: the state is updated move by move and every count is taken
 * by scanning the hyperedge's pins.
 */
typedef struct {
  int64_t gain;
  uint32_t id;
} or_mv;

static int cmp_mv(const void *x, const void *y) { /* gain descending, id ascending */
  const or_mv *a = (const or_mv *)x, *b = (const or_mv *)y;
  if (a->gain != b->gain) return a->gain > b->gain ? -1 : 1;
  return a->id < b->id ? -1 : (a->id > b->id ? 1 : 0);
}

/*
 * O15 -- move chains ([P1] Sec. VI-C, Fig. 5): the sequence as chains of
 * moves, each departing from the destination of the one before.
 *  - The moves are sorted by (source partition, gain desc, id asc).
 *  - Each move gets at most one predecessor and one successor.  In a round,
 *    every move without a successor (a free end) looks at the first
 *    CHAIN_WINDOW moves of the sorted run leaving its destination, takes
 *    those still without a predecessor, and picks the one of largest grade
 *      gain(m) - 1e-6 |size(n) - size(m)| - 1e-7 ||in(n)| - |in(m)||
 *    (kept exact as 10^7 times that, an integer; ties to the smaller id m).
 *    A move picked by several goes to the largest (grade, picker id); the
 *    winner links to it.  Rounds repeat up to CHAIN_ROUNDS times, or until a
 *    round links nothing.
 *  - The links form disjoint paths and cycles.  A path starts at its move
 *    without a predecessor, a cycle at its smallest node id; both follow the
 *    successor links.  Chains are ranked by total gain (desc), then by their
 *    first node (asc), and concatenated.
 * seq[M] gets the nodes in order and seq_chain[M] (optional) the rank of
 * each one's chain.  The window, the tie rules and where a cycle starts are
 * readings; the pages fix the grade, its weights, the window size of 256
 * and the 16 rounds.
 */
#define CHAIN_WINDOW 256
#define CHAIN_ROUNDS 16

typedef struct {
  uint32_t part, id;
  int64_t gain;
} or_smv;

static int cmp_smv(const void *x, const void *y) { /* part asc, gain desc, id asc */
  const or_smv *a = (const or_smv *)x, *b = (const or_smv *)y;
  if (a->part != b->part) return a->part < b->part ? -1 : 1;
  if (a->gain != b->gain) return a->gain > b->gain ? -1 : 1;
  return a->id < b->id ? -1 : (a->id > b->id ? 1 : 0);
}

typedef struct {
  int64_t total;
  uint32_t first, len, start; /* first node, members, position of the first in order[] */
} or_chain;

static int cmp_chain(const void *x, const void *y) { /* total desc, first node asc */
  const or_chain *a = (const or_chain *)x, *b = (const or_chain *)y;
  if (a->total != b->total) return a->total > b->total ? -1 : 1;
  return a->first < b->first ? -1 : (a->first > b->first ? 1 : 0);
}

static int64_t grade_fx(uint32_t n, uint32_t m, const uint32_t *size, const uint32_t *nin,
                        const int64_t *gain) {
  const int64_t ds = size[n] > size[m] ? (int64_t)size[n] - size[m] : (int64_t)size[m] - size[n];
  const int64_t di = nin[n] > nin[m] ? (int64_t)nin[n] - nin[m] : (int64_t)nin[m] - nin[n];
  return 10000000ll * gain[m] - 10 * ds - di;
}

static int or_chain_order(uint32_t N, const uint32_t *size, const uint32_t *nin,
                          const uint32_t *rho, uint32_t k, const uint32_t *move,
                          const int64_t *gain, uint32_t *seq, uint32_t *seq_chain) {
  or_smv *srt = (or_smv *)malloc(sizeof(or_smv) * (N ? N : 1));
  int64_t *pstart = (int64_t *)malloc(sizeof(int64_t) * ((size_t)k + 1));
  uint32_t *pred = (uint32_t *)malloc(sizeof(uint32_t) * (N ? N : 1));
  uint32_t *succ = (uint32_t *)malloc(sizeof(uint32_t) * (N ? N : 1));
  uint32_t *pick = (uint32_t *)malloc(sizeof(uint32_t) * (N ? N : 1));
  uint32_t *winner = (uint32_t *)malloc(sizeof(uint32_t) * (N ? N : 1));
  int64_t *wgrade = (int64_t *)malloc(sizeof(int64_t) * (N ? N : 1));
  uint8_t *seen = (uint8_t *)calloc(N ? N : 1, 1);
  or_chain *ch = (or_chain *)malloc(sizeof(or_chain) * (N ? N : 1));
  uint32_t *order = (uint32_t *)malloc(sizeof(uint32_t) * (N ? N : 1));
  if (!srt || !pstart || !pred || !succ || !pick || !winner || !wgrade || !seen || !ch || !order) {
    free(srt), free(pstart), free(pred), free(succ), free(pick), free(winner), free(wgrade);
    free(seen), free(ch), free(order);
    return OR_ENOMEM;
  }
  uint32_t M = 0;
  for (uint32_t n = 0; n < N; ++n) {
    pred[n] = succ[n] = NONE;
    if (move[n] != NONE) srt[M].part = rho[n], srt[M].id = n, srt[M].gain = gain[n], ++M;
  }
  qsort(srt, M, sizeof(or_smv), cmp_smv);
  /* pstart[p] = first position whose source partition is >= p */
  uint32_t i = 0;
  for (uint32_t p = 0; p <= k; ++p) {
    while (i < M && srt[i].part < p) ++i;
    pstart[p] = i;
  }
  for (int round = 0; round < CHAIN_ROUNDS; ++round) {
    for (uint32_t n = 0; n < N; ++n) pick[n] = NONE, winner[n] = NONE;
    /* every free end picks from its window, with the links of the round before */
    for (uint32_t j = 0; j < M; ++j) {
      const uint32_t n = srt[j].id;
      if (succ[n] != NONE) continue;
      const uint32_t d = move[n];
      int64_t a = pstart[d], b = pstart[d + 1];
      if (b - a > CHAIN_WINDOW) b = a + CHAIN_WINDOW;
      int64_t bg = 0;
      for (int64_t t = a; t < b; ++t) {
        const uint32_t m = srt[t].id;
        if (pred[m] != NONE) continue;
        const int64_t gr = grade_fx(n, m, size, nin, gain);
        if (pick[n] == NONE || gr > bg || (gr == bg && m < pick[n])) pick[n] = m, bg = gr;
      }
    }
    /* each picked move goes to the largest (grade, picker) */
    for (uint32_t n = 0; n < N; ++n) {
      const uint32_t m = pick[n];
      if (m == NONE) continue;
      const int64_t gr = grade_fx(n, m, size, nin, gain);
      if (winner[m] == NONE || gr > wgrade[m] || (gr == wgrade[m] && n > winner[m]))
        winner[m] = n, wgrade[m] = gr;
    }
    uint32_t links = 0;
    for (uint32_t m = 0; m < N; ++m)
      if (winner[m] != NONE) succ[winner[m]] = m, pred[m] = winner[m], ++links;
    if (links == 0) break;
  }
  /* chains: paths from their head, then cycles from their smallest node */
  uint32_t nch = 0, pos = 0;
  for (int pass = 0; pass < 2; ++pass)
    for (uint32_t n = 0; n < N; ++n) {
      if (move[n] == NONE || seen[n]) continue;
      if (pass == 0 && pred[n] != NONE) continue; /* not a path head */
      ch[nch].first = n, ch[nch].start = pos, ch[nch].len = 0, ch[nch].total = 0;
      for (uint32_t v = n; v != NONE && !seen[v]; v = succ[v]) {
        seen[v] = 1;
        order[pos++] = v;
        ch[nch].len++;
        ch[nch].total += gain[v];
      }
      ++nch;
    }
  qsort(ch, nch, sizeof(or_chain), cmp_chain);
  uint32_t o = 0;
  for (uint32_t c = 0; c < nch; ++c)
    for (uint32_t t = 0; t < ch[c].len; ++t) {
      if (seq_chain) seq_chain[o] = c;
      seq[o++] = order[ch[c].start + t];
    }
  free(srt), free(pstart), free(pred), free(succ), free(pick), free(winner), free(wgrade);
  free(seen), free(ch), free(order);
  return o == M ? OR_OK : OR_EINTERNAL;
}

/* pins of e in partition p under part[], all pins or destinations only */
static uint32_t count_in(const or_edges *g, const uint32_t *part, uint32_t e, uint32_t p,
                         int dst_only) {
  const int64_t a = g->e_off[e], b = g->e_off[e + 1], d0 = a + g->e_nsrc[e];
  uint32_t c = 0;
  for (int64_t i = dst_only ? d0 : a; i < b; ++i) c += part[g->e_pins[i]] == p;
  return c;
}

int or_refine(const or_edges *g, const int64_t *n_off, const uint32_t *n_nin,
              const uint32_t *n_inc, const uint32_t *rho, uint32_t k, uint64_t omega,
              uint32_t delta, const uint32_t *move, const int64_t *gain, int chained,
              uint32_t *seq, uint32_t *seq_chain, int64_t *seq_gain, uint32_t *seq_viol,
              uint32_t *n_seq, uint32_t *n_applied, int64_t *gain_applied, uint32_t *rho_out) {
  const uint32_t N = g->n_nodes, E = g->n_edges;
  *n_seq = 0, *n_applied = 0, *gain_applied = 0;
  for (uint32_t n = 0; n < N; ++n) {
    if (rho[n] >= k) return OR_EINVAL;
    if (move[n] != NONE && (move[n] >= k || move[n] == rho[n])) return OR_EINVAL;
  }
  or_mv *mv = (or_mv *)malloc(sizeof(or_mv) * (N ? N : 1));
  uint32_t *cur = (uint32_t *)malloc(sizeof(uint32_t) * (N ? N : 1));
  uint64_t *psize = (uint64_t *)calloc(k ? k : 1, sizeof(uint64_t));
  uint64_t *pinb = (uint64_t *)calloc(k ? k : 1, sizeof(uint64_t));
  uint32_t *mark = (uint32_t *)malloc(sizeof(uint32_t) * (k ? k : 1));
  if (!mv || !cur || !psize || !pinb || !mark) {
    free(mv), free(cur), free(psize), free(pinb), free(mark);
    return OR_ENOMEM;
  }
  /* the sequence */
  uint32_t M = 0;
  for (uint32_t n = 0; n < N; ++n)
    if (move[n] != NONE) mv[M].gain = gain[n], mv[M].id = n, ++M;
  if (chained) {
    const int rc = or_chain_order(N, g->n_size, n_nin, rho, k, move, gain, seq, seq_chain);
    if (rc != OR_OK) {
      free(mv), free(cur), free(psize), free(pinb), free(mark);
      return rc;
    }
  } else {
    qsort(mv, M, sizeof(or_mv), cmp_mv);
    for (uint32_t i = 0; i < M; ++i) {
      seq[i] = mv[i].id;
      if (seq_chain) seq_chain[i] = i;
    }
  }
  /* the starting state */
  for (uint32_t n = 0; n < N; ++n) cur[n] = rho[n], psize[rho[n]] += g->n_size[n];
  for (uint32_t p = 0; p < k; ++p) mark[p] = NONE;
  for (uint32_t e = 0; e < E; ++e)
    for (int64_t i = g->e_off[e] + g->e_nsrc[e]; i < g->e_off[e + 1]; ++i) {
      const uint32_t p = rho[g->e_pins[i]];
      if (mark[p] != e) mark[p] = e, pinb[p]++;
    }
  uint32_t viol = 0;
  for (uint32_t p = 0; p < k; ++p) viol += psize[p] > omega || pinb[p] > delta;
  /* move by move */
  for (uint32_t i = 0; i < M; ++i) {
    const uint32_t n = seq[i], ps = cur[n], pd = move[n];
    int64_t gi = 0;
    for (int64_t j = n_off[n]; j < n_off[n + 1]; ++j) {
      const uint32_t e = n_inc[j];
      if (count_in(g, cur, e, ps, 0) == 1) gi += g->e_w[e];
      if (count_in(g, cur, e, pd, 0) == 0) gi -= g->e_w[e];
    }
    viol -= psize[ps] > omega || pinb[ps] > delta;
    viol -= psize[pd] > omega || pinb[pd] > delta;
    for (int64_t j = n_off[n]; j < n_off[n] + n_nin[n]; ++j) { /* n is a destination of e */
      const uint32_t e = n_inc[j];
      if (count_in(g, cur, e, ps, 1) == 1) pinb[ps]--;
      if (count_in(g, cur, e, pd, 1) == 0) pinb[pd]++;
    }
    psize[ps] -= g->n_size[n];
    psize[pd] += g->n_size[n];
    cur[n] = pd;
    viol += psize[ps] > omega || pinb[ps] > delta;
    viol += psize[pd] > omega || pinb[pd] > delta;
    seq_gain[i] = gi;
    seq_viol[i] = viol;
  }
  /* the best valid prefix */
  int64_t run = 0, best = 0;
  uint32_t best_len = 0;
  for (uint32_t i = 0; i < M; ++i) {
    run += seq_gain[i];
    if (seq_viol[i] == 0 && run > best) best = run, best_len = i + 1;
  }
  for (uint32_t n = 0; n < N; ++n) rho_out[n] = rho[n];
  for (uint32_t i = 0; i < best_len; ++i) rho_out[seq[i]] = move[seq[i]];
  *n_seq = M, *n_applied = best_len, *gain_applied = best;
  free(mv), free(cur), free(psize), free(pinb), free(mark);
  return OR_OK;
}

/*
 * O16 -- Pi matching rounds over the top-Pi candidates ([P1] Sec. V-D).
 * Reading: in round r every node still unmatched proposes to the first entry
 * of its top-Pi list (score desc, id asc) that is still unmatched, with that
 * entry's score; matched nodes propose nothing and, being nobody's choice,
 * are left alone.  Each round's proposal graph then keeps the invariant of
 * Sec. V-A (no cycle longer than two: along a cycle the scores could not
 * drop and the ids would have to fall strictly).  The round's matching (the
 * handshake of O6, or the exact matching of O13 when optimal) adds its pairs.
 * Round 1 is the single-candidate level.  target/score are the pi x N arrays
 * of or_rate_top.
 */
int or_match_rounds(uint32_t N, uint32_t pi, const uint32_t *target, const uint64_t *score,
                    int optimal, uint32_t *match, uint64_t *n_pairs) {
  *n_pairs = 0;
  uint32_t *tr = (uint32_t *)malloc(sizeof(uint32_t) * (N ? N : 1));
  uint64_t *sr = (uint64_t *)malloc(sizeof(uint64_t) * (N ? N : 1));
  uint32_t *mr = (uint32_t *)malloc(sizeof(uint32_t) * (N ? N : 1));
  if (!tr || !sr || !mr) {
    free(tr), free(sr), free(mr);
    return OR_ENOMEM;
  }
  for (uint32_t n = 0; n < N; ++n) match[n] = n;
  int rc = OR_OK;
  for (uint32_t r = 0; r < pi && rc == OR_OK; ++r) {
    for (uint32_t n = 0; n < N; ++n) {
      tr[n] = NONE, sr[n] = 0;
      if (match[n] != n) continue;
      for (uint32_t j = 0; j < pi; ++j) {
        const uint32_t m = target[(size_t)j * N + n];
        if (m != NONE && match[m] == m) {
          tr[n] = m, sr[n] = score[(size_t)j * N + n];
          break;
        }
      }
    }
    uint64_t np = 0;
    rc = optimal ? or_match_dp(N, tr, sr, mr, &np) : or_match(N, tr, sr, mr, &np);
    if (rc != OR_OK) break;
    for (uint32_t n = 0; n < N; ++n)
      if (mr[n] != n) match[n] = mr[n];
    *n_pairs += np;
  }
  free(tr), free(sr), free(mr);
  return rc;
}
