/*
 * chp.h -- C ABI of the constrained hypergraph coarsening library (gfx950).
 *
 * One coarsening level of the multi-level partitioner in
 *   [HP]  Ronzani & Silvano, "Hypergraph Partitioning on GPU with Distinct
 *         Incident Hyperedges and Size Constraints" (TPDS submission), and
 *   [IC]  Ronzani & Silvano, "Incidence Constraints in Hypergraph Partitioning
 *         on GPU" (AsHES 2026 prototype),
 * plus the evaluation of a partition, under the two hard limits of [HP]
 * Sec. II-B: a partition holds at most Omega node weight and at most Delta
 * distinct inbound hyperedges.
 *
 * Conventions shared by every call
 *  - Ids are uint32; 0xFFFFFFFF (CHP_NONE) means "none".  Offsets are int64.
 *    Hyperedge weights and node sizes are uint32.  Ratings are uint64 fixed
 *    point with 40 fractional bits (eta_fx = eta * 2^40, rounded down per
 *    hyperedge term).
 *  - Every array named in a struct or argument is DEVICE memory of the
 *    context's GPU unless its name ends in _host.
 *  - All work is enqueued on the HIP stream given to chp_create.  A call that
 *    returns a host value or must size an allocation synchronises that stream
 *    before it returns; the others return as soon as the work is enqueued.
 *  - Every segment of every CSR is sorted ascending (the canonical form):
 *    a hyperedge holds its sources then its destinations, each run sorted; an
 *    incidence segment holds in(n) then out(n), each run sorted; N(n) sorted.
 *  - A failing call returns a negative CHP_E* code, leaves its outputs
 *    unspecified, never publishes a partial chp_hgraph, and stores a message
 *    retrievable with chp_last_error.  One context must not be used by two
 *    host threads at once.
 */
#ifndef CHP_H
#define CHP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CHP_NONE 0xFFFFFFFFu
#define CHP_FX_SHIFT 40

enum {
  CHP_OK = 0,
  CHP_EINVAL = -1,      /* null pointer, id out of range, duplicate pin, src and dst overlap,
                           empty hyperedge, zero weight or size, bad offsets, rho >= k */
  CHP_ENOMEM = -2,      /* the allocator returned NULL */
  CHP_EOVERFLOW = -3,   /* weight >= 2^24, or a node's sum of rating terms plus the noise
                           cap reaches 2^63 */
  CHP_EINFEASIBLE = -4, /* a single node already breaks Omega or Delta ([HP] Sec. II-B
                           assumes a valid solution exists) */
  CHP_ECYCLE = -5,      /* the proposal graph has a cycle longer than two ([HP] Sec. V-A
                           proves it has none) */
  CHP_EDEVICE = -6      /* a HIP runtime error */
};

/* Device allocator used for every buffer the library owns or needs as
 * scratch.  alloc returns NULL on failure.  Memory is used only on the
 * context's stream, so a stream-ordered caching allocator may recycle a
 * block as soon as free is called. */
typedef void *(*chp_alloc_fn)(size_t bytes, void *user);
typedef void (*chp_free_fn)(void *ptr, void *user);

typedef struct chp_ctx chp_ctx;

/* Create a context bound to the current HIP device and to hip_stream (a
 * hipStream_t; NULL = the default stream).  alloc/free may both be NULL, in
 * which case hipMalloc/hipFree are used.  Returns CHP_OK and *out, or an
 * error (then *out is NULL). */
int chp_create(chp_ctx **out, void *hip_stream, chp_alloc_fn alloc, chp_free_fn free_fn,
               void *user);
void chp_destroy(chp_ctx *ctx);
/* Message of the last failing call on ctx ("" if none).  Owned by ctx. */
const char *chp_last_error(const chp_ctx *ctx);

/* Hyperedge CSR supplied by the caller ([HP] Sec. IV-B, Fig. 2): segment e
 * is e_pins[e_off[e] .. e_off[e+1]), its first e_nsrc[e] pins are src(e),
 * the rest dst(e) ([HP] Sec. II-A).  Any order inside each run is accepted.
 * Borrowed: must stay valid until the call that reads it has completed on
 * the stream. */
typedef struct {
  uint32_t n_nodes, n_edges;
  uint64_t n_pins;       /* == e_off[n_edges] */
  const int64_t *e_off;  /* [E+1] */
  const uint32_t *e_nsrc;/* [E]   */
  const uint32_t *e_pins;/* [P]   */
  const uint32_t *e_w;   /* [E]   omega(e) >= 1 */
  const uint32_t *n_size;/* [N]   size(n) >= 1 (node weight) */
} chp_edges;

/* One level of a hypergraph, owned by the library (allocated through the
 * context's allocator, released with chp_hgraph_free).  Canonical CSR:
 *  e_*:    hyperedges as in chp_edges, each run sorted.
 *  n_off/n_nin/n_inc: incidence ([HP] Sec. IV-B): segment n holds in(n)
 *          ascending, then out(n) ascending; n_nin[n] = |in(n)|.
 *  nb_off/nb: unique neighbourhoods N(n) = (U_{e in I(n)} e) \ {n}, sorted
 *          ([HP] Sec. II-A, V-B).  NULL (nb_total 0) when not built. */
typedef struct {
  uint32_t n_nodes, n_edges;
  uint64_t n_pins;
  int64_t *e_off;
  uint32_t *e_nsrc;
  uint32_t *e_pins;
  uint32_t *e_w;
  uint32_t *n_size;
  int64_t *n_off;
  uint32_t *n_nin;
  uint32_t *n_inc;
  int64_t *nb_off;
  uint32_t *nb;
  uint64_t nb_total;
} chp_hgraph;

/* Limits and rating options.
 *  omega, delta: [HP] Sec. II-B.
 *  noise_on, noise_seed: the symmetric tie-breaking noise of [HP] Sec. V-C,
 *    added once per neighbour pair: mix(seed, min(n,m), max(n,m)) mod (cap+1),
 *    mix = one splitmix64 output (Steele, Lea & Flood, OOPSLA 2014) from the
 *    state seed XOR (min * 2^32 + max), and cap = floor(sum_e t(e) / (10 |E|))
 *    with t(e) the fixed-point per-hyperedge term of Eq. 5. */
typedef struct {
  uint64_t omega;
  uint32_t delta;
  uint32_t noise_on;
  uint64_t noise_seed;
} chp_params;

/* build_incidence ([HP] Sec. IV-B, Fig. 2; Sec. II-A definitions).
 * Validates `in`, copies it into canonical form (runs sorted), builds the
 * incidence CSR and, if build_neighbors != 0, the neighbourhood CSR.
 * Errors, by precedence: EINVAL (bad offsets, e_nsrc > |e|, empty hyperedge,
 * weight 0, size 0, pin >= n_nodes, duplicate pin, src and dst overlap),
 * EOVERFLOW (weight >= 2^24), EINFEASIBLE (size(n) > omega or
 * |in(n)| > delta for some node).  Synchronises.  On success *out is a new
 * library-owned graph. */
int chp_build_incidence(chp_ctx *ctx, const chp_edges *in, const chp_params *prm,
                        int build_neighbors, chp_hgraph *out);

/* rate_and_match: candidate proposal ([HP] Sec. V-A, Eqs. 5-6, Sec. V-C) and
 * the deterministic handshake matching ([IC] Sec. III-A, III-B3).
 *  target[N]   best valid neighbour by (eta desc, id asc), CHP_NONE if none;
 *              valid(n,m) <=> size(n)+size(m) <= omega and
 *              |in(n) u in(m)| = |in(n)| + |in(m)| - inter(n,m) <= delta.
 *  score_fx[N] eta_fx(n, target(n)) (noise included), 0 if none.
 *  match[N]    partner of n, or n itself when unmatched.  Pairs are the
 *              two-cycles of target, then every other node takes its target
 *              iff the target is still free and n is its best proposer
 *              (highest score, smallest id on ties), resolved top-down.
 *  *n_pairs_host number of pairs.
 *  nb_invalid[g->nb_total] (optional, NULL = not written): the invalid-
 *              neighbour flags of [HP] Sec. V-C: byte i is 1 when the pair
 *              (n, g->nb[i]) of N(n)'s entry i breaks either limit, else 0.
 *              Handed to chp_contract they purge the coarse neighbourhoods.
 * Without g->nb (a graph built without neighbours) the neighbourhoods are
 * built here, for batches of consecutive nodes whose neighbour lists fit the
 * batch limit (chp_set_batch_entries), each batch rated before the next is
 * built ([HP] Sec. VII-C); nb_invalid must then be NULL.  Errors: EINVAL,
 * EOVERFLOW, ECYCLE.  Synchronises. */
int chp_rate_and_match(chp_ctx *ctx, const chp_hgraph *g, const chp_params *prm,
                       uint32_t *target, uint64_t *score_fx, uint32_t *match,
                       uint32_t *n_pairs_host, uint8_t *nb_invalid);

/* rate_top_and_match: the top-pi candidates with pi matching rounds
 * ([HP] Sec. V-D).  As chp_rate_and_match (which is this call with pi = 1),
 * except:
 *  target[pi * N], score_fx[pi * N]  row r (entries r*N .. r*N + N - 1) holds
 *              every node's (r+1)-th best valid neighbour by (eta desc, id
 *              asc) and its eta_fx; CHP_NONE and 0 past the node's valid
 *              neighbours.  Row 0 is chp_rate_and_match's target/score_fx.
 *  match[N]    built over pi rounds.  In each round every node not yet
 *              matched proposes to the first entry of its list that is not yet
 *              matched, with that entry's score; matched nodes propose
 *              nothing.  The round's proposals are matched as
 *              chp_rate_and_match matches its targets (the handshake, or the
 *              exact matching under CHP_MATCH_OPTIMAL), and its pairs join
 *              match.  Each round's proposals again form two-cycles at most:
 *              along a longer cycle the scores could not fall and the ids would
 *              have to fall strictly.  Rounds stop early after one that pairs
 *              nothing (the next would propose the same).
 *  *n_pairs_host pairs over all rounds.
 * chp_pair_leftovers then reads row 0 as its target.  pi must be 1 .. 4
 * (EINVAL otherwise).  Synchronises. */
int chp_rate_top_and_match(chp_ctx *ctx, const chp_hgraph *g, const chp_params *prm, uint32_t pi,
                           uint32_t *target, uint64_t *score_fx, uint32_t *match,
                           uint32_t *n_pairs_host, uint8_t *nb_invalid);

/* propose_moves: refinement move proposal ([HP] Sec. VI-A/B, Eq. 13) for the
 * partition rho[N] in [0, k).  With pins(p, e) the pins of e in partition p:
 *  saving(n)  = sum of w(e), e in I(n), pins(rho(n), e) == 1;
 *  loss(n, p) = sum of w(e), e in I(n), pins(p, e) == 0;
 *  move[N]    the p != rho(n) of largest saving(n) - loss(n, p), ties to the
 *             smallest p; with enforce_omega != 0 only partitions whose size
 *             plus size(n) stays within prm->omega; CHP_NONE if there is none
 *             (k == 1, or every other partition full);
 *  gain[N]    saving(n) - loss(n, move(n)) (int64), 0 with no move.
 * Only prm->omega is read.  Errors: EINVAL (k == 0, or some rho[n] >= k).
 * Synchronises. */
int chp_propose_moves(chp_ctx *ctx, const chp_hgraph *g, const uint32_t *rho, uint32_t k,
                      const chp_params *prm, int enforce_omega, uint32_t *move, int64_t *gain);

/* refine_moves: one refinement pass over proposed moves ([HP] Sec. VI-A,
 * VI-C, VI-D, Eqs. 14-15), run after chp_propose_moves on the same rho.
 *  rho[N]      the partition in [0, k); updated in place with the moves applied.
 *  move[N], gain[N]  as written by chp_propose_moves (CHP_NONE = no move).
 * The nodes with a move form the sequence, ordered as chp_set_move_order
 * sets (chains by default).  The in-sequence gain of the i-th move is the
 * connectivity it removes from the partition left by the moves before it:
 * w(e) for each hyperedge e of the node where it is the last pin left in its
 * partition, minus w(e) for each one with no pin in the destination yet.  A
 * partition is invalid while its size exceeds prm->omega or its inbound count
 * (hyperedges with a destination pin in it) exceeds prm->delta.  The prefix
 * applied is the one of largest summed in-sequence gain that leaves no
 * partition invalid; applying nothing (gain 0) is always allowed and ties go
 * to the shorter prefix.
 *  seq[N], seq_gain[N], seq_viol[N] (each optional, NULL = not written): the
 *              nodes in sequence order, their in-sequence gains (int64) and
 *              the invalid partitions after each move (first *n_seq_host
 *              entries).
 *  *n_seq_host moves in the sequence; *n_applied_host the prefix length
 *              applied; *gain_host its summed gain (the connectivity drop).
 * Deterministic.  Errors: EINVAL (k == 0, rho or move >= k, a move to its own
 * partition, N >= 2^29, a hyperedge of 2^30 pins or more), EOVERFLOW (a gain
 * outside [-2^31, 2^31)).  Synchronises. */
/* Order of the move sequence used by chp_refine_moves on ctx.
 * CHP_ORDER_CHAINS (the default): chains of moves ([HP] Sec. VI-C, Fig. 5).
 *   The moves are sorted by (source partition, gain desc, id asc).  In up to
 *   16 rounds (fewer when a round links nothing), every move n without a
 *   successor looks at the first 256 moves leaving its destination, takes
 *   those without a predecessor and picks the m of largest grade
 *   gain(m) - 1e-6 |size(n) - size(m)| - 1e-7 ||in(n)| - |in(m)|| (computed
 *   exactly, in units of 1e-7; ties to the smaller m); a move picked by
 *   several becomes the successor of the largest (grade, picker id).  The
 *   links form paths (started at the move without a predecessor) and cycles
 *   (started at their smallest node); chains, each in successor order, are
 *   ranked by total gain (desc) then first node (asc) and concatenated.
 * CHP_ORDER_GAIN: (gain desc, id asc), every chain of length one (the
 *   pages' ablation without chaining).
 * EINVAL for another value. */
#define CHP_ORDER_CHAINS 0
#define CHP_ORDER_GAIN 1
int chp_set_move_order(chp_ctx *ctx, int order);

int chp_refine_moves(chp_ctx *ctx, const chp_hgraph *g, uint32_t *rho, uint32_t k,
                     const chp_params *prm, const uint32_t *move, const int64_t *gain,
                     uint32_t *seq, int64_t *seq_gain, uint32_t *seq_viol, uint32_t *n_seq_host,
                     uint32_t *n_applied_host, int64_t *gain_host);

/* project_partition ([HP] Sec. III: the partition of a level is carried to
 * the level below through that level's coarsening map).
 *  gamma[n_fine]       coarse id of every node of the finer graph, as written
 *                      by chp_contract.
 *  rho_coarse[n_coarse] partition of every coarse node.
 *  rho_fine[n_fine]    written: rho_coarse[gamma[n]].
 * Errors: EINVAL (null pointer, some gamma[n] >= n_coarse).  Synchronises. */
int chp_project_partition(chp_ctx *ctx, uint32_t n_fine, const uint32_t *gamma, uint32_t n_coarse,
                          const uint32_t *rho_coarse, uint32_t *rho_fine);

/* refine_level: the refinement of one level of the uncoarsening ([HP]
 * Sec. VI-A: the proposal and the application of moves repeat theta times
 * per level, 16 by default; Sec. VI-B: the first half of the repetitions may
 * propose moves that overfill a partition, the second half only moves that fit
 * Omega, and every application keeps only valid prefixes).  Pass r runs
 * chp_propose_moves(enforce_omega = r >= theta / 2), then chp_refine_moves
 * with the context's move order, on rho[N] in place (partitions in [0, k)).
 *  *n_applied_host  moves applied over the passes;
 *  *gain_host       their summed in-sequence gain (the connectivity drop).
 * Errors: those of the two calls.  Synchronises. */
int chp_refine_level(chp_ctx *ctx, const chp_hgraph *g, uint32_t *rho, uint32_t k,
                     const chp_params *prm, uint32_t theta, uint32_t *n_applied_host,
                     int64_t *gain_host);

/* pair_leftovers: best-effort pairing of the nodes left without a partner
 * ([HP] Sec. V-C, last mechanism), run after chp_rate_and_match.
 *  target[N]  as written by chp_rate_and_match (read).
 *  match[N]   as written by chp_rate_and_match; updated in place: nodes with
 *             target NONE and match[n] == n may be paired among themselves.
 *  *n_pairs_host number of new pairs.
 * Those nodes are sorted by (size, id).  Node n binary-searches the last
 * position whose size fits omega - size(n), then takes the first node m != n
 * within 64 positions below it with |in(n)| + |in(m)| <= delta (the union
 * overestimated by the sum, so every pair is valid).  A node chosen by
 * several goes to the smallest id; n pairs with its choice when it won it and
 * nobody chose n.  Deterministic.  Errors: EINVAL.  Synchronises. */
int chp_pair_leftovers(chp_ctx *ctx, const chp_hgraph *g, const chp_params *prm,
                       const uint32_t *target, uint32_t *match, uint32_t *n_pairs_host);

/* contract ([HP] Sec. III and V-E; [IC] Sec. III-B4).
 *  gamma[N]   coarse id of every node: the rank of min(n, match(n)) among
 *             the nodes with match(n) >= n.
 *  *coarse    new library-owned graph: size'(c) = sum of member sizes; one
 *             coarse hyperedge per hyperedge, same id and weight, dst' =
 *             gamma(dst), src' = gamma(src) \ dst'; incidence rebuilt; N'
 *             rebuilt if build_neighbors != 0.
 *  nb_invalid (optional, NULL = none): flags of g's neighbour entries as
 *             written by chp_rate_and_match.  N'(c) then also drops
 *             gamma(m) for every flagged entry m of N(a) or N(b) ([HP]
 *             Sec. V-C: a flag marks every occurrence of that neighbour).
 *             Only invalid pairs are dropped: an invalid (a, m) stays
 *             invalid for (c, gamma(m)).  Needs n_nodes < 2^31 - 1.
 * match must be a symmetric involution (match[match[n]] == n), else EINVAL.
 * Synchronises to size its outputs; the last arrays of *coarse are written
 * in stream order (use them on the same stream, or synchronise before
 * reading them on the host). */
int chp_contract(chp_ctx *ctx, const chp_hgraph *g, const uint32_t *match, uint32_t *gamma,
                 int build_neighbors, chp_hgraph *coarse, const uint8_t *nb_invalid);

/* evaluate_partition ([HP] Eq. 1, Eq. 16, Sec. II-B).
 *  rho[N] in [0,k).  part_size[k] = sum of sizes per part (uint64);
 *  part_inb[k] = |{e : some d in dst(e) has rho(d) = p}|.
 *  summary_host[8] = {connectivity sum_e w (lambda-1), cut-net sum_e w [lambda>1],
 *                     #parts with size > omega, #parts with inbound > delta,
 *                     #empty parts, max part size, max part inbound, sum_e lambda}.
 * EINVAL if k == 0 (with nodes) or some rho[n] >= k.  Synchronises. */
int chp_evaluate_partition(chp_ctx *ctx, const chp_hgraph *g, const uint32_t *rho, uint32_t k,
                           const chp_params *prm, uint64_t *part_size, uint32_t *part_inb,
                           uint64_t summary_host[8]);

/* evaluate_partition_noalloc: chp_evaluate_partition for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, outputs and errors; the
 * caller still supplies rho, part_size and part_inb.  Every scratch buffer
 * comes from a fixed 64 MiB array that the library holds on each GPU it runs
 * on until the process ends (its device address is taken once per device
 * when the first context on that device is created); the call makes no
 * hipMalloc, hipFree or other allocating call and records no timing events.
 * Limits: k * 4 + 3 * n_edges * 4 bytes (each rounded up to 256) plus 512
 * must fit the 64 MiB, else EINVAL before any work; the buffer of hyperedges
 * too long for LDS (2 * their largest pin count * 8 bytes per workgroup, at
 * most 256 workgroups) must fit what is left, else EINVAL.  All calls on one
 * GPU share that GPU's array, whose contents persist between calls (every
 * counter the call needs is cleared by the call itself): calls that overlap
 * in time on one GPU, from any context or stream, race and give wrong
 * results.  Synchronises. */
int chp_evaluate_partition_noalloc(chp_ctx *ctx, const chp_hgraph *g, const uint32_t *rho,
                                   uint32_t k, const chp_params *prm, uint64_t *part_size,
                                   uint32_t *part_inb, uint64_t summary_host[8]);

/* Neighbour entries one rating batch may hold when chp_rate_and_match
 * builds the neighbourhoods itself (a graph without nb); 0 restores the
 * default (3 * 2^30, 12 GiB for the lists plus as much scratch).  A node
 * whose own list is larger gets a batch of its own. */
int chp_set_batch_entries(chp_ctx *ctx, uint64_t entries);

/* Matching used by chp_rate_and_match on ctx.  CHP_MATCH_HANDSHAKE (the
 * default): the greedy handshake described there ([IC] Sec. III-A).
 * CHP_MATCH_OPTIMAL: the exact maximum-weight matching of the proposal
 * pseudo-forest ([HP] Sec. V-D, Eqs. 7-12): edges {n, target(n)} of weight
 * score(n); bottom up ss0(n) = A(n) + max(0, best(n)) and ss1(n) = score(n) +
 * A(n), with A the sum of the children's ss0 and best the largest ss1 - ss0
 * of a child (smallest id on ties); a two-cycle {n, t} pairs when score(n) +
 * A(n) + A(t) > ss0(n) + ss0(t), a node taken by its target pairs with it, any
 * other node takes its best child when best > 0.  Its total score is the
 * largest over all matchings of proposal edges.  EINVAL for another mode. */
#define CHP_MATCH_HANDSHAKE 0
#define CHP_MATCH_OPTIMAL 1
int chp_set_matching(chp_ctx *ctx, int mode);

/* Graphs without neighbour lists: a node with 1..384 incident hyperedges and
 * at least min_visits (and below 2^27) pins over them is rated straight from
 * the incidence, its N(n) held in LDS one id window at a time and never
 * written out; the rest go through the per-batch lists.  Both routes give the
 * same target and score.  min_visits 0 restores the default (16384);
 * UINT64_MAX sends every node through the lists.  hash_keys caps the keys a
 * sparse window may claim before it stops and the next window resumes at the
 * first id it could not hold (0 = the table's capacity, 4608; 1 is taken as
 * 2): a lower cap only adds windows; the results do not change. */
int chp_set_incidence_rating(chp_ctx *ctx, uint64_t min_visits, uint32_t hash_keys);

/* Bins of the rating from the incidence (chp_set_incidence_rating).
 * CHP_INC_BINS_32 (the default; quantised bins in 32-bit LDS words): for a
 *   node whose Delta cannot reject any neighbour (|in(n)| + the largest |in|
 *   of the graph <= delta) and with pi == 1, each bin holds a sum of the terms
 *   t(e) shifted right by the smallest s that keeps the node's term sum below
 *   2^16, two ids to a word in dense id windows (four times the ids of the
 *   64-bit bins); sparse windows hash ids into 32-bit slots.  Those sums bound
 *   eta from below and above, and the neighbours whose bounds can still reach
 *   the best get their exact eta (t(e) summed over the hyperedges n and m
 *   share) at the node's end.  Other nodes (and one whose quantised terms
 *   would lose a hyperedge, or with more than 256 neighbours in reach) go to
 *   the 64-bit bins.
 * CHP_INC_BINS_64: every node through 64-bit bins of exact eta.
 * Both give the same target and score.  EINVAL for another value. */
#define CHP_INC_BINS_32 0
#define CHP_INC_BINS_64 1
int chp_set_incidence_bins(chp_ctx *ctx, int bins);

/* What the last chp_rate_and_match on ctx did about neighbourhoods:
 * *nb_entries = neighbour entries it built batch by batch, *batches = the
 * number of batches and *inc_nodes = the nodes it rated straight from the
 * incidence (all 0 when the graph carried its own lists).  Any pointer may
 * be NULL.  Host values only; no device work. */
int chp_last_rate_stats(const chp_ctx *ctx, uint64_t *nb_entries, uint32_t *batches,
                        uint32_t *inc_nodes);

/* Release every array of g (allocated by this library) and zero *g. */
void chp_hgraph_free(chp_ctx *ctx, chp_hgraph *g);

/* Kernel timing.  With timing on, the library brackets each of its kernel
 * launches with HIP events on the context stream and accumulates, per kernel
 * name, the number of launches and their total duration.  chp_get_timings
 * synchronises, fills up to max entries (names are owned by the library) and
 * returns the number of distinct kernels; chp_reset_timings clears them. */
typedef struct {
  const char *name;
  uint64_t launches;
  double total_ms;
} chp_timing;
int chp_set_timing(chp_ctx *ctx, int on);
/* Time only the kernels whose name starts with prefix (NULL or "" = all);
 * the events of the others are not recorded at all. */
int chp_set_timing_filter(chp_ctx *ctx, const char *prefix);
int chp_get_timings(chp_ctx *ctx, chp_timing *out, int max);
void chp_reset_timings(chp_ctx *ctx);

#ifdef __cplusplus
}
#endif
#endif /* CHP_H */
