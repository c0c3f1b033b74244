// Host-side launchers of the kernels (one translation unit per step).
#pragma once
#include <initializer_list>

#include "common.h"

constexpr u32 LDS_CAP_U32 = 8192;   // u32 keys one workgroup sorts in LDS
constexpr u32 LDS_CAP_U64 = 8192;   // u64 keys one workgroup sorts in LDS
constexpr u32 RATE_SMALL_CAP = 384; // |N(n)| of a node rated by one wave
constexpr u32 RATE_MAX_PI = 4;      // candidates a node may keep ([HP] Sec. V-D uses 4)
constexpr u32 NBM_LDS_CAP = 8192;   // largest coarse neighbour bound merged in LDS

// Runs to sort in place, bucketed by length: class 0 (<= 64 keys, one wave
// each), class 1 (<= LDS_CAP_U32 keys, one workgroup in LDS), class 2
// (longer: one workgroup, global merge sort).  cnt[0..2] = class counts,
// cnt[3] = longest class-2 run, cnt[4] = number of queued hyperedges.
struct RunLists {
  i64 *start[3];
  u32 *len[3];
  u32 *cnt;  // device [8]
};

// Node work lists by class: cnt[0..4] class counts, cnt[5] = largest work of
// the last (global-memory) class, cnt[7] = overflow flag.
struct NbLists {
  u32 *list[5];
  u32 *cnt;  // device [8]
};

// Hyperedge work lists by |e|: <= 64 (wave), <= LDS_CAP_U64 (workgroup LDS),
// longer (workgroup, global merge sort).  cnt[3] = longest class-2 edge.
struct EdgeLists {
  u32 *list[4];  // list[3]: only the coarse incidence's larger LDS class
  u32 *cnt;  // device [8]
};

// ---- k_build.hip : canonical edges, incidence, neighbourhoods -------------
void launch_check_edges(chp_ctx *c, u32 N, u32 E, u64 P, const i64 *e_off, const u32 *e_nsrc,
                        const u32 *e_w, const u32 *n_size);
void launch_edges_canon(chp_ctx *c, u32 N, u32 E, const i64 *e_off, const u32 *e_nsrc,
                        const u32 *pins_in, u32 *pins_out, u32 *bad_edges, RunLists rl);
void launch_sort_runs(chp_ctx *c, u32 *data, RunLists rl, const u32 *host_cnt, u32 *scratch,
                      u64 scratch_per_wg, u32 grid_big);
void launch_edges_check(chp_ctx *c, const i64 *e_off, const u32 *e_nsrc, const u32 *pins,
                        const u32 *list, u32 count);
void launch_degrees(chp_ctx *c, u32 E, const i64 *e_off, const u32 *e_nsrc, const u32 *pins,
                    u32 *indeg, u32 *outdeg);
void launch_node_feas(chp_ctx *c, u32 N, const u32 *indeg, const u32 *outdeg, const u32 *n_size,
                      u64 omega, u32 delta, u32 *deg, u32 *n_nin);
void launch_scatter(chp_ctx *c, u32 E, const i64 *e_off, const u32 *e_nsrc, const u32 *pins,
                    const i64 *n_off, const u32 *n_nin, u32 *cur_in, u32 *cur_out, u32 *n_inc);
void launch_node_runs(chp_ctx *c, u32 N, const i64 *n_off, const u32 *n_nin, RunLists rl);
// nodes lo .. lo + N - 1
// classes: list[0] one wave, list[1] LDS bitmap, list[2] workgroup sort
void launch_nb_classify(chp_ctx *c, u32 lo, u32 N, const i64 *e_off, const u32 *e_nsrc,
                        const u32 *pins, const i64 *n_off, const u32 *n_inc, u32 *bound,
                        NbLists nl, const uint8_t *skip = nullptr);
void launch_nb_build(chp_ctx *c, u32 N, const i64 *e_off, const u32 *pins, const i64 *n_off,
                     const u32 *n_inc, const u32 *bound, const i64 *ooff, u32 *obuf, u32 *count,
                     NbLists nl, const u32 *host_cnt);
void launch_nb_compact(chp_ctx *c, u32 N, const i64 *ooff, const u32 *obuf, const i64 *nb_off,
                       u32 *nb);

// ---- k_rate.hip : terms, noise cap, rating, handshake ---------------------
// capinfo (device u64[4]): cap, d = cap + 1, magic = floor((2^64-1)/d), 0
u32 terms_partials(u32 E);
void launch_terms(chp_ctx *c, u32 E, const i64 *e_off, const u32 *e_w, u64 *t, u64 *partials,
                  u32 nparts, u64 *capinfo);
// Header of a node queued for the rating kernel (48 bytes, read a word per
// lane): n, |N(n)|, |in(n)|, size(n), |I(n)|, nb_off[n], n_off[n].
struct NodeRec {
  u32 n, K, nin, size, deg, pad0;
  i64 nb0, i0;
  u32 pad1, pad2;
};
static_assert(sizeof(NodeRec) == 48, "NodeRec layout");

struct RateArgs {
  u32 N;
  const i64 *e_off;
  const u32 *e_nsrc;
  const u32 *e_pins;
  const u64 *t;
  const i64 *n_off;
  const u32 *n_nin;
  const u32 *n_inc;
  const u32 *n_size;
  const i64 *nb_off;
  const u32 *nb;
  u32 *cur;  // [2 * pins] window cursors of nodes whose hyperedges span several chunks
  uint8_t *flag;  // [nb_total] invalid-neighbour flags to write, or null
  const u64 *capinfo;
  u64 omega;
  u32 delta;
  u32 noise_on;
  u64 seed;
  u32 *target;  // [pi * N]: row r holds every node's (r+1)-th best valid candidate
  u64 *score;   // [pi * N]
  u32 pi;       // rows, 1 .. RATE_MAX_PI
  u32 *flags;
};
// nodes lo .. hi - 1
void launch_rate_classify(chp_ctx *c, const RateArgs &a, u32 lo, u32 hi, NbLists nl,
                          NodeRec *recs, NodeRec *big);
void launch_rate(chp_ctx *c, const RateArgs &a, NbLists nl, const NodeRec *recs, u32 nrec,
                 const NodeRec *big, u32 *work);
// Refinement move proposal: pins(., e) lists (pl[P] packed p << 32 | count in
// each hyperedge's pin range, lam[E] their lengths), the free-capacity
// max-tree over K2 (a power of two >= k) leaves, and the per-node gains
// (launch_gains with host_cnt null classifies into lists / cnt[0..1]; then
// again with the host copy of cnt; cnt[0..2] zeroed before, cnt[2] being the
// heavy path's work counter).
void launch_pins_lists(chp_ctx *c, const i64 *e_off, const u32 *pins, const u32 *rho, u32 k,
                       u64 *pl, u32 *lam, EdgeLists el, const u32 *host_cnt, u64 *scratch,
                       u64 per_wg, u32 grid_big);
void launch_free_tree(chp_ctx *c, u32 k, u32 K2, const u64 *part_size, u64 omega, u64 *tree);
void launch_gains(chp_ctx *c, u32 N, u32 k, u32 K2, int enforce, u64 omega, const i64 *e_off,
                  const u32 *e_w, const u64 *pl, const u32 *lam, const i64 *n_off,
                  const u32 *n_inc, const u32 *n_size, const u32 *rho, const u64 *part_size,
                  const u64 *tree, u32 *move, i64 *gain, u32 *lists, u32 *cnt,
                  const u32 *host_cnt);

// Exact matching on the proposal pseudo-forest (k_match_dp.hip): every
// array N long except small[4] (small[0] = largest depth, zeroed before).
struct DpScratch {
  u32 *par, *anc, *dist, *anc2, *dist2, *byd, *bestc, *small;
  u64 *A, *bestv, *ss0, *diff;
};
// depths by pointer jumping (d.dist, small[0] = the largest; flags ECYCLE
// when a node reaches no root); match set to the identity
void launch_dp_prepare(chp_ctx *c, u32 N, const u32 *target, DpScratch &d, u32 *match);
void launch_dp_count(chp_ctx *c, u32 N, const u32 *dist, u32 *cntd);
// cursor[D+1] = the host offsets offd[0..D] on the device (consumed); the
// levels bottom up, then top down; npairs zeroed before
void launch_dp_levels(chp_ctx *c, u32 N, const u32 *target, const u64 *score, DpScratch &d,
                      u32 D, u32 *cursor, const u32 *offd, u32 *match, u32 *npairs);

// Device-wide sort of n distinct u64 keys; tmp holds n; returns a or tmp.
u64 *sort_keys_u64(chp_ctx *c, u64 *a, u64 *tmp, u64 n);

// ---- k_refine.hip : one refinement pass over proposed moves -----------------
// sequence keys (2^31 - 1 - gain) << 32 | n of the nodes with a move; flags
// EINVAL for rho or move out of range, EOVERFLOW for a gain beyond 32 bits
void launch_seq_keys(chp_ctx *c, u32 N, u32 k, const u32 *rho, const u32 *move, const i64 *gain,
                     u64 *keys, u32 *cnt);
void launch_seq_rank(chp_ctx *c, u32 M, const u64 *keys, u32 *seq, u32 *rank);
// move chains: buffers per position of the (source partition, gain rank)
// order, except posn (by node)
constexpr u32 CHAIN_ROUNDS = 16;  // linking rounds at most
struct ChainBufs {
  u32 *node, *size, *nin, *dest, *pred, *succ, *posn;
  i64 *gain;
  u32 *pick, *wid;
  i64 *pgr, *wgr;
  u32 *anc, *anc2, *mn, *mn2, *cut, *dist, *clen, *cstart;
  i64 *ctot;
  u32 *pstart;  // [k + 1] first position of each source partition's run
  u32 *done;    // pickers whose window has no candidate left
};
void launch_chain_setup(chp_ctx *c, u32 M, u32 k, const u32 *seq, const u32 *rho,
                        const u32 *move, const u32 *n_size, const u32 *n_nin, const i64 *gain,
                        u64 *keys, u64 *ktmp, ChainBufs &B, const u64 **sorted);
void launch_chain_round(chp_ctx *c, u32 M, ChainBufs &B, u32 *links);
void launch_chain_walk(chp_ctx *c, u32 M, ChainBufs &B);
void launch_chain_heads(chp_ctx *c, u32 M, ChainBufs &B, u32 *heads, u64 *hk, u32 *cnt);
void launch_chain_rank_keys(chp_ctx *c, u32 H, const u32 *heads, ChainBufs &B,
                            const u64 *sorted_totals, u64 *keys);
void launch_chain_lens(chp_ctx *c, u32 H, const u64 *keys, ChainBufs &B, u32 *lens);
void launch_chain_place(chp_ctx *c, u32 M, u32 H, const u64 *keys, const i64 *coff,
                        ChainBufs &B, u32 *seq, u32 *rank);
// hyperedges by event capacity: lists[k * E ..], cnt[0..2], cnt[3] = longest class 2
void launch_ev_classify(chp_ctx *c, u32 E, const i64 *e_off, u32 *lists, u32 *cnt);
u64 ev_global_words(u32 max_len);  // scratch words per workgroup of class 2
void launch_ev_edges(chp_ctx *c, u32 E, const i64 *e_off, const u32 *e_nsrc, const u32 *pins,
                     const u32 *e_w, const u32 *rho, const u32 *move, const u32 *rank,
                     i64 *ingain, u32 *dleave, u32 *denter, u32 *inb0, const u32 *lists,
                     const u32 *cnt, const u32 *host_cnt, u64 *scratch, u32 grid_global);
void launch_pev(chp_ctx *c, u32 M, const u32 *seq, const u32 *rho, const u32 *move, u64 *keys);
void launch_pev_vals(chp_ctx *c, u64 Q, const u64 *keys, const u32 *seq, const u32 *n_size,
                     const u32 *dleave, const u32 *denter, i64 *vs, i64 *vi);
void launch_pev_flips(chp_ctx *c, u64 Q, const u64 *keys, const i64 *vs, const i64 *vi,
                      const i64 *Ps, const i64 *Pi, const u64 *size0, const u32 *inb0,
                      u64 omega, u32 delta, i64 *vdelta);
void launch_viol0(chp_ctx *c, u32 k, const u64 *size0, const u32 *inb0, u64 omega, u32 delta,
                  u32 *v0);
void launch_prefix(chp_ctx *c, u32 M, const i64 *ingain, const i64 *Pg, const i64 *vdelta,
                   const i64 *Pv, const u32 *v0, i64 *seq_gain, u32 *seq_viol, u64 *best,
                   u32 *best_len, const u32 *seq, const u32 *move, u32 *rho);

// Best-effort pairing of the unmatched nodes without a target: gather their
// keys (size << 32 | id) into keys (cnt[0..1] zeroed and cnt[2..3] filled
// with NONE before: the gathered nodes' smallest size and |in| go there),
// then, once sorted, choose, claim (claim[N] filled with NONE before) and
// pair into match.
void launch_left_gather(chp_ctx *c, u32 N, const u32 *target, const u32 *match,
                        const u32 *n_size, const u32 *n_nin, u64 *keys, u32 *cnt);
void launch_left_pair(chp_ctx *c, u32 nl, const u64 *keys, const u32 *n_nin, u64 omega,
                      u32 delta, u32 window, u32 *choice, u32 *claim, u32 *match, u32 *npairs);

// Rating straight from the incidence (graphs without neighbour lists): the
// classification lists the nodes of [0, a.N) with 1..384 incident hyperedges
// and min_visits .. 2^27 - 1 incident pins, sets skip[n] for them and writes
// gmax = {max size, max |in|} (cnt and gmax zeroed before); launch_rate_inc
// rates the listed nodes (work zeroed before; host_count = *cnt), a sparse
// window claiming at most hash_keys keys (0 = its full capacity).
void launch_inc_classify(chp_ctx *c, const RateArgs &a, u64 min_visits, uint8_t *skip,
                         NodeRec *recs, u32 *cnt, u32 *gmax);
void launch_rate_inc(chp_ctx *c, const RateArgs &a, const NodeRec *recs, const u32 *cnt,
                     const u32 *gmax, u32 *work, u32 host_count, u32 hash_keys);
// The same nodes with 32-bit bins (k_rate_incq.hip) where Delta cannot bind
// for the node; the nodes it cannot rate are appended to spill / *spill_cnt
// (zeroed before) for launch_rate_inc.
// samp_off / samp: the per-level sample array of launch_samples, or null
// (the samples are then read from the pins).
void launch_rate_incq(chp_ctx *c, const RateArgs &a, const NodeRec *recs, const u32 *cnt,
                      const u32 *gmax, u32 *work, u32 host_count, u32 hash_keys, NodeRec *spill,
                      u32 *spill_cnt, const i64 *samp_off, const u32 *samp);
// Every 16th pin of each run of each hyperedge (source run, then destination
// run) into samp[samp_off[e] ..]; samp_off [E + 1] by a scan of cnt [E] (tmp:
// scan_tmp_words(E)); samp holds samples_bound(E, P) entries.
void launch_samples(chp_ctx *c, u32 E, const i64 *e_off, const u32 *e_nsrc, const u32 *pins,
                    u32 *cnt, i64 *samp_off, i64 *tmp, u32 *samp);
u64 samples_bound(u32 E, u64 P);

struct MatchScratch {
  u64 *bscore;  // [N] zeroed
  u32 *bid;     // [N] filled with NONE
  uint8_t *tk;  // [N]
  u32 *p0, *p1; // [N] pointer-jumping buffers (fallback only)
  uint8_t *x0, *x1;
};
void launch_match(chp_ctx *c, u32 N, const u32 *target, const u64 *score, MatchScratch ms,
                  u32 *match, u32 *npairs);
void launch_match_jump(chp_ctx *c, u32 N, const u32 *target, MatchScratch ms);
void launch_match_write(chp_ctx *c, u32 N, const u32 *target, MatchScratch ms, u32 *match,
                        u32 *npairs);

// ---- k_contract.hip --------------------------------------------------------
void launch_rep(chp_ctx *c, u32 N, const u32 *match, u32 *is_rep);
void launch_gamma(chp_ctx *c, u32 N, const u32 *match, const i64 *rank, const u32 *n_size,
                  u32 *gamma, u32 *c_size, u32 *rep_of);
void launch_edge_classify(chp_ctx *c, u32 E, const i64 *e_off, EdgeLists el);
void launch_edge_contract(chp_ctx *c, const i64 *e_off, const u32 *e_nsrc, const u32 *pins,
                          const u32 *gamma, u32 *opins, u32 *olen, u32 *onsrc, EdgeLists el,
                          const u32 *host_cnt, u64 *scratch, u64 per_wg, u32 grid_big,
                          u32 *rest, bool narrow);  // narrow: every gamma < 2^31 - 1
void launch_pins_compact(chp_ctx *c, u32 E, const i64 *src_off, const u32 *src,
                         const i64 *dst_off, u32 *dst);

// ---- k_coarse.hip : coarse incidence and neighbourhoods from the members ---
void launch_cinc_classify(chp_ctx *c, u32 Nc, const u32 *rep_of, const u32 *match,
                          const i64 *n_off, const u32 *n_nin, u32 *bound, u32 *cnt_in,
                          u32 *cnt_tot, EdgeLists el);
void launch_cinc_build(chp_ctx *c, const i64 *n_off, const u32 *n_nin, const u32 *n_inc,
                       const u32 *rep_of, const u32 *match, const i64 *ooff, u32 *obuf,
                       u32 *cnt_in, u32 *cnt_tot, EdgeLists el, const u32 *host_cnt,
                       u64 *scratch, u64 per_wg, u32 grid_big,
                       bool narrow);  // narrow: every hyperedge id < 2^31 - 1
void launch_cinc_compact(chp_ctx *c, u32 Nc, const u32 *rep_of, const u32 *match,
                         const i64 *n_off, const u32 *n_inc, const i64 *ooff, const u32 *obuf,
                         const i64 *c_off, u32 *c_inc);
void launch_nbm_classify(chp_ctx *c, u32 Nc, const u32 *rep_of, const u32 *match,
                         const i64 *nb_off, u32 *bound, NbLists nl);
void launch_nbm_build(chp_ctx *c, const i64 *nb_off, const u32 *nb, const uint8_t *fl,
                      const u32 *gamma,
                      const u32 *match, const u32 *rep_of, const i64 *ooff, u32 *obuf,
                      u32 *count, NbLists nl, const u32 *host_cnt);

// ---- k_bitmap.hip : sorted distinct lists through an LDS bitmap ------------
void launch_nb_bitmap(chp_ctx *c, u32 N, const i64 *e_off, const u32 *pins, const i64 *n_off,
                      const u32 *n_inc, const u32 *bound, const i64 *ooff, u32 *obuf, u32 *count,
                      const u32 *list, const u32 *cnt, u32 host_count);
void launch_nbm_bitmap(chp_ctx *c, const i64 *nb_off, const u32 *nb, const uint8_t *fl,
                       const u32 *gamma,
                       const u32 *match, const u32 *rep_of, const i64 *ooff, u32 *obuf,
                       u32 *count, const u32 *list, const u32 *cnt, u32 host_count);

// ---- k_eval.hip --------------------------------------------------------------
void launch_eval_nodes(chp_ctx *c, u32 N, const u32 *rho, u32 k, const u32 *n_size,
                       u64 *part_size, u32 *part_cnt);
void launch_eval_edges(chp_ctx *c, const i64 *e_off, const u32 *e_nsrc, const u32 *pins,
                       const u32 *e_w, const u32 *rho, u32 k, u32 *part_inb, u64 *summary,
                       EdgeLists el, const u32 *host_cnt, u64 *scratch, u64 per_wg,
                       u32 grid_big);
void launch_eval_parts(chp_ctx *c, u32 k, const u64 *part_size, const u32 *part_inb,
                       const u32 *part_cnt, u64 omega, u32 delta, u64 *summary);

// ---- small device fills (api.hip) -------------------------------------------
void launch_fill_u32(chp_ctx *c, u32 *p, u64 n, u32 v);
// p[n] = n for n < N
void launch_iota(chp_ctx *c, u32 N, u32 *p);
// One of the pi matching rounds over top-pi lists (rows of stride N): each
// node still unmatched in match proposes to its first still-unmatched entry
// (tr/sr, NONE32/0 otherwise); after the round's matching mr, its pairs join
// match.
void launch_round_prep(chp_ctx *c, u32 N, u32 pi, const u32 *target, const u64 *score,
                       const u32 *match, u32 *tr, u64 *sr);
void launch_round_merge(chp_ctx *c, u32 N, const u32 *mr, u32 *match);
// Several fills in one launch (at most 8 arrays): n elements of u32 (or of
// u64 when wide) set to v.
struct FillItem {
  void *p;
  u64 n;
  u64 v;
  bool wide;
};
struct FillDesc {
  void *p[8];
  u64 n[8];
  u64 v[8];
  u32 wide[8];
  u32 cnt;
};
void launch_fills(chp_ctx *c, std::initializer_list<FillItem> items);
void launch_fill_u64(chp_ctx *c, u64 *p, u64 n, u64 v);
