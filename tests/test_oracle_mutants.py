"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a private copy of ``oracle/chp_oracle.c``
(on the CPU), builds it, and checks that the hand-worked example, the
brute-force comparisons or the closed forms reject it.
"""
import os
import subprocess
import sys
import tempfile

import pytest

import oracle
import test_oracle_pins as pins

MUTANTS = {
    "bc_tie_largest_id": ("(score[c] == score[b] && c < b)", "(score[c] == score[b] && c > b)"),
    "target_tie_largest_id": ("return (a->id > b->id) - (a->id < b->id);",
                              "return (a->id < b->id) - (a->id > b->id);"),
    "inter_counts_out_edges": ("if (e_is_in && i >= d0) inter[m]++;", "if (i >= d0) inter[m]++;"),
    "delta_off_by_one": ("if (u > J->delta) continue;", "if (u > (uint64_t)J->delta + 1) continue;"),
    "omega_ignored": ("if ((uint64_t)g->n_size[n] + g->n_size[m] > J->omega) continue;",
                      "if ((uint64_t)g->n_size[n] > J->omega) continue;"),
    "term_wrong_size": ("t[e] = ((uint64_t)g->e_w[e] << FX_SHIFT) / sz;",
                        "t[e] = ((uint64_t)g->e_w[e] << FX_SHIFT) / (sz > 1 ? sz - 1 : 1);"),
    "noise_asymmetric": ("uint32_t a = n < m ? n : m, b = n < m ? m : n;",
                         "uint32_t a = n, b = m;"),
    "noise_twice": ("if (J->noise_on) eta[m] += or_noise(J->seed, J->cap, n, m);",
                    "if (J->noise_on) eta[m] += 2 * or_noise(J->seed, J->cap, n, m);"),
    "src_keeps_dst_dups": ("if (sorted_has(tmp, ud, sl[i])) continue;", ";"),
    "gamma_rank_by_max": ("uint32_t rep = n < match[n] ? n : match[n];\n    if (rep == n)",
                          "uint32_t rep = n > match[n] ? n : match[n];\n    if (rep == n)"),
    "conn_counts_lambda": ("conn += (uint64_t)g->e_w[e] * (lambda - 1);",
                           "conn += (uint64_t)g->e_w[e] * lambda;"),
    "in_out_swapped": ("if (i < g->e_off[e] + g->e_nsrc[e]) n_inc[fout[n]++] = e;\n      else n_inc[fin[n]++] = e;",
                       "if (i < g->e_off[e] + g->e_nsrc[e]) n_inc[fin[n]++] = e;\n      else n_inc[fout[n]++] = e;"),
    "neighbors_keep_self": ("if (m != n && seen[m] != n) {\n          seen[m] = n;\n          list[cnt++] = m;",
                            "if (seen[m] != n) {\n          seen[m] = n;\n          list[cnt++] = m;"),
    "taken_no_alternation": ("val = !val;", "val = val;"),
    "roots_not_matched_by_default": ("if (tg != NONE && target[tg] == v) { /* v in R */",
                                     "if (0) {"),
    "inbound_counts_sources": ("if (i >= d0 && dmark[p] != e) {", "if (dmark[p] != e) {"),
    "leftover_largest_claimer": ("if (choice[i] != NONE && n < claim[choice[i]]) claim[choice[i]] = n;",
                                 "if (choice[i] != NONE && (claim[choice[i]] == NONE || n > claim[choice[i]])) claim[choice[i]] = n;"),
    "leftover_scan_from_bottom": ("const uint32_t j = lo - 1 - s;", "const uint32_t j = s;"),
    "leftover_claimed_pairs_too": ("if (m != NONE && claim[m] == n && claim[n] == NONE) {",
                                   "if (m != NONE && claim[m] == n) {"),
    "leftover_delta_ignored": ("if ((uint64_t)n_nin[n] + n_nin[m] <= delta) {", "if (1) {"),
    "moves_loss_counts_one_pin": ("if (pins_of(poff, ppart, pcnt, e, p) == 0) loss += g->e_w[e];",
                                  "if (pins_of(poff, ppart, pcnt, e, p) <= 1) loss += g->e_w[e];"),
    "moves_saving_any_pin": ("if (pins_of(poff, ppart, pcnt, e, pn) == 1) saving += g->e_w[e];",
                             "if (pins_of(poff, ppart, pcnt, e, pn) >= 1) saving += g->e_w[e];"),
    "moves_tie_largest_id": ("if (best == NONE || gp > best_gain) best = p, best_gain = gp;",
                             "if (best == NONE || gp >= best_gain) best = p, best_gain = gp;"),
    "dp_roots_pair_on_tie": ("      if (pair > apart) {", "      if (pair >= apart) {"),
    "dp_best_child_largest_id": ("if (bestc[p] == NONE || d > bestv[p] || (d == bestv[p] && n < bestc[p]))",
                                 "if (bestc[p] == NONE || d > bestv[p] || (d == bestv[p] && n > bestc[p]))"),
    "dp_ss1_without_children": ("      ss1[n] = score[n] + A[n];", "      ss1[n] = score[n];"),
    "dp_roots_never_take_children": ("        if (bestc[n] != NONE && bestv[n] > 0) match[n] = bestc[n], match[bestc[n]] = n;\n        if (bestc[t] != NONE && bestv[t] > 0) match[t] = bestc[t], match[bestc[t]] = t;",
                                     ";"),
    "refine_order_gain_ascending": ("const or_mv *a = (const or_mv *)x, *b = (const or_mv *)y;\n  if (a->gain != b->gain) return a->gain > b->gain ? -1 : 1;",
                                    "const or_mv *a = (const or_mv *)x, *b = (const or_mv *)y;\n  if (a->gain != b->gain) return a->gain < b->gain ? -1 : 1;"),
    "refine_gain_in_isolation": ("      if (count_in(g, cur, e, ps, 0) == 1) gi += g->e_w[e];\n      if (count_in(g, cur, e, pd, 0) == 0) gi -= g->e_w[e];",
                                 "      if (count_in(g, rho, e, ps, 0) == 1) gi += g->e_w[e];\n      if (count_in(g, rho, e, pd, 0) == 0) gi -= g->e_w[e];"),
    "refine_inbound_all_pins": ("      if (count_in(g, cur, e, ps, 1) == 1) pinb[ps]--;\n      if (count_in(g, cur, e, pd, 1) == 0) pinb[pd]++;",
                                "      if (count_in(g, cur, e, ps, 0) == 1) pinb[ps]--;\n      if (count_in(g, cur, e, pd, 0) == 0) pinb[pd]++;"),
    "refine_prefix_ties_longest": ("if (seq_viol[i] == 0 && run > best) best = run, best_len = i + 1;",
                                   "if (seq_viol[i] == 0 && run >= best) best = run, best_len = i + 1;"),
    "refine_ignores_violations": ("if (seq_viol[i] == 0 && run > best) best = run, best_len = i + 1;",
                                  "if (run > best) best = run, best_len = i + 1;"),
    "refine_viol_omega_off_by_one": ("    viol += psize[ps] > omega || pinb[ps] > delta;\n    viol += psize[pd] > omega || pinb[pd] > delta;",
                                     "    viol += psize[ps] > omega + 1 || pinb[ps] > delta;\n    viol += psize[pd] > omega + 1 || pinb[pd] > delta;"),
    "chain_window_255": ("#define CHAIN_WINDOW 256", "#define CHAIN_WINDOW 255"),
    "chain_window_257": ("#define CHAIN_WINDOW 256", "#define CHAIN_WINDOW 257"),
    "chain_one_round": ("#define CHAIN_ROUNDS 16", "#define CHAIN_ROUNDS 1"),
    "chain_conflict_smaller_picker": ("if (winner[m] == NONE || gr > wgrade[m] || (gr == wgrade[m] && n > winner[m]))",
                                      "if (winner[m] == NONE || gr > wgrade[m] || (gr == wgrade[m] && n < winner[m]))"),
    "chain_pick_larger_id": ("if (pick[n] == NONE || gr > bg || (gr == bg && m < pick[n])) pick[n] = m, bg = gr;",
                             "if (pick[n] == NONE || gr > bg || (gr == bg && m > pick[n])) pick[n] = m, bg = gr;"),
    "chain_grade_no_inbound": ("return 10000000ll * gain[m] - 10 * ds - di;", "return 10000000ll * gain[m] - 10 * ds;"),
    "chain_grade_alpha_equals_beta": ("return 10000000ll * gain[m] - 10 * ds - di;", "return 10000000ll * gain[m] - ds - di;"),
    "chain_grade_alpha_large": ("return 10000000ll * gain[m] - 10 * ds - di;", "return 10000000ll * gain[m] - 100 * ds - di;"),
    "chain_grade_gain_scale": ("return 10000000ll * gain[m] - 10 * ds - di;", "return 100000000ll * gain[m] - 10 * ds - di;"),
    "chain_grade_of_picker": ("return 10000000ll * gain[m] - 10 * ds - di;", "return 10000000ll * gain[n] - 10 * ds - di;"),
    "chain_rank_ascending": ("if (a->total != b->total) return a->total > b->total ? -1 : 1;",
                             "if (a->total != b->total) return a->total < b->total ? -1 : 1;"),
    "chain_rank_ties_larger_first": ("return a->first < b->first ? -1 : (a->first > b->first ? 1 : 0);\n}\n\nstatic int64_t grade_fx",
                                     "return a->first > b->first ? -1 : (a->first < b->first ? 1 : 0);\n}\n\nstatic int64_t grade_fx"),
    "chain_window_of_source": ("const uint32_t d = move[n];\n      int64_t a = pstart[d]", "const uint32_t d = rho[n];\n      int64_t a = pstart[d]"),
    "chain_sorted_gain_ascending": ("if (a->gain != b->gain) return a->gain > b->gain ? -1 : 1;\n  return a->id < b->id ? -1 : (a->id > b->id ? 1 : 0);\n}\n\ntypedef struct {\n  int64_t total;",
                                    "if (a->gain != b->gain) return a->gain < b->gain ? -1 : 1;\n  return a->id < b->id ? -1 : (a->id > b->id ? 1 : 0);\n}\n\ntypedef struct {\n  int64_t total;"),
    "top_pi_keeps_invalid": ("    if (u > J->delta) continue;\n    J->target[(size_t)got * N + n] = m;",
                             "    J->target[(size_t)got * N + n] = m;"),
    "rounds_propose_to_matched": ("if (m != NONE && match[m] == m) {\n          tr[n] = m, sr[n] = score[(size_t)j * N + n];",
                                  "if (m != NONE) {\n          tr[n] = m, sr[n] = score[(size_t)j * N + n];"),
    "rounds_matched_keep_proposing": ("      if (match[n] != n) continue;\n      for (uint32_t j = 0; j < pi; ++j) {",
                                      "      for (uint32_t j = 0; j < pi; ++j) {"),
    "rounds_last_entry_first": ("        const uint32_t m = target[(size_t)j * N + n];",
                                "        const uint32_t m = target[(size_t)(pi - 1 - j) * N + n];"),
    "rounds_one_round": ("for (uint32_t r = 0; r < pi && rc == OR_OK; ++r) {", "for (uint32_t r = 0; r < 1 && rc == OR_OK; ++r) {"),
    "moves_omega_without_node": ("if (enforce_omega && psize[p] + g->n_size[n] > omega) continue;",
                                 "if (enforce_omega && psize[p] > omega) continue;"),
}


def _checks():
    """A fast subset of the pins."""
    pins.test_hand_incidence_and_neighbors()
    pins.test_hand_rate_unconstrained()
    pins.test_hand_rate_delta_two()
    pins.test_hand_contract_and_evaluate()
    for kw in pins.tiny_cases()[:24:2]:
        pins.test_structures_vs_brute(kw)
        pins.test_rate_match_vs_brute(kw, False)
        pins.test_rate_match_vs_brute(kw, True)
        pins.test_contract_evaluate_vs_brute(kw)
    pins.test_evaluate_closed_forms(1)
    pins.test_leftovers_hand_examples()
    pins.test_leftovers_window_bound()
    pins.test_leftovers_only_unmatched_without_target()
    for seed in range(6):
        pins.test_leftovers_invariants(seed)
    pins.test_moves_hand_example()
    for kw in pins.tiny_cases()[:24:2]:
        pins.test_moves_vs_brute(kw)
    for seed in range(3):
        pins.test_moves_identity_partition(seed)
    pins.test_match_dp_hand_examples()
    for seed in range(12):
        pins.test_match_dp_vs_brute(seed)
    pins.test_rounds_hand_example()
    for kw in pins.tiny_cases()[:24:4]:
        pins.test_rate_top_and_rounds_vs_brute(kw, True)
    pins.test_refine_hand_example()
    pins.test_chain_hand_examples()
    pins.test_chain_window()
    pins.test_chain_grade_weights()
    for kw in pins.tiny_cases()[:24:2]:
        pins.test_refine_vs_brute(kw, False)
        pins.test_refine_vs_brute(kw, True)


def _build_mutant(name, tmpdir):
    old, new = MUTANTS[name]
    src = open(oracle._SRC).read()
    assert src.count(old) == 1, "mutation anchor not found: %s" % name
    path = os.path.join(tmpdir, name + ".c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = os.path.join(tmpdir, name + ".so")
    subprocess.check_call(["gcc", "-O1", "-shared", "-fPIC", "-std=gnu11", "-o", lib, path])
    return lib


def test_unmutated_passes():
    _checks()


RUNNER = """
import sys
sys.path[:0] = [%r, %r]
import oracle
oracle._LIB = oracle._SRC = %r
oracle._lib = None
import test_oracle_mutants as tm
try:
    tm._checks()
except (AssertionError, oracle.OracleError) as ex:
    print("caught:", type(ex).__name__)
    sys.exit(3)
print("not caught")
sys.exit(0)
"""


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    """A planted mistake fails a pin, or makes the mutant crash (both count);
    each mutant runs in a child process so a crash cannot take the suite down."""
    here = os.path.dirname(os.path.abspath(__file__))
    root = os.path.dirname(here)
    with tempfile.TemporaryDirectory() as d:
        lib = _build_mutant(name, d)
        r = subprocess.run([sys.executable, "-c", RUNNER % (root, here, lib)],
                           capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, "planted mistake %s was not detected" % name
