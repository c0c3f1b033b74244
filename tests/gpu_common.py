"""Helpers for the GPU parity tests: run the HIP path and the CPU oracle on
the same seeded inputs and compare every output array bit for bit."""
import numpy as np

import oracle

GRAPH_ARRAYS = [("e_off", np.int64), ("e_nsrc", np.uint32), ("e_pins", np.uint32),
                ("e_w", np.uint32), ("n_size", np.uint32), ("n_off", np.int64),
                ("n_nin", np.uint32), ("n_inc", np.uint32), ("nb_off", np.int64),
                ("nb", np.uint32)]


def assert_graph_equal(dg, og, what, neighbors=True):
    """Device graph (chp.HGraph) vs oracle.Graph, array by array."""
    assert dg.n_nodes == og.n_nodes and dg.n_edges == og.n_edges, what
    assert dg.n_pins == og.n_pins, what
    for name, dt in GRAPH_ARRAYS:
        if name.startswith("nb") and not neighbors:
            continue
        got = dg.host(name)
        want = getattr(og, name)
        assert got is not None and want is not None, "%s: %s missing" % (what, name)
        got = got.view(dt) if got.dtype != dt else got
        if not np.array_equal(got, want.astype(dt)):
            bad = np.nonzero(got != want.astype(dt))[0]
            raise AssertionError("%s: %s differs at %d positions, first %s (got %s want %s)"
                                 % (what, name, bad.size, bad[:5].tolist(),
                                    got[bad[:5]].tolist(), want[bad[:5]].tolist()))


def assert_equal(got, want, what):
    if not np.array_equal(got, want):
        bad = np.nonzero(got != want)[0]
        raise AssertionError("%s differs at %d of %d positions, first %s (got %s want %s)"
                             % (what, bad.size, want.size, bad[:5].tolist(),
                                got[bad[:5]].tolist(), want[bad[:5]].tolist()))


def run_level_pair(chp, ctx, dg, og, omega, delta, noise_on, seed, neighbors=True, tag="",
                   purge=False, leftovers=False, optimal=False, pi=1):
    """One level on both sides; compares target, score, match, pairs, gamma
    and the coarse graph (with purge, also the invalid-neighbour flags, and
    the coarse neighbourhoods purged; with leftovers, after the best-effort
    pairing of the nodes left without a partner).  Returns (device coarse,
    oracle Level, device gamma).  With pi > 1 the device call is
    rate_top_and_match and the whole (pi, N) candidate lists are compared
    with the oracle's top-pi rating; target/score below are then row 0."""
    flags = ctx.new_flags(dg) if purge else None
    ctx.set_matching(optimal)
    try:
        if pi > 1:
            tl, sl, match, npairs = ctx.rate_top_and_match(dg, pi, omega, delta, noise_on, seed,
                                                           flags=flags)
            otl, osl = oracle.rate_top(og, omega, delta, noise_on, seed, pi)
            assert_equal(chp.to_host(tl, np.uint32).reshape(-1), otl.reshape(-1),
                         tag + " top-pi targets")
            assert_equal(chp.to_host(sl, np.uint64).reshape(-1), osl.reshape(-1),
                         tag + " top-pi scores")
            tgt, score = tl[0], sl[0]
        else:
            tgt, score, match, npairs = ctx.rate_and_match(dg, omega, delta, noise_on, seed,
                                                           flags=flags)
    finally:
        ctx.set_matching(False)
    if leftovers:
        npairs += ctx.pair_leftovers(dg, tgt, match, omega, delta)
    lv = oracle.level(og, omega, delta, noise_on, seed, build_neighbors=neighbors,
                      purge_invalid=purge, leftovers=leftovers, optimal=optimal, pi=pi)
    assert_equal(chp.to_host(tgt, np.uint32), lv.target, tag + " target")
    assert_equal(chp.to_host(score, np.uint64), lv.score, tag + " score")
    assert_equal(chp.to_host(match, np.uint32), lv.match, tag + " match")
    if purge:
        got = flags.cpu().numpy()[: og.nb.shape[0]]
        assert_equal(got, lv.flags, tag + " flags")
    assert npairs == lv.n_pairs, tag + " pairs"
    if npairs == 0:
        return None, lv, None
    gamma, cg = ctx.contract(dg, match, neighbors, flags=flags)
    assert_equal(chp.to_host(gamma, np.uint32), lv.gamma, tag + " gamma")
    assert_graph_equal(cg, lv.coarse, tag + " coarse", neighbors)
    return cg, lv, gamma


def eval_pair(chp, ctx, dg, og, rho, k, omega, delta, tag=""):
    ps, pi, summ = ctx.evaluate_partition(dg, chp.to_device(rho), k, omega, delta)
    ops, opi, osumm = oracle.evaluate(og, rho, k, omega, delta)
    assert_equal(chp.to_host(ps, np.uint64), ops, tag + " part_size")
    assert_equal(chp.to_host(pi, np.uint32), opi, tag + " part_inb")
    assert_equal(summ, osumm, tag + " summary")
    return summ
