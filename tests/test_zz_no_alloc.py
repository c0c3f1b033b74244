"""chp_evaluate_partition_noalloc (the evaluation for callers that cannot
allocate) against chp_evaluate_partition, through the C ABI: the same
part sizes, part inbound counts and summary, two calls in a row on the
library's fixed scratch (the second on a smaller graph and partition, so it
runs over what the first left there), no call of the allocation callback,
and sizes beyond the fixed scratch refused before any work."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def chp():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import constrained_hypergraph_partitioning_amd as m
    m.load_library()
    return m


def say(*a):
    print("[case]", *a, flush=True)


def concat(h1, h2):
    """One edge CSR holding h1's hyperedges, then h2's (same nodes)."""
    e_off = np.concatenate([h1.e_off, h1.e_off[-1] + h2.e_off[1:]])
    return synth.Hypergraph(h1.spec, e_off, np.concatenate([h1.e_nsrc, h2.e_nsrc]),
                            np.concatenate([h1.e_pins, h2.e_pins]),
                            np.concatenate([h1.e_w, h2.e_w]), h1.n_size)


def graphs():
    # 30,000 nodes: short hyperedges (wave and LDS classes) plus eight of
    # 8,300..12,000 pins (the class sorted in global scratch)
    a = concat(synth.generate(synth.custom(synth.UNIFORM, 30000, 30000, 2, 200, 8, 3,
                                           1 << 20, 1 << 20, 21)),
               synth.generate(synth.custom(synth.UNIFORM, 30000, 8, 8300, 12000, 8, 1,
                                           1 << 20, 1 << 20, 22)))
    b = synth.generate(synth.config(2, n_nodes=8000))
    return [("mixed 30k, k 5000", a, 5000), ("ring 8k, k 300", b, 300)]


def test_noalloc_matches_evaluate_partition(chp):
    import torch
    ctx = chp.Context(0)
    omega, delta = 1 << 20, 1 << 20
    for tag, h, k in graphs():
        say("noalloc", tag)
        g = ctx.build_incidence(*chp.upload_edges(h), omega, delta, False)
        rho = chp.to_device(synth.uniform_u32(7, 3, h.n_nodes, k))
        ps, pi, summ = ctx.evaluate_partition(g, rho, k, omega, delta)
        want_ps = chp.to_host(ps, np.uint64)
        want_pi = chp.to_host(pi, np.uint32)
        # outputs pre-filled with garbage: the call must overwrite all of them
        ps2 = torch.full((k,), -1, dtype=torch.int64, device=ctx.device)
        pi2 = torch.full((k,), -1, dtype=torch.int32, device=ctx.device)
        torch.cuda.synchronize()
        before = ctx.n_allocs
        summ2 = ctx.evaluate_partition_noalloc(g, rho, k, omega, delta, ps2, pi2)
        torch.cuda.synchronize()
        assert ctx.n_allocs == before, "the no-allocation call allocated"
        assert np.array_equal(chp.to_host(ps2, np.uint64), want_ps), tag + " part_size"
        assert np.array_equal(chp.to_host(pi2, np.uint32), want_pi), tag + " part_inb"
        assert np.array_equal(summ2, summ), tag + " summary"
        g.free()


def test_noalloc_refuses_beyond_its_scratch(chp):
    import torch
    ctx = chp.Context(0)
    h = synth.generate(synth.config(1))
    g = ctx.build_incidence(*chp.upload_edges(h), 16, 64, False)
    k = 17_000_000  # 68 MB of part counters: above the 64 MiB scratch
    rho = chp.to_device(synth.uniform_u32(7, 4, h.n_nodes, k))
    ps = torch.empty(k, dtype=torch.int64, device=ctx.device)
    pi = torch.empty(k, dtype=torch.int32, device=ctx.device)
    say("noalloc limit")
    with pytest.raises(chp.ChpError) as ei:
        ctx.evaluate_partition_noalloc(g, rho, k, 16, 64, ps, pi)
    assert ei.value.code == chp.EINVAL
    # the context still works afterwards
    _, _, summ = ctx.evaluate_partition(g, rho, k, 16, 64)
    assert int(summ[4]) >= k - h.n_nodes
