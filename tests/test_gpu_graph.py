"""Matrix-core calls captured into HIP graphs.

A matrix-core call (prefill M) made while its stream is captured takes its
scratch from a buffer owned by the graph (a user object of the graph) instead
of stream-ordered allocation nodes; released buffers go back to a per-device
pool for later captures.  Every replay must give the eager bits, with eager
calls and other graphs between the replays, and again after graphs are
destroyed and new ones captured from the pool.  No memset is recorded: the
outputs are cleared by torch's fill kernel outside the graphs.
"""
import gc

import numpy as np
import pytest

import oracle
import synth
from test_gpu_parity import assert_close, dev, host

pytestmark = pytest.mark.gpu


def bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


def _inputs():
    m, n, k, gs = 192, 320, 1024, 64
    x, q, s, b = synth.affine_case(5100, m, n, k, gs)
    w0, x0 = synth.q4_0_case(5101, m, n, k)
    return (m, n, k, gs), (x, q, s, b), (w0, x0)


def _capture(torch, fn):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def test_captured_prefill_calls_replay_the_eager_bits(lib):
    import torch
    (m, n, k, gs), (x, q, s, b), (w0, x0) = _inputs()
    dx, dq, ds, db, dw0, dx0 = dev(x), dev(q), dev(s), dev(b), dev(w0), dev(x0)
    eager_a = host(lib.qmm_affine_t(dx, dq, ds, db, gs))
    eager_q = host(lib.qgemv_q4_0(dw0, dx0, n, k))
    assert_close(eager_a, oracle.decode_affine(q, s, b, n, k, gs), x, "eager affine prefill")
    assert_close(eager_q, oracle.decode_q4_0(w0, n, k), x0, "eager q4_0 prefill")

    ya, ya2, yq = (torch.empty((m, n), dtype=torch.float32, device="cuda") for _ in range(3))
    # three matrix-core calls in one graph: three graph-owned buffers
    g1 = _capture(torch, lambda: (lib.qmm_affine_t(dx, dq, ds, db, gs, y=ya),
                                  lib.qgemv_q4_0(dw0, dx0, n, k, y=yq),
                                  lib.qmm_affine_t(dx, dq, ds, db, gs, y=ya2)))
    za = torch.empty((m, n), dtype=torch.float32, device="cuda")
    g2 = _capture(torch, lambda: lib.qmm_affine_t(dx, dq, ds, db, gs, y=za))
    for rep in range(4):
        for t in (ya, ya2, yq, za):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g1.replay()
        if rep % 2:
            g2.replay()
        # an eager call between the replays (stream-ordered scratch)
        mid = host(lib.qmm_affine_t(dx, dq, ds, db, gs))
        if not rep % 2:
            g2.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(host(ya)), bits(eager_a)), f"replay {rep}: first affine call"
        assert np.array_equal(bits(host(ya2)), bits(eager_a)), f"replay {rep}: second affine call"
        assert np.array_equal(bits(host(yq)), bits(eager_q)), f"replay {rep}: q4_0 call"
        assert np.array_equal(bits(host(za)), bits(eager_a)), f"replay {rep}: second graph"
        assert np.array_equal(bits(mid), bits(eager_a)), f"replay {rep}: eager call"
    # destroy both graphs (their buffers return to the pool), capture new ones
    del g1, g2
    gc.collect()
    torch.cuda.synchronize()
    for round_ in range(2):
        yb = torch.empty((m, n), dtype=torch.float32, device="cuda")
        yc = torch.empty((m, n), dtype=torch.float32, device="cuda")
        g3 = _capture(torch, lambda: (lib.qgemv_q4_0(dw0, dx0, n, k, y=yc),
                                      lib.qmm_affine_t(dx, dq, ds, db, gs, y=yb)))
        for rep in range(3):
            yb.fill_(float("nan"))
            yc.fill_(float("nan"))
            g3.replay()
            torch.cuda.synchronize()
            assert np.array_equal(bits(host(yb)), bits(eager_a)), f"pool round {round_} replay {rep}"
            assert np.array_equal(bits(host(yc)), bits(eager_q)), f"pool round {round_} replay {rep}"
        del g3
        gc.collect()
        torch.cuda.synchronize()


def test_captured_call_with_a_larger_scratch_than_the_pool_holds(lib):
    """A capture whose scratch exceeds every released buffer allocates a new one."""
    import torch
    m, n, k, gs = 512, 256, 2048, 64
    x, q, s, b = synth.affine_case(5102, m, n, k, gs)
    dx, dq, ds, db = dev(x), dev(q), dev(s), dev(b)
    eager = host(lib.qmm_affine_t(dx, dq, ds, db, gs))
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")
    g = _capture(torch, lambda: lib.qmm_affine_t(dx, dq, ds, db, gs, y=y))
    for rep in range(3):
        y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(host(y)), bits(eager)), f"replay {rep}"
    assert_close(eager, oracle.decode_affine(q, s, b, n, k, gs), x, "eager 512x256x2048")
