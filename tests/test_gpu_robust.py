"""GPU robustness: unaligned activations, HIP graph capture and replay,
concurrent streams.  Every result is checked against the eager result of the
same call (bitwise) and against the f64 oracle (tolerance)."""
import numpy as np
import pytest

import oracle
import synth
from test_gpu_parity import assert_close, dev, host

pytestmark = pytest.mark.gpu


def bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


def offset_x(x, floats=1):
    """x on the device at a 4-byte (not 16-byte) aligned address."""
    import torch
    buf = torch.zeros(x.size + floats, dtype=torch.float32, device="cuda")
    buf[floats:] = torch.from_numpy(np.ascontiguousarray(x).ravel()).cuda()
    return buf[floats:].view(x.shape)


@pytest.mark.parametrize("m", [1, 3, 8])
def test_q4_k_unaligned_x(lib, m):
    n, k = 70, 1024
    w, x = synth.q4_k_case(7000 + m, m, n, k)
    y = host(lib.qgemv_q4_k(dev(w), offset_x(x), n, k))
    y0 = host(lib.qgemv_q4_k(dev(w), dev(x), n, k))
    assert np.array_equal(bits(y), bits(y0))
    assert_close(y, oracle.decode_q4_k(w, n, k), x, f"q4_k unaligned x m{m}")


@pytest.mark.parametrize("m", [2, 130])
def test_affine_unaligned_x_both_paths(lib, m):
    n, k, gs = 96, 512, 64
    x, q, s, b = synth.affine_case(7100 + m, m, n, k, gs)
    y = host(lib.qmm_affine_t(offset_x(x), dev(q), dev(s), dev(b), gs))
    y0 = host(lib.qmm_affine_t(dev(x), dev(q), dev(s), dev(b), gs))
    assert np.array_equal(bits(y), bits(y0))
    assert_close(y, oracle.decode_affine(q, s, b, n, k, gs), x, f"affine unaligned x m{m}")


def test_graph_replays_match_eager(lib):
    """Capture a GEMV (Q4_K, M=1), a matrix-core product (affine, M=130, which
    allocates stream-ordered scratch inside the capture) and a split in one HIP
    graph; replay it three times with eager work and synchronizations in
    between, on changing inputs, and compare every replay with eager calls."""
    import torch
    n, k, gs, m = 256, 1024, 64, 130
    w, x1 = synth.q4_k_case(7200, 1, n, k)
    xa, q, s, b = synth.affine_case(7201, m, n, k, gs)
    dw, dq, ds, db = dev(w), dev(q), dev(s), dev(b)
    dx1, dxa = dev(x1), dev(xa)
    y1 = torch.empty((1, n), dtype=torch.float32, device="cuda")
    ya = torch.empty((m, n), dtype=torch.float32, device="cuda")
    qo = torch.empty((m, 64), dtype=torch.float32, device="cuda")
    ko = torch.empty((m, 64), dtype=torch.float32, device="cuda")
    vo = torch.empty((m, 128), dtype=torch.float32, device="cuda")

    def step():
        lib.qgemv_q4_k(dw, dx1, n, k, y=y1)
        lib.qmm_affine_t(dxa, dq, ds, db, gs, y=ya)
        lib.qkv_split_f32(ya, m, 64, 64, 128, q=qo, k=ko, v=vo)

    step()  # warm up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    rng = synth.rng(7202)
    for rep in range(3):
        nx1 = synth.normal_f32(rng, (1, k))
        nxa = synth.normal_f32(rng, (m, k))
        dx1.copy_(torch.from_numpy(nx1))
        dxa.copy_(torch.from_numpy(nxa))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [host(t).copy() for t in (y1, ya, qo, ko, vo)]
        # eager work between replays: the same calls, results compared bitwise
        e1 = host(lib.qgemv_q4_k(dw, dx1, n, k))
        ea = host(lib.qmm_affine_t(dxa, dq, ds, db, gs))
        assert np.array_equal(bits(got[0]), bits(e1)), rep
        assert np.array_equal(bits(got[1]), bits(ea)), rep
        assert np.array_equal(np.concatenate(got[2:], axis=1).view(np.uint32), bits(ea)), rep
        assert_close(got[0], oracle.decode_q4_k(w, n, k), nx1, f"graph q4_k rep {rep}")
        assert_close(got[1], oracle.decode_affine(q, s, b, n, k, gs), nxa, f"graph affine rep {rep}")
    del g


def test_two_streams_do_not_interfere(lib):
    """The same products issued on two streams at once (each call's scratch is
    stream-ordered) give the eager single-stream bits."""
    import torch
    n, k, gs, m = 128, 512, 64, 100
    xa, q, s, b = synth.affine_case(7300, m, n, k, gs)
    w, x1 = synth.q4_0_case(7301, 3, n, k)
    dxa, dq, ds, db, dw, dx1 = dev(xa), dev(q), dev(s), dev(b), dev(w), dev(x1)
    ref_a = host(lib.qmm_affine_t(dxa, dq, ds, db, gs))
    ref_q = host(lib.qgemv_q4_0(dw, dx1, n, k))
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    outs = []
    for _ in range(4):
        with torch.cuda.stream(s1):
            outs.append(("a", lib.qmm_affine_t(dxa, dq, ds, db, gs)))
        with torch.cuda.stream(s2):
            outs.append(("q", lib.qgemv_q4_0(dw, dx1, n, k)))
    torch.cuda.synchronize()
    for kind, t in outs:
        assert np.array_equal(bits(host(t)), bits(ref_a if kind == "a" else ref_q))
