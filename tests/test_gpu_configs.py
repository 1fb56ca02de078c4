"""Full-size parity on the benchmark workloads, in the launch configuration
bench.py times (same entry points, same shapes, default variant choice).
The oracle finishes every one of these in seconds on the host, so every output
element is compared, not a sample."""
import numpy as np
import pytest

import oracle
import synth
from test_gpu_parity import assert_close, dev, host

pytestmark = pytest.mark.gpu

CFG = synth.CONFIGS


def test_config_q4_0_gemv_1024(lib):
    c = CFG["q4_0_gemv_1024"]
    w, x = synth.q4_0_case(c["seed"], c["m"], c["n"], c["k"])
    y = host(lib.qgemv_q4_0(dev(w), dev(x), c["n"], c["k"]))
    assert_close(y, oracle.decode_q4_0(w, c["n"], c["k"]), x, "C q4_0 1024")


def test_config_q4_k_gemv_4096(lib):
    c = CFG["q4_k_gemv_4096"]
    w, x = synth.q4_k_case(c["seed"], c["m"], c["n"], c["k"])
    y = host(lib.qgemv_q4_k(dev(w), dev(x), c["n"], c["k"]))
    assert_close(y, oracle.decode_q4_k(w, c["n"], c["k"]), x, "C q4_k 4096")


@pytest.mark.parametrize("m", [1, 4, 8])
def test_config_dual_q4_0_4096(lib, m):
    c = CFG["dual_q4_0_4096"]
    wa, wb, x8 = synth.dual_q4_0_case(c["seed"], c["m"], c["n"], c["k"])
    x = np.ascontiguousarray(x8[:m])
    dwa, dwb, dx = dev(wa), dev(wb), dev(x)
    ya, yb = lib.qgemv_dual_q4_0(dwa, dwb, dx, c["n"], c["k"])
    sa = host(lib.qgemv_q4_0(dwa, dx, c["n"], c["k"]))
    sb = host(lib.qgemv_q4_0(dwb, dx, c["n"], c["k"]))
    ya, yb = host(ya), host(yb)
    assert np.array_equal(ya.view(np.uint32), sa.view(np.uint32))
    assert np.array_equal(yb.view(np.uint32), sb.view(np.uint32))
    assert_close(ya, oracle.decode_q4_0(wa, c["n"], c["k"]), x, f"C dual a m{m}")
    assert_close(yb, oracle.decode_q4_0(wb, c["n"], c["k"]), x, f"C dual b m{m}")


@pytest.mark.parametrize("m", [1, 8])
def test_config_affine_12288x4096(lib, m):
    c = CFG["affine_12288x4096_gs64"]
    x8, q, s, b = synth.affine_case(c["seed"], c["m"], c["n"], c["k"], c["gs"])
    x = np.ascontiguousarray(x8[:m])
    y = host(lib.qmm_affine_t(dev(x), dev(q), dev(s), dev(b), c["gs"]))
    assert_close(y, oracle.decode_affine(q, s, b, c["n"], c["k"], c["gs"]), x, f"C affine m{m}")


def test_config_prefill_qkv_512x2048(lib):
    c = CFG["prefill_qkv_512x2048"]
    x, q, s, b = synth.affine_case(c["seed"], c["m"], c["n"], c["k"], c["gs"])
    assert c["m"] >= lib.qg_get_mfma_min_m()  # the matrix-core path is the one timed
    qkv = lib.qmm_affine_t(dev(x), dev(q), dev(s), dev(b), c["gs"])
    qo, ko, vo = lib.qkv_split_f32(qkv, c["m"], c["q_sp"], c["k_sp"], c["v_sp"])
    qkv_h = host(qkv)
    assert_close(qkv_h, oracle.decode_affine(q, s, b, c["n"], c["k"], c["gs"]), x, "C prefill gemm")
    rq, rk, rv = oracle.qkv_split_f32(qkv_h, c["m"], c["q_sp"], c["k_sp"], c["v_sp"])
    for got, ref in ((qo, rq), (ko, rk), (vo, rv)):
        assert np.array_equal(host(got).view(np.uint32), ref.view(np.uint32))


# ------------------------------------------------------------------ follow-on paths, full size
NXT = synth.NEXT_CONFIGS


def test_config_q4_k_qkv_multi_4096(lib):
    c = NXT["q4_k_qkv_multi_4096"]
    ns, k = list(c["ns"]), c["k"]
    ws, x = synth.q4_k_multi_case(c["seed"], c["m"], ns, k)
    dws, dx = [dev(w) for w in ws], dev(x)
    y = host(lib.qgemv_q4_k_multi(dws, dx, ns, k))
    col = 0
    for w, dw, n in zip(ws, dws, ns):
        single = host(lib.qgemv_q4_k(dw, dx, n, k))
        assert np.array_equal(y[:, col:col + n].view(np.uint32), single.view(np.uint32))
        assert_close(y[:, col:col + n], oracle.decode_q4_k(w, n, k), x, f"C multi col {col}")
        col += n


@pytest.mark.parametrize("m", [1, 8])
def test_config_affine_b4_12288x4096(lib, m):
    import torch
    c = NXT["affine_b4_12288x4096_gs64"]
    x8, q, s, b = synth.affine_case(c["seed"], c["m"], c["n"], c["k"], c["gs"])
    x = np.ascontiguousarray(x8[:m])
    wp = synth.pack_b4_u32(q)
    dx, ds, db = dev(x), dev(s), dev(b)
    y = host(lib.qmm_affine_t_packed(dx, torch.from_numpy(wp.view(np.int32)).cuda(), ds, db, c["gs"]))
    y8 = host(lib.qmm_affine_t(dx, dev(q), ds, db, c["gs"]))
    assert np.array_equal(y.view(np.uint32), y8.view(np.uint32))
    assert_close(y, oracle.decode_affine_b4(wp, s, b, c["n"], c["k"], c["gs"]), x, f"C packed m{m}")


def test_config_q4_0_prefill_512x4096(lib):
    c = NXT["q4_0_prefill_512x4096"]
    assert c["m"] >= lib.qg_get_mfma_min_m()  # the matrix-core path is the one timed
    w, x = synth.q4_0_case(c["seed"], c["m"], c["n"], c["k"])
    y = host(lib.qgemv_q4_0(dev(w), dev(x), c["n"], c["k"]))
    assert_close(y, oracle.decode_q4_0(w, c["n"], c["k"]), x, "C q4_0 prefill")


def test_config_prefill_qkv_fused_512x2048(lib):
    c = CFG["prefill_qkv_512x2048"]
    x, q, s, b = synth.affine_case(c["seed"], c["m"], c["n"], c["k"], c["gs"])
    dx, dq, ds, db = dev(x), dev(q), dev(s), dev(b)
    outs = lib.qmm_affine_t_qkv(dx, dq, ds, db, c["gs"], c["q_sp"], c["k_sp"], c["v_sp"])
    qkv = lib.qmm_affine_t(dx, dq, ds, db, c["gs"])
    refs = lib.qkv_split_f32(qkv, c["m"], c["q_sp"], c["k_sp"], c["v_sp"])
    for got, ref in zip(outs, refs):
        assert np.array_equal(host(got).view(np.uint32), host(ref).view(np.uint32))
    y = np.concatenate([host(t) for t in outs], axis=1)
    assert_close(y, oracle.decode_affine(q, s, b, c["n"], c["k"], c["gs"]), x, "C fused qkv")


def test_config_prefills_replayed_from_a_graph(lib):
    """bench.py times the prefill products as graph replays, where their
    scratch belongs to the graph: the replays give the eager bits, and the
    affine product is within the bar of the oracle."""
    import torch
    c = CFG["prefill_qkv_512x2048"]
    x, q, s, b = synth.affine_case(c["seed"], c["m"], c["n"], c["k"], c["gs"])
    dx, dq, ds, db = dev(x), dev(q), dev(s), dev(b)
    n0 = NXT["q4_0_prefill_512x4096"]
    w0, x0 = synth.q4_0_case(n0["seed"], n0["m"], n0["n"], n0["k"])
    dw0, dx0 = dev(w0), dev(x0)
    eager_a = host(lib.qmm_affine_t(dx, dq, ds, db, c["gs"]))
    eager_q = host(lib.qgemv_q4_0(dw0, dx0, n0["n"], n0["k"]))
    eager_f = [host(t) for t in lib.qmm_affine_t_qkv(dx, dq, ds, db, c["gs"], c["q_sp"], c["k_sp"], c["v_sp"])]
    ya = torch.empty((c["m"], c["n"]), dtype=torch.float32, device="cuda")
    yq = torch.empty((n0["m"], n0["n"]), dtype=torch.float32, device="cuda")
    fo = [torch.empty((c["m"], sp), dtype=torch.float32, device="cuda") for sp in (c["q_sp"], c["k_sp"], c["v_sp"])]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lib.qmm_affine_t(dx, dq, ds, db, c["gs"], y=ya)
        lib.qgemv_q4_0(dw0, dx0, n0["n"], n0["k"], y=yq)
        lib.qmm_affine_t_qkv(dx, dq, ds, db, c["gs"], c["q_sp"], c["k_sp"], c["v_sp"], q_out=fo[0], k_out=fo[1],
                             v_out=fo[2])
    bits = lambda a: np.ascontiguousarray(a).view(np.uint32)
    for rep in range(2):
        for t in [ya, yq, *fo]:
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(host(ya)), bits(eager_a)), f"replay {rep}: affine prefill"
        assert np.array_equal(bits(host(yq)), bits(eager_q)), f"replay {rep}: q4_0 prefill"
        for got, ref in zip(fo, eager_f):
            assert np.array_equal(bits(host(got)), bits(ref)), f"replay {rep}: fused q|k|v"
    assert_close(host(ya), oracle.decode_affine(q, s, b, c["n"], c["k"], c["gs"]), x, "C prefill gemm, replayed")
    del g
