"""GPU parity of the follow-on paths, through the C ABI, against the f64 oracle:

* Q4_0 and Q4_K products on the matrix cores (prefill rows of x),
* the dual Q4_0 projection on the matrix cores (bitwise equal to two singles),
* the multi-part Q4_K projection (each part bitwise equal to a single call),
* packed 4-bit affine codes (bitwise equal to the u8 codes),
* the fused affine projection + q|k|v split (bitwise equal to product then split).

Bar: bitwise where an equality is stated, otherwise
max |y_gpu - y_oracle| / sum_k |x w| <= 1e-5, and both on the small-M (GEMV)
path and on the matrix-core path (forced with qg_set_mfma_min_m(1))."""
import numpy as np
import pytest

import oracle
import synth
from test_gpu_parity import assert_close, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture
def force_mfma(lib):
    old = lib.qg_get_mfma_min_m()
    lib.qg_set_mfma_min_m(1)
    yield
    lib.qg_set_mfma_min_m(old)


def bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


# ------------------------------------------------------------------ Q4_0 / Q4_K on the matrix cores
@pytest.mark.parametrize("m,n,k", [(1, 9, 128), (64, 64, 256), (130, 77, 512), (33, 300, 2048),
                                   (3, 5, 96)])  # K % 64 != 0: GEMV even when forced
def test_q4_0_mfma_matches_oracle(lib, force_mfma, m, n, k):
    w, x = synth.q4_0_case(6000 + m + n + k, m, n, k)
    y = host(lib.qgemv_q4_0(dev(w), dev(x), n, k))
    assert_close(y, oracle.decode_q4_0(w, n, k), x, f"q4_0 mfma {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", [(1, 7, 256), (64, 64, 256), (77, 130, 1024), (129, 33, 4096)])
def test_q4_k_mfma_matches_oracle(lib, force_mfma, m, n, k):
    w, x = synth.q4_k_case(6100 + m + n + k, m, n, k)
    y = host(lib.qgemv_q4_k(dev(w), dev(x), n, k))
    assert_close(y, oracle.decode_q4_k(w, n, k), x, f"q4_k mfma {m}x{n}x{k}")


def test_q4_k_mfma_random_bytes_all_scale_paths(lib, force_mfma):
    n, k, m = 37, 1024, 70
    g = synth.rng(19)
    w = g.integers(0, 256, size=(n, k // 256 * 144), dtype=np.uint8)
    sb = w.reshape(n, k // 256, 144)
    sb[..., 1] = (sb[..., 1] & 0x03) | 0x20  # d, dmin in a tame fp16 range
    sb[..., 3] = (sb[..., 3] & 0x03) | 0x20
    x = synth.normal_f32(g, (m, k))
    y = host(lib.qgemv_q4_k(dev(w), dev(x), n, k))
    assert_close(y, oracle.decode_q4_k(w, n, k), x, "q4_k mfma random bytes")


def test_q4_0_mfma_onehot_is_bitwise(lib, force_mfma):
    n, k = 40, 256
    w, _ = synth.q4_0_case(79, 1, n, k)
    dec = oracle.decode_q4_0(w, n, k)
    cols = np.array([0, 1, 31, 32, 63, 64, 200, 255])
    x = np.zeros((len(cols), k), np.float32)
    x[np.arange(len(cols)), cols] = 1.0
    y = host(lib.qgemv_q4_0(dev(w), dev(x), n, k))
    assert np.array_equal(y, dec[:, cols].T.astype(np.float32))


@pytest.mark.parametrize("m,n,k", [(70, 64, 512), (128, 33, 1024)])
def test_dual_mfma_bitwise_equals_two_singles(lib, force_mfma, m, n, k):
    wa, wb, x = synth.dual_q4_0_case(6200 + m + n + k, m, n, k)
    dwa, dwb, dx = dev(wa), dev(wb), dev(x)
    ya, yb = lib.qgemv_dual_q4_0(dwa, dwb, dx, n, k)
    sa = lib.qgemv_q4_0(dwa, dx, n, k)
    sb = lib.qgemv_q4_0(dwb, dx, n, k)
    ya, yb, sa, sb = host(ya), host(yb), host(sa), host(sb)
    assert np.array_equal(bits(ya), bits(sa))
    assert np.array_equal(bits(yb), bits(sb))
    assert_close(ya, oracle.decode_q4_0(wa, n, k), x, "dual mfma a")
    assert_close(yb, oracle.decode_q4_0(wb, n, k), x, "dual mfma b")


# ------------------------------------------------------------------ multi-part Q4_K
# more than four parts run as several launches of up to four parts each
MULTI = [(1, (5, 130, 64), 256), (3, (7, 1, 40), 1024), (8, (64, 64), 2048), (1, (33,) * 8, 512),
         (1, (300, 5, 1024, 17, 64, 1, 2, 100), 4096), (4, (40, 3, 17, 90, 33), 4096)]


def _check_multi(lib, m, ns, k, seed, tag):
    ws, x = synth.q4_k_multi_case(seed, m, ns, k)
    dws, dx = [dev(w) for w in ws], dev(x)
    y = host(lib.qgemv_q4_k_multi(dws, dx, list(ns), k))
    ref = oracle.qgemv_multi(oracle.decode_q4_k, list(zip(ws, ns)), x, m, k)
    assert y.shape == ref.shape
    col = 0
    for w, dw, n in zip(ws, dws, ns):
        single = host(lib.qgemv_q4_k(dw, dx, n, k))
        assert np.array_equal(bits(y[:, col:col + n]), bits(single)), f"{tag}: part at column {col}"
        assert_close(y[:, col:col + n], oracle.decode_q4_k(w, n, k), x, f"{tag} col {col}")
        col += n
    # separate outputs, one per part
    ys = lib.qgemv_q4_k_multi(dws, dx, list(ns), k, ys=[None] * len(ns))
    col = 0
    for t, n in zip(ys, ns):
        assert np.array_equal(bits(host(t)), bits(y[:, col:col + n]))
        col += n


@pytest.mark.parametrize("m,ns,k", MULTI)
def test_q4_k_multi_parts_bitwise_equal_singles(lib, m, ns, k):
    _check_multi(lib, m, ns, k, 6300 + m + k, f"multi m{m}")


@pytest.mark.parametrize("m,ns,k", [(70, (5, 130, 64), 256), (128, (200, 17), 1024)])
def test_q4_k_multi_mfma(lib, force_mfma, m, ns, k):
    _check_multi(lib, m, ns, k, 6400 + m + k, f"multi mfma m{m}")


def test_q4_k_multi_hand_parts(lib):
    """[hand super-block, zero block, hand block] with x = ones gives
    [39, 0, 39] (the hand-worked value of tests/golden/q4_k_hand_block.json)."""
    import json
    import os
    from conftest import GOLDEN
    fx = json.load(open(os.path.join(GOLDEN, "q4_k_hand_block.json")))
    hand = np.frombuffer(bytes.fromhex(fx["bytes_hex"]), dtype=np.uint8)[None, :].copy()
    zero = np.zeros_like(hand)
    x = np.ones((1, 256), np.float32)
    y = host(lib.qgemv_q4_k_multi([dev(hand), dev(zero), dev(hand)], dev(x), [1, 1, 1], 256))
    assert list(y[0]) == [fx["y_ones"], 0.0, fx["y_ones"]]


# ------------------------------------------------------------------ packed 4-bit affine
PACKED = [(1, 13, 64, 32), (3, 50, 1024, 64), (8, 129, 4096, 64), (1, 33, 2048, 128),
          (2, 20, 4096, 1024), (5, 31, 256, 16),
          (2, 11, 48, 16), (3, 7, 40, 8), (1, 5, 16, 2)]  # K % 16 != 0 or gs < 16: plain kernel


def _check_packed(lib, m, n, k, gs, seed, tag):
    x, q, s, b = synth.affine_case(seed, m, n, k, gs)
    wp = synth.pack_b4_u32(q)
    import torch
    dx, ds, db = dev(x), dev(s), dev(b)
    y = host(lib.qmm_affine_t_packed(dx, torch.from_numpy(wp.view(np.int32)).cuda(), ds, db, gs))
    y8 = host(lib.qmm_affine_t(dx, dev(q), ds, db, gs))
    assert np.array_equal(bits(y), bits(y8)), f"{tag}: packed differs from u8 codes"
    assert_close(y, oracle.decode_affine_b4(wp, s, b, n, k, gs), x, tag)


@pytest.mark.parametrize("m,n,k,gs", PACKED)
def test_packed_bitwise_equals_u8_codes(lib, m, n, k, gs):
    _check_packed(lib, m, n, k, gs, 6500 + m + n + k + gs, f"packed {m}x{n}x{k} gs{gs}")


@pytest.mark.parametrize("m,n,k,gs", [(64, 64, 256, 32), (130, 77, 1024, 64), (33, 200, 2048, 512)])
def test_packed_mfma_bitwise_equals_u8_codes(lib, force_mfma, m, n, k, gs):
    _check_packed(lib, m, n, k, gs, 6600 + m + n + k + gs, f"packed mfma {m}x{n}x{k} gs{gs}")


def test_packed_page_byte_identity_inputs(lib):
    """Input recipe of the page's packed-vs-unpacked byte-identity test (sin of a
    ramp for x, modular codes, ramped scales and biases), m32 n64 k128 gs32."""
    import torch
    m, n, k, gs = 32, 64, 128, 32
    i = np.arange(m * k, dtype=np.float32)
    x = (np.sin(i * np.float32(0.017) + np.float32(0.3)) * np.float32(0.4)).astype(np.float32).reshape(m, k)
    q = ((np.arange(n * k) * 7 + 5) % 16).astype(np.uint8).reshape(n, k)
    g = np.arange(n * (k // gs), dtype=np.float32)
    s = (np.float32(0.04) + g * np.float32(0.001)).astype(np.float32).reshape(n, k // gs)
    b = (np.float32(-0.15) + g * np.float32(0.007)).astype(np.float32).reshape(n, k // gs)
    wp = synth.pack_b4_u32(q)
    dx, ds, db = dev(x), dev(s), dev(b)
    y = host(lib.qmm_affine_t_packed(dx, torch.from_numpy(wp.view(np.int32)).cuda(), ds, db, gs))
    y8 = host(lib.qmm_affine_t(dx, dev(q), ds, db, gs))
    assert np.array_equal(bits(y), bits(y8))
    assert_close(y, oracle.decode_affine(q, s, b, n, k, gs), x, "packed page inputs")


# ------------------------------------------------------------------ fused projection + split
QKV = [(1, 64, 32, 8, 4, 20), (8, 256, 64, 100, 37, 200), (3, 96, 32, 1, 1, 1), (5, 512, 128, 64, 64, 128)]


def _check_qkv(lib, m, k, gs, qs, ks, vs, seed, tag):
    n = qs + ks + vs
    x, q, s, b = synth.affine_case(seed, m, n, k, gs)
    dx, dq, ds, db = dev(x), dev(q), dev(s), dev(b)
    qo, ko, vo = lib.qmm_affine_t_qkv(dx, dq, ds, db, gs, qs, ks, vs)
    y = lib.qmm_affine_t(dx, dq, ds, db, gs)
    rq, rk, rv = lib.qkv_split_f32(y, m, qs, ks, vs)
    for got, ref in ((qo, rq), (ko, rk), (vo, rv)):
        assert np.array_equal(bits(host(got)), bits(host(ref))), tag
    oq, ok, ov = oracle.qmm_affine_t_qkv(x, q, s, b, m, k, gs, qs, ks, vs)
    dec = oracle.decode_affine(q, s, b, n, k, gs)
    assert_close(np.concatenate([host(qo), host(ko), host(vo)], axis=1), dec, x, tag)
    assert oq.shape == host(qo).shape and ok.shape == host(ko).shape and ov.shape == host(vo).shape


@pytest.mark.parametrize("m,k,gs,qs,ks,vs", QKV)
def test_qkv_fused_bitwise_equals_product_then_split(lib, m, k, gs, qs, ks, vs):
    _check_qkv(lib, m, k, gs, qs, ks, vs, 6700 + m + k + qs, f"qkv fused m{m}")


@pytest.mark.parametrize("m,k,gs,qs,ks,vs", [(70, 256, 64, 128, 128, 256), (130, 512, 32, 100, 37, 200)])
def test_qkv_fused_mfma(lib, force_mfma, m, k, gs, qs, ks, vs):
    _check_qkv(lib, m, k, gs, qs, ks, vs, 6800 + m + k + qs, f"qkv fused mfma m{m}")


def test_qkv_fused_hand(lib):
    import json
    import os
    from conftest import GOLDEN
    fx = json.load(open(os.path.join(GOLDEN, "affine_qkv_hand.json")))
    x = np.array(fx["x"], np.float32)
    q = np.array(fx["q"], np.uint8)
    s = np.array(fx["scales"], np.float32)
    b = np.array(fx["biases"], np.float32)
    qo, ko, vo = lib.qmm_affine_t_qkv(dev(x), dev(q), dev(s), dev(b), fx["group_size"],
                                      fx["q_sp"], fx["k_sp"], fx["v_sp"])
    assert np.array_equal(host(qo), np.array(fx["q_out"], np.float32))
    assert np.array_equal(host(ko), np.array(fx["k_out"], np.float32))
    assert np.array_equal(host(vo), np.array(fx["v_out"], np.float32))


# ------------------------------------------------------------------ matrix-core tile shapes
def test_mfma_tile_shape_does_not_change_bits(lib, force_mfma):
    """Four 2048-row parts at M = 256 give the launch 4x the column tiles of one
    part alone, so the multi-part launch and the single calls take different
    tile shapes (128x128 vs 64x128 on a 256-CU part); each part must still
    equal its single call bit for bit."""
    m, ns, k = 256, (2048, 2048, 2048, 2048), 256
    ws, x = synth.q4_k_multi_case(6900, m, ns, k)
    dws, dx = [dev(w) for w in ws], dev(x)
    y = host(lib.qgemv_q4_k_multi(dws, dx, list(ns), k))
    col = 0
    for w, dw, n in zip(ws, dws, ns):
        single = host(lib.qgemv_q4_k(dw, dx, n, k))
        assert np.array_equal(bits(y[:, col:col + n]), bits(single)), f"part at column {col}"
        col += n
    assert_close(y[:, :2048], oracle.decode_q4_k(ws[0], 2048, k), x, "tile shapes")


@pytest.mark.parametrize("fmt,gs", [("affine", 32), ("affine", 64), ("affine", 128), ("affine", 512),
                                    ("q4_0", 32), ("q4_k", 32)])
def test_mfma_two_steps_per_barrier_same_bits(lib, fmt, gs):
    """At M = 512 an 8192-row product runs on 128 x 128 tiles with one 64-column
    K step per barrier, and its first 2048 rows alone on 64 x 128 tiles with
    two steps per barrier (K a multiple of 128); the outputs they share must
    be the same bits (groups of 32 codes: two groups per step; 128 and 512:
    a group spans steps and stages)."""
    m, n, n_small, k = 512, 8192, 2048, 1024
    if fmt == "affine":
        x, q, s, b = synth.affine_case(7000 + gs, m, n, k, gs)
        dx = dev(x)
        full = host(lib.qmm_affine_t(dx, dev(q), dev(s), dev(b), gs))
        small = host(lib.qmm_affine_t(dx, dev(np.ascontiguousarray(q[:n_small])),
                                      dev(np.ascontiguousarray(s[:n_small])), dev(np.ascontiguousarray(b[:n_small])), gs))
        ref = oracle.decode_affine(np.ascontiguousarray(q[:64]), s[:64], b[:64], 64, k, gs)
    else:
        case = synth.q4_0_case if fmt == "q4_0" else synth.q4_k_case
        w, x = case(7100, m, n, k)
        f = lib.qgemv_q4_0 if fmt == "q4_0" else lib.qgemv_q4_k
        dx = dev(x)
        full = host(f(dev(w), dx, n, k))
        small = host(f(dev(np.ascontiguousarray(w[:n_small])), dx, n_small, k))
        dec = oracle.decode_q4_0 if fmt == "q4_0" else oracle.decode_q4_k
        ref = dec(np.ascontiguousarray(w[:64]), 64, k)
    assert np.array_equal(bits(full[:, :n_small]), bits(small)), f"{fmt} gs{gs}"
    assert_close(small[:, :64], ref, x, f"{fmt} gs{gs} two steps")
