"""GPU parity: the HIP path (through the C ABI) against the f64 oracle.

Bar: bitwise for qkv_split, for dual vs two singles, for one-hot x and for
exactly representable products; otherwise
    max |y_gpu - y_oracle| / sum_k |x[m,k] w[n,k]|  <=  1e-5
(the tolerance of the product, stated for every floating-point result).
"""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

TOL = 1e-5


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_close(y_gpu, w64, x, tag=""):
    ref = oracle.gemv_f64(w64, x)
    bound = oracle.abs_bound(w64, x)
    err = np.abs(y_gpu.astype(np.float64) - ref.astype(np.float64))
    zero = bound == 0
    assert np.all(y_gpu[zero] == 0), tag
    ratio = np.where(zero, 0.0, err / np.where(zero, 1.0, bound))
    worst = float(ratio.max()) if ratio.size else 0.0
    assert worst <= TOL, f"{tag}: max err/bound = {worst:.3e}"
    return worst


# ------------------------------------------------------------------ Q4_0
Q40_SHAPES = [
    (1, 1, 64), (1, 7, 64), (2, 33, 128), (3, 130, 256), (5, 64, 1024), (8, 100, 2048),
    (9, 17, 4096), (17, 5, 640), (1, 300, 4160),      # K % 64 == 0: chunked kernel
    (1, 9, 32), (4, 13, 96), (3, 70, 1056),           # K % 64 == 32: plain kernel
]


@pytest.mark.parametrize("m,n,k", Q40_SHAPES)
def test_q4_0_matches_oracle(lib, m, n, k):
    w, x = synth.q4_0_case(1000 + m * 7 + n + k, m, n, k)
    y = host(lib.qgemv_q4_0(dev(w), dev(x), n, k))
    assert_close(y, oracle.decode_q4_0(w, n, k), x, f"q4_0 {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", [(1, 40, 128), (3, 9, 1024), (8, 5, 96)])
def test_q4_0_onehot_is_bitwise(lib, m, n, k):
    w, _ = synth.q4_0_case(77, 1, n, k)
    dec = oracle.decode_q4_0(w, n, k)
    cols = np.random.default_rng(5).choice(k, size=m, replace=False)
    x = np.zeros((m, k), np.float32)
    x[np.arange(m), cols] = 1.0
    y = host(lib.qgemv_q4_0(dev(w), dev(x), n, k))
    assert np.array_equal(y, dec[:, cols].T.astype(np.float32))


# ------------------------------------------------------------------ Q4_K
Q4K_SHAPES = [(1, 1, 256), (1, 7, 512), (2, 33, 1024), (4, 65, 2048), (1, 130, 4096),
              (8, 12, 4096), (3, 64, 8192), (11, 19, 768)]


@pytest.mark.parametrize("m,n,k", Q4K_SHAPES)
def test_q4_k_matches_oracle(lib, m, n, k):
    w, x = synth.q4_k_case(2000 + m * 7 + n + k, m, n, k)
    y = host(lib.qgemv_q4_k(dev(w), dev(x), n, k))
    assert_close(y, oracle.decode_q4_k(w, n, k), x, f"q4_k {m}x{n}x{k}")


def test_q4_k_random_bytes_all_scale_paths(lib):
    """Arbitrary super-block bytes (finite d, dmin) exercise every 6-bit scale/min path."""
    n, k, m = 37, 1024, 3
    g = synth.rng(9)
    w = g.integers(0, 256, size=(n, k // 256 * 144), dtype=np.uint8)
    sb = w.reshape(n, k // 256, 144)
    sb[..., 1] = (sb[..., 1] & 0x03) | 0x20  # d, dmin in a tame fp16 range
    sb[..., 3] = (sb[..., 3] & 0x03) | 0x20
    x = synth.normal_f32(g, (m, k))
    y = host(lib.qgemv_q4_k(dev(w), dev(x), n, k))
    assert_close(y, oracle.decode_q4_k(w, n, k), x, "q4_k random bytes")


def test_q4_k_misaligned_weights_use_plain_kernel(lib):
    import torch
    n, k = 9, 512
    w, x = synth.q4_k_case(99, 2, n, k)
    buf = torch.zeros(w.size + 4, dtype=torch.uint8, device="cuda")
    buf[4:] = dev(w.ravel())
    y = host(lib.qgemv_q4_k(buf[4:], dev(x), n, k))
    assert_close(y, oracle.decode_q4_k(w, n, k), x, "q4_k offset 4")


def test_q4_k_onehot_is_bitwise(lib):
    n, k = 21, 1024
    w, _ = synth.q4_k_case(78, 1, n, k)
    dec = oracle.decode_q4_k(w, n, k)
    for col in (0, 31, 32, 63, 64, 255, 256, 1023):
        x = np.zeros((1, k), np.float32)
        x[0, col] = 1.0
        y = host(lib.qgemv_q4_k(dev(w), dev(x), n, k))
        assert np.array_equal(y[0], dec[:, col].astype(np.float32)), col


# ------------------------------------------------------------------ dual
@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 8, 9])
@pytest.mark.parametrize("n,k", [(64, 4096), (77, 1024), (5, 96)])
def test_dual_bitwise_equals_two_singles(lib, m, n, k):
    wa, wb, x = synth.dual_q4_0_case(3000 + m + n + k, m, n, k)
    dwa, dwb, dx = dev(wa), dev(wb), dev(x)
    ya, yb = lib.qgemv_dual_q4_0(dwa, dwb, dx, n, k)
    sa = lib.qgemv_q4_0(dwa, dx, n, k)
    sb = lib.qgemv_q4_0(dwb, dx, n, k)
    ya, yb, sa, sb = host(ya), host(yb), host(sa), host(sb)
    assert np.array_equal(ya.view(np.uint32), sa.view(np.uint32))
    assert np.array_equal(yb.view(np.uint32), sb.view(np.uint32))
    assert_close(ya, oracle.decode_q4_0(wa, n, k), x, "dual a")
    assert_close(yb, oracle.decode_q4_0(wb, n, k), x, "dual b")


# ------------------------------------------------------------------ affine
AFF_SHAPES = [
    (1, 1, 64, 64), (1, 13, 64, 32), (7, 13, 64, 32), (8, 16, 64, 32), (5, 9, 96, 32),
    (2, 50, 1024, 64), (8, 129, 4096, 64), (1, 33, 2048, 128), (3, 20, 4096, 1024),
    (4, 31, 256, 16),
    (2, 11, 48, 16), (3, 7, 40, 8), (2, 9, 24, 4), (1, 5, 18, 2),  # plain kernel
]


@pytest.mark.parametrize("m,n,k,gs", AFF_SHAPES)
def test_affine_matches_oracle(lib, m, n, k, gs):
    x, q, s, b = synth.affine_case(4000 + m + n + k + gs, m, n, k, gs)
    y = host(lib.qmm_affine_t(dev(x), dev(q), dev(s), dev(b), gs))
    assert_close(y, oracle.decode_affine(q, s, b, n, k, gs), x, f"affine {m}x{n}x{k} gs{gs}")


def test_affine_full_byte_codes(lib):
    x, q, s, b = synth.affine_case(41, 3, 40, 512, 64, code_max=255)
    y = host(lib.qmm_affine_t(dev(x), dev(q), dev(s), dev(b), 64))
    assert_close(y, oracle.decode_affine(q, s, b, 40, 512, 64), x, "affine codes 0..255")


def test_affine_page_sincos_inputs(lib):
    """Input recipe of the page's qmm_affine_t test (sin of a ramp, modular codes,
    ramped scales and biases), m8 n16 k64 gs32, held to the library's tolerance."""
    m, n, k, gs = 8, 16, 64, 32
    i = np.arange(m * k, dtype=np.float32)
    x = (np.sin(i * np.float32(0.013) - np.float32(0.4)) * np.float32(0.6)).astype(np.float32).reshape(m, k)
    q = ((np.arange(n * k) * 11 + 3) % 16).astype(np.uint8).reshape(n, k)
    g = np.arange(n * (k // gs), dtype=np.float32)
    s = (np.float32(0.05) + g * np.float32(0.003)).astype(np.float32).reshape(n, k // gs)
    b = (np.float32(-0.2) + g * np.float32(0.011)).astype(np.float32).reshape(n, k // gs)
    y = host(lib.qmm_affine_t(dev(x), dev(q), dev(s), dev(b), gs))
    assert_close(y, oracle.decode_affine(q, s, b, n, k, gs), x, "affine sincos")


# ------------------------------------------------------------------ MFMA prefill path
@pytest.fixture
def force_mfma(lib):
    old = lib.qg_get_mfma_min_m()
    lib.qg_set_mfma_min_m(1)
    yield
    lib.qg_set_mfma_min_m(old)


@pytest.mark.parametrize("m,n,k,gs", [
    (1, 16, 64, 64), (16, 16, 64, 32), (128, 128, 256, 64), (130, 129, 512, 64),
    (77, 300, 1024, 128), (256, 64, 2048, 512), (40, 70, 1024, 256), (33, 257, 192, 32), (5, 9, 128, 64),
    (3, 11, 2048, 1024),  # group_size above 512: takes the GEMV path even when forced
])
def test_affine_mfma_matches_oracle(lib, force_mfma, m, n, k, gs):
    x, q, s, b = synth.affine_case(5000 + m + n + k + gs, m, n, k, gs)
    y = host(lib.qmm_affine_t(dev(x), dev(q), dev(s), dev(b), gs))
    assert_close(y, oracle.decode_affine(q, s, b, n, k, gs), x, f"mfma {m}x{n}x{k} gs{gs}")


def test_affine_mfma_full_byte_codes_and_wide_x(lib, force_mfma):
    g = synth.rng(51)
    m, n, k, gs = 64, 96, 512, 64
    _, q, s, b = synth.affine_case(52, 1, n, k, gs, code_max=255)
    x = (synth.normal_f32(g, (m, k)) * np.exp2(g.integers(-20, 20, size=(m, 1)))).astype(np.float32)
    y = host(lib.qmm_affine_t(dev(x), dev(q), dev(s), dev(b), gs))
    assert_close(y, oracle.decode_affine(q, s, b, n, k, gs), x, "mfma wide x")


def test_affine_mfma_exact_inputs_bitwise(lib, force_mfma):
    """Integer x (|x| <= 4), power-of-two scales and biases: every partial sum is
    exact in f32, so GPU and oracle agree bit for bit."""
    g = synth.rng(53)
    m, n, k, gs = 40, 70, 256, 64
    x = g.integers(-4, 5, size=(m, k)).astype(np.float32)
    q = g.integers(0, 16, size=(n, k), dtype=np.uint8)
    s = np.exp2(g.integers(-3, 2, size=(n, k // gs))).astype(np.float32)
    b = (np.exp2(g.integers(-3, 2, size=(n, k // gs))) * g.choice([-1, 1], size=(n, k // gs))).astype(np.float32)
    y = host(lib.qmm_affine_t(dev(x), dev(q), dev(s), dev(b), gs))
    ref = oracle.qmm_affine_t(x, q, s, b, m, n, k, gs)
    assert np.array_equal(y, ref)


# ------------------------------------------------------------------ qkv split
@pytest.mark.parametrize("seq,qs,ks,vs", [(1, 4, 4, 8), (7, 12, 4, 20), (3, 5, 3, 2), (2, 1, 1, 1),
                                          (33, 128, 64, 256)])
def test_qkv_split_bitwise(lib, seq, qs, ks, vs):
    qkv = synth.qkv_payload(seq, qs, ks, vs)
    q, k, v = lib.qkv_split_f32(dev(qkv), seq, qs, ks, vs)
    rq, rk, rv = oracle.qkv_split_f32(qkv, seq, qs, ks, vs)
    for got, ref in ((q, rq), (k, rk), (v, rv)):
        assert np.array_equal(host(got).view(np.uint32), ref.view(np.uint32))


def test_qkv_split_special_values_bitwise(lib):
    seq, qs, ks, vs = 3, 8, 4, 12
    bits = synth.rng(61).integers(0, 2**32, size=(seq, qs + ks + vs), dtype=np.uint32)
    bits[0, :4] = [0x80000000, 0x7FC00001, 0xFF800000, 0x00000001]  # -0, NaN payload, -inf, denormal
    qkv = bits.view(np.float32)
    q, k, v = lib.qkv_split_f32(dev(qkv), seq, qs, ks, vs)
    got = np.concatenate([host(q), host(k), host(v)], axis=1)
    assert np.array_equal(got.view(np.uint32), bits)


# ------------------------------------------------------------------ determinism
def test_repeat_calls_are_bitwise_identical(lib):
    w, x = synth.q4_k_case(71, 4, 512, 4096)
    dw, dx = dev(w), dev(x)
    a = host(lib.qgemv_q4_k(dw, dx, 512, 4096))
    for _ in range(3):
        assert np.array_equal(host(lib.qgemv_q4_k(dw, dx, 512, 4096)), a)
