"""The matrix-core GEMV with x in registers (Q4_0, Q4_K and affine codes with
group size >= 64; from 3 rows of x, up to 8 per launch, K a multiple of 512 up
to 4096) against the f64 oracle, and its stated equalities: the dual Q4_0 and
the multi-part Q4_K products bitwise equal to single calls, packed affine codes
bitwise equal to u8 codes, the fused q|k|v product bitwise equal to the
product then the split, each row of x independent of the others, Q4_0 blocks
of codes 8 giving exactly zero, the hand-worked Q4_K super-block exactly.
Without QG_KERNEL_XR in the kernel mask the other kernels run, whose results
must agree within the same tolerance.  Shapes outside that range (K = 4160, 8192, 256) take the
FMA kernels and are checked the same way."""
import os

import numpy as np
import pytest

import oracle
import synth
from test_gpu_parity import assert_close, dev, host

pytestmark = pytest.mark.gpu


def bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


def without_xr(lib, call):
    """The call with the x-resident matrix-core GEMV switched off."""
    with lib.kernels(mask=lib.QG_KERNEL_ALL & ~lib.QG_KERNEL_XR):
        return call()


# M from 3 to 40 (one to five launches of up to 8 rows), K from one wave (512)
# to eight (4096) and 3072 (six waves), ragged N (1, 15, 17 rows: partial
# 16-row groups); then shapes that stay on the FMA kernels
CASES = [(3, 1, 512), (3, 17, 1024), (8, 33, 2048), (5, 100, 3072), (8, 300, 4096), (4, 16, 4096),
         (9, 40, 4096), (16, 15, 1024), (40, 65, 512), (7, 1000, 4096),
         (4, 20, 4160), (3, 9, 8192), (6, 30, 256)]


@pytest.mark.parametrize("m,n,k", CASES)
def test_q4_0_xr_against_oracle_and_fma_path(lib, m, n, k):
    w, x = synth.q4_0_case(9400 + m + n, m, n, k)
    dw, dx = dev(w), dev(x)
    y = host(lib.qgemv_q4_0(dw, dx, n, k))
    w64 = oracle.decode_q4_0(w, n, k)
    assert_close(y, w64, x, f"q4_0 xr m{m} n{n} k{k}")
    y_fma = without_xr(lib, lambda: host(lib.qgemv_q4_0(dw, dx, n, k)))
    assert_close(y_fma, w64, x, "fma path")
    # a second call gives the same bits (no state carried between calls)
    assert np.array_equal(bits(y), bits(host(lib.qgemv_q4_0(dw, dx, n, k))))


@pytest.mark.parametrize("m,n,k", [(3, 50, 4096), (4, 4096, 4096), (8, 257, 2048), (5, 31, 512), (13, 19, 1024)])
def test_dual_xr_bitwise_equals_two_singles(lib, m, n, k):
    wa, wb, x = synth.dual_q4_0_case(9500 + m + n, m, n, k)
    dwa, dwb, dx = dev(wa), dev(wb), dev(x)
    ya, yb = (host(t) for t in lib.qgemv_dual_q4_0(dwa, dwb, dx, n, k))
    assert np.array_equal(bits(ya), bits(host(lib.qgemv_q4_0(dwa, dx, n, k))))
    assert np.array_equal(bits(yb), bits(host(lib.qgemv_q4_0(dwb, dx, n, k))))
    assert_close(ya, oracle.decode_q4_0(wa, n, k), x, f"dual a m{m}")
    assert_close(yb, oracle.decode_q4_0(wb, n, k), x, f"dual b m{m}")


def test_xr_rows_of_x_are_independent(lib):
    """Output row m depends on x row m only: the same x row gives the same bits
    at any position of an 8-row tile and of a 3-row launch."""
    n, k = 70, 4096
    w, x = synth.q4_0_case(9600, 8, n, k)
    dw = dev(w)
    y8 = host(lib.qgemv_q4_0(dw, dev(x), n, k))
    for pos in (0, 3, 7):
        x3 = np.stack([x[(pos + 1) % 8], x[pos], x[(pos + 2) % 8]])
        y3 = host(lib.qgemv_q4_0(dw, dev(x3), n, k))
        assert np.array_equal(bits(y3[1]), bits(y8[pos])), pos


def test_xr_blocks_of_eights_give_exact_zero(lib):
    """Rows whose blocks all hold codes 8 (w = 0 for any scale) give exactly 0
    for any x, and a row holding the hand block [d = 0.5, qs[0] = 0x1F,
    qs[1] = 0x80, rest 0x88] at block 3 gives 3.5 x[96] - 4 x[97] - 3.5 x[112],
    exactly for integer x."""
    n, k, m = 33, 2048, 6
    g = np.random.default_rng(9700)
    blocks = np.zeros((n, k // 32, 18), np.uint8)
    d = np.frombuffer(np.float16(g.uniform(0.01, 2.0, size=n * (k // 32))).astype(np.float16).tobytes(),
                      np.uint8).reshape(n, k // 32, 2)
    blocks[:, :, 0:2] = d
    blocks[:, :, 2:] = 0x88
    blocks[5, 3, 0:2] = np.frombuffer(np.float16(0.5).tobytes(), np.uint8)
    blocks[5, 3, 2] = 0x1F
    blocks[5, 3, 3] = 0x80
    w = blocks.reshape(-1)
    dw = dev(w)
    xi = g.integers(-4, 5, size=(m, k)).astype(np.float32)
    y = host(lib.qgemv_q4_0(dw, dev(xi), n, k))
    want = np.zeros((m, n), np.float32)
    want[:, 5] = 3.5 * xi[:, 96] - 4.0 * xi[:, 97] - 3.5 * xi[:, 112]
    assert np.array_equal(bits(y), bits(want))
    xn = synth.normal_f32(g, (m, k))
    y = host(lib.qgemv_q4_0(dw, dev(xn), n, k))
    rest = [i for i in range(n) if i != 5]
    assert np.array_equal(bits(y[:, rest]), bits(np.zeros((m, n - 1), np.float32)))
    assert_close(y, oracle.decode_q4_0(w, n, k), xn, "eights")


def test_xr_non_finite_x_stays_in_its_row(lib):
    n, k, m = 40, 1024, 5
    w, x = synth.q4_0_case(9800, m, n, k)
    x[2, 77] = np.inf
    x[4, 5] = np.nan
    y = host(lib.qgemv_q4_0(dev(w), dev(x), n, k))
    finite = [0, 1, 3]
    assert np.all(np.isfinite(y[finite]))
    assert_close(y[finite], oracle.decode_q4_0(w, n, k), x[finite], "finite rows")
    assert not np.any(np.isfinite(y[4]))


# ------------------------------------------------------------------ Q4_K
Q4K_CASES = [(3, 1, 512), (4, 17, 1024), (8, 33, 2048), (5, 100, 3072), (8, 300, 4096), (9, 40, 4096),
             (16, 15, 1024), (7, 1000, 4096), (4, 20, 4352), (3, 9, 8192), (6, 30, 256)]


@pytest.mark.parametrize("m,n,k", Q4K_CASES)
def test_q4_k_xr_against_oracle_and_fma_path(lib, m, n, k):
    w, x = synth.q4_k_case(9900 + m + n, m, n, k)
    dw, dx = dev(w), dev(x)
    y = host(lib.qgemv_q4_k(dw, dx, n, k))
    w64 = oracle.decode_q4_k(w, n, k)
    assert_close(y, w64, x, f"q4_k xr m{m} n{n} k{k}")
    y_fma = without_xr(lib, lambda: host(lib.qgemv_q4_k(dw, dx, n, k)))
    assert_close(y_fma, w64, x, "fma path")
    assert np.array_equal(bits(y), bits(host(lib.qgemv_q4_k(dw, dx, n, k))))


@pytest.mark.parametrize("m,ns,k", [(3, (7, 1, 40), 1024), (8, (64, 64), 2048), (5, (33,) * 8, 512),
                                    (4, (4096, 1024, 1024), 4096)])
def test_q4_k_multi_xr_bitwise_equals_singles(lib, m, ns, k):
    ws, x = synth.q4_k_multi_case(10000 + m + k, m, ns, k)
    dws, dx = [dev(w) for w in ws], dev(x)
    y = host(lib.qgemv_q4_k_multi(dws, dx, list(ns), k))
    col = 0
    for w, dw, n in zip(ws, dws, ns):
        assert np.array_equal(bits(y[:, col:col + n]), bits(host(lib.qgemv_q4_k(dw, dx, n, k)))), col
        assert_close(y[:, col:col + n], oracle.decode_q4_k(w, n, k), x, f"multi xr col {col}")
        col += n


def test_q4_k_xr_hand_super_block_exact(lib):
    """The hand-worked super-block (d = 1, dmin = 0.5, scale bytes 0xC1 at 0,
    0x42 at 4, 0x23 at 8; code bytes 0x52 at 0, 0x07 at 64) in the first of two
    super-blocks, a zero super-block in the second, at 4 rows of integer x: the
    products are exact, so the result equals the oracle's bit for bit; with
    x = ones it is the worked value."""
    import json
    from conftest import GOLDEN
    fx = json.load(open(os.path.join(GOLDEN, "q4_k_hand_block.json")))
    hand = np.frombuffer(bytes.fromhex(fx["bytes_hex"]), dtype=np.uint8)
    row = np.concatenate([hand, np.zeros(144, np.uint8)])
    w = np.stack([row, np.zeros_like(row), row]).reshape(-1)
    n, k = 3, 512
    g = np.random.default_rng(10100)
    x = g.integers(-4, 5, size=(4, k)).astype(np.float32)
    x[0] = 1.0
    y = host(lib.qgemv_q4_k(dev(w), dev(x), n, k))
    want = (x.astype(np.float64) @ oracle.decode_q4_k(w, n, k).T).astype(np.float32)
    assert np.array_equal(bits(y), bits(want))
    assert list(y[0]) == [fx["y_ones"], 0.0, fx["y_ones"]]


# ------------------------------------------------------------------ affine codes
AFF_CASES = [(3, 1, 512, 64, 15), (4, 17, 1024, 512, 255), (8, 33, 2048, 128, 15), (5, 100, 3072, 1024, 255),
             (8, 300, 4096, 64, 15), (9, 40, 4096, 256, 255), (16, 15, 1024, 64, 15), (7, 600, 4096, 64, 255),
             (4, 20, 1024, 32, 255), (3, 9, 8192, 64, 15), (6, 30, 1536, 64, 15)]


@pytest.mark.parametrize("m,n,k,gs,code_max", AFF_CASES)
def test_affine_xr_against_oracle_and_other_path(lib, m, n, k, gs, code_max):
    x, q, s, b = synth.affine_case(10200 + m + n, m, n, k, gs, code_max)
    dx, dq, ds, db = dev(x), dev(q), dev(s), dev(b)
    y = host(lib.qmm_affine_t(dx, dq, ds, db, gs))
    w64 = oracle.decode_affine(q, s, b, n, k, gs)
    assert_close(y, w64, x, f"affine xr m{m} n{n} k{k} gs{gs}")
    y_other = without_xr(lib, lambda: host(lib.qmm_affine_t(dx, dq, ds, db, gs)))
    assert_close(y_other, w64, x, "other path")
    assert np.array_equal(bits(y), bits(host(lib.qmm_affine_t(dx, dq, ds, db, gs))))


@pytest.mark.parametrize("m,n,k,gs", [(3, 29, 512, 64), (8, 64, 4096, 64), (6, 31, 2048, 128), (12, 5, 1024, 1024)])
def test_packed_xr_bitwise_equals_u8(lib, m, n, k, gs):
    import torch
    x, q, s, b = synth.affine_case(10300 + m + n, m, n, k, gs)
    wp = torch.from_numpy(synth.pack_b4_u32(q).view(np.int32)).cuda()
    dx, ds, db = dev(x), dev(s), dev(b)
    y = host(lib.qmm_affine_t_packed(dx, wp, ds, db, gs))
    assert np.array_equal(bits(y), bits(host(lib.qmm_affine_t(dx, dev(q), ds, db, gs))))
    assert_close(y, oracle.decode_affine(q, s, b, n, k, gs), x, f"packed xr m{m}")


@pytest.mark.parametrize("m", [3, 8, 11])
def test_fused_qkv_xr_bitwise_equals_product_then_split(lib, m):
    k, gs, qs, ks, vs = 1024, 64, 96, 40, 17
    n = qs + ks + vs
    x, q, s, b = synth.affine_case(10400 + m, m, n, k, gs)
    dx, dq, ds, db = dev(x), dev(q), dev(s), dev(b)
    got = [host(t) for t in lib.qmm_affine_t_qkv(dx, dq, ds, db, gs, qs, ks, vs)]
    y = lib.qmm_affine_t(dx, dq, ds, db, gs)
    for a, r in zip(got, lib.qkv_split_f32(y, m, qs, ks, vs)):
        assert np.array_equal(bits(a), bits(host(r)))
    assert_close(np.concatenate(got, axis=1), oracle.decode_affine(q, s, b, n, k, gs), x, f"fused qkv xr m{m}")


@pytest.mark.parametrize("fmt", ["q4_0", "q4_k", "affine"])
def test_xr_unaligned_x_gives_the_same_bits(lib, fmt):
    """x at a 4-byte (not 16-byte) aligned address: the x loads are dword-aligned
    vector loads, so the result is the same bits as with aligned x."""
    import torch
    m, n, k, gs = 5, 37, 2048, 64
    if fmt == "q4_0":
        w, x = synth.q4_0_case(10500, m, n, k)
        call = lambda dx: lib.qgemv_q4_0(dev(w), dx, n, k)
    elif fmt == "q4_k":
        w, x = synth.q4_k_case(10501, m, n, k)
        call = lambda dx: lib.qgemv_q4_k(dev(w), dx, n, k)
    else:
        x, q, s, b = synth.affine_case(10502, m, n, k, gs)
        call = lambda dx: lib.qmm_affine_t(dx, dev(q), dev(s), dev(b), gs)
    buf = torch.zeros(x.size + 1, dtype=torch.float32, device="cuda")
    xu = buf[1:].view(m, k)
    xu.copy_(torch.from_numpy(x).cuda())
    assert xu.data_ptr() % 16 == 4
    assert np.array_equal(bits(host(call(xu))), bits(host(call(dev(x)))))


# ---------------------------------------------- many row groups per workgroup
def _random_blocks(rng, n, k, fmt):
    """Random but valid weight bytes (any nibbles and scale bytes, finite
    fp16 d / dmin of either sign) without running a quantizer over N x K
    values."""
    if fmt == "q4_0":
        w = rng.integers(0, 256, size=(n, k // 32, 18), dtype=np.uint8)
        d = (rng.uniform(0.001, 0.01, size=(n, k // 32)) * rng.choice([-1.0, 1.0], size=(n, k // 32)))
        w[:, :, 0:2] = d.astype(np.float16).view(np.uint8).reshape(n, k // 32, 2)
    else:
        w = rng.integers(0, 256, size=(n, k // 256, 144), dtype=np.uint8)
        d = rng.uniform(0.001, 0.01, size=(n, k // 256, 2))
        w[:, :, 0:4] = d.astype(np.float16).view(np.uint8).reshape(n, k // 256, 4)
    return w.reshape(n, -1)


@pytest.mark.parametrize("fmt,m,n,k", [("q4_0", 8, 16400, 4096), ("q4_k", 5, 16403, 4096), ("q4_0", 4, 33001, 2048),
                                       ("packed", 8, 16411, 4096), ("u8", 3, 8200, 4096)])
def test_xr_many_row_groups_per_workgroup(lib, fmt, m, n, k):
    """More than four row groups per workgroup: the wave partials of up to four
    groups wait in LDS slots for one barrier, in two alternating buffers.  Every
    output row must equal the same rows computed by a call with few groups
    (the arithmetic of an output does not depend on the other rows of the
    call), and a slice agrees with the oracle."""
    import torch
    rng = np.random.default_rng(10600 + m + n)
    x = rng.standard_normal((m, k)).astype(np.float32)
    gs = 64
    if fmt in ("q4_0", "q4_k"):
        w = _random_blocks(rng, n, k, fmt)
        f = lib.qgemv_q4_0 if fmt == "q4_0" else lib.qgemv_q4_k
        call = lambda rows: f(dev(np.ascontiguousarray(w[rows])), dev(x), rows.stop - rows.start, k)
        ref = lambda rows: (oracle.decode_q4_0 if fmt == "q4_0" else oracle.decode_q4_k)(
            np.ascontiguousarray(w[rows]), rows.stop - rows.start, k)
    else:
        q = rng.integers(0, 16, size=(n, k), dtype=np.uint8)
        s = rng.uniform(0.001, 0.01, size=(n, k // gs)).astype(np.float32)
        b = (0.02 * rng.standard_normal((n, k // gs))).astype(np.float32)
        if fmt == "u8":
            call = lambda rows: lib.qmm_affine_t(dev(x), dev(np.ascontiguousarray(q[rows])),
                                                 dev(np.ascontiguousarray(s[rows])), dev(np.ascontiguousarray(b[rows])), gs)
        else:
            wp = synth.pack_b4_u32(q).view(np.int32)
            call = lambda rows: lib.qmm_affine_t_packed(dev(x), torch.from_numpy(np.ascontiguousarray(wp[rows])).cuda(),
                                                        dev(np.ascontiguousarray(s[rows])), dev(np.ascontiguousarray(b[rows])), gs)
        ref = lambda rows: oracle.decode_affine(np.ascontiguousarray(q[rows]), s[rows], b[rows], rows.stop - rows.start, k, gs)
    y = host(call(slice(0, n)))
    # slices starting on 16-row group boundaries keep each row's place in its group
    for rows in (slice(0, 48), slice(16 * (n // 32), 16 * (n // 32) + 40), slice(16 * ((n - 37) // 16), n)):
        got = y[:, rows]
        assert np.array_equal(bits(got), bits(host(call(rows)))), f"{fmt} rows {rows}"
    tail = slice(16 * ((n - 37) // 16), n)
    assert_close(y[:, tail], ref(tail), x, f"{fmt} xr m{m} n{n} k{k} tail")
    assert_close(y[:, 0:48], ref(slice(0, 48)), x, f"{fmt} xr m{m} n{n} k{k} head")
