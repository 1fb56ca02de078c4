"""The matrix-core Q4_0 GEMV with x in registers (2..8 rows of x per launch,
K a multiple of 512 up to 4096) against the f64 oracle, and its stated
equalities: the dual product bitwise equal to two single calls, each row of x
independent of the others, blocks of codes 8 giving exactly zero.  The tuning
switch QG_GEMV_XR=0 selects the FMA kernels, whose results must agree within
the same tolerance.  Shapes outside that range (K = 4160, 8192, 256) take the
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


def with_env(val, call):
    old = os.environ.get("QG_GEMV_XR")
    try:
        os.environ["QG_GEMV_XR"] = val
        return call()
    finally:
        if old is None:
            os.environ.pop("QG_GEMV_XR", None)
        else:
            os.environ["QG_GEMV_XR"] = old


# M from 2 to 40 (one to five launches of up to 8 rows), K from one wave (512)
# to eight (4096) and 3072 (six waves), ragged N (1, 15, 17 rows: partial
# 16-row groups); then shapes that stay on the FMA kernels
CASES = [(2, 1, 512), (3, 17, 1024), (8, 33, 2048), (5, 100, 3072), (8, 300, 4096), (4, 16, 4096),
         (9, 40, 4096), (16, 15, 1024), (40, 65, 512), (7, 1000, 4096),
         (4, 20, 4160), (3, 9, 8192), (6, 30, 256)]


@pytest.mark.parametrize("m,n,k", CASES)
def test_q4_0_xr_against_oracle_and_fma_path(lib, m, n, k):
    w, x = synth.q4_0_case(9400 + m + n, m, n, k)
    dw, dx = dev(w), dev(x)
    y = host(lib.qgemv_q4_0(dw, dx, n, k))
    w64 = oracle.decode_q4_0(w, n, k)
    assert_close(y, w64, x, f"q4_0 xr m{m} n{n} k{k}")
    y_fma = with_env("0", lambda: host(lib.qgemv_q4_0(dw, dx, n, k)))
    assert_close(y_fma, w64, x, "fma path")
    # a second call gives the same bits (no state carried between calls)
    assert np.array_equal(bits(y), bits(host(lib.qgemv_q4_0(dw, dx, n, k))))


@pytest.mark.parametrize("m,n,k", [(2, 50, 4096), (4, 4096, 4096), (8, 257, 2048), (5, 31, 512), (13, 19, 1024)])
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
    at any position of an 8-row tile and in a 2-row launch."""
    n, k = 70, 4096
    w, x = synth.q4_0_case(9600, 8, n, k)
    dw = dev(w)
    y8 = host(lib.qgemv_q4_0(dw, dev(x), n, k))
    for pos in (0, 3, 7):
        x2 = np.stack([x[(pos + 1) % 8], x[pos]])
        y2 = host(lib.qgemv_q4_0(dw, dev(x2), n, k))
        assert np.array_equal(bits(y2[1]), bits(y8[pos])), pos


def test_xr_blocks_of_eights_give_exact_zero(lib):
    """Rows whose blocks all hold codes 8 (w = 0 for any scale) give exactly 0;
    a row of the hand block [d = 0.5, qs[0] = 0x1F, qs[1] = 0x80, rest 0x88]
    followed by such blocks gives -4 sum x[.., 1] ... exactly the oracle value
    for integer x."""
    n, k, m = 33, 2048, 6
    g = np.random.default_rng(9700)
    blocks = np.zeros((n, k // 32, 18), np.uint8)
    d = np.frombuffer(np.float16(g.uniform(0.01, 2.0, size=n * (k // 32))).astype(np.float16).tobytes(),
                      np.uint8).reshape(n, k // 32, 2)
    blocks[:, :, 0:2] = d
    blocks[:, :, 2:] = 0x88
    # row 5: the hand block at block 3
    blocks[5, 3, 0:2] = np.frombuffer(np.float16(0.5).tobytes(), np.uint8)
    blocks[5, 3, 2] = 0x1F
    blocks[5, 3, 3] = 0x80
    w = blocks.reshape(-1)
    x = g.integers(-4, 5, size=(m, k)).astype(np.float32)
    y = host(lib.qgemv_q4_0(dev(w), dev(x), n, k))
    want = np.zeros((m, n), np.float32)
    # hand block: w[0] = 3.5, w[1] = -4.0, w[16] = -3.5, others 0 (columns 96 + j)
    want[:, 5] = 3.5 * x[:, 96] - 4.0 * x[:, 97] - 3.5 * x[:, 112]
    assert np.array_equal(bits(y), bits(want))
    assert_close(y, oracle.decode_q4_0(w, n, k), x, "eights")


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
