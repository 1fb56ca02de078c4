"""The matrix-core GEMV for 2..8 rows of x per launch (u8 and packed affine
codes, group size >= 64, K a multiple of 512 with K/512 in {1, 2, 4, 8})
against the f64 oracle, and its stated equalities: packed codes bitwise equal
to u8 codes, the fused q|k|v product bitwise equal to the product then the
split.  Without QG_KERNEL_MMA in the kernel mask the FMA kernels run, whose
results must agree within the same tolerance.  Shapes outside that range (group size
32, K = 256 or 1536) take the FMA kernels and are checked the same way."""
import numpy as np
import pytest

import oracle
import synth
from test_gpu_parity import assert_close, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _no_xr(lib):
    """From 3 rows of x the x-resident matrix-core GEMV takes these products;
    it is switched off here so that this kernel is the one tested at every M
    (tests/test_gpu_xr.py covers the other)."""
    with lib.kernels(mask=lib.QG_KERNEL_ALL & ~lib.QG_KERNEL_XR):
        yield


def bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


def fma_only(lib, call):
    """The call with the FMA kernels only (no matrix-core GEMV)."""
    with lib.kernels(mask=lib.QG_KERNEL_KSLICED):
        return call()


# M from 2 to 40 (one to five launches of up to 8 rows), K from one pair of
# 32-column blocks per wave (512) to eight (4096), group sizes 64 .. 1024,
# ragged N, all codes 0..255; then three shapes that stay on the FMA kernels
CASES = [(2, 1, 512, 64, 15), (3, 17, 1024, 512, 255), (8, 33, 1024, 128, 15), (5, 100, 2048, 1024, 255),
         (8, 300, 4096, 64, 15), (9, 40, 4096, 256, 255), (16, 77, 2048, 64, 15), (40, 65, 1024, 512, 255),
         (4, 20, 1024, 32, 255), (3, 9, 256, 64, 15), (6, 30, 1536, 64, 15)]


@pytest.mark.parametrize("m,n,k,gs,code_max", CASES)
def test_affine_mma_against_oracle_and_fma_path(lib, m, n, k, gs, code_max):
    x, q, s, b = synth.affine_case(9100 + m + n, m, n, k, gs, code_max)
    dx, dq, ds, db = dev(x), dev(q), dev(s), dev(b)
    y = host(lib.qmm_affine_t(dx, dq, ds, db, gs))
    w64 = oracle.decode_affine(q, s, b, n, k, gs)
    assert_close(y, w64, x, f"affine mma m{m} n{n} k{k} gs{gs}")
    y_fma = fma_only(lib, lambda: host(lib.qmm_affine_t(dx, dq, ds, db, gs)))
    assert_close(y_fma, w64, x, "fma path")
    # a second call gives the same bits (no state carried between calls)
    assert np.array_equal(bits(y), bits(host(lib.qmm_affine_t(dx, dq, ds, db, gs))))


@pytest.mark.parametrize("m,n,k,gs", [(2, 29, 512, 64), (8, 64, 4096, 64), (6, 31, 2048, 128), (12, 5, 1024, 256)])
def test_packed_mma_bitwise_equals_u8(lib, m, n, k, gs):
    import torch
    x, q, s, b = synth.affine_case(9200 + m + n, m, n, k, gs)
    wp = torch.from_numpy(synth.pack_b4_u32(q).view(np.int32)).cuda()
    dx, ds, db = dev(x), dev(s), dev(b)
    y = host(lib.qmm_affine_t_packed(dx, wp, ds, db, gs))
    assert np.array_equal(bits(y), bits(host(lib.qmm_affine_t(dx, dev(q), ds, db, gs))))
    assert_close(y, oracle.decode_affine(q, s, b, n, k, gs), x, f"packed mma m{m}")


@pytest.mark.parametrize("m", [2, 8, 11])
def test_fused_qkv_mma_bitwise_equals_product_then_split(lib, m):
    k, gs, qs, ks, vs = 1024, 64, 96, 40, 17
    n = qs + ks + vs
    x, q, s, b = synth.affine_case(9300 + m, m, n, k, gs)
    dx, dq, ds, db = dev(x), dev(q), dev(s), dev(b)
    got = [host(t) for t in lib.qmm_affine_t_qkv(dx, dq, ds, db, gs, qs, ks, vs)]
    y = lib.qmm_affine_t(dx, dq, ds, db, gs)
    for a, r in zip(got, lib.qkv_split_f32(y, m, qs, ks, vs)):
        assert np.array_equal(bits(a), bits(host(r)))
    assert_close(np.concatenate(got, axis=1), oracle.decode_affine(q, s, b, n, k, gs), x, f"fused qkv mma m{m}")


def test_rows_of_x_are_independent(lib):
    """Rows of x sharing a launch do not leak into each other: the M = 8
    product equals, row by row, the same rows computed at M = 2 (both on the
    matrix-core kernel; the block products of one row do not depend on the
    others)."""
    n, k, gs = 50, 2048, 64
    x, q, s, b = synth.affine_case(9400, 8, n, k, gs)
    dq, ds, db = dev(q), dev(s), dev(b)
    y8 = host(lib.qmm_affine_t(dev(x), dq, ds, db, gs))
    for r0 in (0, 2, 6):
        y2 = host(lib.qmm_affine_t(dev(x[r0:r0 + 2]), dq, ds, db, gs))
        assert np.array_equal(bits(y8[r0:r0 + 2]), bits(y2)), f"rows {r0}.."
