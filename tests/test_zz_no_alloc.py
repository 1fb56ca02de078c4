"""qmm_affine_t_noalloc (the allocation-free variant of qmm_affine_t, for
callers that cannot allocate) through the C ABI against qmm_affine_t: the
same bits on the matrix-core path (static scratch) and on the GEMV path (no
scratch), on two calls in a row, the second with a smaller input that reuses
the scratch the first one left behind."""
import numpy as np
import pytest

import oracle
import synth
from test_gpu_parity import assert_close, dev, host

pytestmark = pytest.mark.gpu


def bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


def _case(lib, seed, m, n, k, gs):
    import torch
    x, q, s, b = synth.affine_case(seed, m, n, k, gs)
    dx, dq, ds, db = dev(x), dev(q), dev(s), dev(b)
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
    lib.qmm_affine_t_noalloc(dx, dq, ds, db, gs, y)
    want = host(lib.qmm_affine_t(dx, dq, ds, db, gs))
    return host(y), want, (x, q, s, b)


def test_noalloc_equals_qmm_affine_t_on_two_calls(lib):
    assert lib.qg_get_mfma_min_m() <= 512
    # first call: the prefill shape (x 512 x 2048: 4.06 MiB of scratch)
    y1, w1, (x, q, s, b) = _case(lib, 5100, 512, 8192, 2048, 64)
    assert np.array_equal(bits(y1), bits(w1))
    rows = np.arange(0, 512, 37)
    assert_close(y1[rows], oracle.decode_affine(q, s, b, 8192, 2048, 64), x[rows], "noalloc prefill (sampled rows)")
    # second call, smaller: the scratch holds the first call's values
    y2, w2, (x, q, s, b) = _case(lib, 5101, 70, 300, 1024, 128)
    assert np.array_equal(bits(y2), bits(w2))
    assert_close(y2, oracle.decode_affine(q, s, b, 300, 1024, 128), x, "noalloc second call")


def test_noalloc_gemv_path_and_limit(lib):
    y, w, _ = _case(lib, 5102, 4, 500, 4096, 64)  # few rows of x: no scratch
    assert np.array_equal(bits(y), bits(w))
    import torch
    m, n, k = 2048, 64, 4096  # 2 * 16 MiB of x_hi/x_lo: beyond the static buffer
    x = torch.zeros((m, k), dtype=torch.float32, device="cuda")
    q = torch.zeros((n, k), dtype=torch.uint8, device="cuda")
    sb = torch.zeros((n, k // 64), dtype=torch.float32, device="cuda")
    y = torch.zeros((m, n), dtype=torch.float32, device="cuda")
    with pytest.raises(lib.QGError, match="static buffer"):
        lib.qmm_affine_t_noalloc(x, q, sb, sb.clone(), 64, y)
