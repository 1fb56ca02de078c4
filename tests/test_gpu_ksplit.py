"""The K-sliced GEMV (one x row: Q4_0, Q4_K, u8 and packed affine codes,
single and multi-part) against the chunked GEMV it replaces at M = 1: the two
kernels make the same additions in the same order, so their outputs must agree
bit for bit (without QG_KERNEL_KSLICED in the kernel mask the chunked kernel runs), and
both against the f64 oracle."""

import numpy as np
import pytest

import oracle
import synth
from test_gpu_parity import assert_close, dev, host

pytestmark = pytest.mark.gpu


def bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


def both(call):
    """(K-sliced result, chunked result) of one call.  The matrix-core GEMVs,
    which take products from 2 or 3 rows of x on, are switched off for both."""
    import gemm_qgemv_q4_amd as qg
    with qg.kernels(mask=qg.QG_KERNEL_KSLICED):
        a = call()
    with qg.kernels(mask=0):
        b = call()
    return a, b


# K from one super-block to 64 (one to four chunks per lane, ragged last lanes;
# from K = 4096 on, 64 lanes per row and 8 waves)
@pytest.mark.parametrize("n,k", [(1, 256), (15, 512), (17, 1024), (33, 2304), (300, 4096),
                                 (70, 5888), (40, 8192), (4099, 4096), (25, 12544), (11, 16384)])
def test_q4_k_ksplit_equals_chunked(lib, n, k):
    w, x = synth.q4_k_case(8100 + n, 1, n, k)
    dw, dx = dev(w), dev(x)
    a, b = both(lambda: host(lib.qgemv_q4_k(dw, dx, n, k)))
    assert np.array_equal(bits(a), bits(b))
    assert_close(a, oracle.decode_q4_k(w, n, k), x, f"q4_k ksplit n{n} k{k}")


@pytest.mark.parametrize("n,k", [(3, 64), (257, 4096), (31, 8128), (20, 12288), (9, 16384)])
def test_q4_0_ksplit_equals_chunked(lib, n, k):
    w, x = synth.q4_0_case(8200 + n, 1, n, k)
    dw, dx = dev(w), dev(x)
    a, b = both(lambda: host(lib.qgemv_q4_0(dw, dx, n, k)))
    assert np.array_equal(bits(a), bits(b))
    assert_close(a, oracle.decode_q4_0(w, n, k), x, f"q4_0 ksplit n{n} k{k}")


@pytest.mark.parametrize("n,k", [(50, 4096), (19, 2048 + 64), (21, 16384)])
def test_dual_ksplit_equals_chunked_and_single_calls(lib, n, k):
    """The dual product on the K-sliced kernel equals the chunked kernel and
    two single calls, bit for bit."""
    wa, wb, x = synth.dual_q4_0_case(8300 + n, 1, n, k)
    dwa, dwb, dx = dev(wa), dev(wb), dev(x)
    (a0, a1), (b0, b1) = both(lambda: tuple(host(t) for t in lib.qgemv_dual_q4_0(dwa, dwb, dx, n, k)))
    assert np.array_equal(bits(a0), bits(b0)) and np.array_equal(bits(a1), bits(b1))
    single = host(lib.qgemv_q4_0(dwb, dx, n, k))
    assert np.array_equal(bits(a1), bits(single))


def test_multi_ksplit_equals_chunked_and_single(lib):
    ns, k = (96, 40, 17), 4096
    ws, x = synth.q4_k_multi_case(8400, 1, ns, k)
    dws, dx = [dev(w) for w in ws], dev(x)
    a, b = both(lambda: host(lib.qgemv_q4_k_multi(dws, dx, list(ns), k)))
    assert np.array_equal(bits(a), bits(b))
    col = 0
    for w, dw, n in zip(ws, dws, ns):
        assert np.array_equal(bits(a[:, col:col + n]), bits(host(lib.qgemv_q4_k(dw, dx, n, k))))
        col += n


def test_unaligned_x_ksplit(lib):
    import torch
    n, k = 40, 4096
    w, x = synth.q4_k_case(8500, 1, n, k)
    buf = torch.zeros(x.size + 1, dtype=torch.float32, device="cuda")
    buf[1:] = torch.from_numpy(np.ascontiguousarray(x).ravel()).cuda()
    xo = buf[1:].view(x.shape)
    dw = dev(w)
    a, b = both(lambda: host(lib.qgemv_q4_k(dw, xo, n, k)))
    assert np.array_equal(bits(a), bits(b))
    assert np.array_equal(bits(a), bits(host(lib.qgemv_q4_k(dw, dev(x), n, k))))


# affine codes: 32-code chunks, 64 lanes per row (8 waves of 8 lanes each);
# K from 2048 (one chunk per lane) to 8192 (four), ragged last lanes (K = 2432
# ends a wave's slice of 8 chunks part way, K = 3072 leaves whole slices past
# the row's end), group sizes 32 to 512 (each chunk's scale and bias loaded
# after all of the row group's codes)
@pytest.mark.parametrize("n,k,gs,code_max", [(1, 2048, 64, 15), (17, 2208, 32, 255), (40, 4096, 64, 15),
                                             (33, 6144, 512, 255), (300, 8192, 128, 15), (2049, 4096, 64, 255),
                                             (77, 2432, 64, 255), (19, 2432, 128, 15), (50, 3072, 128, 15),
                                             (9, 3072, 64, 255)])
def test_affine_ksplit_equals_chunked(lib, n, k, gs, code_max):
    x, q, s, b = synth.affine_case(8600 + n, 1, n, k, gs, code_max)
    dx, dq, ds, db = dev(x), dev(q), dev(s), dev(b)
    a, c = both(lambda: host(lib.qmm_affine_t(dx, dq, ds, db, gs)))
    assert np.array_equal(bits(a), bits(c))
    assert_close(a, oracle.decode_affine(q, s, b, n, k, gs), x, f"affine ksplit n{n} k{k} gs{gs}")


@pytest.mark.parametrize("n,k,gs", [(29, 4096, 64), (64, 2208, 32), (5, 8192, 256), (13, 2432, 128), (21, 3072, 64)])
def test_packed_ksplit_equals_chunked_and_u8(lib, n, k, gs):
    import torch
    x, q, s, b = synth.affine_case(8700 + n, 1, n, k, gs)
    wp = torch.from_numpy(synth.pack_b4_u32(q).view(np.int32)).cuda()
    dx, ds, db = dev(x), dev(s), dev(b)
    a, c = both(lambda: host(lib.qmm_affine_t_packed(dx, wp, ds, db, gs)))
    assert np.array_equal(bits(a), bits(c))
    assert np.array_equal(bits(a), bits(host(lib.qmm_affine_t(dx, dev(q), ds, db, gs))))


def test_fused_qkv_ksplit_equals_chunked_and_split(lib):
    k, gs, qs, ks, vs = 4096, 64, 96, 40, 17
    n = qs + ks + vs
    x, q, s, b = synth.affine_case(8800, 1, n, k, gs)
    dx, dq, ds, db = dev(x), dev(q), dev(s), dev(b)
    a, c = both(lambda: tuple(host(t) for t in lib.qmm_affine_t_qkv(dx, dq, ds, db, gs, qs, ks, vs)))
    for u, v in zip(a, c):
        assert np.array_equal(bits(u), bits(v))
    y = lib.qmm_affine_t(dx, dq, ds, db, gs)
    for got, ref in zip(a, lib.qkv_split_f32(y, 1, qs, ks, vs)):
        assert np.array_equal(bits(got), bits(host(ref)))


# two to four rows of x (tiles of 2 or 4 rows, 4 waves per workgroup at K >= 2048)
@pytest.mark.parametrize("m,n,k", [(2, 33, 2048), (3, 300, 4096), (4, 70, 8192), (4, 4099, 4096),
                                   (2, 4099, 4096), (2, 17, 16384)])
def test_q4_k_ksplit_rows_of_x_equal_chunked(lib, m, n, k):
    w, x = synth.q4_k_case(9700 + m + n, m, n, k)
    dw, dx = dev(w), dev(x)
    a, b = both(lambda: host(lib.qgemv_q4_k(dw, dx, n, k)))
    assert np.array_equal(bits(a), bits(b))
    assert_close(a, oracle.decode_q4_k(w, n, k), x, f"q4_k ksplit m{m} n{n} k{k}")


@pytest.mark.parametrize("m", [2, 4])
def test_dual_and_multi_ksplit_rows_of_x_equal_chunked(lib, m):
    n, k = 40, 4096
    wa, wb, x = synth.dual_q4_0_case(9800 + m, m, n, k)
    dwa, dwb, dx = dev(wa), dev(wb), dev(x)
    (a0, a1), (b0, b1) = both(lambda: tuple(host(t) for t in lib.qgemv_dual_q4_0(dwa, dwb, dx, n, k)))
    assert np.array_equal(bits(a0), bits(b0)) and np.array_equal(bits(a1), bits(b1))
    with lib.kernels(mask=lib.QG_KERNEL_KSLICED):  # the single call on the dual's kernels
        assert np.array_equal(bits(a0), bits(host(lib.qgemv_q4_0(dwa, dx, n, k))))
    assert_close(a1, oracle.decode_q4_0(wb, n, k), x, f"dual ksplit m{m}")
    ns = (96, 40, 17)
    ws, xm = synth.q4_k_multi_case(9850 + m, m, ns, k)
    dws, dxm = [dev(w) for w in ws], dev(xm)
    a, b = both(lambda: host(lib.qgemv_q4_k_multi(dws, dxm, list(ns), k)))
    assert np.array_equal(bits(a), bits(b))


# Row counts whose 16-row groups fill the CUs in whole rounds (or one round at
# least three quarters full) take 16-wave workgroups (one per CU) at 64 lanes
# per row; the additions are the same.
@pytest.mark.parametrize("fmt,n,k", [("q4_k", 4096, 4096), ("q4_k", 3600, 8192), ("q4_0", 4000, 4096),
                                     ("q4_0", 3900, 6144), ("q4_k", 8192, 4096), ("q4_0", 12288, 4096)])
def test_sixteen_wave_groups_equal_chunked(lib, fmt, n, k):
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    groups = -(-n // 16)
    if not (3 * cus <= 4 * groups <= 4 * cus or groups % cus == 0):
        pytest.skip(f"{n} rows are not whole rounds of 16-row groups on {cus} CUs")
    if fmt == "q4_k":
        w, x = synth.q4_k_case(8600 + n, 1, n, k)
        call, dec = lib.qgemv_q4_k, oracle.decode_q4_k
    else:
        w, x = synth.q4_0_case(8600 + n, 1, n, k)
        call, dec = lib.qgemv_q4_0, oracle.decode_q4_0
    dw, dx = dev(w), dev(x)
    a, b = both(lambda: host(call(dw, dx, n, k)))
    assert np.array_equal(bits(a), bits(b))
    assert_close(a, dec(w, n, k), x, f"{fmt} 16 waves n{n} k{k}")


# A dual Q4_0 product at one x row whose two streams together make whole rounds
# of 16-row groups (or one round at least three quarters full) runs as one
# stream of twice the row groups on 16 waves: ragged N, one and two chunks
# per lane.
@pytest.mark.parametrize("n,k", [(4096, 4096), (1999, 4096), (1536, 6144), (2048, 8192)])
def test_dual_pair_launch_equals_chunked_and_single_calls(lib, n, k):
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    groups = 2 * -(-n // 16)
    if not (3 * cus <= 4 * groups <= 4 * cus or groups % cus == 0):
        pytest.skip(f"2 x {n} rows are not whole rounds of 16-row groups on {cus} CUs")
    wa, wb, x = synth.dual_q4_0_case(8800 + n, 1, n, k)
    dwa, dwb, dx = dev(wa), dev(wb), dev(x)
    a, b = both(lambda: tuple(host(t) for t in lib.qgemv_dual_q4_0(dwa, dwb, dx, n, k)))
    for s in range(2):
        assert np.array_equal(bits(a[s]), bits(b[s])), f"stream {s}: pair launch vs chunked kernel"
    assert np.array_equal(bits(a[0]), bits(host(lib.qgemv_q4_0(dwa, dx, n, k))))
    assert np.array_equal(bits(a[1]), bits(host(lib.qgemv_q4_0(dwb, dx, n, k))))
    assert_close(a[0], oracle.decode_q4_0(wa, n, k), x, f"dual pair a n{n} k{k}")
    assert_close(a[1], oracle.decode_q4_0(wb, n, k), x, f"dual pair b n{n} k{k}")


def test_sixteen_wave_multi_part_equals_single_calls(lib):
    """Parts of 2048 + 1024 + 1024 rows (one round of 16-row groups): each part
    equals its single call and the chunked kernel."""
    ns, k = (2048, 1024, 1024), 4096
    ws, x = synth.q4_k_multi_case(8700, 1, ns, k)
    dws, dx = [dev(w) for w in ws], dev(x)
    a, b = both(lambda: host(lib.qgemv_q4_k_multi(dws, dx, list(ns), k)))
    assert np.array_equal(bits(a), bits(b))
    col = 0
    for w, dw, nn in zip(ws, dws, ns):
        single = host(lib.qgemv_q4_k(dw, dx, nn, k))
        assert np.array_equal(bits(a[:, col:col + nn]), bits(single))
        col += nn
    assert_close(a[:, :ns[0]], oracle.decode_q4_k(ws[0], ns[0], k), x, "multi part 0")
