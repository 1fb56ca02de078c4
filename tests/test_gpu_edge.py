"""Edge cases on every kernel path, through the C ABI, against the f64 oracle.

* Q4_0 rows whose blocks all hold codes 8 (w = (q - 8) d = 0 for any d) give
  exactly 0 for any finite x, and rows with exactly one nonzero weight are held
  to the 1e-5 bar even when that weight's x is tiny next to the rest of its
  block (a decode that adds d q x and subtracts 8 d x separately loses that
  term to cancellation).  Paths: the K-sliced GEMV (one and two rows of x,
  32 and 64 lanes per row, 4-row tiles), the chunked GEMV, the x-resident
  matrix-core GEMV, the matrix-core GEMM and the plain kernel, single and dual
  ([dual] mlx-native fused_dual_proj_q4_0.rs: value (nibble - 8) * d).
* The dual product and the multi-part Q4_K product stay bitwise equal to the
  single calls when the weight tensors have different alignments, so that
  they take different kernels ([dual] module doc: byte-identical to two single
  dispatches; [q4k] ferrum-kernels q4_k_gemv_v2.rs, dispatch_gemv_q4k_v2_offset:
  parts at byte offsets into one shared buffer).
* The plain kernel at long K (misaligned Q4_K at K = 8192, affine group size
  16 at K = 4096, Q4_0 with K % 64 = 32) stays within the bar.
"""
import numpy as np
import pytest

import oracle
import synth
from test_gpu_parity import assert_close, dev, host

pytestmark = pytest.mark.gpu


def bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


def at_offset(arr, off):
    """A device uint8 copy of `arr` whose address is 256-byte aligned + off."""
    import torch
    raw = np.ascontiguousarray(arr).reshape(-1).view(np.uint8)
    buf = torch.empty(raw.size + 512, dtype=torch.uint8, device="cuda")
    base = (-buf.data_ptr()) % 256
    t = buf[base + off: base + off + raw.size]
    t.copy_(torch.from_numpy(raw))
    assert t.data_ptr() % 256 == off
    return t


def sparse_q4_0(seed, n, k, hot):
    """Q4_0 weights [n, k]: every block has a random d (|d| in [0.01, 2]) and
    codes 8, except that each row in `hot` has one element with a code other
    than 8.  Returns the bytes and {row: k index of its nonzero weight}."""
    g = synth.rng(seed)
    nb = k // 32
    blocks = np.full((n, nb, 18), 0x88, np.uint8)
    d = (g.uniform(0.01, 2.0, size=(n, nb)) * g.choice([-1.0, 1.0], size=(n, nb))).astype(np.float16)
    blocks[:, :, 0:2] = d.view(np.uint8).reshape(n, nb, 2)
    where = {}
    for r in hot:
        b = int(g.integers(0, nb))
        e = int(g.integers(0, 32))
        q = int(g.choice([c for c in range(16) if c != 8]))
        byte = blocks[r, b, 2 + (e & 15)]
        blocks[r, b, 2 + (e & 15)] = (byte & 0xF0) | q if e < 16 else (byte & 0x0F) | (q << 4)
        where[r] = 32 * b + e
    return blocks.reshape(n, nb * 18), where


def tiny_at(x, cols, seed):
    """x with the given columns scaled down to ~1e-3 of the others."""
    g = synth.rng(seed)
    x = x * 10.0
    for c in set(cols):
        x[:, c] = (g.standard_normal(x.shape[0]) * 1e-3).astype(np.float32)
    return x.astype(np.float32)


# (m, k, kernel mask or None for the default, which path the call takes)
ZERO_PATHS = [
    (1, 4096, None, "K-sliced, 64 lanes per row"),
    (1, 4096, 0, "chunked GEMV"),
    (1, 1024, None, "K-sliced, 32 lanes per row"),
    (2, 4096, None, "K-sliced, two rows of x"),
    (4, 2048, 1, "K-sliced 4-row tiles"),
    (8, 2048, 0, "chunked GEMV, 8-row tiles"),
    (3, 4096, None, "x-resident matrix cores"),
    (8, 2048, None, "x-resident matrix cores"),
    (70, 1024, None, "matrix-core GEMM"),
    (2, 4128, None, "plain kernel (K % 64 = 32)"),
]


@pytest.mark.parametrize("m,k,mask,path", ZERO_PATHS)
def test_q4_0_zero_blocks_and_single_weights(lib, m, k, mask, path):
    n = 80
    hot = list(range(0, n, 5))
    w, where = sparse_q4_0(4100 + m + k, n, k, hot)
    x = tiny_at(synth.normal_f32(synth.rng(4200 + m), (m, k)), where.values(), 4300 + m)
    w64 = oracle.decode_q4_0(w, n, k)
    dw, dx = dev(w), dev(x)
    with lib.kernels(mask=mask if mask is not None else lib.QG_KERNEL_ALL):
        y = host(lib.qgemv_q4_0(dw, dx, n, k))
        ya, yb = (host(t) for t in lib.qgemv_dual_q4_0(dw, dev(w[::-1].copy()), dx, n, k))
    cold = [r for r in range(n) if r not in where]
    assert np.all(y[:, cold] == 0), f"{path}: rows of codes 8 must give exactly 0"
    assert_close(y, w64, x, f"{path}: single nonzero weights")
    assert np.array_equal(bits(ya), bits(y)), f"{path}: dual stream a"
    assert np.all(yb[:, [n - 1 - r for r in cold]] == 0), f"{path}: dual stream b"
    assert_close(yb, w64[::-1], x, f"{path}: dual stream b")


def test_q4_0_zero_blocks_are_exact_for_any_finite_x(lib):
    """Rows of codes 8 stay exactly 0 for huge, tiny and denormal x."""
    n, k = 24, 4096
    w, _ = sparse_q4_0(4400, n, k, [])
    x = np.stack([np.full(k, 3.0e38, np.float32), np.full(k, -1e-40, np.float32),
                  synth.normal_f32(synth.rng(4401), (k,)) * 1e30]).astype(np.float32)
    for m in (1, 2, 3):
        y = host(lib.qgemv_q4_0(dev(w), dev(x[:m].copy()), n, k))
        assert np.all(y == 0), m


# ------------------------------------------------------------------ mixed alignment
@pytest.mark.parametrize("m", [1, 2, 3, 4, 8, 70])
def test_dual_with_misaligned_second_weight_equals_singles(lib, m):
    """w_a 16-byte aligned, w_b at +4 bytes: from 3 rows of x w_a alone may use
    the x-resident kernel (16-byte loads); both results still equal the single
    calls bit for bit."""
    n, k = 65, 4096
    wa, wb, x = synth.dual_q4_0_case(4500 + m, m, n, k)
    dwa, dwb, dx = at_offset(wa, 0), at_offset(wb, 4), dev(x)
    ya, yb = (host(t) for t in lib.qgemv_dual_q4_0(dwa, dwb, dx, n, k))
    assert np.array_equal(bits(ya), bits(host(lib.qgemv_q4_0(dwa, dx, n, k))))
    assert np.array_equal(bits(yb), bits(host(lib.qgemv_q4_0(dwb, dx, n, k))))
    assert_close(ya, oracle.decode_q4_0(wa, n, k), x, f"dual a m{m}")
    assert_close(yb, oracle.decode_q4_0(wb, n, k), x, f"dual b m{m}")
    # and with the roles swapped
    za, zb = (host(t) for t in lib.qgemv_dual_q4_0(dwb, dwa, dx, n, k))
    assert np.array_equal(bits(za), bits(yb)) and np.array_equal(bits(zb), bits(ya))


@pytest.mark.parametrize("m", [1, 4, 70])
def test_multi_with_one_misaligned_part_equals_singles(lib, m):
    """Parts at 16-byte aligned addresses and one at +4 bytes (which only the
    plain kernel reads): every part equals its single call bit for bit."""
    ns, k = (96, 40, 17), 2048
    ws, x = synth.q4_k_multi_case(4600 + m, m, ns, k)
    dws = [at_offset(ws[0], 0), at_offset(ws[1], 4), at_offset(ws[2], 16)]
    dx = dev(x)
    y = host(lib.qgemv_q4_k_multi(dws, dx, list(ns), k))
    col = 0
    for w, dw, nn in zip(ws, dws, ns):
        single = host(lib.qgemv_q4_k(dw, dx, nn, k))
        assert np.array_equal(bits(y[:, col:col + nn]), bits(single)), f"part at column {col}, m{m}"
        assert_close(single, oracle.decode_q4_k(w, nn, k), x, f"multi part m{m}")
        col += nn


# ------------------------------------------------------------------ plain kernel at long K
def test_plain_q4_k_misaligned_long_k(lib):
    m, n, k = 2, 33, 8192
    w, x = synth.q4_k_case(4700, m, n, k)
    y = host(lib.qgemv_q4_k(at_offset(w, 4), dev(x), n, k))
    assert_close(y, oracle.decode_q4_k(w, n, k), x, "plain q4_k k8192")


def test_plain_affine_small_groups_long_k(lib):
    m, n, k, gs = 2, 40, 4096, 16
    x, q, s, b = synth.affine_case(4701, m, n, k, gs)
    y = host(lib.qmm_affine_t(dev(x), dev(q), dev(s), dev(b), gs))
    assert_close(y, oracle.decode_affine(q, s, b, n, k, gs), x, "plain affine gs16 k4096")


def test_plain_q4_0_odd_blocks_long_k(lib):
    m, n, k = 3, 50, 4128
    w, x = synth.q4_0_case(4702, m, n, k)
    y = host(lib.qgemv_q4_0(dev(w), dev(x), n, k))
    assert_close(y, oracle.decode_q4_0(w, n, k), x, "plain q4_0 k4128")
