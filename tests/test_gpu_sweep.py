"""A seeded sweep over the kernel-choice space: every entry point at shapes,
alignments and settings drawn from a fixed generator, each against the f64
oracle (1e-5 of sum |x w|), plus the bitwise equalities the header states
(dual = two singles, multi-part = singles, packed = u8 codes) under the same
settings.

The draws cover M on both sides of every kernel threshold (1, 2, 3..8, 9..63,
the matrix-core threshold and above, also with the threshold lowered to 2),
K from one block to 4096 including K % 64 = 32 and K not a multiple of 512,
ragged N, affine group sizes 16..256, weights at byte offsets 0, 4 and 16
(which send misaligned tensors to other kernels), and the kernel mask with
and without the optional kernels.  Each case prints its parameters first, so
a failure names its case.
"""
import numpy as np
import pytest

import oracle
import synth
from test_gpu_edge import at_offset
from test_gpu_parity import assert_close, dev, host

pytestmark = pytest.mark.gpu

N_CASES = 128
MS = [1, 2, 3, 4, 5, 8, 9, 17, 63, 64, 65, 130]


def bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


def draw(i):
    g = synth.rng(9000 + i)
    fmt = ["q4_0", "q4_k", "affine", "packed", "dual", "multi"][i % 6]
    m = int(g.choice(MS))
    n = int(g.integers(1, 258))
    if fmt in ("q4_0", "dual"):
        k = int(g.choice([64, 96, 512, 1024, 1056, 2048, 4096]))
        off = int(g.choice([0, 4, 16]))
    elif fmt in ("q4_k", "multi"):
        k = int(g.choice([256, 512, 1024, 2304, 4096]))
        off = int(g.choice([0, 4, 16]))
    else:
        k = int(g.choice([64, 128, 512, 1024, 2048, 4096]))
        off = int(g.choice([0, 4, 16])) if fmt == "affine" else int(g.choice([0, 4, 8, 16]))
    gs = int(g.choice([gs for gs in (16, 32, 64, 128, 256) if k % gs == 0]))
    mask = int(g.choice([7, 0, 1, 2, 4]))
    mfma_min_m = int(g.choice([64, 64, 2]))
    return dict(i=i, fmt=fmt, m=m, n=n, k=k, gs=gs, off=off, mask=mask, mfma_min_m=mfma_min_m, seed=9100 + i)


CASES = [draw(i) for i in range(N_CASES)]


@pytest.mark.parametrize("c", CASES, ids=lambda c: f"{c['i']}-{c['fmt']}-m{c['m']}-n{c['n']}-k{c['k']}")
def test_sweep(lib, c):
    print(f"sweep case {c}", flush=True)
    fmt, m, n, k, gs, off, seed = c["fmt"], c["m"], c["n"], c["k"], c["gs"], c["off"], c["seed"]
    tag = f"case {c}"
    with lib.kernels(mask=c["mask"], mfma_min_m=c["mfma_min_m"]):
        if fmt == "q4_0":
            w, x = synth.q4_0_case(seed, m, n, k)
            y = host(lib.qgemv_q4_0(at_offset(w, off), dev(x), n, k))
            assert_close(y, oracle.decode_q4_0(w, n, k), x, tag)
        elif fmt == "q4_k":
            w, x = synth.q4_k_case(seed, m, n, k)
            y = host(lib.qgemv_q4_k(at_offset(w, off), dev(x), n, k))
            assert_close(y, oracle.decode_q4_k(w, n, k), x, tag)
        elif fmt == "dual":
            wa, wb, x = synth.dual_q4_0_case(seed, m, n, k)
            dwa, dwb, dx = at_offset(wa, off), at_offset(wb, 0), dev(x)
            ya, yb = (host(t) for t in lib.qgemv_dual_q4_0(dwa, dwb, dx, n, k))
            assert np.array_equal(bits(ya), bits(host(lib.qgemv_q4_0(dwa, dx, n, k)))), tag
            assert np.array_equal(bits(yb), bits(host(lib.qgemv_q4_0(dwb, dx, n, k)))), tag
            assert_close(ya, oracle.decode_q4_0(wa, n, k), x, tag)
            assert_close(yb, oracle.decode_q4_0(wb, n, k), x, tag)
        elif fmt == "multi":
            ns = (n, max(1, n // 3), 17)
            ws, x = synth.q4_k_multi_case(seed, m, ns, k)
            dws = [at_offset(ws[0], off), at_offset(ws[1], 0), at_offset(ws[2], 16)]
            dx = dev(x)
            y = host(lib.qgemv_q4_k_multi(dws, dx, list(ns), k))
            col = 0
            for w, dw, nn in zip(ws, dws, ns):
                single = host(lib.qgemv_q4_k(dw, dx, nn, k))
                assert np.array_equal(bits(y[:, col:col + nn]), bits(single)), tag
                assert_close(single, oracle.decode_q4_k(w, nn, k), x, tag)
                col += nn
        else:
            x, q, s, b = synth.affine_case(seed, m, n, k, gs)
            dx, ds, db = dev(x), dev(s), dev(b)
            w64 = oracle.decode_affine(q, s, b, n, k, gs)
            if fmt == "affine":
                y = host(lib.qmm_affine_t(dx, at_offset(q, off).view(n, k), ds, db, gs))
                assert_close(y, w64, x, tag)
            else:
                wp = synth.pack_b4_u32(q)
                dwp = at_offset(wp, off)
                import torch
                dwp32 = dwp.view(torch.int32).view(n, k // 8)
                yp = host(lib.qmm_affine_t_packed(dx, dwp32, ds, db, gs))
                yu = host(lib.qmm_affine_t(dx, dev(q), ds, db, gs))
                assert_close(yp, w64, x, tag)
                # same codes, same settings: the packed and u8 paths take the
                # same kernel when both are aligned for it
                if off % 16 == 0:
                    assert np.array_equal(bits(yp), bits(yu)), tag
