"""Weights beyond 2 GiB: every byte offset into the weights is 64-bit, so rows
past the 2^31-byte mark decode and multiply like the first ones.  The oracle
checks a sample of rows (the first ones, rows around the middle and rows whose
bytes lie past 2^31) against the same f64 definition as everywhere else:
    max |y_gpu - y_oracle| / sum_k |x[m,k] w[n,k]|  <=  1e-5
Inputs are drawn on the GPU (they do not fit the host comfortably); the oracle
decodes the sampled rows' bytes copied back from the device."""
import numpy as np
import pytest

import oracle
import synth
from test_gpu_parity import assert_close, dev, host

pytestmark = pytest.mark.gpu

LIMIT = 1 << 31


def sample_rows(n, row_bytes):
    first_beyond = LIMIT // row_bytes + 1  # the first row that starts past 2^31 bytes
    rows = {0, 1, 2, n // 2, n // 2 + 1, first_beyond - 1, first_beyond, first_beyond + 1, n - 2, n - 1}
    rows |= set(np.random.Generator(np.random.PCG64(5)).integers(0, n, 22).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < n), dtype=np.int64)


def test_q4_0_weights_beyond_2gib(lib):
    import torch
    k = 1024
    row_bytes = (k // 32) * 18
    n = LIMIT // row_bytes + 80_000  # 2.19 GB of weights
    print(f"q4_0 M=1 N={n} K={k}: {n * row_bytes / 1e9:.2f} GB", flush=True)
    w = synth.q4_0_random_device(901, n, k)
    x = synth.normal_f32(synth.rng(902), (1, k))
    y = host(lib.qgemv_q4_0(w, dev(x), n, k))
    rows = sample_rows(n, row_bytes)
    wr = w.view(n, row_bytes)[torch.from_numpy(rows).cuda()].cpu().numpy()
    assert_close(y[:, rows], oracle.decode_q4_0(wr.reshape(-1), len(rows), k), x, "q4_0 > 2 GiB")
    del w
    torch.cuda.empty_cache()


def test_affine_codes_beyond_2gib(lib):
    import torch
    k, gs = 4096, 64
    n = LIMIT // k + 20_000  # 2.28 GB of u8 codes
    print(f"affine M=2 N={n} K={k} gs={gs}: {n * k / 1e9:.2f} GB of codes", flush=True)
    q, s, b = synth.affine_random_device(903, n, k, gs)
    x = synth.normal_f32(synth.rng(904), (2, k))
    y = host(lib.qmm_affine_t(dev(x), q, s, b, gs))
    rows = torch.from_numpy(sample_rows(n, k)).cuda()
    dec = oracle.decode_affine(q[rows].cpu().numpy(), s[rows].cpu().numpy(), b[rows].cpu().numpy(), len(rows), k, gs)
    assert_close(y[:, rows.cpu().numpy()], dec, x, "affine > 2 GiB")
    del q, s, b
    torch.cuda.empty_cache()
