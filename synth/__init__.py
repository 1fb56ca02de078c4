"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks.

This module only *produces* inputs: random f32 tensors and the packed 4-bit
weight encodings made from them.  It holds no decoding and no products; the
oracle (``oracle/``) and the HIP library (``gemm_qgemv_q4_amd``) each decode
the bytes written here with code of their own.

Encodings written here (byte layouts; where the pages are silent these are
readings of them, the same ones the oracle uses):

* ``block_q4_0`` -- 18 bytes per 32 weights: little-endian fp16 ``d`` then 16
  bytes ``qs``; the low nibble of ``qs[j]`` is element ``j``, the high nibble is
  element ``j+16``; the value is ``(nibble - 8) * d``
  (mlx-native ``fused_dual_proj_q4_0.rs``, dispatch preconditions).
* ``block_q4_K`` -- 144 bytes per 256 weights: fp16 ``d``, fp16 ``dmin``, 12
  bytes of packed 6-bit sub-block scales and mins, 128 bytes of nibbles
  (ferrum-kernels ``q4_k_gemv_v2.rs``, module doc and ``nb01``).
* MLX-style affine groups -- u8 codes ``[N, K]`` plus f32 ``scales`` and
  ``biases`` ``[N, K/group_size]`` (mlx-native ``qmm_affine.rs``, CPU oracle in
  the tests module).
* Packed 4-bit affine codes -- u32 ``[N, K/8]``, the code of element
  ``8*kp + j`` in bits ``4j .. 4j+3`` of word ``kp`` (mlx-native
  ``qmm_affine.rs``, the ``pack_b4_to_u32`` test helper).

Quantizers are plain input generators: any code assignment is a valid input,
so their rounding choices do not affect parity.
"""
from __future__ import annotations

import numpy as np

QK4_0 = 32
BLOCK_Q4_0_BYTES = 18
QK_K = 256
BLOCK_Q4_K_BYTES = 144


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def normal_f32(g: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    """Draw N(0, std^2) in f64 and cast to f32."""
    return (g.standard_normal(size=shape) * std).astype(np.float32)


# ---------------------------------------------------------------- Q4_0
def quantize_q4_0(w: np.ndarray) -> np.ndarray:
    """Encode f32 ``w[N, K]`` (K % 32 == 0) into ``uint8[N, K/32*18]``.

    Per block: ``amax`` is the element of largest magnitude with its sign,
    ``d32 = amax / -8``, ``d = fp16(d32)`` (round to nearest even), and
    ``q = clamp(floor(w / d32 + 8.5), 0, 15)``.  An all-zero block gets d = 0
    and q = 8.
    """
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    assert k % QK4_0 == 0
    blk = w.reshape(n, k // QK4_0, QK4_0).astype(np.float64)
    idx = np.argmax(np.abs(blk), axis=2)
    amax = np.take_along_axis(blk, idx[..., None], axis=2)[..., 0]
    d32 = np.where(amax == 0, 0.0, amax / -8.0)
    d16 = d32.astype(np.float16)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(d32[..., None] != 0, blk / d32[..., None], 0.0)
    q = np.clip(np.floor(t + 8.5), 0, 15).astype(np.uint8)
    out = np.empty((n, k // QK4_0, BLOCK_Q4_0_BYTES), dtype=np.uint8)
    out[..., 0:2] = d16.view(np.uint8).reshape(n, k // QK4_0, 2)
    out[..., 2:] = q[..., :16] | (q[..., 16:] << 4)
    return out.reshape(n, k // QK4_0 * BLOCK_Q4_0_BYTES)


# ---------------------------------------------------------------- Q4_K
def _pack_q4k_scales(sc: np.ndarray, mn: np.ndarray) -> np.ndarray:
    """Pack 8 six-bit scales and 8 six-bit mins per super-block into 12 bytes.

    Bytes 0..3 hold scales 0..3 in their low 6 bits and the top two bits of
    scales 4..7 in bits 6..7; bytes 4..7 do the same for mins; bytes 8..11
    hold the low nibbles of scale 4+i (bits 0..3) and min 4+i (bits 4..7).
    """
    sc = sc.astype(np.uint8)
    mn = mn.astype(np.uint8)
    out = np.zeros(sc.shape[:-1] + (12,), dtype=np.uint8)
    for i in range(4):
        out[..., i] = (sc[..., i] & 63) | ((sc[..., i + 4] >> 4) << 6)
        out[..., i + 4] = (mn[..., i] & 63) | ((mn[..., i + 4] >> 4) << 6)
        out[..., i + 8] = (sc[..., i + 4] & 15) | ((mn[..., i + 4] & 15) << 4)
    return out


def quantize_q4_k(w: np.ndarray) -> np.ndarray:
    """Encode f32 ``w[N, K]`` (K % 256 == 0) into ``uint8[N, K/256*144]``.

    A plain min/max quantizer (not an iterative search): per 32-element
    sub-block ``mn = max(0, -min w)`` and ``scf = (max w + mn) / 15``; per
    super-block ``d = fp16(max scf / 63)`` and ``dmin = fp16(max mn / 63)``;
    ``sc = clamp(round(scf/d), 0, 63)``, ``m = clamp(round(mn/dmin), 0, 63)``
    and ``q = clamp(round((w + dmin*m) / (d*sc)), 0, 15)``.
    """
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    assert k % QK_K == 0
    nsb = k // QK_K
    sub = w.reshape(n, nsb, 8, 32).astype(np.float64)
    mn = np.maximum(0.0, -sub.min(axis=3))
    scf = (sub.max(axis=3) + mn) / 15.0
    d = (scf.max(axis=2) / 63.0).astype(np.float16)
    dmin = (mn.max(axis=2) / 63.0).astype(np.float16)
    d64 = d.astype(np.float64)[..., None]
    dm64 = dmin.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        sc = np.where(d64 > 0, np.rint(scf / d64), 0.0)
        m = np.where(dm64 > 0, np.rint(mn / dm64), 0.0)
    sc = np.clip(sc, 0, 63)
    m = np.clip(m, 0, 63)
    step = d64 * sc
    off = dm64 * m
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(step[..., None] > 0,
                     np.rint((sub + off[..., None]) / step[..., None]), 0.0)
    q = np.clip(q, 0, 15).astype(np.uint8).reshape(n, nsb, 256)
    out = np.empty((n, nsb, BLOCK_Q4_K_BYTES), dtype=np.uint8)
    out[..., 0:2] = d.view(np.uint8).reshape(n, nsb, 2)
    out[..., 2:4] = dmin.view(np.uint8).reshape(n, nsb, 2)
    out[..., 4:16] = _pack_q4k_scales(sc.astype(np.uint8), m.astype(np.uint8))
    qc = q.reshape(n, nsb, 4, 64)
    out[..., 16:] = (qc[..., :32] | (qc[..., 32:] << 4)).reshape(n, nsb, 128)
    return out.reshape(n, nsb * BLOCK_Q4_K_BYTES)


# ---------------------------------------------------------------- affine
def affine_weights(g: np.random.Generator, n: int, k: int, group_size: int,
                   code_max: int = 15):
    """u8 codes uniform in [0, code_max], scales ~ U(0.001, 0.01), biases ~ N(0, 0.02)."""
    q = g.integers(0, code_max + 1, size=(n, k), dtype=np.uint8)
    s = g.uniform(0.001, 0.01, size=(n, k // group_size)).astype(np.float32)
    b = normal_f32(g, (n, k // group_size), 0.02)
    return q, s, b


# ---------------------------------------------------------------- workloads
def q4_0_case(seed: int, m: int, n: int, k: int):
    g = rng(seed)
    w = normal_f32(g, (n, k), 0.02)
    x = normal_f32(g, (m, k))
    return quantize_q4_0(w), x


def q4_k_case(seed: int, m: int, n: int, k: int):
    g = rng(seed)
    w = normal_f32(g, (n, k), 0.02)
    x = normal_f32(g, (m, k))
    return quantize_q4_k(w), x


def dual_q4_0_case(seed: int, m: int, n: int, k: int):
    g = rng(seed)
    wa = normal_f32(g, (n, k), 0.02)
    wb = normal_f32(g, (n, k), 0.02)
    x = normal_f32(g, (m, k))
    return quantize_q4_0(wa), quantize_q4_0(wb), x


def affine_case(seed: int, m: int, n: int, k: int, group_size: int, code_max: int = 15):
    g = rng(seed)
    q, s, b = affine_weights(g, n, k, group_size, code_max)
    x = normal_f32(g, (m, k))
    return x, q, s, b


def pack_b4_u32(codes: np.ndarray) -> np.ndarray:
    """u8 codes ``[N, K]`` (each 0..15, K % 8 == 0) -> u32 ``[N, K/8]``."""
    c = np.asarray(codes, dtype=np.uint32)
    n, k = c.shape
    assert k % 8 == 0 and int(c.max(initial=0)) <= 15
    c = c.reshape(n, k // 8, 8)
    out = np.zeros((n, k // 8), dtype=np.uint32)
    for j in range(8):
        out |= c[..., j] << np.uint32(4 * j)
    return out


def q4_k_multi_case(seed: int, m: int, ns, k: int):
    """One Q4_K weight per part (rows ``ns[p]``), then x ``[m, k]``."""
    g = rng(seed)
    ws = [quantize_q4_k(normal_f32(g, (n, k), 0.02)) for n in ns]
    x = normal_f32(g, (m, k))
    return ws, x


def qkv_payload(seq: int, q_sp: int, k_sp: int, v_sp: int) -> np.ndarray:
    """f32 [seq, q_sp+k_sp+v_sp] whose elements are distinct integers (exact in f32
    up to 2^24 elements), so every output element names its source position."""
    ch = q_sp + k_sp + v_sp
    assert seq * ch < (1 << 24)
    return np.arange(seq * ch, dtype=np.float32).reshape(seq, ch)


# The five workloads the benchmark and the full-size parity tests use.
CONFIGS = {
    "q4_0_gemv_1024": dict(kind="q4_0", seed=101, m=1, n=1024, k=1024),
    "q4_k_gemv_4096": dict(kind="q4_k", seed=102, m=1, n=4096, k=4096),
    "dual_q4_0_4096": dict(kind="dual_q4_0", seed=103, m=8, n=4096, k=4096),
    "affine_12288x4096_gs64": dict(kind="affine", seed=104, m=8, n=12288, k=4096, gs=64),
    "prefill_qkv_512x2048": dict(kind="prefill", seed=105, m=512, n=8192, k=2048, gs=64,
                                 q_sp=2048, k_sp=2048, v_sp=4096),
}


# Workloads of the follow-on paths (multi-part Q4_K decode projection, packed
# 4-bit affine GEMV, Q4_0 prefill on the matrix cores); the fused projection +
# split reuses "prefill_qkv_512x2048" above.
NEXT_CONFIGS = {
    "q4_k_qkv_multi_4096": dict(kind="q4_k_multi", seed=106, m=1, ns=(4096, 1024, 1024), k=4096),
    "affine_b4_12288x4096_gs64": dict(kind="affine_b4", seed=107, m=8, n=12288, k=4096, gs=64),
    "q4_0_prefill_512x4096": dict(kind="q4_0", seed=108, m=512, n=4096, k=4096),
}


# ---------------------------------------------------------------- device-side
# Inputs too large to build on the host (weights beyond 2 GiB): random bytes
# drawn on the GPU with a seeded torch generator.  Only the byte patterns are
# chosen here; no value is decoded.

def q4_0_random_device(seed: int, n: int, k: int, device: str = "cuda"):
    """block_q4_0 rows [n][k/32] with random nibbles and fp16 d in [2^-6, 2^-5)
    (exponent field 9, random mantissa), as a flat uint8 tensor on `device`."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    blocks = n * (k // QK4_0)
    w = torch.randint(0, 256, (blocks, BLOCK_Q4_0_BYTES), dtype=torch.uint8, device=device, generator=gen)
    w[:, 1] = (w[:, 1] & 0x03) | 0x24  # fp16 high byte: sign 0, exponent 01001
    return w.view(-1)


def affine_random_device(seed: int, n: int, k: int, group_size: int, device: str = "cuda"):
    """u8 codes [n, k] in 0..15 and f32 scales, biases [n, k/group_size] with
    scale ~ U(0.001, 0.01) and bias ~ N(0, 0.02), on `device`."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    q = torch.randint(0, 16, (n, k), dtype=torch.uint8, device=device, generator=gen)
    g = k // group_size
    s = torch.rand((n, g), dtype=torch.float32, device=device, generator=gen) * 0.009 + 0.001
    b = torch.randn((n, g), dtype=torch.float32, device=device, generator=gen) * 0.02
    return q, s, b
