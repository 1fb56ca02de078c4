"""CPU oracle for the 4-bit dequantize-fused GEMV / skinny-GEMM family.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the HIP library (``gemm_qgemv_q4_amd``) and imports nothing from it.

What it computes, and where the pages define it:

* Every product is ``y[m, n] = sum_k x[m, k] * w[n, k]`` where ``w`` is the
  dequantized weight; the weights are decoded to f64 from the packed bytes,
  the dot products are taken in f64 and the result is rounded to f32 once.
  This follows the f64 CPU reference ``qmm_affine_t_cpu`` in the tests of
  mlx-native ``qmm_affine.rs`` (dequantize ``q*s + b`` in f64, accumulate in
  f64, cast to f32 at the end); the same plain definition is used for the two
  GGML block formats.
* ``block_q4_0``: fp16 ``d`` then 16 nibble bytes, value ``(nibble - 8) * d``
  (mlx-native ``fused_dual_proj_q4_0.rs``, preconditions of
  ``dispatch_fused_dual_proj_q4_0``: an fp16 scale followed by 16 bytes of
  nibbles).  Which nibble is which element is not on the pages; the reading
  used here is the low nibble of byte j for element j and the high nibble for
  element j+16.
* ``block_q4_K``: 144 bytes per 256 weights, row-major ``[N][K/256]``
  (ferrum-kernels ``q4_k_gemv_v2.rs``, module doc and ``nb01``).  The field
  layout is not on the pages; the reading used is the GGML ``block_q4_K``
  layout written out below.
* The fused dual projection equals two single Q4_0 products
  (mlx-native ``fused_dual_proj_q4_0.rs``, module doc: what the kernel computes).
* ``qkv_split_f32`` copies columns ``[0,q_sp)``, ``[q_sp,q_sp+k_sp)`` and
  ``[q_sp+k_sp, qkv_ch)`` of each token row into q, k, v
  (mlx-native ``qkv_split.rs``, module doc and ``dispatch_qkv_split_f32``).
* Packed 4-bit affine codes: eight codes per u32 word, the code of element
  ``8*kp + j`` in bits ``4j .. 4j+3`` of word ``kp`` (mlx-native
  ``qmm_affine.rs``, the ``pack_b4_to_u32`` helper of its tests); the product
  is the affine one of the unpacked codes (the byte-identity test of the
  packed kernel against the unpacked one on the same page).
* Multi-part projections: several weight tensors of one format share x and
  each writes a disjoint column slice of one output (ferrum-kernels
  ``q4_k_gemv_v2.rs``, doc of ``dispatch_gemv_q4k_v2_offset``: the parts of a
  fused projection written into slices of a shared output buffer).
* The fused projection + split: the affine product of a fused q|k|v weight,
  split as ``qkv_split_f32`` splits it (mlx-native ``qkv_split.rs``, module
  doc: the split follows the fused-QKV projection).

Pins (tests/test_oracle_pins.py) tie each function to hand-decoded blocks
under tests/golden/, closed forms, exact rational brute force and the
quantize-then-decode round trip.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "f16_bits_to_f64", "decode_q4_0", "decode_q4_k", "decode_affine",
    "gemv_f64", "abs_bound", "qgemv_q4_0", "qgemv_q4_k", "qgemv_dual_q4_0",
    "qmm_affine_t", "qkv_split_f32", "q4k_scale_min",
    "unpack_b4_u32", "decode_affine_b4", "qmm_affine_t_packed",
    "qgemv_multi", "qmm_affine_t_qkv",
]


def f16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """IEEE binary16 bit patterns (uint16) -> f64, subnormals included (exact)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def _le16(lo: np.ndarray, hi: np.ndarray) -> np.ndarray:
    return lo.astype(np.uint16) | (hi.astype(np.uint16) << 8)


def decode_q4_0(w: np.ndarray, n: int, k: int) -> np.ndarray:
    """Packed ``block_q4_0`` rows (uint8 ``[n, k/32*18]``) -> f64 ``[n, k]``.

    Per block: ``d`` = fp16 at bytes 0..1 (little endian); byte ``2+j`` holds
    element ``j`` in its low nibble and element ``j+16`` in its high nibble;
    value = ``(nibble - 8) * d``.
    """
    assert k % 32 == 0
    blk = np.asarray(w, dtype=np.uint8).reshape(n, k // 32, 18)
    d = f16_bits_to_f64(_le16(blk[..., 0], blk[..., 1]))
    qs = blk[..., 2:18].astype(np.int64)
    nib = np.concatenate([qs & 0x0F, qs >> 4], axis=-1)  # elements 0..15, 16..31
    return ((nib - 8).astype(np.float64) * d[..., None]).reshape(n, k)


def q4k_scale_min(scales12: np.ndarray):
    """Unpack the 12 scale bytes of a ``block_q4_K`` into (sc[8], m[8]) integers.

    For sub-block j < 4 the 6-bit scale is the low 6 bits of byte j and the
    6-bit min is the low 6 bits of byte j+4.  For j >= 4 the low 4 bits come
    from byte j+4 (scale: low nibble, min: high nibble) and the top 2 bits from
    bits 6..7 of byte j-4 (scale) or byte j (min).
    """
    s = np.asarray(scales12, dtype=np.int64)
    sc = np.empty(s.shape[:-1] + (8,), dtype=np.int64)
    mn = np.empty_like(sc)
    for j in range(8):
        if j < 4:
            sc[..., j] = s[..., j] & 63
            mn[..., j] = s[..., j + 4] & 63
        else:
            sc[..., j] = (s[..., j + 4] & 0x0F) | ((s[..., j - 4] >> 6) << 4)
            mn[..., j] = (s[..., j + 4] >> 4) | ((s[..., j] >> 6) << 4)
    return sc, mn


def decode_q4_k(w: np.ndarray, n: int, k: int) -> np.ndarray:
    """Packed ``block_q4_K`` rows (uint8 ``[n, k/256*144]``) -> f64 ``[n, k]``.

    Per super-block: fp16 ``d`` @0, fp16 ``dmin`` @2, 12 scale bytes @4, 128
    nibble bytes @16.  Nibble bytes come in 4 chunks of 32: the low nibble of
    ``qs[32c + l]`` is element ``64c + l`` (sub-block 2c), the high nibble is
    element ``64c + 32 + l`` (sub-block 2c+1).  Value of an element in
    sub-block j: ``d * sc[j] * q - dmin * m[j]``.
    """
    assert k % 256 == 0
    sb = np.asarray(w, dtype=np.uint8).reshape(n, k // 256, 144)
    d = f16_bits_to_f64(_le16(sb[..., 0], sb[..., 1]))
    dmin = f16_bits_to_f64(_le16(sb[..., 2], sb[..., 3]))
    sc, mn = q4k_scale_min(sb[..., 4:16])
    qs = sb[..., 16:144].astype(np.int64).reshape(n, k // 256, 4, 32)
    q = np.concatenate([qs & 0x0F, qs >> 4], axis=-1).reshape(n, k // 256, 8, 32)
    val = (d[..., None, None] * sc[..., None].astype(np.float64) * q.astype(np.float64)
           - dmin[..., None, None] * mn[..., None].astype(np.float64))
    return val.reshape(n, k)


def decode_affine(q: np.ndarray, scales: np.ndarray, biases: np.ndarray,
                  n: int, k: int, group_size: int) -> np.ndarray:
    """u8 codes ``[n, k]`` with f32 ``scales``/``biases`` ``[n, k/gs]`` -> f64
    ``w = q * s + b`` (mlx-native ``qmm_affine.rs``, ``qmm_affine_t_cpu``)."""
    assert k % group_size == 0
    qq = np.asarray(q, dtype=np.uint8).reshape(n, k).astype(np.float64)
    s = np.asarray(scales, dtype=np.float32).reshape(n, k // group_size).astype(np.float64)
    b = np.asarray(biases, dtype=np.float32).reshape(n, k // group_size).astype(np.float64)
    s_full = np.repeat(s, group_size, axis=1)
    b_full = np.repeat(b, group_size, axis=1)
    return qq * s_full + b_full


def gemv_f64(w64: np.ndarray, x: np.ndarray) -> np.ndarray:
    """``y[m, n] = sum_k x[m, k] * w[n, k]`` in f64, rounded once to f32."""
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    return (x64 @ w64.T).astype(np.float32)


def abs_bound(w64: np.ndarray, x: np.ndarray) -> np.ndarray:
    """``sum_k |x[m, k] * w[n, k]|`` in f64: the scale of the parity tolerance."""
    x64 = np.abs(np.asarray(x, dtype=np.float32).astype(np.float64))
    return x64 @ np.abs(w64).T


def qgemv_q4_0(w: np.ndarray, x: np.ndarray, m: int, n: int, k: int) -> np.ndarray:
    """f32 ``y[m, n]`` for Q4_0 weights ``[n][k/32]`` and f32 ``x[m, k]``."""
    return gemv_f64(decode_q4_0(w, n, k), np.asarray(x).reshape(m, k))


def qgemv_q4_k(w: np.ndarray, x: np.ndarray, m: int, n: int, k: int) -> np.ndarray:
    """f32 ``y[m, n]`` for Q4_K weights ``[n][k/256]`` and f32 ``x[m, k]``."""
    return gemv_f64(decode_q4_k(w, n, k), np.asarray(x).reshape(m, k))


def qgemv_dual_q4_0(w_a: np.ndarray, w_b: np.ndarray, x: np.ndarray,
                    m: int, n: int, k: int):
    """Two single Q4_0 products sharing ``x`` (the dual projection's contract)."""
    return qgemv_q4_0(w_a, x, m, n, k), qgemv_q4_0(w_b, x, m, n, k)


def qmm_affine_t(x: np.ndarray, q: np.ndarray, scales: np.ndarray, biases: np.ndarray,
                 m: int, n: int, k: int, group_size: int) -> np.ndarray:
    """f32 ``y = x * (s*q + b)^T`` with the weights dequantized in f64."""
    return gemv_f64(decode_affine(q, scales, biases, n, k, group_size),
                    np.asarray(x).reshape(m, k))


def qkv_split_f32(qkv: np.ndarray, seq: int, q_sp: int, k_sp: int, v_sp: int):
    """Split ``qkv[seq, q_sp+k_sp+v_sp]`` into contiguous q, k, v (bit copies)."""
    a = np.asarray(qkv, dtype=np.float32).reshape(seq, q_sp + k_sp + v_sp)
    return (np.ascontiguousarray(a[:, :q_sp]),
            np.ascontiguousarray(a[:, q_sp:q_sp + k_sp]),
            np.ascontiguousarray(a[:, q_sp + k_sp:]))


def unpack_b4_u32(w_packed: np.ndarray, n: int, k: int) -> np.ndarray:
    """u32 words ``[n, k/8]`` -> u8 codes ``[n, k]``: element ``8*kp + j`` is
    bits ``4j .. 4j+3`` of word ``kp`` (low nibble first)."""
    assert k % 8 == 0
    wp = np.asarray(w_packed, dtype=np.uint32).reshape(n, k // 8)
    out = np.empty((n, k // 8, 8), dtype=np.uint8)
    for j in range(8):
        out[..., j] = (wp >> np.uint32(4 * j)) & np.uint32(0xF)
    return out.reshape(n, k)


def decode_affine_b4(w_packed: np.ndarray, scales: np.ndarray, biases: np.ndarray,
                     n: int, k: int, group_size: int) -> np.ndarray:
    """Packed 4-bit affine weights -> f64 ``w = q * s + b``."""
    return decode_affine(unpack_b4_u32(w_packed, n, k), scales, biases, n, k, group_size)


def qmm_affine_t_packed(x: np.ndarray, w_packed: np.ndarray, scales: np.ndarray,
                        biases: np.ndarray, m: int, n: int, k: int, group_size: int) -> np.ndarray:
    """f32 ``y = x * (s*q + b)^T`` with the codes packed eight per u32."""
    return gemv_f64(decode_affine_b4(w_packed, scales, biases, n, k, group_size),
                    np.asarray(x).reshape(m, k))


def qgemv_multi(decode, parts, x: np.ndarray, m: int, k: int) -> np.ndarray:
    """Multi-part projection: ``parts`` is a list of ``(w_p, n_p)`` in one
    format, ``decode(w, n, k)`` its decoder.  Returns f32 ``y[m, sum n_p]``
    with part p in columns ``[sum_{q<p} n_q, sum_{q<=p} n_q)``."""
    xm = np.asarray(x).reshape(m, k)
    return np.concatenate([gemv_f64(decode(w, n, k), xm) for w, n in parts], axis=1)


def qmm_affine_t_qkv(x: np.ndarray, q: np.ndarray, scales: np.ndarray, biases: np.ndarray,
                     m: int, k: int, group_size: int, q_sp: int, k_sp: int, v_sp: int):
    """The affine product of a fused ``[q_sp + k_sp + v_sp, k]`` weight, split
    into contiguous q ``[m, q_sp]``, k ``[m, k_sp]``, v ``[m, v_sp]``."""
    n = q_sp + k_sp + v_sp
    y = qmm_affine_t(x, q, scales, biases, m, n, k, group_size)
    return qkv_split_f32(y, m, q_sp, k_sp, v_sp)
