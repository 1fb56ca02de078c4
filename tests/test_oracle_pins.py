"""Pins for the CPU oracle: hand-decoded blocks, textbook values, closed forms,
exact rational brute force and the quantize -> decode round trip.

Each test checks the oracle against something other than itself, so that a
dropped term, a wrong sign or index, a swapped nibble or a transposed operand
fails at least one of them.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from conftest import GOLDEN


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ------------------------------------------------------------- fp16 values
def test_f16_textbook_values():
    fx = _load("f16_values.json")
    for hx, val in fx["pairs"]:
        got = oracle.f16_bits_to_f64(np.array([int(hx, 16)], dtype=np.uint16))[0]
        assert got == val and np.signbit(got) == np.signbit(val), (hx, got, val)


# ------------------------------------------------------------- Q4_0
def test_q4_0_hand_block():
    fx = _load("q4_0_hand_block.json")
    w = np.frombuffer(bytes.fromhex(fx["bytes_hex"]), dtype=np.uint8)[None, :]
    dec = oracle.decode_q4_0(w, 1, 32)[0]
    expect = np.zeros(32)
    for i, v in fx["nonzero"].items():
        expect[int(i)] = v
    assert np.array_equal(dec, expect)
    ones = np.ones((1, 32), np.float32)
    ar = np.arange(32, dtype=np.float32)[None, :]
    assert oracle.qgemv_q4_0(w, ones, 1, 1, 32)[0, 0] == fx["y_ones"]
    assert oracle.qgemv_q4_0(w, ar, 1, 1, 32)[0, 0] == fx["y_arange"]


def test_q4_0_all_0x88_block_is_zero():
    blk = np.array([0x00, 0x3C] + [0x88] * 16, dtype=np.uint8)[None, :]
    assert np.array_equal(oracle.decode_q4_0(blk, 1, 32), np.zeros((1, 32)))


def test_q4_0_is_affine_with_group_32():
    """A Q4_0 block is an affine group of 32 with s = d and b = -8 d (the page's
    affine definition, mlx-native qmm_affine.rs); codes taken straight from the
    bytes here."""
    g = synth.rng(7)
    n, k = 5, 96
    w = g.integers(0, 256, size=(n, k // 32 * 18), dtype=np.uint8)
    blk = w.reshape(n, k // 32, 18)
    blk[..., 1] &= 0x3B  # keep d finite
    d = blk[..., 0:2].copy().view(np.float16)[..., 0].astype(np.float32)
    qs = blk[..., 2:].astype(np.uint8)
    codes = np.concatenate([qs & 15, qs >> 4], axis=-1).reshape(n, k)
    via_affine = oracle.decode_affine(codes, d, -8 * d, n, k, 32)
    assert np.array_equal(oracle.decode_q4_0(w, n, k), via_affine)


def test_q4_0_quantize_roundtrip():
    g = synth.rng(11)
    n, k = 16, 256
    w = synth.normal_f32(g, (n, k), 0.02)
    packed = synth.quantize_q4_0(w)
    assert packed.shape == (n, k // 32 * 18)
    dec = oracle.decode_q4_0(packed, n, k)
    d = np.abs(packed.reshape(n, k // 32, 18)[..., 0:2].copy().view(np.float16)[..., 0]
               .astype(np.float64))
    err = np.abs(dec - w.astype(np.float64)).reshape(n, k // 32, 32)
    assert np.all(err <= 1.01 * d[..., None] + 1e-12)
    assert np.sqrt(np.mean(err ** 2)) < 0.2 * np.sqrt(np.mean(w.astype(np.float64) ** 2))


def test_q4_0_zero_block_quantizes_to_code_8():
    packed = synth.quantize_q4_0(np.zeros((1, 32), np.float32))
    assert packed[0, 0] == 0 and packed[0, 1] == 0
    assert np.all(packed[0, 2:] == 0x88)


# ------------------------------------------------------------- Q4_K
def test_q4_k_hand_block():
    fx = _load("q4_k_hand_block.json")
    w = np.frombuffer(bytes.fromhex(fx["bytes_hex"]), dtype=np.uint8)[None, :]
    sc, mn = oracle.q4k_scale_min(w[:, 4:16])
    assert sc[0].tolist() == fx["sc"] and mn[0].tolist() == fx["m"]
    dec = oracle.decode_q4_k(w, 1, 256)[0]
    for i, v in fx["values"].items():
        assert dec[int(i)] == v, (i, dec[int(i)], v)
    ones = np.ones((1, 256), np.float32)
    assert oracle.qgemv_q4_k(w, ones, 1, 1, 256)[0, 0] == fx["y_ones"]


def test_q4_k_is_affine_with_group_32():
    """Each Q4_K sub-block is an affine group of 32 with s = d*sc and b = -dmin*m."""
    g = synth.rng(8)
    n, k = 3, 512
    w = g.integers(0, 256, size=(n, k // 256 * 144), dtype=np.uint8)
    sb = w.reshape(n, k // 256, 144)
    sb[..., 1] &= 0x3B
    sb[..., 3] &= 0x3B
    d = sb[..., 0:2].copy().view(np.float16)[..., 0].astype(np.float64)
    dmin = sb[..., 2:4].copy().view(np.float16)[..., 0].astype(np.float64)
    sc, mn = oracle.q4k_scale_min(sb[..., 4:16])
    qs = sb[..., 16:].reshape(n, k // 256, 4, 32)
    codes = np.concatenate([qs & 15, qs >> 4], axis=-1).reshape(n, k)
    s = (d[..., None] * sc).reshape(n, k // 32).astype(np.float32)
    b = (-dmin[..., None] * mn).reshape(n, k // 32).astype(np.float32)
    # d*sc and dmin*m are exact in f32 (11-bit x 6-bit significands)
    assert np.array_equal(s.astype(np.float64), (d[..., None] * sc).reshape(n, k // 32))
    via_affine = oracle.decode_affine(codes, s, b, n, k, 32)
    assert np.array_equal(oracle.decode_q4_k(w, n, k), via_affine)


def test_q4_k_scale_packing_roundtrip_all_values():
    """Every 6-bit (scale, min) pair survives the 12-byte packing of the generator."""
    vals = np.arange(64, dtype=np.uint8)
    for rot in range(8):
        sc = np.roll(vals, rot)[:8][None, :]
        mn = np.roll(vals[::-1], rot)[:8][None, :]
        for base in range(0, 64, 8):
            sc_b = (sc + base) % 64
            mn_b = (mn + 3 * base) % 64
            packed = synth._pack_q4k_scales(sc_b, mn_b)
            s2, m2 = oracle.q4k_scale_min(packed)
            assert np.array_equal(s2, sc_b.astype(np.int64))
            assert np.array_equal(m2, mn_b.astype(np.int64))


def test_q4_k_quantize_roundtrip():
    g = synth.rng(12)
    n, k = 8, 512
    w = synth.normal_f32(g, (n, k), 0.02)
    packed = synth.quantize_q4_k(w)
    assert packed.shape == (n, k // 256 * 144)
    dec = oracle.decode_q4_k(packed, n, k)
    sb = packed.reshape(n, k // 256, 144)
    d = sb[..., 0:2].copy().view(np.float16)[..., 0].astype(np.float64)
    dmin = sb[..., 2:4].copy().view(np.float16)[..., 0].astype(np.float64)
    sc, _ = oracle.q4k_scale_min(sb[..., 4:16])
    step = (d[..., None] * sc)[..., None]  # [n, nsb, 8, 1]
    err = np.abs(dec - w.astype(np.float64)).reshape(n, k // 256, 8, 32)
    assert np.all(err <= step + dmin[..., None, None] + 1e-9)
    assert np.sqrt(np.mean(err ** 2)) < 0.2 * np.sqrt(np.mean(w.astype(np.float64) ** 2))


# ------------------------------------------------------------- affine
def test_affine_hand():
    fx = _load("affine_hand.json")
    q = np.array(fx["q"], np.uint8)
    s = np.array(fx["scales"], np.float32)
    b = np.array(fx["biases"], np.float32)
    x = np.array(fx["x"], np.float32)
    n, k, gs = fx["n"], fx["k"], fx["group_size"]
    assert np.array_equal(oracle.decode_affine(q, s, b, n, k, gs), np.array(fx["w"]))
    assert np.array_equal(oracle.qmm_affine_t(x, q, s, b, 1, n, k, gs), np.array(fx["y"], np.float32))


def test_affine_constant_closed_form():
    g = synth.rng(3)
    m, n, k, gs = 3, 4, 128, 32
    x = synth.normal_f32(g, (m, k))
    q = np.full((n, k), 9, np.uint8)
    s = np.full((n, k // gs), 0.25, np.float32)
    b = np.full((n, k // gs), -1.5, np.float32)
    y = oracle.qmm_affine_t(x, q, s, b, m, n, k, gs)
    expect = (9 * 0.25 - 1.5) * x.astype(np.float64).sum(axis=1)
    assert np.allclose(y, np.repeat(expect[:, None], n, axis=1).astype(np.float32), rtol=0, atol=1e-6)


def test_affine_onehot_picks_group_of_column():
    g = synth.rng(4)
    n, k, gs = 6, 64, 8
    x, q, s, b = synth.affine_case(5, 1, n, k, gs, code_max=255)
    for col in (0, 7, 8, 37, 63):
        e = np.zeros((1, k), np.float32)
        e[0, col] = 1.0
        y = oracle.qmm_affine_t(e, q, s, b, 1, n, k, gs)[0]
        want = (q[:, col].astype(np.float64) * s[:, col // gs] + b[:, col // gs]).astype(np.float32)
        assert np.array_equal(y, want), col


# ------------------------------------------------------------- qkv split
def test_qkv_split_hand():
    fx = _load("qkv_split_hand.json")
    qkv = np.array(fx["qkv"], np.float32)
    q, k, v = oracle.qkv_split_f32(qkv, fx["seq"], fx["q_sp"], fx["k_sp"], fx["v_sp"])
    assert q.tolist() == fx["q"] and k.tolist() == fx["k"] and v.tolist() == fx["v"]


def test_qkv_split_reconstructs_with_distinct_payloads():
    seq, qs, ks, vs = 7, 12, 4, 20
    qkv = synth.qkv_payload(seq, qs, ks, vs)
    q, k, v = oracle.qkv_split_f32(qkv, seq, qs, ks, vs)
    assert q.shape == (seq, qs) and k.shape == (seq, ks) and v.shape == (seq, vs)
    assert np.array_equal(np.concatenate([q, k, v], axis=1).view(np.uint32), qkv.view(np.uint32))
    # every payload appears exactly once
    allv = np.concatenate([q.ravel(), k.ravel(), v.ravel()])
    assert np.array_equal(np.sort(allv), np.arange(seq * (qs + ks + vs), dtype=np.float32))


# ------------------------------------------------------------- products
@pytest.mark.parametrize("fmt", ["q4_0", "q4_k", "affine"])
def test_onehot_x_gives_decoded_column(fmt):
    """y(e_k)[n] = w[n, k]: catches a transposed operand in the product."""
    n, k = 7, 512
    if fmt == "q4_0":
        w, _ = synth.q4_0_case(21, 1, n, k)
        dec = oracle.decode_q4_0(w, n, k)
        f = lambda x: oracle.qgemv_q4_0(w, x, 1, n, k)
    elif fmt == "q4_k":
        w, _ = synth.q4_k_case(22, 1, n, k)
        dec = oracle.decode_q4_k(w, n, k)
        f = lambda x: oracle.qgemv_q4_k(w, x, 1, n, k)
    else:
        _, q, s, b = synth.affine_case(23, 1, n, k, 64)
        dec = oracle.decode_affine(q, s, b, n, k, 64)
        f = lambda x: oracle.qmm_affine_t(x, q, s, b, 1, n, k, 64)
    for col in (0, 1, 31, 32, 255, 256, 511):
        e = np.zeros((1, k), np.float32)
        e[0, col] = 1.0
        assert np.array_equal(f(e)[0], dec[:, col].astype(np.float32)), col


def _exact_q4_0_row(row_bytes, k):
    out = []
    for b in range(k // 32):
        blk = row_bytes[18 * b:18 * b + 18]
        d = Fraction(float(np.frombuffer(bytes(blk[0:2]), dtype=np.float16)[0]))
        vals = [0] * 32
        for j in range(16):
            vals[j] = (blk[2 + j] & 15) - 8
            vals[j + 16] = (blk[2 + j] >> 4) - 8
        out += [d * v for v in vals]
    return out


def test_bruteforce_fraction_q4_0():
    """Exact rational sums, rounded once to f32, equal the oracle's f32 output."""
    m, n, k = 3, 4, 64
    w, x = synth.q4_0_case(31, m, n, k)
    y = oracle.qgemv_q4_0(w, x, m, n, k)
    for r in range(m):
        for c in range(n):
            wv = _exact_q4_0_row(w[c].tolist(), k)
            exact = sum(Fraction(float(x[r, i])) * wv[i] for i in range(k))
            assert y[r, c] == np.float32(float(exact)), (r, c)


def test_bruteforce_fraction_affine():
    m, n, k, gs = 2, 3, 64, 16
    x, q, s, b = synth.affine_case(32, m, n, k, gs, code_max=255)
    y = oracle.qmm_affine_t(x, q, s, b, m, n, k, gs)
    for r in range(m):
        for c in range(n):
            exact = Fraction(0)
            for i in range(k):
                wv = Fraction(int(q[c, i])) * Fraction(float(s[c, i // gs])) + Fraction(float(b[c, i // gs]))
                exact += Fraction(float(x[r, i])) * wv
            assert y[r, c] == np.float32(float(exact)), (r, c)


def test_dual_is_two_singles():
    wa, wb, x = synth.dual_q4_0_case(41, 3, 8, 128)
    ya, yb = oracle.qgemv_dual_q4_0(wa, wb, x, 3, 8, 128)
    assert np.array_equal(ya, oracle.qgemv_q4_0(wa, x, 3, 8, 128))
    assert np.array_equal(yb, oracle.qgemv_q4_0(wb, x, 3, 8, 128))
    assert not np.array_equal(ya, yb)


def test_linearity_in_x():
    """y(2x) == 2 y(x) exactly (scaling by 2 is exact in every step)."""
    w, x = synth.q4_k_case(42, 2, 5, 256)
    y1 = oracle.qgemv_q4_k(w, x, 2, 5, 256)
    y2 = oracle.qgemv_q4_k(w, 2 * x, 2, 5, 256)
    assert np.array_equal(y2, 2 * y1)


def test_abs_bound_hand_worked():
    """bound = sum_k |x w| term by term, worked by hand (tests/golden/abs_bound_hand.json):
    a bound of |sum_k x w| (entry (0, 1): y = 0, bound 4), a transposed
    operand (shape [2, 3]) or a dropped |.| on either factor fails it."""
    fx = _load("abs_bound_hand.json")
    x = np.array(fx["x"], np.float32)
    w64 = np.array(fx["w"], np.float64)
    bound = oracle.abs_bound(w64, x)
    assert bound.shape == (2, 3)
    assert np.array_equal(bound, np.array(fx["bound"]))
    assert np.array_equal(oracle.gemv_f64(w64, x), np.array(fx["y"], np.float32))


def test_abs_bound_q4_0_zero_rows():
    """A Q4_0 row whose weights are all zero (codes 8 with d != 0, or d = 0)
    has bound 0 and product exactly 0; one code 9 gives bound = |y| = d x[k]."""
    fx = _load("abs_bound_hand.json")
    w = np.stack([np.frombuffer(bytes.fromhex(h), np.uint8) for h in fx["q4_0_rows_hex"]])
    x = (np.arange(64, dtype=np.float32) + 1)[None, :]
    w64 = oracle.decode_q4_0(w, 2, 64)
    assert np.array_equal(oracle.abs_bound(w64, x)[0], np.array(fx["q4_0_bound"]))
    y = oracle.qgemv_q4_0(w, x, 1, 2, 64)[0]
    assert np.array_equal(y, np.array(fx["q4_0_y"], np.float32))
    assert y[1] == 0.0 and not np.signbit(y[1])


def test_abs_bound_dominates_result():
    x, q, s, b = synth.affine_case(43, 2, 9, 128, 32)
    w64 = oracle.decode_affine(q, s, b, 9, 128, 32)
    y = oracle.qmm_affine_t(x, q, s, b, 2, 9, 128, 32)
    bound = oracle.abs_bound(w64, x)
    assert np.all(np.abs(y.astype(np.float64)) <= bound * (1 + 1e-6))
    assert np.all(bound > 0)


# ------------------------------------------------------------- packed 4-bit affine
def test_affine_b4_hand_words():
    fx = _load("affine_b4_hand.json")
    n, k, gs = fx["n"], fx["k"], fx["group_size"]
    wp = np.array([[int(h, 16) for h in fx["words_hex"]]], dtype=np.uint32)
    s = np.array(fx["scales"], np.float32)
    b = np.array(fx["biases"], np.float32)
    assert np.array_equal(oracle.unpack_b4_u32(wp, n, k)[0], np.arange(16))
    assert np.array_equal(oracle.decode_affine_b4(wp, s, b, n, k, gs), np.array(fx["w"]))
    ones = np.ones((1, k), np.float32)
    ar = np.arange(k, dtype=np.float32)[None, :]
    assert oracle.qmm_affine_t_packed(ones, wp, s, b, 1, n, k, gs)[0, 0] == fx["y_ones"]
    assert oracle.qmm_affine_t_packed(ar, wp, s, b, 1, n, k, gs)[0, 0] == fx["y_arange"]


def test_affine_b4_equals_unpacked_codes():
    """Packing code j of each 8-code run into bits 4j..4j+3 (integer loop here)
    and decoding must give the affine weights of the plain u8 codes."""
    g = synth.rng(23)
    n, k, gs = 6, 64, 32
    codes = g.integers(0, 16, size=(n, k), dtype=np.uint8)
    words = np.zeros((n, k // 8), dtype=np.uint32)
    for r in range(n):
        for kp in range(k // 8):
            v = 0
            for j in range(8):
                v |= int(codes[r, 8 * kp + j]) << (4 * j)
            words[r, kp] = v
    s = g.uniform(0.001, 0.01, size=(n, k // gs)).astype(np.float32)
    b = g.normal(0.0, 0.02, size=(n, k // gs)).astype(np.float32)
    assert np.array_equal(oracle.decode_affine_b4(words, s, b, n, k, gs),
                          oracle.decode_affine(codes, s, b, n, k, gs))
    assert np.array_equal(synth.pack_b4_u32(codes), words)


# ------------------------------------------------------------- multi-part projection
def test_q4_k_multi_parts_land_in_their_columns():
    """Parts [hand block, zero block, hand block] with x = ones: the hand
    super-block gives 39 (its worked value), an all-zero super-block gives 0,
    and each part lands in its own column."""
    fx = _load("q4_k_hand_block.json")
    hand = np.frombuffer(bytes.fromhex(fx["bytes_hex"]), dtype=np.uint8)[None, :]
    zero = np.zeros_like(hand)
    x = np.ones((1, 256), np.float32)
    y = oracle.qgemv_multi(oracle.decode_q4_k, [(hand, 1), (zero, 1), (hand, 1)], x, 1, 256)
    assert y.shape == (1, 3)
    assert list(y[0]) == [fx["y_ones"], 0.0, fx["y_ones"]]
    two = np.concatenate([zero, hand])
    y2 = oracle.qgemv_multi(oracle.decode_q4_k, [(two, 2), (hand, 1)], x, 1, 256)
    assert list(y2[0]) == [0.0, fx["y_ones"], fx["y_ones"]]


# ------------------------------------------------------------- fused projection + split
def test_affine_qkv_hand():
    fx = _load("affine_qkv_hand.json")
    x = np.array(fx["x"], np.float32)
    q = np.array(fx["q"], np.uint8)
    s = np.array(fx["scales"], np.float32)
    b = np.array(fx["biases"], np.float32)
    qo, ko, vo = oracle.qmm_affine_t_qkv(x, q, s, b, fx["m"], fx["k"], fx["group_size"],
                                         fx["q_sp"], fx["k_sp"], fx["v_sp"])
    assert np.array_equal(qo, np.array(fx["q_out"], np.float32))
    assert np.array_equal(ko, np.array(fx["k_out"], np.float32))
    assert np.array_equal(vo, np.array(fx["v_out"], np.float32))
