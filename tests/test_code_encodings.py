"""Number-format facts the kernels rely on, checked on the host from the
formats' definitions (no GPU):

* read as OCP FP8 E4M3 (1 sign bit, 4 exponent bits with bias 7, 3 mantissa
  bits, subnormals at exponent 0), the bytes 0..15 are exactly q / 512, so a
  conversion with scale 2^9 returns the 4-bit code q exactly;
* every code 0..255 is exact in bf16 (8 significant bits), so the matrix-core
  kernels take the codes as bf16 operands without rounding;
* splitting an f32 x into hi = bf16(x) and lo = bf16(x - hi) leaves a
  relative error of at most 2^-17 (the bound the matrix-core paths use), and
  x - hi itself is exact in f32."""
import numpy as np


def e4m3_value(byte: int) -> float:
    sign = -1.0 if byte & 0x80 else 1.0
    exp = (byte >> 3) & 0xF
    man = byte & 0x7
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round f32 to bf16 (nearest, ties to even) and back to f32."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    r = ((b + 0x7FFF + lsb) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def test_e4m3_bytes_0_to_15_are_code_over_512():
    for q in range(16):
        assert e4m3_value(q) * 512.0 == float(q), q
    # a byte holding two nibbles is not a code: the masking before the conversion matters
    assert e4m3_value(0x5A) * 512.0 != float(0x5A & 0xF)


def test_codes_0_to_255_are_exact_in_bf16():
    q = np.arange(256, dtype=np.float32)
    assert np.array_equal(bf16_round(q), q)


def test_hi_lo_bf16_split_error_bound():
    g = np.random.default_rng(11)
    x = np.concatenate([g.standard_normal(100000).astype(np.float32),
                        (g.standard_normal(1000) * 1e-30).astype(np.float32),
                        (g.standard_normal(1000) * 1e30).astype(np.float32)])
    hi = bf16_round(x)
    rem = x - hi
    # the remainder is exact in f32 (hi shares x's exponent range)
    assert np.array_equal(rem.astype(np.float64), x.astype(np.float64) - hi.astype(np.float64))
    lo = bf16_round(rem)
    err = np.abs(x.astype(np.float64) - hi.astype(np.float64) - lo.astype(np.float64))
    assert np.all(err <= np.abs(x.astype(np.float64)) * 2.0 ** -17)
