"""Pins for the oracle's quantizers and rounding (CPU only).

Each test checks the oracle against something it does not compute itself:
hand-worked codes, the definition of correct rounding checked with exact
rationals, derived error bounds, exactly representable special cases, and
bit patterns fixed by the IEEE/bfloat16/fp16 formats.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import qlora_oracle as O

F32 = np.float32


def _is_correctly_rounded_f32(value: np.float32, exact: Fraction) -> bool:
    """True when ``value`` is a float32 nearest to the rational ``exact``."""
    v = F32(value)
    up = np.nextafter(v, F32(np.inf))
    dn = np.nextafter(v, F32(-np.inf))
    d = abs(Fraction(float(v)) - exact)
    return d <= abs(Fraction(float(up)) - exact) and d <= abs(Fraction(float(dn)) - exact)


# --------------------------- int8, worked by hand ---------------------------

def test_w8_hand_worked_channel():
    # one output channel (column of W [K, N]) with abs-max 1.0:
    # inv = 127, codes = rint(127 * w): 127, rint(-63.5) = -64 (tie to even),
    # rint(31.75) = 32, 0
    W = np.array([[1.0], [-0.5], [0.25], [0.0]], dtype=F32)
    codes, sw = O.quantize_w8(W)
    assert codes.shape == (1, 4) and codes.dtype == np.int8
    assert codes.tolist() == [[127, -64, 32, 0]]
    assert _is_correctly_rounded_f32(sw[0], Fraction(1, 127))


def test_w8_ties_to_even_and_layout():
    # abs-max 127 makes inv exactly 1, so the codes are rint of the values
    col0 = [127.0, 0.5, 1.5, 2.5, -0.5, -2.5, 3.5, -126.5]
    col1 = [2.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 1.0]   # abs-max 2: inv 63.5
    W = np.array([col0, col1], dtype=F32).T           # [K=8, N=2]
    codes, sw = O.quantize_w8(W)
    assert codes.shape == (2, 8)                      # [N, K], K contiguous
    assert codes[0].tolist() == [127, 0, 2, 2, 0, -2, 4, -126]
    assert sw[0] == F32(1.0)
    # 1.0 * 63.5 = 63.5 -> 64 (tie to even)
    assert codes[1].tolist() == [127, 0, 0, 0, 0, 0, 0, 64]
    assert _is_correctly_rounded_f32(sw[1], Fraction(2, 127))


def test_w8_error_bound_and_full_range():
    rng = np.random.default_rng(7)
    W = (rng.standard_normal((300, 40)) * 0.05).astype(F32)
    W[:, 3] *= 1e-20       # tiny but normal channel
    W[:, 5] *= 1e20        # huge channel
    codes, sw = O.quantize_w8(W)
    assert codes.min() >= -127 and codes.max() <= 127
    deq = O.dequant_w8(codes, sw)              # [K, N] float64, exact
    err = np.abs(W.astype(np.float64) - deq)
    # two float32 divides and one multiply: |w - q s| <= s (1/2 + 2^-15)
    bound = sw.astype(np.float64)[None, :] * (0.5 + 2.0 ** -15)
    assert np.all(err <= bound)
    assert np.all(np.abs(codes).max(axis=1) == 127)
    for n in range(W.shape[1]):
        a = Fraction(float(np.abs(W[:, n]).max()))
        assert _is_correctly_rounded_f32(sw[n], a / 127)


def test_w8_exact_when_channel_is_on_grid():
    # channel = integer multiples of 2^e with abs-max 127 * 2^e: inv = 2^-e and
    # scale = 2^e are exact, so dequantization returns W bit for bit
    rng = np.random.default_rng(3)
    K, N = 64, 6
    ints = rng.integers(-127, 128, size=(K, N))
    ints[0] = 127
    ints[1, ::2] = -127
    e = np.array([-10, -3, 0, 2, 7, -20])
    W = (ints * (2.0 ** e)[None, :]).astype(F32)
    codes, sw = O.quantize_w8(W)
    assert np.array_equal(sw, (2.0 ** e).astype(F32))
    assert np.array_equal(codes.T.astype(np.int64), ints)
    assert np.array_equal(O.dequant_w8(codes, sw), W.astype(np.float64))


def test_w8_degenerate_channels():
    W = np.ones((4, 5), dtype=F32)
    W[:, 0] = 0.0                                   # all zero
    W[:, 1] = [1e-45, 0.0, -1e-45, 0.0]             # 127/absmax overflows
    W[2, 2] = np.nan                                # NaN
    W[1, 3] = -np.inf                               # infinity
    codes, sw = O.quantize_w8(W)
    assert sw[0] == 0 and not codes[0].any()
    assert sw[1] == 0 and not codes[1].any()
    assert np.isnan(sw[2]) and not codes[2].any()
    assert np.isnan(sw[3]) and not codes[3].any()
    assert sw[4] == F32(1.0) / F32(127.0) and np.all(codes[4] == 127)


def test_rows_match_channels_transposed():
    # a row of x is quantized exactly as an output channel of W would be
    rng = np.random.default_rng(11)
    x = rng.standard_normal((9, 33)).astype(F32)
    xq, sx = O.quantize_rows(x)
    codes, sw = O.quantize_w8(x.T)
    assert np.array_equal(xq, codes) and np.array_equal(sx, sw)
    assert xq.shape == (9, 33) and sx.shape == (9,)


def test_requantizing_dequantized_weight_is_stable():
    # quantize(deq(quantize(W))) keeps the codes and moves the scale <= 1 ulp
    rng = np.random.default_rng(5)
    W = (rng.standard_normal((128, 16)) * 0.03).astype(F32)
    c1, s1 = O.quantize_w8(W)
    c2, s2 = O.quantize_w8(O.dequant_w8(c1, s1).astype(F32))
    assert np.array_equal(c1, c2)
    ulp = np.abs(np.nextafter(s1, F32(np.inf)) - s1)
    assert np.all(np.abs(s2 - s1) <= ulp)


# ------------------------------ integer product -----------------------------

def test_int8_acc_matches_integer_loops():
    rng = np.random.default_rng(2)
    xq = rng.integers(-127, 128, size=(3, 7)).astype(np.int8)
    codes = rng.integers(-127, 128, size=(4, 7)).astype(np.int8)
    acc = O.int8_acc(xq, codes)
    for m in range(3):
        for n in range(4):
            want = sum(int(xq[m, k]) * int(codes[n, k]) for k in range(7))
            assert acc[m, n] == want


def test_int8_acc_extreme_is_exact():
    K = 16384
    xq = np.full((2, K), 127, dtype=np.int8)
    xq[1] = -127
    codes = np.full((1, K), 127, dtype=np.int8)
    acc = O.int8_acc(xq, codes)
    assert acc[0, 0] == K * 127 * 127 and acc[1, 0] == -K * 127 * 127


# ------------------------------ result rounding -----------------------------

@pytest.mark.parametrize("bits32,bits16", [
    (0x3F800000, 0x3F80),   # 1.0
    (0x3F808000, 0x3F80),   # 1 + 2^-8: tie, keep even 1.0
    (0x3F818000, 0x3F82),   # 1 + 3*2^-8: tie, round up to even
    (0x3F808001, 0x3F81),   # just above the tie
    (0x3F807FFF, 0x3F80),   # just below the tie
    (0xBF808001, 0xBF81),   # negative
    (0x7F7FFFFF, 0x7F80),   # largest float32 rounds to +inf
    (0x7F800000, 0x7F80),   # +inf stays
    (0x00000001, 0x0000),   # smallest subnormal rounds to +0
    (0x80000000, 0x8000),   # -0 stays
])
def test_bf16_rounding_bit_patterns(bits32, bits16):
    v = np.array([bits32], dtype=np.uint32).view(F32)
    assert int(O.f32_to_bf16_bits(v)[0]) == bits16


def test_bf16_nan_stays_nan():
    v = np.array([0x7F800001, 0xFFC00000], dtype=np.uint32).view(F32)
    out = O.bf16_bits_to_f32(O.f32_to_bf16_bits(v))
    assert np.all(np.isnan(out))


def test_round_to_bf16_is_nearest():
    rng = np.random.default_rng(1)
    v = rng.standard_normal(2000) * 10.0
    r = O.round_to(v, "bf16").astype(np.float64)
    v32 = v.astype(F32).astype(np.float64)
    # nearest bf16: error at most half a bf16 ulp (2^-8 relative to 2^exp)
    ulp = 2.0 ** (np.floor(np.log2(np.abs(v32))) - 7)
    assert np.all(np.abs(r - v32) <= ulp / 2)


# ---------------------------------- 4-bit -----------------------------------

def test_nibble_pack_layout_and_roundtrip():
    q = np.array([[1, -1, -8, 7, 0, 5]], dtype=np.int8)
    p = O.pack_nibbles(q)
    # even k in the low nibble, two's complement
    assert p.tolist() == [[0xF1, 0x78, 0x50]]
    allq = np.array([[a, b] for a in range(-8, 8) for b in range(-8, 8)],
                    dtype=np.int8).reshape(1, -1)
    assert np.array_equal(O.unpack_nibbles(O.pack_nibbles(allq)), allq)


def test_w4_error_bound_range_and_layout():
    rng = np.random.default_rng(9)
    K, N = 512, 24
    W = (rng.standard_normal((K, N)) * 0.02).astype(F32)
    packed, sc = O.quantize_w4(W)
    assert packed.shape == (N, K // 2) and packed.dtype == np.uint8
    assert sc.shape == (N, K // 128) and sc.dtype == np.float16
    q = O.unpack_nibbles(packed)
    assert q.min() >= -7 and q.max() <= 7
    # every group reaches the end of the range
    assert np.all(np.abs(q.reshape(N, K // 128, 128)).max(axis=2) == 7)
    deq = O.dequant_w4(packed, sc)
    scale_k = np.repeat(sc.astype(np.float64), 128, axis=1).T     # [K, N]
    assert np.all(np.abs(W - deq) <= scale_k * (0.5 + 2.0 ** -15))
    # the stored scale is the nearest fp16 of fl32(absmax / 7)
    a = np.abs(W.T.reshape(N, K // 128, 128)).max(axis=2)
    s32 = (a / F32(7)).astype(np.float64)
    rel = np.abs(sc.astype(np.float64) - s32) / s32
    assert np.all(rel <= 2.0 ** -11)


def test_w4_exact_on_power_of_two_grid():
    rng = np.random.default_rng(4)
    K, N = 256, 3
    ints = rng.integers(-7, 8, size=(K, N))
    ints[0] = 7
    ints[128] = -7
    e = np.array([-6, -1, 3])
    W = (ints * (2.0 ** e)[None, :]).astype(F32)
    packed, sc = O.quantize_w4(W)
    assert np.array_equal(sc.astype(np.float64), np.repeat((2.0 ** e)[:, None], 2, axis=1))
    assert np.array_equal(O.dequant_w4(packed, sc), W.astype(np.float64))


def test_w4_fp16_scale_ties_and_overflow():
    K = 128
    W = np.zeros((K, 3), dtype=F32)
    # absmax / 7 = 1 + 2^-11 exactly: halfway between fp16 1.0 and 1 + 2^-10,
    # ties to even -> 1.0
    W[0, 0] = F32(7.0 * (1.0 + 2.0 ** -11))
    # absmax / 7 = 1 + 3 * 2^-11: tie, rounds up to the even 1 + 2^-9
    W[0, 1] = F32(7.0 * (1.0 + 3.0 * 2.0 ** -11))
    # absmax / 7 = 70000 > 65504: the fp16 scale overflows -> NaN marker
    W[0, 2] = F32(7.0 * 70000.0)
    packed, sc = O.quantize_w4(W)
    assert sc[0, 0] == np.float16(1.0)
    assert sc[1, 0] == np.float16(1.0 + 2.0 ** -9)
    assert np.isnan(sc[2, 0])
    q = O.unpack_nibbles(packed)
    assert q[0, 0] == 7 and q[1, 0] == 7 and not q[2].any()


def test_w4_zero_group():
    W = np.zeros((256, 2), dtype=F32)
    W[200, 1] = 0.5
    packed, sc = O.quantize_w4(W)
    assert sc[0, 0] == 0 and sc[0, 1] == 0 and sc[1, 0] == 0
    assert not packed[0].any()
    assert O.unpack_nibbles(packed)[1, 200] == 7
