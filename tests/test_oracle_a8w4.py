"""Pins for the oracle's integer 4-bit forward (int8 activations x 4-bit
weights, per-group rescaling), CPU only:

* the per-group integer sums against a plain loop that decodes the nibbles
  itself;
* activations that quantize exactly (integer rows whose abs-max is 127, so
  the row scale is 1) reduce it to the dequantized float product, exactly;
* for general activations it stays within the activation quantizer's error
  bound of the float product: |y - y_float| <= (1/2 + 2^-15) sx sum_k |deq4|.
"""

import numpy as np

from oracle import qlora_oracle as O

F32 = np.float32


def _layer(seed, M, K, N, r=2, xint=False):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((K, N)) * 0.02).astype(F32)
    packed, scales = O.quantize_w4(W)
    if xint:
        x = rng.integers(-127, 128, (M, K)).astype(F32)
        x[:, 0] = 127.0                      # every row's abs-max is 127
    else:
        x = rng.standard_normal((M, K)).astype(F32)
    A = (rng.standard_normal((K, r)) * 0.01).astype(F32)
    B = (rng.standard_normal((r, N)) * 0.01).astype(F32)
    return x, packed, scales, A, B


def _nibble(byte, hi):
    v = (int(byte) >> 4) & 15 if hi else int(byte) & 15
    return v - 16 if v >= 8 else v


def test_group_sums_against_a_plain_loop():
    x, packed, _, _, _ = _layer(0, 2, 256, 3)
    xq, _ = O.quantize_rows(x)
    acc = O.int4_group_acc(xq, packed)
    assert acc.shape == (2, 2, 3)
    for g in range(2):
        for m in range(2):
            for n in range(3):
                want = 0
                for k in range(128 * g, 128 * g + 128):
                    want += int(xq[m, k]) * _nibble(packed[n, k // 2], k % 2)
                assert acc[g, m, n] == want


def test_exact_activations_reduce_to_the_float_product():
    x, packed, scales, A, B = _layer(1, 4, 384, 5, xint=True)
    xq, sx = O.quantize_rows(x)
    assert np.all(sx == 1.0) and np.array_equal(xq.astype(F32), x)
    y8, t8, _, _ = O.fwd_a8w4_f64(x, packed, scales, A, B, 8.0)
    yf, tf = O.fwd_w4_f64(x, packed, scales, A, B, 8.0)
    assert np.array_equal(t8, tf)
    assert np.array_equal(y8, yf)


def test_error_bound_against_the_float_product():
    x, packed, scales, A, B = _layer(2, 6, 512, 7, r=4)
    y8, _, _, sx = O.fwd_a8w4_f64(x, packed, scales, A, B, 8.0)
    yf, _ = O.fwd_w4_f64(x, packed, scales, A, B, 8.0)
    deq = O.dequant_w4(packed, scales)                  # [K, N]
    bound = (0.5 + 2.0 ** -15) * sx.astype(np.float64)[:, None] * np.abs(deq).sum(axis=0)[None, :]
    assert np.all(np.abs(y8 - yf) <= bound * (1 + 1e-12) + 1e-300)
    # and the quantization error is really there (the two forwards differ)
    assert np.any(y8 != yf)
