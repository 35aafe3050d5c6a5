"""Pins for the oracle's forward and backward (CPU only).

* exact rational brute force of y = x deq(W) + s x (A B) on tiny inputs,
  written as the merged product (the unmerged and merged LoRA forms agree);
* B = 0 reduces the layer to the plain quantized product; A = 0 kills dB;
* inputs on the quantization grid reduce it to the textbook float product;
* dA, dB from central finite differences (the loss <dy, y> is linear in A
  and in B, so differences are exact up to rounding);
* dx from finite differences of the float surrogate x deq(W) + s x A B, and
  the adjoint identity <dy, x W> = <dy W^T, x>.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import qlora_oracle as O

F32 = np.float32


def _tiny(seed, M=3, K=4, N=4, r=2):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(F32)
    W = (rng.standard_normal((K, N)) * 0.1).astype(F32)
    A = (rng.standard_normal((K, r)) * 0.1).astype(F32)
    B = (rng.standard_normal((r, N)) * 0.1).astype(F32)
    dy = rng.standard_normal((M, N)).astype(F32)
    return x, W, A, B, dy


@pytest.mark.parametrize("seed,r", [(0, 1), (1, 2), (2, 2)])
def test_forward_equals_exact_merged_product(seed, r):
    x, W, A, B, _ = _tiny(seed, r=r)
    alpha = 8.0
    codes, sw = O.quantize_w8(W)
    xq, sx = O.quantize_rows(x)
    y64, t64, *_ = O.fwd_w8_f64(x, codes, sw, A, B, alpha)
    s = Fraction(alpha) / r
    M, K = x.shape
    N = W.shape[1]
    for m in range(M):
        for n in range(N):
            # base: dequantized activations times dequantized weights
            base = sum(Fraction(int(xq[m, k])) * Fraction(float(sx[m]))
                       * Fraction(int(codes[n, k])) * Fraction(float(sw[n]))
                       for k in range(K))
            # adapter merged into one matrix: x (s A B)
            lora = sum(Fraction(float(x[m, k])) * s
                       * sum(Fraction(float(A[k, j])) * Fraction(float(B[j, n]))
                             for j in range(r))
                       for k in range(K))
            want = float(base + lora)
            assert y64[m, n] == pytest.approx(want, rel=1e-14, abs=1e-15)
    for m in range(M):
        for j in range(r):
            want = float(sum(Fraction(float(x[m, k])) * Fraction(float(A[k, j]))
                             for k in range(K)))
            assert t64[m, j] == pytest.approx(want, rel=1e-14, abs=1e-15)


def test_zero_B_is_plain_quantized_product():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((16, 64)).astype(F32)
    W = (rng.standard_normal((64, 32)) * 0.05).astype(F32)
    A = (rng.standard_normal((64, 4)) * 0.01).astype(F32)
    B = np.zeros((4, 32), F32)
    codes, sw = O.quantize_w8(W)
    y64, _, xq, sx, acc = O.fwd_w8_f64(x, codes, sw, A, B, 32.0)
    plain = acc.astype(np.float64) * sx.astype(np.float64)[:, None] * sw.astype(np.float64)[None, :]
    assert np.array_equal(y64, plain)


def test_on_grid_inputs_give_the_float_lora_layer():
    # x rows and W channels on power-of-two grids with full-range maxima are
    # quantized without loss, so the layer equals x W + s (x A) B in floats
    rng = np.random.default_rng(8)
    M, K, N, r = 8, 32, 12, 4
    xi = rng.integers(-127, 128, size=(M, K)); xi[:, 0] = 127
    wi = rng.integers(-127, 128, size=(K, N)); wi[5] = -127
    x = (xi * 2.0 ** -4).astype(F32)
    W = (wi * 2.0 ** -9).astype(F32)
    A = (rng.standard_normal((K, r)) * 0.01).astype(F32)
    B = (rng.standard_normal((r, N)) * 0.01).astype(F32)
    codes, sw = O.quantize_w8(W)
    y64, *_ = O.fwd_w8_f64(x, codes, sw, A, B, 16.0)
    xd, Wd, Ad, Bd = (a.astype(np.float64) for a in (x, W, A, B))
    want = xd @ Wd + 4.0 * (xd @ Ad) @ Bd
    np.testing.assert_allclose(y64, want, rtol=1e-13, atol=1e-13)


def _loss(x, codes, sw, A, B, alpha, dy):
    y64, *_ = O.fwd_w8_f64(x, codes, sw, A, B, alpha)
    return float(np.sum(y64 * dy.astype(np.float64)))


def test_dA_dB_match_central_differences():
    x, W, A, B, dy = _tiny(5, M=5, K=6, N=7, r=2)
    alpha = 4.0
    codes, sw = O.quantize_w8(W)
    dx, dA, dB, _ = O.bwd_f64(x, dy, O.dequant_w8(codes, sw), A, B, alpha)
    h = 2.0 ** -10
    A64, B64 = A.astype(np.float64), B.astype(np.float64)

    def loss64(Am, Bm):
        # the oracle's own (pinned) forward, with float64 adapter weights
        return _loss(x, codes, sw, Am, Bm, alpha, dy)

    for k in range(A.shape[0]):
        for j in range(A.shape[1]):
            e = np.zeros_like(A64); e[k, j] = h
            fd = (loss64(A64 + e, B64) - loss64(A64 - e, B64)) / (2 * h)
            assert dA[k, j] == pytest.approx(fd, rel=1e-9, abs=1e-12)
    for j in range(B.shape[0]):
        for n in range(B.shape[1]):
            e = np.zeros_like(B64); e[j, n] = h
            fd = (loss64(A64, B64 + e) - loss64(A64, B64 - e)) / (2 * h)
            assert dB[j, n] == pytest.approx(fd, rel=1e-9, abs=1e-12)


def test_dx_matches_surrogate_differences_and_adjoint():
    x, W, A, B, dy = _tiny(6, M=4, K=5, N=6, r=2)
    alpha = 8.0
    codes, sw = O.quantize_w8(W)
    Wd = O.dequant_w8(codes, sw)
    dx, *_ = O.bwd_f64(x, dy, Wd, A, B, alpha)
    s = alpha / A.shape[1]
    A64, B64, dy64 = A.astype(np.float64), B.astype(np.float64), dy.astype(np.float64)

    def surrogate(xm):  # the straight-through float view of the layer
        return float(np.sum((xm @ Wd + s * (xm @ A64) @ B64) * dy64))

    x64 = x.astype(np.float64)
    h = 2.0 ** -12
    for m in range(x.shape[0]):
        for k in range(x.shape[1]):
            e = np.zeros_like(x64); e[m, k] = h
            fd = (surrogate(x64 + e) - surrogate(x64 - e)) / (2 * h)
            assert dx[m, k] == pytest.approx(fd, rel=1e-9, abs=1e-12)
    # adjoint identity for the frozen part alone
    lhs = float(np.sum(dy64 * (x64 @ Wd)))
    rhs = float(np.sum((dy64 @ Wd.T) * x64))
    assert lhs == pytest.approx(rhs, rel=1e-13)


def test_zero_adapter_halves():
    x, W, A, B, dy = _tiny(7, M=6, K=8, N=5, r=2)
    codes, sw = O.quantize_w8(W)
    Wd = O.dequant_w8(codes, sw)
    dx, dA, dB, _ = O.bwd_f64(x, dy, Wd, A, np.zeros_like(B), 16.0)
    assert not dA.any()
    assert np.array_equal(dx, dy.astype(np.float64) @ Wd.T)
    _, dA2, dB2, _ = O.bwd_f64(x, dy, Wd, np.zeros_like(A), B, 16.0)
    assert not dB2.any()


def test_w4_forward_backward_against_rationals():
    rng = np.random.default_rng(12)
    M, K, N, r = 2, 128, 3, 1
    x = rng.standard_normal((M, K)).astype(F32)
    W = (rng.standard_normal((K, N)) * 0.02).astype(F32)
    A = (rng.standard_normal((K, r)) * 0.01).astype(F32)
    B = (rng.standard_normal((r, N)) * 0.01).astype(F32)
    packed, sc = O.quantize_w4(W)
    y64, _ = O.fwd_w4_f64(x, packed, sc, A, B, 8.0)
    q = O.unpack_nibbles(packed)
    for m in range(M):
        for n in range(N):
            want = sum(Fraction(float(x[m, k])) * int(q[n, k]) * Fraction(float(sc[n, k // 128]))
                       for k in range(K))
            want += 8 * sum(Fraction(float(x[m, k])) * Fraction(float(A[k, 0])) for k in range(K)) \
                * Fraction(float(B[0, n]))
            assert y64[m, n] == pytest.approx(float(want), rel=1e-13, abs=1e-14)


def test_merge_with_zero_B_keeps_codes():
    rng = np.random.default_rng(13)
    W = (rng.standard_normal((64, 8)) * 0.03).astype(F32)
    A = (rng.standard_normal((64, 4)) * 0.01).astype(F32)
    codes, sw = O.quantize_w8(W)
    c2, s2 = O.merge_w8(codes, sw, A, np.zeros((4, 8), F32), 16.0)
    assert np.array_equal(c2, codes)
    assert np.all(np.abs(s2 - sw) <= np.abs(np.nextafter(sw, F32(1)) - sw))


@pytest.mark.parametrize("seed,r", [(21, 1), (22, 3)])
def test_merged_weight_is_the_nearest_float32(seed, r):
    """W' is the float32 nearest to the exact deq(W) + s A B (checked with
    rational arithmetic), for every element of a small layer."""
    rng = np.random.default_rng(seed)
    K, N, alpha = 6, 5, 8.0
    W = (rng.standard_normal((K, N)) * 0.05).astype(F32)
    A = (rng.standard_normal((K, r)) * 0.3).astype(F32)
    B = (rng.standard_normal((r, N)) * 0.3).astype(F32)
    codes, sw = O.quantize_w8(W)
    Wm = O.merged_weight_w8(codes, sw, A, B, alpha)
    s = Fraction(float(np.float32(alpha) / np.float32(r)))
    for k in range(K):
        for n in range(N):
            exact = int(codes[n, k]) * Fraction(float(sw[n])) + s * sum(
                Fraction(float(A[k, j])) * Fraction(float(B[j, n])) for j in range(r))
            got = Fraction(float(Wm[k, n]))
            lo = Fraction(float(np.nextafter(Wm[k, n], np.float32(-np.inf))))
            hi = Fraction(float(np.nextafter(Wm[k, n], np.float32(np.inf))))
            # nearest: no neighbouring float32 is strictly closer
            assert abs(got - exact) <= abs(lo - exact) and abs(got - exact) <= abs(hi - exact)


def test_merge_error_bound_and_merged_forward():
    """The merged codes are W' on its own channel grid (error <= half a step,
    plus the slack of the float32 quantizer), so the merged forward stays
    within that bound of the unmerged float product."""
    rng = np.random.default_rng(23)
    K, N, r, alpha = 48, 24, 4, 16.0
    W = (rng.standard_normal((K, N)) * 0.05).astype(F32)
    A = (rng.standard_normal((K, r)) * 0.05).astype(F32)
    B = (rng.standard_normal((r, N)) * 0.05).astype(F32)
    codes, sw = O.quantize_w8(W)
    Wm = O.merged_weight_w8(codes, sw, A, B, alpha).astype(np.float64)
    c2, s2 = O.merge_w8(codes, sw, A, B, alpha)
    step = s2.astype(np.float64)[None, :]
    assert np.all(np.abs(O.dequant_w8(c2, s2) - Wm) <= step * (0.5 + 2.0 ** -15))
    assert np.all(np.abs(c2).max(axis=1) == 127)
    x = rng.standard_normal((5, K)).astype(np.float64)
    s = float(np.float32(alpha) / np.float32(r))
    unmerged = x @ O.dequant_w8(codes, sw) + s * (x @ A.astype(np.float64)) @ B.astype(np.float64)
    merged = x @ O.dequant_w8(c2, s2)
    bound = np.abs(x) @ np.ones((K, 1)) * step * (0.5 + 2.0 ** -15) + 1e-12 * np.abs(unmerged).max()
    assert np.all(np.abs(merged - unmerged) <= bound + 1e-6 * np.abs(unmerged))


def test_rounded_outputs_are_nearest():
    x, W, A, B, dy = _tiny(9, M=4, K=16, N=8, r=2)
    codes, sw = O.quantize_w8(W)
    y64, *_ = O.fwd_w8_f64(x, codes, sw, A, B, 4.0)
    yb, _ = O.fwd_w8(x, codes, sw, A, B, 4.0, "bf16")
    yf, _ = O.fwd_w8(x, codes, sw, A, B, 4.0, "f32")
    assert np.array_equal(yf, y64.astype(F32))
    ulp = 2.0 ** (np.floor(np.log2(np.abs(yf.astype(np.float64)))) - 7)
    assert np.all(np.abs(yb.astype(np.float64) - yf) <= ulp / 2)
