"""Pins of the oracle's outlier-compensated int8 weight (keras-llm-light
README, "Simplified Int8Variable quantization"): the percentile cut, the
affine grid, the exact restore of the outliers and the layer built on the
reconstructed weight, each checked against something other than the
oracle's own formula: brute-force counting, numpy's inverted-CDF percentile,
closed forms on a constructed example, error bounds, and algebraic identities
of the product."""

import numpy as np
import pytest

from oracle import qlora_oracle as O

F32, F64 = np.float32, np.float64


def _student(shape, seed):
    rng = np.random.default_rng(seed)
    return (0.02 * rng.standard_t(3, size=shape)).astype(F32)


def _brute_percentile(v, num, den):
    """Smallest element x with at least num/den of the elements <= x, found by
    counting (no sort, no rank formula): 1000 * #(v <= x) >= 999 * n."""
    flat = v.ravel()
    n = flat.size
    best = None
    for x in np.unique(flat):
        if den * np.count_nonzero(flat <= x) >= num * n:
            best = x
            break
    return best


@pytest.mark.parametrize("shape,seed", [((37, 53), 0), ((64, 48), 1), ((40, 50), 2), ((16, 16), 3)])
def test_cut_is_the_nearest_rank_percentile_by_counting(shape, seed):
    W = _student(shape, seed)
    q = O.quantize_w8o(W)
    assert q["lo"] == _brute_percentile(W, 1, 1000)
    assert q["hi"] == _brute_percentile(W, 999, 1000)


@pytest.mark.parametrize("shape,seed", [((37, 53), 4), ((256, 384), 5), ((128, 96), 6)])
def test_cut_matches_numpy_inverted_cdf(shape, seed):
    # numpy's "inverted_cdf" percentile is the nearest-rank definition; these
    # sizes keep q n / 100 away from integers so its float arithmetic is exact
    W = _student(shape, seed)
    n = W.size
    for qq in (0.1, 99.9):
        assert abs(qq * n / 100 - round(qq * n / 100)) > 1e-3
    q = O.quantize_w8o(W)
    lo, hi = np.percentile(W, [0.1, 99.9], method="inverted_cdf")
    assert q["lo"] == F32(lo) and q["hi"] == F32(hi)


@pytest.mark.parametrize("n_rows,n_cols", [(256, 256), (37, 53), (1000, 16)])
def test_outlier_counts_for_distinct_values(n_rows, n_cols):
    # distinct values: exactly ceil(n/1000) - 1 below the cut and
    # n - ceil(999 n / 1000) above it
    n = n_rows * n_cols
    rng = np.random.default_rng(n)
    W = (rng.permutation(n).astype(F64) / n - 0.5).astype(F32).reshape(n_rows, n_cols)
    assert np.unique(W).size == n
    q = O.quantize_w8o(W)
    below = np.count_nonzero(W[q["rows"], q["cols"]] < q["lo"])
    above = np.count_nonzero(W[q["rows"], q["cols"]] > q["hi"])
    assert below == -(-n // 1000) - 1
    assert above == n - -(-999 * n // 1000)
    assert below + above == q["rows"].size


def test_constructed_example_closed_forms():
    # 2000 distinct values (j - 1000) / 100, j = 0..1999, shuffled into 40 x 50:
    # rank ceil(2000 / 1000) = 2 -> lo = -9.99; rank ceil(1998) -> hi = 9.97;
    # one outlier below (-10.00) and two above (9.98, 9.99)
    rng = np.random.default_rng(7)
    vals = ((np.arange(2000) - 1000) / 100).astype(F32)
    W = rng.permutation(vals).reshape(40, 50)
    q = O.quantize_w8o(W)
    assert q["lo"] == F32(-9.99) and q["hi"] == F32(9.97)
    got = sorted(float(v) for v in q["vals"])
    assert got == [float(np.float16(-10.0)), float(np.float16(9.98)), float(np.float16(9.99))]
    pos = {float(W[k, n]) for k, n in zip(q["rows"], q["cols"])}
    assert pos == {float(F32(-10.0)), float(F32(9.98)), float(F32(9.99))}
    # grid: lo -> 0, hi -> 255, 0 -> rint(9.99 * 255 / 19.96) = rint(127.6) = 128
    def value_of(x):
        k, n = np.argwhere(W == F32(x))[0]
        return int(q["value"][k, n])
    assert value_of(-9.99) == 0 and value_of(9.97) == 255 and value_of(0.0) == 128
    assert value_of(-10.0) == 0 and value_of(9.99) == 255        # clipped before coding
    assert abs(float(q["scale"]) - 19.96 / 255) < 1e-6


@pytest.mark.parametrize("shape,seed", [((256, 384), 8), ((512, 64), 9)])
def test_reconstruction_error_bounds(shape, seed):
    W = _student(shape, seed)
    q = O.quantize_w8o(W)
    Wr = O.dequant_w8o(q)
    mask = np.zeros(W.shape, bool)
    mask[q["rows"], q["cols"]] = True
    # outliers: restored exactly as fp16 (relative error <= 2^-11)
    assert np.array_equal(Wr[mask], W[mask].astype(np.float16).astype(F32))
    assert np.all(np.abs(Wr[mask] - W[mask]) <= np.abs(W[mask]) * 2.0 ** -11)
    # the rest: within half a step of the grid (plus float32 rounding of the
    # reconstruction and of the code computation)
    slack = 4 * np.finfo(F32).eps * max(abs(float(q["lo"])), abs(float(q["hi"])))
    assert np.all(np.abs(Wr[~mask] - W[~mask]) <= float(q["scale"]) / 2 + slack)
    # every clipped element lies inside the cut, every outlier outside it
    assert np.all((W[~mask] >= q["lo"]) & (W[~mask] <= q["hi"]))


def test_constant_weight_has_no_grid_and_no_outliers():
    W = np.full((32, 48), 0.25, F32)
    q = O.quantize_w8o(W)
    assert q["scale"] == 0 and q["rows"].size == 0
    assert np.all(q["value"] == 0)
    assert np.array_equal(O.dequant_w8o(q), W)


def test_small_tensors_have_no_outliers():
    # n <= 1000: both cuts are the extremes
    W = _student((16, 48), 10)
    q = O.quantize_w8o(W)
    assert q["lo"] == W.min() and q["hi"] == W.max() and q["rows"].size == 0


def test_device_codes_layout():
    W = _student((64, 48), 11)
    q = O.quantize_w8o(W)
    c = O.w8o_device_codes(q)
    assert c.shape == (48, 64) and c.dtype == np.int8
    assert np.array_equal(c.T.astype(np.int16) + 128, q["value"].astype(np.int16))


@pytest.mark.parametrize("M", [1, 5, 33])
def test_forward_equals_the_affine_decomposition(M):
    # base = sx * (scale * (xq . (value - 128)^T) + (lo + 128 scale) rowsum(xq)
    #              + xq . D), D = Wr - (lo + value * scale) nonzero only at
    # outliers: the exact integer product of the int8 path plus a rank-one
    # bias term and the sparse correction -- a different route to the same sum
    K, N, r = 256, 96, 4
    rng = np.random.default_rng(12 + M)
    W = _student((K, N), 13)
    q = O.quantize_w8o(W)
    x = rng.standard_normal((M, K)).astype(F32)
    A = (0.01 * rng.standard_normal((K, r))).astype(F32)
    B = (0.01 * rng.standard_normal((r, N))).astype(F32)
    y, t, xq, sx = O.fwd_w8o_f64(x, q, A, B, 16.0)
    codes = O.w8o_device_codes(q)
    acc = O.int8_acc(xq, codes).astype(F64)
    sc, lo = F64(q["scale"]), F64(q["lo"])
    dense = lo + q["value"].astype(F64) * sc
    D = np.zeros((K, N))
    D[q["rows"], q["cols"]] = q["vals"].astype(F64) - dense[q["rows"], q["cols"]]
    rowsum = xq.astype(F64).sum(axis=1)
    base = sx.astype(F64)[:, None] * (sc * acc + (lo + 128 * sc) * rowsum[:, None] + xq.astype(F64) @ D)
    s = O.lora_scale(16.0, r)
    ref = base + s * (x.astype(F64) @ A.astype(F64)) @ B.astype(F64)
    # Wr is rounded to float32 per element; the decomposition is not
    scale_y = np.sqrt(np.mean(ref ** 2))
    assert np.max(np.abs(y - ref)) <= 1e-5 * scale_y


def test_forward_with_zero_adapter_is_the_quantized_product():
    K, N, M = 128, 64, 7
    rng = np.random.default_rng(14)
    W = _student((K, N), 15)
    q = O.quantize_w8o(W)
    x = rng.standard_normal((M, K)).astype(F32)
    A = (0.01 * rng.standard_normal((K, 4))).astype(F32)
    y, _, xq, sx = O.fwd_w8o_f64(x, q, A, np.zeros((4, N), F32), 32.0)
    # brute force over k on a few outputs
    Wr = O.dequant_w8o(q).astype(F64)
    for m, n in [(0, 0), (3, 17), (6, 63)]:
        ref = sum(float(xq[m, k]) * Wr[k, n] for k in range(K)) * float(sx[m])
        assert abs(y[m, n] - ref) <= 1e-12 * max(1.0, abs(ref))


def test_backward_is_the_adjoint_of_the_base_product():
    # <dy, x Wr> = <dy Wr^T, x>: a transposed or mis-indexed weight in dx fails
    K, N, M = 192, 80, 9
    rng = np.random.default_rng(16)
    W = _student((K, N), 17)
    q = O.quantize_w8o(W)
    Wr = O.dequant_w8o(q)
    x = rng.standard_normal((M, K))
    dy = rng.standard_normal((M, N))
    A = np.zeros((K, 4))
    B = np.zeros((4, N))
    dx, dA, dB, _ = O.bwd_f64(x, dy, Wr, A, B, 8.0)
    lhs = np.sum(dy * (x @ Wr.astype(F64)))
    rhs = np.sum(dx * x)
    assert abs(lhs - rhs) <= 1e-10 * (abs(lhs) + 1)
    assert np.all(dA == 0) and np.all(dB == 0)
