"""GPU parity of the outlier-compensated int8 format (keras-llm-light README,
"Simplified Int8Variable quantization") through the C ABI, against the CPU
oracle: the cut, the grid step, the codes and the outlier list bit-exact;
forward outputs and gradients within the bf16 tolerance."""

from __future__ import annotations

import sys

import numpy as np
import pytest

from helpers import RTOL, assert_close, to_numpy
from oracle import qlora_oracle as O
from quantized_frozen_weight_amd import binding as Q
from quantized_frozen_weight_amd import workloads as WL

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    Q.lib()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def student(K, N, seed):
    rng = np.random.default_rng(seed)
    return (0.02 * rng.standard_t(3, size=(K, N))).astype(np.float32)


def check_quantized(W, codes, side):
    K, N = W.shape
    q = O.quantize_w8o(W)
    head, rowptr, col, val = Q.qlora_outliers(side, K, N)
    assert head["lo"] == q["lo"] and head["hi"] == q["hi"], (head, q["lo"], q["hi"])
    assert head["scale"].view(np.uint32) == np.float32(q["scale"]).view(np.uint32)
    assert np.array_equal(codes.cpu().numpy(), O.w8o_device_codes(q))
    nnz = q["rows"].size
    assert head["nnz"] == nnz
    want_ptr = np.searchsorted(q["rows"], np.arange(K + 1)).astype(np.int32)
    assert np.array_equal(rowptr, want_ptr)
    assert np.array_equal(col, q["cols"].astype(np.int32))
    assert np.array_equal(val.view(np.uint16), q["vals"].view(np.uint16))
    return q


QUANT_CASES = [
    ("student 256x384", lambda: student(256, 384, 1)),
    ("student ragged 208x80", lambda: student(208, 80, 2)),
    ("tiny 16x48 (no outliers)", lambda: student(16, 48, 3)),
    ("constant 32x48", lambda: np.full((32, 48), 0.25, np.float32)),
    ("distinct 256x256", lambda: ((np.random.default_rng(4).permutation(65536) / 65536.0 - 0.5)
                                  .astype(np.float32).reshape(256, 256))),
    ("ties 512x112", lambda: np.round(student(512, 112, 5) * 200).astype(np.float32) / 200),
    ("negative 128x64", lambda: -np.abs(student(128, 64, 6)) - 1.0),
    ("gemma up 2048x16384", lambda: WL.weight(WL.WORKLOADS[4], 0)),
    ("gemma down 16384x2048", lambda: WL.weight(WL.WORKLOADS[4], 2)),
]


@pytest.mark.parametrize("name,make", QUANT_CASES, ids=[c[0] for c in QUANT_CASES])
def test_w8o_quantize_bit_exact(name, make):
    W = make()
    say("w8o quantize", name, W.shape)
    codes, side = Q.qlora_quantize(dev(W), "w8o")
    torch.cuda.synchronize()
    check_quantized(W, codes, side)


def test_w8o_quantize_twice_same_bytes():
    # the side buffer's lists do not depend on what it held before
    W = student(320, 192, 7)
    say("w8o quantize twice")
    codes, side = Q.qlora_quantize(dev(W), "w8o")
    side2 = torch.full_like(side, 0xA5)
    codes2 = torch.full_like(codes, 7)
    Q.lib().qlora_quantize(Q._ptr(dev(W)), 320, 192, Q.QLORA_W8O, Q._ptr(codes2),
                           Q._ptr(side2), Q._stream())
    torch.cuda.synchronize()
    check_quantized(W, codes2, side2)


class W8OCase:
    """One outlier-compensated layer: inputs, device tensors, oracle answers."""

    def __init__(self, M, K, N, r=8, alpha=16.0, seed=0, W=None, zero_B=False):
        rng = np.random.default_rng(seed)
        self.M, self.K, self.N, self.r, self.alpha = M, K, N, r, alpha
        self.W = student(K, N, seed + 1) if W is None else W
        self.A = (0.01 * rng.standard_normal((K, r))).astype(np.float32)
        self.B = (np.zeros((r, N), np.float32) if zero_B
                  else (0.01 * rng.standard_normal((r, N))).astype(np.float32))
        x32 = rng.standard_normal((M, K)).astype(np.float32)
        dy32 = rng.standard_normal((M, N)).astype(np.float32)
        self.x_t, self.x = WL.as_compute_dtype(x32, "bf16")
        self.dy_t, self.dy = WL.as_compute_dtype(dy32, "bf16")
        self.x_t, self.dy_t = self.x_t.cuda(), self.dy_t.cuda()
        codes, side = Q.qlora_quantize(dev(self.W), "w8o")
        self.lin = Q.QLinear(K, N, r, alpha, "w8o", codes, side, dev(self.A), dev(self.B))
        self.q = O.quantize_w8o(self.W)


def run_fwd_bwd(c: W8OCase):
    y, t = Q.qlora_fwd(c.lin, c.x_t)
    dx, dA, dB = Q.qlora_bwd(c.lin, c.x_t, c.dy_t, t=t)
    torch.cuda.synchronize()
    return to_numpy(y), to_numpy(t), to_numpy(dx), to_numpy(dA), to_numpy(dB)


def check_fwd_bwd(c: W8OCase, what):
    y, t, dx, dA, dB = run_fwd_bwd(c)
    ye, te = O.fwd_w8o(c.x, c.q, c.A, c.B, c.alpha, "bf16")
    dxe, dAe, dBe = O.bwd(c.x, c.dy, O.dequant_w8o(c.q), c.A, c.B, c.alpha, "bf16")
    tol = RTOL["bf16"]
    assert_close(t, te, RTOL["f32"], f"{what} t")
    assert_close(y, ye, tol, f"{what} y")
    assert_close(dx, dxe, tol, f"{what} dx")
    assert_close(dA, dAe, RTOL["f32"], f"{what} dA")
    assert_close(dB, dBe, RTOL["f32"], f"{what} dB")


LAYER_CASES = [
    (100, 256, 384, 8, 0),      # ragged rows, several tiles
    (33, 208, 80, 4, 1),        # ragged k block (208 = 128 + 80) and columns (80)
    (1, 512, 128, 16, 2),       # one row
    (257, 1024, 192, 32, 3),    # rank 32, a ragged row tile
    (64, 2048, 1024, 8, 4),     # several 128-wide k blocks
    (70, 208, 2080, 4, 5),      # split contraction: 4 splits, ragged last stage
    (40, 128, 8192, 8, 6),      # 8 splits; the later ones start past 64 stages
    (9, 8208, 64, 8, 7),        # long rows: code sums over four waves; forward split 4 ways
    (130, 4096, 80, 4, 8),      # forward split 4 ways over 2 x 2 ragged 128 x 64 tiles
]


@pytest.mark.parametrize("M,K,N,r,seed", LAYER_CASES)
def test_w8o_layer(M, K, N, r, seed):
    say("w8o layer", M, K, N, r)
    check_fwd_bwd(W8OCase(M, K, N, r=r, seed=seed), f"M{M} K{K} N{N} r{r}")


def test_w8o_zero_adapter_is_the_quantized_product():
    c = W8OCase(96, 384, 256, zero_B=True, seed=5)
    say("w8o B = 0")
    y, _ = Q.qlora_fwd(c.lin, c.x_t)
    torch.cuda.synchronize()
    ye, _ = O.fwd_w8o(c.x, c.q, c.A, c.B, c.alpha, "bf16")
    assert_close(to_numpy(y), ye, RTOL["bf16"], "y (B = 0)")


def test_w8o_integer_product_bit_exact():
    # the forward's integer part: acc = xq (v - 128)^T, exact
    c = W8OCase(70, 384, 208, seed=6)
    say("w8o acc")
    acc = Q.qlora_fwd_acc(c.lin, c.x_t)
    torch.cuda.synchronize()
    xq, _ = O.quantize_rows(c.x)
    assert np.array_equal(acc.cpu().numpy(), O.int8_acc(xq, O.w8o_device_codes(c.q)))


def test_w8o_many_outliers_in_one_cell():
    # 200 planted outliers in one 16 x 16 block: more than one wave's worth
    # in a forward cell (128 k x 32 n) and a backward cell (64 n x 64 k)
    K, N = 512, 512
    W = student(K, N, 40)
    W[200:216, 300:316] = np.linspace(5, 6, 256, dtype=np.float32).reshape(16, 16)
    W[100:116, 40:56] = -np.linspace(5, 6, 256, dtype=np.float32).reshape(16, 16)
    c = W8OCase(80, K, N, W=W, seed=41)
    cell = c.q["rows"][(c.q["rows"] >= 200) & (c.q["rows"] < 216)]
    assert cell.size >= 200
    say("w8o dense outlier block")
    check_fwd_bwd(c, "dense outlier block")


GEMMA = WL.with_format(WL.WORKLOADS[4], "w8o")


@pytest.mark.parametrize("layer", [0, 2], ids=["up 2048->16384", "down 16384->2048"])
def test_w8o_gemma_full_size(layer):
    # the 2B-decoder feed-forward kernels at full size, 512 tokens
    K, N = GEMMA.layers[layer]
    say("w8o gemma", layer, K, N)
    W = WL.weight(GEMMA, layer)
    c = W8OCase(GEMMA.M, K, N, r=GEMMA.r, alpha=GEMMA.alpha, W=W, seed=50 + layer)
    check_fwd_bwd(c, f"gemma layer {layer}")
