"""qlora_bwd_noalloc (the backward for callers that cannot allocate: its
scratch is the library's static device array) against qlora_bwd with a
workspace of the caller's, through the C ABI: two calls in a row, the
second on a smaller layer, each bitwise equal to qlora_bwd's results."""

from __future__ import annotations

import ctypes
import sys

import numpy as np
import pytest

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


def _bits(a):
    return a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32)


def _layer(spec):
    w = WL.small(*spec)
    K, N = w.layers[0]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    codes, scales = Q.qlora_quantize(dev(WL.weight(w, 0)), w.wfmt)
    lin = Q.QLinear(K, N, w.r, w.alpha, w.wfmt, codes, scales, dev(WL.lora_A(w, 0)),
                    dev(WL.lora_B(w, 0)))
    x_t, _ = WL.as_compute_dtype(WL.activations(w, 0), w.dtype)
    dy_t, _ = WL.as_compute_dtype(WL.out_grad(w, 0), w.dtype)
    return w, lin, x_t.cuda(), dy_t.cuda()


def test_noalloc_backward_matches_workspace_backward():
    lib = Q.lib()
    st = torch.cuda.current_stream().cuda_stream
    # the 1024 x 1024 MLP layer, then a smaller ragged layer of another rank
    for spec in [(2, 1024, 1024, 1024, 8), (2, 257, 512, 272, 4)]:
        w, lin, x, dy = _layer(spec)
        say(f"no-alloc backward: M={w.M} K,N={w.layers[0]} r={w.r}")
        M, K, N, r = w.M, lin.K, lin.N, w.r
        dt = Q.QLORA_BF16
        y, t = Q.qlora_fwd(lin, x)
        dx1, dA1, dB1 = Q.qlora_bwd(lin, x, dy, t=t)
        dx2 = torch.full((M, K), 7.0, dtype=torch.bfloat16, device="cuda")
        dA2 = torch.full((K, r), 7.0, dtype=torch.float32, device="cuda")
        dB2 = torch.full((r, N), 7.0, dtype=torch.float32, device="cuda")
        cs = lin.cstruct()
        assert lib.qlora_bwd_noalloc(ctypes.byref(cs), M, dt, x.data_ptr(), dy.data_ptr(),
                                     t.data_ptr(), dx2.data_ptr(), dA2.data_ptr(),
                                     dB2.data_ptr(), st) == 0
        torch.cuda.synchronize()
        assert torch.equal(_bits(dx1), _bits(dx2)), "dx differs"
        assert torch.equal(_bits(dA1), _bits(dA2)), "dA differs"
        assert torch.equal(_bits(dB1), _bits(dB2)), "dB differs"


def test_noalloc_rejects_a_layer_past_the_scratch():
    """A layer whose backward needs more than the static scratch is refused
    before anything is enqueued (the Gemma 2048 -> 16384 layer at 512 rows
    keeps 32 MiB of split partial products)."""
    w, lin, x, dy = _layer((2, 512, 2048, 16384, 8))
    assert Q.qlora_bwd_workspace(lin, 512, Q.QLORA_BF16) > Q.QLORA_NOALLOC_SCRATCH_BYTES
    cs = lin.cstruct()
    dx = torch.empty((512, 2048), dtype=torch.bfloat16, device="cuda")
    dA = torch.empty((2048, 8), dtype=torch.float32, device="cuda")
    dB = torch.empty((8, 16384), dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    assert Q.lib().qlora_bwd_noalloc(ctypes.byref(cs), 512, Q.QLORA_BF16, x.data_ptr(),
                                     dy.data_ptr(), None, dx.data_ptr(), dA.data_ptr(),
                                     dB.data_ptr(), st) == Q.QLORA_EWORKSPACE
