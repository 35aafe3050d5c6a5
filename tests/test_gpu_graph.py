"""The forward and backward captured in a HIP graph, the way the step is timed.

Every replay must give the same bytes as eager calls on the same inputs: the
kernels' reductions have a fixed order, so the results do not depend on the
output or workspace addresses. The replays run one after another with eager
calls and synchronizations between them, and new inputs are copied into the
captured buffers before some of them, so a replay that read stale inputs, or
a workspace region that a replay relies on but does not rewrite, would show
up as a mismatch. One shape per kernel family: 64-row and 128-wide backward
tiles, the split backward contraction, the split forward with the split
long-row pass, outlier-compensated int8, 4-bit, and the float32 path.
"""

from __future__ import annotations

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
    Q.lib()   # raises if libqlora.so is missing: no silent fallback


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bits(t):
    """The tensor's bytes as integers, for a bitwise comparison."""
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


SPECS = [
    # (cid, M, K, N, r, weight format or None for the workload's own)
    (2, 1024, 1024, 1024, 8, None),   # 64-row backward tiles (the MLP layers)
    (3, 512, 768, 2304, 4, None),     # 128-wide backward and forward tiles
    (2, 130, 2048, 8320, 4, None),    # backward contraction split 8 ways
    (2, 100, 16384, 256, 8, None),    # forward split 8 ways, long rows split over k
    (4, 64, 4096, 1024, 8, "w8o"),    # outlier-compensated int8
    (5, 77, 256, 4160, 8, None),      # 4-bit, input gradient split
    (1, 130, 128, 144, 16, None),     # float32
]


@pytest.mark.parametrize("cid,M,K,N,r,fmt", SPECS)
def test_graph_replay_matches_eager(cid, M, K, N, r, fmt):
    w = WL.small(cid, M, K, N, r)
    if fmt is not None:
        w = WL.with_format(w, fmt)
    say(f"graph: {w.name} M={M} K={K} N={N} r={r} {w.dtype} {w.wfmt}")
    codes, scales = Q.qlora_quantize(dev(WL.weight(w, 0)), w.wfmt)
    lin = Q.QLinear(K, N, w.r, w.alpha, w.wfmt, codes, scales,
                    dev(WL.lora_A(w, 0)), dev(WL.lora_B(w, 0)))
    x1 = WL.as_compute_dtype(WL.activations(w, 0, M), w.dtype)[0].cuda()
    dy1 = WL.as_compute_dtype(WL.out_grad(w, 0, M), w.dtype)[0].cuda()
    # a second input set: rows rolled, gradient columns reversed
    x2 = torch.roll(x1, 1, 0).contiguous()
    dy2 = torch.flip(dy1, (1,)).contiguous()

    # the captured buffers, one workspace for both calls
    dt = 0 if w.dtype == "f32" else 1
    nws = max(Q.qlora_fwd_workspace(lin, M, dt), Q.qlora_bwd_workspace(lin, M, dt))
    ws = torch.empty((nws,), dtype=torch.uint8, device="cuda")
    x, dy = x1.clone(), dy1.clone()
    y = torch.empty((M, N), dtype=x.dtype, device="cuda")
    t = torch.empty((M, w.r), dtype=torch.float32, device="cuda")
    dx = torch.empty((M, K), dtype=x.dtype, device="cuda")
    dA = torch.empty((K, w.r), dtype=torch.float32, device="cuda")
    dB = torch.empty(Q._b_shape(lin), dtype=torch.float32, device="cuda")

    def step():
        Q.qlora_fwd(lin, x, y=y, t=t, ws=ws)
        Q.qlora_bwd(lin, x, dy, t=t, dx=dx, dA=dA, dB=dB, ws=ws)

    def eager(xi, dyi):
        ye, te = Q.qlora_fwd(lin, xi)
        dxe, dAe, dBe = Q.qlora_bwd(lin, xi, dyi, t=te)
        return ye, te, dxe, dAe, dBe

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    names = ("y", "t", "dx", "dA", "dB")
    for it, (xi, dyi) in enumerate([(x1, dy1), (x2, dy2), (x2, dy2), (x1, dy1)]):
        x.copy_(xi)
        dy.copy_(dyi)
        g.replay()
        torch.cuda.synchronize()
        got = [a.clone() for a in (y, t, dx, dA, dB)]
        ref = eager(xi, dyi)
        torch.cuda.synchronize()
        for n, a, b in zip(names, got, ref):
            assert torch.equal(bits(a), bits(b)), f"replay {it}: {n} differs from the eager call"
    say("graph: 4 replays match")
