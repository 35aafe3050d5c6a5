"""qlora_bwd_finish_batch: the adapter gradients of many layers in one launch
per 32 layers, bitwise equal to each layer's own qlora_bwd.

The layers mix every backward path (64-row and 128-wide int8 tiles, the split
contraction, 4-bit, float32) and split counts from 1 to 65, so one launch
holds jobs of different split counts (each still summed in its own split
order), and 35 layers take two launches.
"""

from __future__ import annotations

import sys

import numpy as np
import pytest

from quantized_frozen_weight_amd import binding as Q
from quantized_frozen_weight_amd import workloads as WL

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    Q.lib()   # raises if libqlora.so is missing: no silent fallback


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


SPECS = [
    # (cid, M, K, N, r)
    (2, 1024, 1024, 1024, 8),   # 64-row tiles, 16 row blocks
    (3, 300, 768, 400, 4),      # 128-wide tiles
    (2, 130, 2048, 8320, 4),    # split contraction
    (5, 77, 256, 272, 8),       # 4-bit
    (1, 130, 128, 144, 16),     # float32
    (2, 4100, 96, 48, 8),       # 65 row blocks: more than one pass of loads
] + [(2, 33 + 7 * i, 64, 48 + 16 * (i % 3), 1 + i % 8) for i in range(29)]


def layer(spec):
    cid, M, K, N, r = spec
    w = WL.small(cid, M, K, N, r)
    codes, scales = Q.qlora_quantize(dev(WL.weight(w, 0)), w.wfmt)
    lin = Q.QLinear(K, N, w.r, w.alpha, w.wfmt, codes, scales,
                    dev(WL.lora_A(w, 0)), dev(WL.lora_B(w, 0)))
    x = WL.as_compute_dtype(WL.activations(w, 0, M), w.dtype)[0].cuda()
    dy = WL.as_compute_dtype(WL.out_grad(w, 0, M), w.dtype)[0].cuda()
    return lin, x, dy


@pytest.mark.parametrize("packed", [False, True], ids=["own workspaces", "packed workspaces"])
def test_finish_batch_matches_per_layer_backward(packed):
    print(f"[case] finish batch: {len(SPECS)} layers, packed={packed}", file=sys.stderr,
          flush=True)
    layers = [layer(s) for s in SPECS]
    refs, items, ts = [], [], []
    for lin, x, dy in layers:
        _, t = Q.qlora_fwd(lin, x)
        _, dA, dB = Q.qlora_bwd(lin, x, dy, t=t)
        refs.append((dA, dB))
        ts.append(t)
    # packed: layer k's workspace starts where the partial sums of layers
    # 0..k-1 end (they run in that order), and the scratch of each call lies
    # over the layers after it
    views, o, total = [], 0, 0
    for lin, x, _ in layers:
        dt = Q.QLORA_F32 if x.dtype == torch.float32 else Q.QLORA_BF16
        need = Q.qlora_bwd_workspace(lin, x.shape[0], dt)
        views.append((o, need))
        total = max(total, o + need)
        o += Q.qlora_bwd_partials_bytes(lin, x.shape[0], dt)
    pack = torch.empty((total,), dtype=torch.uint8, device="cuda")
    for (lin, x, dy), t, (off, need) in zip(layers, ts, views):
        ws = pack[off:off + need] if packed else None   # else a workspace per layer
        _, ws = Q.qlora_bwd_partial(lin, x, dy, t=t, ws=ws)
        items.append((lin, x.shape[0], x.dtype, ws))
    got = Q.qlora_bwd_finish_batch(items)
    torch.cuda.synchronize()
    for n, ((dA, dB), (gA, gB)) in enumerate(zip(refs, got)):
        assert torch.equal(dA.view(torch.int32), gA.view(torch.int32)), f"layer {n} {SPECS[n]}: dA"
        assert torch.equal(dB.view(torch.int32), gB.view(torch.int32)), f"layer {n} {SPECS[n]}: dB"
