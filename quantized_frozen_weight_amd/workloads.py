"""Seeded synthetic workloads for the frozen-weight + LoRA linear.

This module only draws random tensors and names shapes. It holds none of the
method's arithmetic (no quantizer, no product, no rounding rule of the
method): the tests hand the same bytes to the CPU oracle and to the HIP
library, and the benchmark uses it to fill device buffers.

The shapes stand in for the workloads the pages train on (the datasets and
trained weights themselves are not used):

* ``single``   -- one 256->256 linear, fp32 compute (a small parity case).
* ``mlp``      -- the MNIST MLP of "Introduce QLoRA-like technique"
                  (benchmark.py: Flatten(784) then 32 Dense(1024) layers, batch
                  1024); LoRA rank 8, alpha 16, bf16 compute.
* ``gpt2``     -- GPT-2 base linears at 32 sequences of 128 tokens ("GPT2 &
                  Gemma Finetuning" of the same page; sequence length 128 in
                  "Parameter-efficient fine-tuning of GPT-2 with LoRA").
* ``gemma``    -- the Gemma-2B feed-forward kernels [2048,16384] and
                  [16384,2048] listed in the block-memory table of the
                  keras-llm-light README ("Weights quantization"), 512 tokens,
                  Student-t(3) weights to create outlier channels.
* ``w4``       -- the 4096 x 4096 4-bit layer with a 4096 x 4 fp32 adapter that
                  "How to fine-tune the 4-bit model?" describes.

Seeds follow ``1000*config + tensor_id + 10*layer`` with tensor ids
x=1, W=2, A=3, B=4, dy=5, so every tensor of every layer is reproducible on
its own.
"""

from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import List, Tuple

import numpy as np

TID_X, TID_W, TID_A, TID_B, TID_DY = 1, 2, 3, 4, 5


@dataclass(frozen=True)
class Workload:
    cid: int                       # 1..5
    name: str
    M: int                         # rows (tokens or batch)
    layers: Tuple[Tuple[int, int], ...]  # (K, N) per layer
    r: int
    alpha: float
    dtype: str                     # "f32" or "bf16": x, y, dy, dx
    wfmt: str                      # "w8", "w4g128" or "w8o"
    w_dist: Tuple = ("normal", 0.02)
    x_sigma: float = 1.0
    lora_sigma: float = 0.01
    dy_sigma: float = 1.0
    notes: str = ""

    def seed(self, tid: int, layer: int = 0) -> int:
        return 1000 * self.cid + tid + 10 * layer

    def ops_per_layer(self, K: int, N: int, M: int | None = None) -> int:
        """Algorithmic operations of one fwd+bwd of a K->N layer.

        Two per multiply-add: the base product (2MKN), the dx product (2MKN)
        and the six rank-r products x.A, t.B, dy.B^T, t^T.dy, x^T.u, u.A^T.
        """
        M = self.M if M is None else M
        return 4 * M * K * N + 6 * M * self.r * (K + N)

    def total_ops(self) -> int:
        return sum(self.ops_per_layer(K, N) for K, N in self.layers)


WORKLOADS = {
    1: Workload(1, "single", 64, ((256, 256),), r=4, alpha=32.0, dtype="f32",
                wfmt="w8", w_dist=("normal", 0.05)),
    2: Workload(2, "mlp", 1024, ((784, 1024),) + ((1024, 1024),) * 31, r=8,
                alpha=16.0, dtype="bf16", wfmt="w8", w_dist=("normal", 0.03)),
    3: Workload(3, "gpt2", 4096,
                ((768, 2304), (768, 768), (768, 3072), (3072, 768)), r=4,
                alpha=32.0, dtype="bf16", wfmt="w8", w_dist=("normal", 0.02)),
    4: Workload(4, "gemma", 512,
                ((2048, 16384), (2048, 16384), (16384, 2048)), r=8, alpha=16.0,
                dtype="bf16", wfmt="w8", w_dist=("student_t", 3.0, 0.02)),
    5: Workload(5, "w4", 2048, ((4096, 4096),), r=4, alpha=8.0, dtype="bf16",
                wfmt="w4g128", w_dist=("normal", 0.02)),
}


def _draw(seed: int, shape, dist) -> np.ndarray:
    rng = np.random.default_rng(seed)
    kind = dist[0]
    if kind == "normal":
        return (rng.standard_normal(shape, dtype=np.float32)
                * np.float32(dist[1]))
    if kind == "student_t":
        t = rng.standard_t(dist[1], size=shape).astype(np.float32)
        return t * np.float32(dist[2])
    raise ValueError(kind)


def weight(w: Workload, layer: int) -> np.ndarray:
    """Float weight [K, N] (the pages' kernel orientation)."""
    K, N = w.layers[layer]
    return _draw(w.seed(TID_W, layer), (K, N), w.w_dist)


def lora_A(w: Workload, layer: int) -> np.ndarray:
    K, _ = w.layers[layer]
    return _draw(w.seed(TID_A, layer), (K, w.r), ("normal", w.lora_sigma))


def lora_B(w: Workload, layer: int) -> np.ndarray:
    _, N = w.layers[layer]
    return _draw(w.seed(TID_B, layer), (w.r, N), ("normal", w.lora_sigma))


def activations(w: Workload, layer: int, M: int | None = None) -> np.ndarray:
    K, _ = w.layers[layer]
    M = w.M if M is None else M
    return _draw(w.seed(TID_X, layer), (M, K), ("normal", w.x_sigma))


def out_grad(w: Workload, layer: int, M: int | None = None) -> np.ndarray:
    _, N = w.layers[layer]
    M = w.M if M is None else M
    return _draw(w.seed(TID_DY, layer), (M, N), ("normal", w.dy_sigma))


def as_compute_dtype(a: np.ndarray, dtype: str):
    """Return (torch CPU tensor in the compute dtype, float32 numpy copy of it).

    For bf16 the cast is torch's own float32->bfloat16 conversion; the numpy
    copy holds exactly the values the device will see, widened to float32.
    """
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
        return t, t.float().numpy()
    if dtype == "f32":
        return t.clone(), t.numpy().copy()
    raise ValueError(dtype)


def with_format(w: Workload, wfmt: str) -> Workload:
    """The same workload (same seeds, so the same tensors) stored in another
    weight format, e.g. the Gemma kernels as outlier-compensated int8
    ("w8o", keras-llm-light README, "Simplified Int8Variable quantization")."""
    return replace(w, wfmt=wfmt, name=f"{w.name}_{wfmt}")


def small(cid: int, M: int, K: int, N: int, r: int | None = None) -> Workload:
    """A shrunken single-layer variant of workload ``cid`` for quick parity."""
    base = WORKLOADS[cid]
    return Workload(100 + cid, base.name + "_small", M, ((K, N),),
                    r=base.r if r is None else r, alpha=base.alpha,
                    dtype=base.dtype, wfmt=base.wfmt, w_dist=base.w_dist)
