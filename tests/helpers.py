"""Shared test helpers: tolerance rule and device round trips."""

from __future__ import annotations

import numpy as np

# Tolerances: float32 compute 1e-5, bf16 compute (outputs and all gradients)
# 2e-2, relative per element against max(|oracle|, rms(oracle)) so that
# entries near zero are judged on the tensor's scale.
RTOL = {"f32": 1e-5, "bf16": 2e-2}
# float32 outputs of every workload: t = x A (saved by the forward) and the
# adapter gradients dA, dB (the adapter is float32 in every workload)
RTOL_F32 = RTOL["f32"]


def rel_errors(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    rms = float(np.sqrt(np.mean(want * want))) if want.size else 0.0
    denom = np.maximum(np.abs(want), rms)
    denom = np.where(denom == 0, 1.0, denom)
    elem = np.abs(got - want) / denom
    nw = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300))
    return elem, nw


def assert_close(got, want, rtol, what=""):
    """Per-element relative check; NaN and +-inf must sit at the same places
    (an infinity must match exactly), the finite rest within rtol."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.array_equal(np.isnan(got), np.isnan(want)), f"{what}: NaN pattern differs"
    assert np.array_equal(np.isposinf(got), np.isposinf(want)), f"{what}: +inf pattern differs"
    assert np.array_equal(np.isneginf(got), np.isneginf(want)), f"{what}: -inf pattern differs"
    ok = np.isfinite(want)
    elem, nw = rel_errors(got[ok], want[ok])
    worst = float(elem.max()) if elem.size else 0.0
    assert worst <= rtol, f"{what}: max rel err {worst:.3e} > {rtol} (normwise {nw:.3e})"
    return worst, nw


def to_numpy(t):
    """Device tensor -> numpy (bf16 widened to float32 exactly)."""
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.numpy()


def same_bits_f32(a, b):
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = np.ascontiguousarray(b, dtype=np.float32)
    both_nan = np.isnan(a) & np.isnan(b)
    return bool(np.all((a.view(np.uint32) == b.view(np.uint32)) | both_nan))


def same_bits_f16(a, b):
    a = np.ascontiguousarray(a, dtype=np.float16)
    b = np.ascontiguousarray(b, dtype=np.float16)
    both_nan = np.isnan(a) & np.isnan(b)
    return bool(np.all((a.view(np.uint16) == b.view(np.uint16)) | both_nan))
