"""Pins for the multi-head layout maps of the oracle (CPU only): the layer
computed per head with np.einsum on [heads, K, hd] / [heads, r, hd] tensors
(the EinsumDense form "mk,hkd->mhd") equals the plain layer on the mapped
[K, N] / [r, N] tensors, forward and adapter gradients; the maps invert each
other and put output n at head n // hd, position n % hd."""

import numpy as np

from oracle import qlora_oracle as O


def _heads(seed, M=5, K=12, H=3, hd=4, r=2):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K))
    Wh = rng.standard_normal((H, K, hd))
    A = rng.standard_normal((K, r))
    Bh = rng.standard_normal((H, r, hd))
    dy = rng.standard_normal((M, H, hd))
    return x, Wh, A, Bh, dy


def test_maps_place_each_output_and_invert():
    H, rows, hd = 3, 2, 4
    T = np.arange(H * rows * hd).reshape(H, rows, hd)
    P = O.heads_to_plain(T)
    for h in range(H):
        for j in range(rows):
            for d in range(hd):
                assert P[j, h * hd + d] == T[h, j, d]
    assert np.array_equal(O.plain_to_heads(P, H), T)


def test_per_head_einsum_equals_the_plain_layer():
    x, Wh, A, Bh, dy = _heads(3)
    s = 8.0
    t = x @ A
    y_heads = np.einsum("mk,hkd->mhd", x, Wh) + s * np.einsum("mj,hjd->mhd", t, Bh)
    W, B = O.heads_to_plain(Wh), O.heads_to_plain(Bh)
    y_plain = x @ W + s * (t @ B)
    np.testing.assert_allclose(y_heads.reshape(x.shape[0], -1), y_plain, rtol=1e-13, atol=1e-13)
    # adapter gradients of <dy, y>: dB per head, dA, and dx
    dB_heads = s * np.einsum("mj,mhd->hjd", t, dy)
    dyp = dy.reshape(dy.shape[0], -1)
    np.testing.assert_allclose(dB_heads, O.plain_to_heads(s * t.T @ dyp, Wh.shape[0]),
                               rtol=1e-13, atol=1e-13)
    u_heads = np.einsum("mhd,hjd->mj", dy, Bh)
    np.testing.assert_allclose(u_heads, dyp @ B.T, rtol=1e-13, atol=1e-13)
    dx_heads = np.einsum("mhd,hkd->mk", dy, Wh) + s * u_heads @ A.T
    np.testing.assert_allclose(dx_heads, dyp @ W.T + s * (dyp @ B.T) @ A.T, rtol=1e-13, atol=1e-13)
