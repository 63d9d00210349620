"""Pins of the oracle's query/key/value projection (oracle.qkv_proj) to facts outside itself.

The projection is y = x W^T split into [query heads | key heads | value heads] (head-major, d
fastest), with RoPE on the query and key heads at positions 0 .. T-1 (agentlenshq NanoEuler page,
"핵심 아키텍처 및 설계" and "기술 사양").  The pins: brute force on tiny inputs with D = 2 (a
rotation by t radians), one-hot weights that select input columns, linearity in the weights, and
consistency with the attention oracle's own rotation of raw projections.
"""
import math

import numpy as np
import pytest

import oracle


def test_brute_force_tiny():
    """Pure-Python sums and explicit 2-D rotations: D = 2, so the pair rotates by t radians."""
    rng = np.random.default_rng(3)
    B, T, C, Hq, Hkv, D = 2, 4, 3, 2, 1, 2
    x = rng.standard_normal((B, T, C))
    w = rng.standard_normal(((Hq + 2 * Hkv) * D, C))
    q, k, v = oracle.qkv_proj(x, w, Hq, Hkv, theta=10000.0)
    for b in range(B):
        for t in range(T):
            feats = [sum(x[b][t][c] * w[f][c] for c in range(C)) for f in range((Hq + 2 * Hkv) * D)]
            for head in range(Hq + 2 * Hkv):
                y0, y1 = feats[head * D], feats[head * D + 1]
                if head < Hq + Hkv:         # query and key heads are rotated by angle t
                    y0, y1 = y0 * math.cos(t) - y1 * math.sin(t), y0 * math.sin(t) + y1 * math.cos(t)
                if head < Hq:
                    got = q[b, head, t]
                elif head < Hq + Hkv:
                    got = k[b, head - Hq, t]
                else:
                    got = v[b, head - Hq - Hkv, t]
                assert abs(got[0] - y0) < 1e-12 and abs(got[1] - y1) < 1e-12


@pytest.mark.parametrize("theta", [0.0, 10000.0])
def test_one_hot_weights_select_columns(theta):
    """Feature f reads input column sel[f] only: the outputs are those columns, placed by head and
    rotated (theta > 0) exactly as the attention oracle's RoPE rotates a [B, H, T, D] tensor."""
    rng = np.random.default_rng(5)
    B, T, C, Hq, Hkv, D = 2, 7, 16, 3, 1, 8
    N = (Hq + 2 * Hkv) * D
    sel = rng.integers(0, C, size=N)
    w = np.zeros((N, C))
    w[np.arange(N), sel] = 1.0
    x = rng.standard_normal((B, T, C))
    q, k, v = oracle.qkv_proj(x, w, Hq, Hkv, theta=theta)
    picked = x[:, :, sel]                                # [B, T, N]
    heads = picked.reshape(B, T, Hq + 2 * Hkv, D).transpose(0, 2, 1, 3)
    q0, k0, v0 = heads[:, :Hq], heads[:, Hq:Hq + Hkv], heads[:, Hq + Hkv:]
    if theta > 0:
        q0, k0 = oracle.rope(q0, theta), oracle.rope(k0, theta)
    assert np.array_equal(v, v0)
    np.testing.assert_allclose(q, q0, rtol=0, atol=1e-15)
    np.testing.assert_allclose(k, k0, rtol=0, atol=1e-15)


def test_linear_in_weights():
    rng = np.random.default_rng(7)
    B, T, C, Hq, Hkv, D = 1, 9, 24, 4, 2, 16
    x = rng.standard_normal((B, T, C))
    w1 = rng.standard_normal(((Hq + 2 * Hkv) * D, C))
    w2 = rng.standard_normal(w1.shape)
    a = 0.37
    lhs = oracle.qkv_proj(x, a * w1 + w2, Hq, Hkv)
    r1, r2 = oracle.qkv_proj(x, w1, Hq, Hkv), oracle.qkv_proj(x, w2, Hq, Hkv)
    for got, y1, y2 in zip(lhs, r1, r2):
        np.testing.assert_allclose(got, a * y1 + y2, rtol=1e-12, atol=1e-12)


def test_consistent_with_attention_rotation():
    """Attention over the rotated projections without RoPE equals attention over the raw
    projections with RoPE: both rotate position t of every head by the same R_t."""
    rng = np.random.default_rng(11)
    B, T, C, Hq, Hkv, D = 1, 20, 32, 4, 2, 8
    x = rng.standard_normal((B, T, C))
    w = rng.standard_normal(((Hq + 2 * Hkv) * D, C)) / np.sqrt(C)
    qr, kr, vr = oracle.qkv_proj(x, w, Hq, Hkv, theta=10000.0)
    q0, k0, v0 = oracle.qkv_proj(x, w, Hq, Hkv, theta=0.0)
    o1, L1 = oracle.attention(qr, kr, vr, theta=0.0)
    o2, L2 = oracle.attention(q0, k0, v0, theta=10000.0)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(L1, L2, rtol=1e-12, atol=1e-12)


def test_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.qkv_proj(np.zeros((1, 2, 8)), np.zeros((10, 7)), 1, 1)
    with pytest.raises(ValueError):
        oracle.qkv_proj(np.zeros((1, 2, 8)), np.zeros((10, 8)), 2, 1)
