"""Pins of the oracle's attention block (oracle.block) and its RMSNorm.

The block's analytic gradients (with respect to x, the norm gain, the packed projection weights
and the output projection) are checked against central finite differences in double, the check
the agentlenshq NanoEuler page ("검증 및 안정성") describes for the whole model; RMSNorm against
its definition in closed form.
"""
import numpy as np
import pytest

import oracle


def test_rmsnorm_closed_form():
    x = np.array([[3.0, 4.0]])                      # mean square 12.5
    g = np.array([2.0, 0.5])
    np.testing.assert_allclose(oracle.rmsnorm(x, g, eps=0.0), [[3 / np.sqrt(12.5) * 2, 4 / np.sqrt(12.5) * 0.5]],
                               rtol=1e-15)
    y = oracle.rmsnorm(np.random.default_rng(1).standard_normal((4, 7)), np.ones(7), eps=0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-13)   # unit RMS with unit gain


def fd_errors(B, T, C, Hq, Hkv, D, theta, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, T, C))
    g = 1.0 + 0.1 * rng.standard_normal(C)
    wq = rng.standard_normal(((Hq + 2 * Hkv) * D, C)) / np.sqrt(C)
    wo = rng.standard_normal((C, Hq * D)) / np.sqrt(Hq * D)
    dy = rng.standard_normal((B, T, C))
    _, dx, dg, dwq, dwo = oracle.block(x, g, wq, wo, dy, Hq, Hkv, theta=theta)

    def loss():
        return np.sum(oracle.block(x, g, wq, wo, dy, Hq, Hkv, theta=theta)[0] * dy)

    h = 1e-5
    errs = {}
    for name, arr, grad in (("x", x, dx), ("g", g, dg), ("wqkv", wq, dwq), ("wo", wo, dwo)):
        num = np.zeros_like(arr)
        for i in np.ndindex(arr.shape):
            old = arr[i]
            arr[i] = old + h
            lp = loss()
            arr[i] = old - h
            lm = loss()
            arr[i] = old
            num[i] = (lp - lm) / (2 * h)
        errs[name] = np.abs(num - grad).max() / np.abs(grad).max()
    return errs


@pytest.mark.parametrize("shape,theta", [((1, 5, 16, 2, 1, 8), 10000.0), ((2, 4, 8, 2, 2, 4), 10.0),
                                         ((1, 6, 12, 3, 1, 4), 0.0)])
def test_block_gradients_match_central_differences(shape, theta):
    errs = fd_errors(*shape, theta=theta, seed=sum(shape))
    assert max(errs.values()) < 1e-7, errs


def test_block_output_is_residual_plus_projection():
    """y - x equals the attention output of the normalised input, heads concatenated, times wo^T."""
    rng = np.random.default_rng(4)
    B, T, C, Hq, Hkv, D = 1, 6, 16, 2, 1, 8
    x = rng.standard_normal((B, T, C))
    g = np.ones(C)
    wq = rng.standard_normal(((Hq + 2 * Hkv) * D, C)) / 4
    wo = rng.standard_normal((C, Hq * D)) / 4
    y = oracle.block(x, g, wq, wo, np.zeros_like(x), Hq, Hkv)[0]
    q, k, v = oracle.qkv_proj(oracle.rmsnorm(x, g), wq, Hq, Hkv)
    o, _ = oracle.attention(q, k, v, theta=0.0)
    np.testing.assert_allclose(y - x, o.transpose(0, 2, 1, 3).reshape(B, T, Hq * D) @ wo.T, rtol=1e-12, atol=1e-12)
