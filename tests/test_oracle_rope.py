"""Pins for the oracle's RoPE (rotary position embedding on queries and keys).

The rotation is checked against an independent complex-number formulation: pair (x[2i], x[2i+1])
is the complex number x[2i] + 1j*x[2i+1], multiplied by exp(1j * t * w_i) with
w_i = theta^(-2i/D).  Also: R_0 = I, norm preservation, R^T R = I, and the relative-position
property <R_m q, R_n k> = <R_(m+c) q, R_(n+c) k> that makes RoPE encode relative positions
(byte-level GPT page, "Core Mechanics").
"""
import numpy as np
import pytest

import gen
import oracle


def rope_complex(x, theta, pos_offset=0, inverse=False):
    B, H, T, D = x.shape
    z = x[..., 0::2] + 1j * x[..., 1::2]
    w = theta ** (-(2.0 * np.arange(D // 2)) / D)
    t = np.arange(T) + pos_offset
    rot = np.exp(1j * np.outer(t, w))
    if inverse:
        rot = np.conj(rot)
    z = z * rot[None, None]
    y = np.empty_like(x)
    y[..., 0::2] = z.real
    y[..., 1::2] = z.imag
    return y


@pytest.mark.parametrize("theta", [10.0, 10000.0, 500000.0])
@pytest.mark.parametrize("D", [2, 8, 64])
@pytest.mark.parametrize("pos_offset", [0, 37])
def test_rope_matches_complex_formulation(theta, D, pos_offset):
    x = gen.tensor(11, 0, "q", (2, 3, 50, D)).astype(np.float64)
    for inverse in (False, True):
        got = oracle.rope(x, theta, inverse=inverse, pos_offset=pos_offset)
        want = rope_complex(x, theta, pos_offset, inverse)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_rope_d2_rotates_by_position_in_radians():
    # D = 2: the only frequency is theta^0 = 1, so position t rotates by exactly t radians.
    x = np.zeros((1, 1, 4, 2))
    x[..., 0] = 1.0
    y = oracle.rope(x, 10000.0)
    t = np.arange(4)
    np.testing.assert_allclose(y[0, 0, :, 0], np.cos(t), atol=1e-15)
    np.testing.assert_allclose(y[0, 0, :, 1], np.sin(t), atol=1e-15)


def test_rope_identity_norm_inverse_relative():
    x = gen.tensor(12, 0, "k", (1, 2, 64, 16)).astype(np.float64)
    y = oracle.rope(x, 10000.0)
    np.testing.assert_array_equal(y[:, :, 0], x[:, :, 0])          # R_0 = I
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    back = oracle.rope(y, 10000.0, inverse=True)
    np.testing.assert_allclose(back, x, atol=1e-13)                 # R^T R = I
    off = oracle.rope(x, 10000.0, pos_offset=5)
    np.testing.assert_allclose(off[:, :, :59], oracle.rope(x, 10000.0)[:, :, 5:] * 0 +
                               rope_complex(x, 10000.0, 5)[:, :, :59], atol=1e-12)
    # relative property: <R_m q, R_n k> depends on m - n only
    q = x[0, 0, 3]
    k = x[0, 1, 9]
    def at(v, p):
        arr = np.zeros((1, 1, p + 1, 16))
        arr[0, 0, p] = v
        return oracle.rope(arr, 10000.0)[0, 0, p]
    a = at(q, 20) @ at(k, 7)
    b = at(q, 33) @ at(k, 20)
    assert abs(a - b) < 1e-12


def test_rope_theta_zero_is_identity():
    x = gen.tensor(13, 0, "q", (1, 1, 8, 4)).astype(np.float64)
    np.testing.assert_array_equal(oracle.rope(x, 0.0), x)
