"""Pins of the decode oracle (oracle.decode) against the full causal attention oracle.

A decode call is the last n rows of the full forward over the first kv_len[b] positions, with
the cache holding the keys rotated at their own positions.  The full oracle (itself pinned by
finite differences, closed forms and library routines in test_oracle_forward.py) is run on the
raw keys with its own RoPE, so the position convention (token i of sequence b at kv_len[b] - n + i),
the causal prefix among the new tokens, the GQA head map, the scale and L are all checked.
"""
import numpy as np
import pytest

import oracle


def _case(B, Hq, Hkv, T, D, seed):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, Hq, T, D))
    k = r.standard_normal((B, Hkv, T, D))
    v = r.standard_normal((B, Hkv, T, D))
    return q, k, v


@pytest.mark.parametrize("n,Hq,Hkv", [(1, 4, 2), (3, 4, 2), (5, 3, 3), (2, 6, 1)])
@pytest.mark.parametrize("theta", [10000.0, 10.0, 0.0])
def test_decode_is_last_rows_of_full_attention(n, Hq, Hkv, theta):
    B, T, D = 3, 21, 8
    q, k, v = _case(B, Hq, Hkv, T, D, 11 + n)
    kv_len = [21, 13, n]                                   # ragged, including a cache of only the new tokens
    kc = oracle.rope(k, theta) if theta > 0 else k         # cache: keys rotated at their positions
    qn = np.zeros((B, Hq, n, D))
    for b in range(B):
        qn[b] = q[b, :, kv_len[b] - n:kv_len[b]]
    o, L = oracle.decode(qn, kc, v, kv_len, theta=theta, scale=0.37)
    for b in range(B):
        lb = kv_len[b]
        of, Lf = oracle.attention(q[b:b + 1, :, :lb], k[b:b + 1, :, :lb], v[b:b + 1, :, :lb], theta=theta,
                                  scale=0.37)
        np.testing.assert_allclose(o[b], of[0, :, lb - n:], rtol=0, atol=1e-12)
        np.testing.assert_allclose(L[b], Lf[0, :, lb - n:], rtol=0, atol=1e-12)


def test_rows_past_kv_len_are_ignored():
    B, Hq, Hkv, T, D, n = 2, 4, 2, 16, 8, 2
    q, k, v = _case(B, Hq, Hkv, T, D, 5)
    kv_len = [10, 16]
    o1, L1 = oracle.decode(q[:, :, :n], k, v, kv_len, theta=0.0)
    k2, v2 = k.copy(), v.copy()
    k2[0, :, 10:] = 1e6                                     # garbage beyond the valid rows
    v2[0, :, 10:] = np.nan
    o2, L2 = oracle.decode(q[:, :, :n], k2, v2, kv_len, theta=0.0)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(L1, L2)


def test_single_visible_key():
    # the first token of a sequence sees only itself: o = v_0, L = scale * q.k
    B, Hq, Hkv, T, D = 1, 2, 1, 4, 8
    q, k, v = _case(B, Hq, Hkv, T, D, 7)
    o, L = oracle.decode(q[:, :, :1], k, v, [1], theta=0.0, scale=0.5)
    np.testing.assert_allclose(o[0, :, 0], np.repeat(v[0, :, 0], 2, axis=0), rtol=0, atol=1e-15)
    np.testing.assert_allclose(L[0, :, 0], 0.5 * (q[0, :, 0] @ k[0, 0, 0]), rtol=0, atol=1e-12)
