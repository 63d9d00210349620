"""Pins for the oracle's forward pass: O and the natural-log row logsumexp L.

Independent references: torch's float64 CPU scaled_dot_product_attention (is_causal=True) with
K/V heads repeated contiguously (query head h reads kv head h // G), torch.logsumexp over the
masked score matrix, and closed forms.
"""
import numpy as np
import pytest
import torch

import gen
import oracle
from test_oracle_rope import rope_complex


def torch_ref(q, k, v, theta, scale=None):
    """O and L from torch float64 on the CPU, RoPE by complex multiplication."""
    B, Hq, T, D = q.shape
    G = Hq // k.shape[1]
    if theta > 0:
        q = rope_complex(q, theta)
        k = rope_complex(k, theta)
    s = scale if scale else 1.0 / np.sqrt(D)
    qt = torch.from_numpy(np.ascontiguousarray(q))
    kt = torch.from_numpy(np.ascontiguousarray(k)).repeat_interleave(G, dim=1)
    vt = torch.from_numpy(np.ascontiguousarray(v)).repeat_interleave(G, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=s)
    S = s * torch.matmul(qt, kt.transpose(-1, -2).contiguous())
    mask = torch.ones(T, T, dtype=torch.bool).triu(1)
    L = torch.logsumexp(S.masked_fill(mask, float("-inf")), dim=-1)
    return o.numpy(), L.numpy()


CASES = [
    # seed, B, Hq, Hkv, T, D, theta
    (1, 1, 2, 1, 9, 4, 0.0),
    (2, 2, 4, 2, 33, 8, 10000.0),
    (3, 1, 6, 2, 40, 16, 10.0),
    (4, 1, 3, 3, 17, 32, 10000.0),
    (5, 2, 4, 1, 64, 8, 10000.0),
]


@pytest.mark.parametrize("case", CASES)
def test_forward_vs_torch_float64(case):
    seed, B, Hq, Hkv, T, D, theta = case
    q, k, v, _ = gen.small_case(seed, B, Hq, Hkv, T, D)
    o, L = oracle.attention(q, k, v, theta=theta)
    o_ref, L_ref = torch_ref(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), theta)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, L_ref, rtol=0, atol=1e-12)


def test_explicit_scale():
    q, k, v, _ = gen.small_case(6, 1, 2, 2, 12, 8)
    o, L = oracle.attention(q, k, v, theta=10000.0, scale=0.3)
    o_ref, L_ref = torch_ref(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                             10000.0, 0.3)
    np.testing.assert_allclose(o, o_ref, atol=1e-12)
    np.testing.assert_allclose(L, L_ref, atol=1e-12)


def test_single_position_closed_form():
    # T = 1: the only key is the query's own position (R_0 = I): O = V, L = s <q, k>.
    q, k, v, _ = gen.small_case(7, 2, 4, 2, 1, 8)
    o, L = oracle.attention(q, k, v, theta=10000.0)
    G = 2
    kk = np.repeat(k, G, axis=1).astype(np.float64)
    vv = np.repeat(v, G, axis=1).astype(np.float64)
    np.testing.assert_array_equal(o, vv)
    np.testing.assert_allclose(L[..., 0], np.sum(q * kk, axis=-1)[..., 0] / np.sqrt(8), atol=1e-15)


def test_zero_keys_closed_form():
    # K = 0: every visible score is 0, so P_ij = 1/(i+1), O_i is the prefix mean of V and
    # L_i = ln(i+1) (natural log, diagonal included).
    T, D = 50, 8
    q, k, v, _ = gen.small_case(8, 1, 2, 1, T, D)
    k = np.zeros_like(k)
    o, L = oracle.attention(q, k, v, theta=10000.0)
    prefix = np.cumsum(v[0, 0].astype(np.float64), axis=0) / np.arange(1, T + 1)[:, None]
    for h in range(2):
        np.testing.assert_allclose(o[0, h], prefix, atol=1e-14)
        np.testing.assert_allclose(L[0, h], np.log(np.arange(1, T + 1)), atol=1e-14)


def test_softmax_rows_sum_to_one_and_exact_causal_zeros():
    # With V_j = e_j (one-hot, T <= D), O_i is exactly row i of P.
    T, D = 24, 32
    q, k, _, _ = gen.small_case(9, 1, 2, 1, T, D)
    v = np.zeros((1, 1, T, D))
    v[0, 0, np.arange(T), np.arange(T)] = 1.0
    o, _ = oracle.attention(q, k, v, theta=10000.0)
    P = o[0, :, :, :T]
    np.testing.assert_allclose(P.sum(-1), 1.0, atol=1e-13)
    assert np.all(P[:, np.triu_indices(T, 1)[0], np.triu_indices(T, 1)[1]] == 0.0)
    assert np.all(P[:, np.arange(T), np.arange(T)] > 0.0)
    assert np.all(o[0, :, :, T:] == 0.0)


def test_causal_invariance_forward_bitwise():
    T, i0 = 40, 17
    q, k, v, _ = gen.small_case(10, 1, 4, 2, T, 8)
    o1, L1 = oracle.attention(q, k, v, theta=10000.0)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    rq, rk, rv, _ = gen.small_case(99, 1, 4, 2, T, 8)
    q2[:, :, i0 + 1:] = rq[:, :, i0 + 1:] * 5
    k2[:, :, i0 + 1:] = rk[:, :, i0 + 1:] * 5
    v2[:, :, i0 + 1:] = rv[:, :, i0 + 1:] * 5
    o2, L2 = oracle.attention(q2, k2, v2, theta=10000.0)
    np.testing.assert_array_equal(o1[:, :, :i0 + 1], o2[:, :, :i0 + 1])
    np.testing.assert_array_equal(L1[:, :, :i0 + 1], L2[:, :, :i0 + 1])
    assert not np.array_equal(o1[:, :, i0 + 1:], o2[:, :, i0 + 1:])


def test_gqa_equals_mha_with_repeated_kv():
    q, k, v, _ = gen.small_case(11, 2, 6, 2, 20, 8)
    o_g, L_g = oracle.attention(q, k, v, theta=10000.0)
    o_m, L_m = oracle.attention(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), theta=10000.0)
    np.testing.assert_array_equal(o_g, o_m)
    np.testing.assert_array_equal(L_g, L_m)


def test_group_subset_matches_full():
    q, k, v, do = gen.small_case(12, 2, 4, 2, 16, 8)
    full = oracle.attention(q, k, v, do, theta=10000.0)
    part = oracle.attention(q, k, v, do, theta=10000.0, groups=[(1, 0)])
    o, L, dq, dk, dv = part
    np.testing.assert_array_equal(o[1, 0:2], full[0][1, 0:2])
    np.testing.assert_array_equal(dq[1, 0:2], full[2][1, 0:2])
    np.testing.assert_array_equal(dk[1, 0], full[3][1, 0])
    assert np.isnan(o[0]).all() and np.isnan(dk[1, 1]).all()


def test_hand_worked_example_t2_d2():
    # Worked by hand.  D = 2, so the single RoPE frequency is 1 and position t rotates by t rad.
    # q0 = (1,0), q1 = (0,1), k0 = k1 = (1,0), v0 = (1,2), v1 = (3,4), s = 1/sqrt(2).
    # Rotated: q~1 = (-sin 1, cos 1), k~1 = (cos 1, sin 1); q~0 = k~0 = (1, 0).
    # Row 0: only key 0, O_0 = v0, L_0 = s.
    # Row 1: S_10 = -s sin 1, S_11 = s(-sin1 cos1 + cos1 sin1) = 0, so with e = exp(-s sin 1):
    #   P_10 = e/(1+e), P_11 = 1/(1+e), O_1 = P_10 v0 + P_11 v1, L_1 = ln(1 + e).
    q = np.array([[[[1.0, 0.0], [0.0, 1.0]]]])
    k = np.array([[[[1.0, 0.0], [1.0, 0.0]]]])
    v = np.array([[[[1.0, 2.0], [3.0, 4.0]]]])
    s = 1 / np.sqrt(2)
    e = np.exp(-s * np.sin(1.0))
    o, L = oracle.attention(q, k, v, theta=10000.0)
    np.testing.assert_allclose(o[0, 0, 0], [1.0, 2.0], atol=1e-15)
    np.testing.assert_allclose(o[0, 0, 1], e / (1 + e) * np.array([1, 2]) + 1 / (1 + e) * np.array([3, 4]),
                               atol=1e-15)
    np.testing.assert_allclose(L[0, 0], [s, np.log1p(e)], atol=1e-15)
