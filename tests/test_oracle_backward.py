"""Pins for the oracle's backward pass (dQ, dK, dV for the loss <dO, O>).

The pages check every analytic gradient against central finite differences in double precision
(agentlenshq page "NanoEuler: C와 CUDA로 밑바닥부터 구축한 GPT-2 규모의 LLM", section
"검증 및 안정성"); the first test does exactly that.  The others compare with torch float64 autograd
through SDPA (RoPE applied by complex multiplication), and check closed forms and invariants.
"""
import numpy as np
import pytest
import torch

import gen
import oracle
from test_oracle_rope import rope_complex


def loss(q, k, v, do, theta):
    o, _ = oracle.attention(q, k, v, theta=theta, nthreads=1)
    return float(np.sum(o * do))


@pytest.mark.parametrize("shape", [(1, 2, 1, 5, 4), (2, 4, 2, 7, 8), (1, 3, 3, 6, 4)])
@pytest.mark.parametrize("theta", [0.0, 10.0, 10000.0])
def test_central_finite_differences(shape, theta):
    B, Hq, Hkv, T, D = shape
    q, k, v, do = [x.astype(np.float64) for x in gen.small_case(20 + T, B, Hq, Hkv, T, D)]
    _, _, dq, dk, dv = oracle.attention(q, k, v, do, theta=theta, nthreads=1)
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.empty_like(x)
        flat = x.reshape(-1)
        for idx in range(flat.size):
            h = 1e-5 * max(1.0, abs(flat[idx]))
            old = flat[idx]
            flat[idx] = old + h
            lp = loss(q, k, v, do, theta)
            flat[idx] = old - h
            lm = loss(q, k, v, do, theta)
            flat[idx] = old
            fd.reshape(-1)[idx] = (lp - lm) / (2 * h)
        err = np.max(np.abs(fd - g)) / np.max(np.abs(g))
        assert err < 1e-7, (name, err)


def torch_grads(q, k, v, do, theta):
    B, Hq, T, D = q.shape
    G = Hq // k.shape[1]
    qt = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    kt = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    vt = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    w = theta ** (-(2.0 * torch.arange(D // 2, dtype=torch.float64)) / D)
    ang = torch.outer(torch.arange(T, dtype=torch.float64), w)
    rot = torch.polar(torch.ones_like(ang), ang)

    def rope(x):
        xc = torch.view_as_complex(x.reshape(*x.shape[:-1], D // 2, 2))
        return torch.view_as_real(xc * rot).reshape(x.shape)

    kr = rope(kt).repeat_interleave(G, dim=1)
    vr = vt.repeat_interleave(G, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(rope(qt), kr, vr, is_causal=True)
    (o * torch.tensor(do, dtype=torch.float64)).sum().backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


@pytest.mark.parametrize("case", [(31, 2, 4, 2, 33, 8, 10000.0), (32, 1, 6, 3, 50, 16, 10.0),
                                  (33, 1, 2, 2, 64, 32, 10000.0)])
def test_backward_vs_torch_autograd(case):
    seed, B, Hq, Hkv, T, D, theta = case
    q, k, v, do = [x.astype(np.float64) for x in gen.small_case(seed, B, Hq, Hkv, T, D)]
    _, _, dq, dk, dv = oracle.attention(q, k, v, do, theta=theta)
    tq, tk, tv = torch_grads(q, k, v, do, theta)
    for a, b in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12 * max(1.0, np.abs(b).max()))


def test_single_position_backward():
    # T = 1: P = 1, so dS = 0: dQ = dK = 0 exactly, dV = dO (summed over the group).
    q, k, v, do = gen.small_case(34, 1, 4, 2, 1, 8)
    _, _, dq, dk, dv = oracle.attention(q, k, v, do, theta=10000.0)
    assert np.all(dq == 0.0) and np.all(dk == 0.0)
    np.testing.assert_allclose(dv, do.reshape(1, 2, 2, 1, 8).sum(2), atol=1e-15)


def test_rotated_dk_sums_to_zero():
    # sum_j dS_ij = 0 for every row, hence sum_t R_t dK[b, g, t] = 0 for every (b, g).
    q, k, v, do = gen.small_case(35, 2, 4, 2, 45, 16)
    _, _, dq, dk, dv = oracle.attention(q, k, v, do, theta=10000.0)
    s = oracle.rope(dk, 10000.0).sum(axis=2)
    assert np.abs(s).max() < 1e-12 * np.abs(dk).max() * 45


def test_gqa_grads_equal_summed_mha_grads():
    q, k, v, do = gen.small_case(36, 1, 6, 2, 19, 8)
    _, _, dq, dk, dv = oracle.attention(q, k, v, do, theta=10000.0)
    _, _, dq_m, dk_m, dv_m = oracle.attention(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1),
                                              do, theta=10000.0)
    np.testing.assert_allclose(dq, dq_m, atol=1e-14)
    np.testing.assert_allclose(dk, dk_m.reshape(1, 2, 3, 19, 8).sum(2), atol=1e-13)
    np.testing.assert_allclose(dv, dv_m.reshape(1, 2, 3, 19, 8).sum(2), atol=1e-13)


def test_dv_linear_in_do_and_independent_of_v():
    q, k, v, do = gen.small_case(37, 1, 2, 1, 12, 8)
    _, _, _, _, dv1 = oracle.attention(q, k, v, do, theta=10000.0)
    _, _, _, _, dv2 = oracle.attention(q, k, v * 3.0 + 1.0, 2.0 * do, theta=10000.0)
    np.testing.assert_allclose(dv2, 2.0 * dv1, atol=1e-13)


def test_causal_invariance_dq_bitwise():
    T, i0 = 30, 11
    q, k, v, do = gen.small_case(38, 1, 2, 1, T, 8)
    _, _, dq1, _, _ = oracle.attention(q, k, v, do, theta=10000.0)
    q2, k2, v2, do2 = q.copy(), k.copy(), v.copy(), do.copy()
    for a in (q2, k2, v2, do2):
        a[:, :, i0 + 1:] = 3.0 * a[:, :, i0 + 1:] + 0.5
    _, _, dq2, _, _ = oracle.attention(q2, k2, v2, do2, theta=10000.0)
    np.testing.assert_array_equal(dq1[:, :, :i0 + 1], dq2[:, :, :i0 + 1])
