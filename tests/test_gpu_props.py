"""GPU properties that hold at any size: standalone RoPE vs the oracle, the RoPE table, bitwise
forward determinism, bitwise determinism of the bf16 and float32 backward (no atomics anywhere:
partial sums are added in a fixed order), causal invariance of the forward (and of dQ, bitwise),
GQA = MHA with repeated K/V, and the sum_t R_t dK_t = 0 identity at full size.
"""
import numpy as np
import pytest
import torch

import causal_gqa_flashattention_ne_amd as ne
import gen
import oracle
from parity_util import TOL, rel_err, run_gpu, to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [32, 64])
@pytest.mark.parametrize("pos_offset,inverse", [(0, False), (0, True), (37, False), (5, True)])
def test_rope_apply_vs_oracle(dtype, D, pos_offset, inverse):
    x = gen.tensor(40 + D, 0, "q", (2, 3, 77, D), dtype=dtype)
    xd = to_dev(x, dtype)
    y = to_np(ne.rope_apply(xd, 10000.0, inverse=inverse, pos_offset=pos_offset))
    ref = oracle.rope(x, 10000.0, inverse=inverse, pos_offset=pos_offset)
    tol = 1e-6 if dtype == "f32" else 2 ** -8
    assert rel_err(y, ref) <= tol
    # in place
    ne.rope_apply(xd, 10000.0, inverse=inverse, pos_offset=pos_offset, out=xd)
    assert np.array_equal(to_np(xd), y)


def test_rope_table_values():
    T, D, theta = 2048, 64, 10000.0
    cs = ne.rope_table(T, D, theta, "cuda:0").cpu().numpy()
    w = theta ** (-(2.0 * np.arange(D // 2)) / D)
    ang = np.outer(np.arange(T), w)
    ref = np.stack([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32)
    # double evaluation rounded to float32: at most one float32 ulp apart from numpy's libm
    ulp = np.spacing(np.abs(ref).astype(np.float32))
    assert np.all(np.abs(cs - ref) <= ulp)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_forward_bitwise_deterministic_and_causal_invariant(dtype):
    B, Hq, Hkv, T, D, i0 = 2, 4, 2, 300, 64, 141
    q, k, v, do = gen.small_case(91, B, Hq, Hkv, T, D, dtype)
    a = run_gpu(q, k, v, do, dtype)
    b = run_gpu(q, k, v, do, dtype)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    r = gen.small_case(92, B, Hq, Hkv, T, D, dtype)
    q2, k2, v2, do2 = (x.copy() for x in (q, k, v, do))
    for dst, src in zip((q2, k2, v2, do2), r):
        dst[:, :, i0 + 1:] = src[:, :, i0 + 1:]
    c = run_gpu(q2, k2, v2, do2, dtype)
    assert np.array_equal(a[0][:, :, :i0 + 1], c[0][:, :, :i0 + 1])
    assert np.array_equal(a[1][:, :, :i0 + 1], c[1][:, :, :i0 + 1])
    # dQ of earlier rows depends only on earlier positions (both paths sum in a fixed order: bits)
    assert np.array_equal(c[2][:, :, :i0 + 1], a[2][:, :, :i0 + 1])


@pytest.mark.parametrize("shape", [(2, 6, 2, 300, 64), "gpt116m-layer-bf16"])
def test_backward_bitwise_deterministic_bf16(shape):
    # the bf16 backward sums with no atomics (dK/dV over the group's heads in registers, dQ once
    # per query block), so two runs on the same inputs agree bit for bit, also on the full layer
    if isinstance(shape, str):
        w = next(x for x in gen.WORKLOADS.values() if x.name == shape)
        q, k, v, do = gen.layer_inputs(w)
    else:
        B, Hq, Hkv, T, D = shape
        q, k, v, do = gen.small_case(71, B, Hq, Hkv, T, D, "bf16")
    a = run_gpu(q, k, v, do, "bf16")
    b = run_gpu(q, k, v, do, "bf16")
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("T", [200, 300])
def test_backward_bitwise_deterministic_f32(T):
    # float32: no atomics either: dQ through one slice per 128-key tile and dK / dV through
    # per-share slices, each added in order by the finalize pass, so every output repeats bit for
    # bit (T = 300: three key tiles, so rows past 256 sum three dQ slices)
    q, k, v, do = gen.small_case(72, 2, 4, 2, T, 32, "f32")
    a = run_gpu(q, k, v, do, "f32")
    b = run_gpu(q, k, v, do, "f32")
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gqa_equals_mha_with_repeated_kv(dtype):
    B, Hq, Hkv, T, D = 1, 6, 2, 200, 64
    G = Hq // Hkv
    q, k, v, do = gen.small_case(93, B, Hq, Hkv, T, D, dtype)
    g = run_gpu(q, k, v, do, dtype)
    m = run_gpu(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), do, dtype)
    assert np.array_equal(g[0], m[0]) and np.array_equal(g[1], m[1])
    assert rel_err(g[2], m[2]) <= TOL[dtype] / 10
    # the MHA run rounds each head's dK/dV to the element type before the sum; the GQA kernel
    # sums the heads in float32 first, so the two agree to the parity bar, not bitwise
    for i in (3, 4):
        summed = m[i].reshape(B, Hkv, G, T, D).sum(2)
        assert rel_err(g[i], summed) <= TOL[dtype]


def test_rotated_dk_sums_to_zero_full_size():
    w = gen.WORKLOADS[3]
    q, k, v, do = gen.layer_inputs(w)
    _, _, dq, dk, dv = run_gpu(q, k, v, do, w.dtype)
    s = oracle.rope(dk, w.theta).sum(axis=2)           # [B, Hkv, D]
    # each sum cancels to roughly the rounding noise of T terms
    assert np.abs(s).max() <= 0.05 * np.abs(dk).max() * np.sqrt(w.T)
    assert np.isfinite(dq).all() and np.isfinite(dv).all()


def test_python_binding_rejects_bad_inputs():
    q = torch.zeros(1, 4, 16, 64, device="cuda:0", dtype=torch.bfloat16)
    k = torch.zeros(1, 3, 16, 64, device="cuda:0", dtype=torch.bfloat16)
    with pytest.raises(ne.NeError) as ei:
        ne.attn_fwd(q, k, k)
    assert ei.value.code == -2
    with pytest.raises(ValueError):
        ne.attn_fwd(q, q[:, :2].contiguous().float(), q[:, :2].contiguous())
    with pytest.raises(ValueError):
        ne.attn_fwd(q.transpose(2, 3), q, q)
