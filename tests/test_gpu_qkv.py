"""GPU parity of the query/key/value projection (ne_qkv_proj) against the double oracle.

Both sides read the same bf16 x and w (the oracle widens them to double).  The GPU accumulates in
fp32 over C terms (error below C * 2^-24 relative, 5e-5 at C = 768) and rounds each output once
to bf16: round to nearest even with 8 significand bits errs by at most 2^-8 = 3.9e-3 relative to
the output's magnitude.  Hence the bar e(X) = max|gpu - ref| / max|ref| <= 4e-3 per output tensor,
compared over whole tensors.
"""
import sys

import numpy as np
import pytest
import torch

import causal_gqa_flashattention_ne_amd as ne
import gen
import oracle

pytestmark = pytest.mark.gpu
TOL = 4e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_case(seed, B, T, C, Hq, Hkv, D, theta=10000.0):
    dev = torch.device("cuda:0")
    x, w = gen.qkv_case(seed, B, T, C, Hq, Hkv, D)
    ref = oracle.qkv_proj(x, w, Hq, Hkv, theta=theta)
    xd = torch.from_numpy(x).to(dev).to(torch.bfloat16).contiguous()
    wd = torch.from_numpy(w).to(dev).to(torch.bfloat16).contiguous()
    got = ne.qkv_proj(xd, wd, Hq, Hkv, rope_theta=theta)
    errs = []
    for name, g, r in zip("qkv", got, ref):
        g = g.float().cpu().numpy()
        assert g.shape == r.shape
        assert np.isfinite(g).all()
        errs.append(np.abs(g - r).max() / np.abs(r).max())
    log("  qkv B%d T%d C%d Hq%d Hkv%d D%d theta %s: e(q) %.2e e(k) %.2e e(v) %.2e"
        % (B, T, C, Hq, Hkv, D, theta, *errs))
    assert max(errs) <= TOL, errs


CASES = [
    # seed, B, T, C, Hq, Hkv, D
    (1, 2, 100, 128, 4, 2, 32),        # ragged token tail (200 rows), several feature tiles
    (2, 1, 513, 768, 12, 4, 64),       # the 116M width, 513 tokens
    (3, 3, 64, 256, 2, 1, 128),        # head_dim 128
    (4, 2, 77, 64, 3, 1, 32),          # 160 features: a partial feature tile; C = one k step
    (5, 1, 1, 192, 2, 2, 64),          # a single token
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%d-T%d-C%d-H%d-%d-D%d" % c[1:])
def test_qkv_parity(case):
    log("qkv case %s" % (case,))
    run_case(*case)


def test_qkv_rope_off():
    log("qkv rope off")
    run_case(6, 2, 130, 256, 4, 2, 64, theta=0.0)


def test_qkv_workload_full_size():
    wl = gen.QKV_WORKLOADS[1]
    log("qkv workload %s" % wl.name)
    run_case(wl.seed, wl.B, wl.T, wl.C, wl.Hq, wl.Hkv, wl.D, theta=wl.theta)


def test_qkv_feeds_attention():
    """The projection's rotated outputs through the library's forward without RoPE equal the
    forward with RoPE over the un-rotated projection (both from the library)."""
    dev = torch.device("cuda:0")
    x, w = gen.qkv_case(8, 2, 96, 256, 4, 2, 64)
    xd = torch.from_numpy(x).to(dev).to(torch.bfloat16).contiguous()
    wd = torch.from_numpy(w).to(dev).to(torch.bfloat16).contiguous()
    qr, kr, vr = ne.qkv_proj(xd, wd, 4, 2, rope_theta=10000.0)
    o1, l1 = ne.attn_fwd(qr, kr, vr, rope_theta=0.0)
    q_ref, k_ref, v_ref = oracle.qkv_proj(x, w, 4, 2, theta=10000.0)
    o_ref, l_ref = oracle.attention(gen.round_bf16(q_ref.astype(np.float32)), gen.round_bf16(k_ref.astype(np.float32)),
                                    gen.round_bf16(v_ref.astype(np.float32)), theta=0.0)
    e_o = np.abs(o1.float().cpu().numpy() - o_ref).max() / np.abs(o_ref).max()
    e_l = np.abs(l1.cpu().numpy() - l_ref).max() / np.abs(l_ref).max()
    log("  projection -> attention: e(O) %.2e e(L) %.2e" % (e_o, e_l))
    assert e_o <= 2e-2 and e_l <= 2e-2
