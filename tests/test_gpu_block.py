"""The attention block on the GPU (the library's projection, attention and RoPE kernels inside a
pre-norm block, block.py) against the double-precision oracle block, whose gradients are pinned
by central finite differences.

Both sides read the same bf16 x, gain and weights.  The GPU side rounds the normalised input, the
projections, O and dO to bf16 between its steps, so each output is held to the bf16 bar of the
attention itself, e(X) = max|gpu - ref| / max|ref| <= 2e-2, for y, dx, dg, dWqkv and dWo.
"""
import sys

import numpy as np
import pytest
import torch

import gen
import oracle
from causal_gqa_flashattention_ne_amd.block import block_forward_backward

pytestmark = pytest.mark.gpu
TOL = 2e-2


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("B,T,C,Hq,Hkv,D,theta", [
    (2, 64, 768, 12, 4, 64, 10000.0),       # the 116M model's block width and heads
    (1, 200, 256, 4, 2, 64, 10000.0),       # ragged T
    (2, 96, 128, 2, 1, 32, 0.0),            # no RoPE
    (1, 130, 256, 2, 1, 128, 10000.0),      # head_dim 128
])
def test_block_matches_oracle(B, T, C, Hq, Hkv, D, theta):
    log("block B%d T%d C%d Hq%d Hkv%d D%d theta %s" % (B, T, C, Hq, Hkv, D, theta))
    dev = torch.device("cuda:0")
    seed = 900 + T + C
    x, wqkv = gen.qkv_case(seed, B, T, C, Hq, Hkv, D)
    rng = np.random.default_rng(seed)
    g = gen.round_bf16((1.0 + 0.1 * rng.standard_normal(C)).astype(np.float32))
    wo = gen.round_bf16((rng.standard_normal((C, Hq * D)) / np.sqrt(Hq * D)).astype(np.float32))
    dy = gen.round_bf16(rng.standard_normal((B, T, C)).astype(np.float32))
    ref = oracle.block(x, g, wqkv, wo, dy, Hq, Hkv, theta=theta)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev).to(torch.bfloat16).contiguous()
    got = block_forward_backward(t(x), t(g), t(wqkv), t(wo), t(dy), Hq, Hkv, rope_theta=theta)
    errs = {}
    for name, a, r in zip(("y", "dx", "dg", "dwqkv", "dwo"), got, ref):
        a = a.cpu().numpy()
        assert a.shape == r.shape and np.isfinite(a).all()
        errs[name] = float(np.abs(a - r).max() / np.abs(r).max())
    log("  " + " ".join("e(%s) %.2e" % kv for kv in errs.items()))
    assert max(errs.values()) <= TOL, errs
