"""GPU parity at the largest attention shape the C ABI accepts.

A [B, Hq, T, D] tensor may hold at most 2^31 - 1 elements; here the query, output and gradient
tensors hold 2^31 - 32768 (B = 65535, Hq = 8, Hkv = 2, T = 64, D = 64, bf16, RoPE on), so every
element offset, grid size and per-row index of the forward, the backward and the training pair
runs near the top of its range (about 30 GB of buffers).  Inputs are drawn on the device
(gen.device_normals); the first, a middle and the last kv group (all their query heads and
positions) are read back and compared with the oracle at the bf16 bar, relative to each
output's largest magnitude within the group.
"""
import sys

import numpy as np
import pytest
import torch

import causal_gqa_flashattention_ne_amd as ne
import gen
import oracle
from parity_util import TOL, rel_err

pytestmark = pytest.mark.gpu

B, HQ, HKV, T, D = 65535, 8, 2, 64, 64
G = HQ // HKV
GROUPS = [(0, 0), (B // 2, 1), (B - 1, HKV - 1)]


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def group_slices(b, g, *tensors):
    """float64 numpy copies of batch b, kv group g: [1, G, T, D] query-side, [1, 1, T, D] kv-side."""
    out = []
    for t in tensors:
        sl = t[b:b + 1, g * G:(g + 1) * G] if t.shape[1] == HQ else t[b:b + 1, g:g + 1]
        out.append(sl.float().cpu().numpy().astype(np.float64))
    return out


def check_groups(q, k, v, do, o, lse, dq, dk, dv, label):
    for b, g in GROUPS:
        qs, ks, vs, dos = group_slices(b, g, q, k, v, do)
        ref = oracle.attention(qs, ks, vs, dos, theta=10000.0)
        got = group_slices(b, g, o, lse.unsqueeze(-1), dq, dk, dv)
        got[1] = got[1][..., 0]
        errs = {n: rel_err(x, r) for n, x, r in zip(("o", "L", "dq", "dk", "dv"), got, ref)}
        log("%s group (%d, %d): %s" % (label, b, g, {n: "%.2e" % e for n, e in errs.items()}))
        bad = {n: e for n, e in errs.items() if not e <= TOL["bf16"]}
        assert not bad, "%s group (%d, %d): %s" % (label, b, g, bad)


def test_max_elements_bf16_forward_backward_and_training_pair():
    assert B * HQ * T * D == (1 << 31) - 32768
    dev = torch.device("cuda:0")
    q = gen.device_normals(61, (B, HQ, T, D), dev, torch.bfloat16)
    k = gen.device_normals(62, (B, HKV, T, D), dev, torch.bfloat16)
    v = gen.device_normals(63, (B, HKV, T, D), dev, torch.bfloat16)
    do = gen.device_normals(64, (B, HQ, T, D), dev, torch.bfloat16, sigma=0.1)
    log("inputs drawn: %d elements per query-side tensor" % q.numel())
    o, lse = ne.attn_fwd(q, k, v)
    dq, dk, dv = ne.attn_bwd(q, k, v, o, lse, do)
    torch.cuda.synchronize()
    check_groups(q, k, v, do, o, lse, dq, dk, dv, "fwd/bwd")
    o2, lse2, dq2, dk2, dv2 = ne.attn_train(q, k, v, do)
    torch.cuda.synchronize()
    assert torch.equal(o2, o) and torch.equal(lse2, lse)
    del o, lse, dq, dk, dv
    check_groups(q, k, v, do, o2, lse2, dq2, dk2, dv2, "training pair")
