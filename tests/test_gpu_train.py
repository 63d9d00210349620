"""GPU tests of the training pair (ne_attn_fwd_train / ne_attn_bwd_train sharing one workspace).

The pair computes the same operation as ne_attn_fwd / ne_attn_bwd; the forward keeps its rotated
queries and keys for the backward instead of the preprocess recomputing them.  The forward's O and
L are identical to the plain forward's.  The rotations themselves run in different kernels (the
forward and the key-rotation kernel instead of the preprocess), where the compiler may fuse the
rotation's multiply-adds differently, so a rotated operand can differ in its last bit and flip an
occasional bf16 rounding of a gradient: the gradients are held to 1e-2 of the plain pair's (the
backward then reuses exactly the operands the forward's L came from).  The benchmark's workloads,
which run through the training pair, are compared with the double oracle over whole tensors at
full size (bf16 bar 2e-2).
"""
import sys

import numpy as np
import pytest

import gen
from parity_util import check, run_gpu, run_gpu_train

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("dtype,B,Hq,Hkv,T,D,theta", [
    ("bf16", 2, 4, 2, 129, 64, 10000.0),
    ("bf16", 1, 6, 2, 300, 32, 10000.0),
    ("bf16", 2, 4, 4, 200, 64, 0.0),          # no RoPE: the keys are copied into the workspace
    ("bf16", 1, 4, 2, 150, 128, 10000.0),
    ("f32", 2, 4, 2, 100, 64, 10000.0),       # float32: the plain pair underneath
])
def test_train_pair_equals_plain_pair(dtype, B, Hq, Hkv, T, D, theta):
    log("train vs plain %s B%d Hq%d Hkv%d T%d D%d theta %s" % (dtype, B, Hq, Hkv, T, D, theta))
    q, k, v, do = gen.small_case(7000 + T + D, B, Hq, Hkv, T, D, dtype)
    plain = run_gpu(q, k, v, do, dtype, theta)
    train = run_gpu_train(q, k, v, do, dtype, theta)
    diffs = {}
    for name, a, b in zip(("O", "L", "dQ", "dK", "dV"), plain, train):
        assert not np.isnan(b).any(), name
        diffs[name] = float(np.abs(a - b).max() / np.abs(a).max())
    log("  relative differences from the plain pair: %s" % diffs)
    assert diffs["O"] == 0.0 and diffs["L"] == 0.0, diffs
    assert max(diffs.values()) <= 1e-2, diffs


@pytest.mark.parametrize("cfg", [3, 5])
def test_train_pair_workload_full_size(cfg):
    w = gen.WORKLOADS[cfg]
    log("train pair workload %s" % w.name)
    q, k, v, do = gen.layer_inputs(w, 0)
    check(q, k, v, do, w.dtype, theta=w.theta, label=w.name + " (training pair)", train=True)


def test_train_pair_every_layer_of_the_stack():
    """The 16-layer stack as the benchmark runs it: every layer's inputs resident at once, one
    workspace shared by all layers, and one step (training forward, preprocess, backward main per
    layer, in layer order) before any output is read; then every layer's whole output tensors
    against the oracle."""
    import torch

    import causal_gqa_flashattention_ne_amd as ne
    import oracle
    from parity_util import TOL, compare, to_dev, to_np

    w = gen.WORKLOADS[4]
    dev = torch.device("cuda:0")
    cs = ne.rope_table(w.T, w.D, w.theta, dev)
    p = ne.make_params(w.B, w.Hq, w.Hkv, w.T, w.D, ne.NE_DTYPE_BF16, None, cs)
    ws = torch.full((ne.bwd_workspace_bytes(p),), 0xFF, dtype=torch.uint8, device=dev)
    host, dev_in, outs = [], [], []
    for layer in range(w.layers):
        q, k, v, do = gen.layer_inputs(w, layer)
        host.append((q, k, v, do))
        dev_in.append(tuple(to_dev(x, w.dtype) for x in (q, k, v, do)))
        qd, kd = dev_in[-1][0], dev_in[-1][1]
        outs.append((torch.full_like(qd, float("nan")),
                     torch.full((w.B, w.Hq, w.T), float("nan"), dtype=torch.float32, device=dev),
                     torch.full_like(qd, float("nan")), torch.full_like(kd, float("nan")),
                     torch.full_like(kd, float("nan"))))
    for (qd, kd, vd, dod), (o, lse, dq, dk, dv) in zip(dev_in, outs):
        ne.attn_fwd_train_into(p, qd, kd, vd, o, lse, ws)
        ne.attn_bwd_train_preprocess_into(p, qd, kd, o, lse, dod, ws)
        ne.attn_bwd_main_into(p, qd, kd, vd, lse, dod, dq, dk, dv, ws)
    torch.cuda.synchronize()
    for layer, ((q, k, v, do), t) in enumerate(zip(host, outs)):
        ref = oracle.attention(q, k, v, do, theta=w.theta)
        errs = compare(tuple(to_np(x) for x in t), ref, w.dtype)
        log("stack layer %d errors %s" % (layer, errs))
        bad = {n: e for n, e in errs.items() if not e <= TOL[w.dtype]}
        assert not bad, "layer %d: %s" % (layer, errs)
