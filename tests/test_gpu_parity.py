"""GPU parity: the HIP path (through the C ABI) against the double-precision oracle.

Small shapes span several tiles and ragged tails and are checked element by element in full.
The five workloads run at their full sizes in the benchmark's launch configuration and their whole
output tensors are compared (every kv group), since the bar is relative to the scale of the whole
tensor.
"""
import sys

import numpy as np
import pytest

import gen
from parity_util import check

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


SWEEP = []
for dtype in ("f32", "bf16"):
    for (T, D, Hq, Hkv) in [(1, 32, 2, 1), (2, 64, 2, 2), (17, 32, 4, 2), (63, 64, 3, 1), (64, 64, 4, 1),
                            (65, 32, 4, 4), (127, 64, 6, 2), (128, 32, 4, 2), (129, 64, 8, 2),
                            (200, 64, 3, 3), (300, 32, 4, 1), (513, 64, 4, 2)]:
        SWEEP.append((dtype, 2, Hq, Hkv, T, D))


@pytest.mark.parametrize("case", SWEEP, ids=lambda c: "%s-B%d-H%d-%d-T%d-D%d" % c)
def test_small_shapes(case):
    dtype, B, Hq, Hkv, T, D = case
    log("case %s" % (case,))
    q, k, v, do = gen.small_case(1000 + T + D, B, Hq, Hkv, T, D, dtype)
    check(q, k, v, do, dtype, label=str(case))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("theta,scale", [(0.0, None), (10.0, None), (10000.0, 0.3)])
def test_rope_off_small_theta_and_explicit_scale(dtype, theta, scale):
    log("theta %s scale %s %s" % (theta, scale, dtype))
    q, k, v, do = gen.small_case(77, 1, 4, 2, 150, 64, dtype)
    check(q, k, v, do, dtype, theta=theta, scale=scale, label="theta=%s" % theta)


@pytest.mark.parametrize("cfg", [1, 2])
def test_workload_full_f32(cfg):
    w = gen.WORKLOADS[cfg]
    for layer in range(w.layers):
        log("workload %d layer %d" % (cfg, layer))
        q, k, v, do = gen.layer_inputs(w, layer)
        check(q, k, v, do, w.dtype, theta=w.theta, label="%s layer %d" % (w.name, layer))


@pytest.mark.parametrize("cfg,layers", [(3, [0]), (4, [0, 15]), (5, [0])])
def test_workload_full_size(cfg, layers):
    """Whole output tensors at the full workload size against the oracle (every kv group)."""
    w = gen.WORKLOADS[cfg]
    for layer in layers:
        log("workload %d layer %d (all groups)" % (cfg, layer))
        q, k, v, do = gen.layer_inputs(w, layer)
        errs = check(q, k, v, do, w.dtype, theta=w.theta, label="%s layer %d" % (w.name, layer))
        log("  errors %s" % errs)
