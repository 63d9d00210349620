"""GPU parity at head_dim 128 (bf16 path) against the double-precision oracle.

Small shapes span several 64-row tiles and ragged tails and are compared element by element; the
head_dim-128 variant of the 116M layer (6 query heads of 128 over 2 kv heads, B = 16, T = 512)
runs at full size and its whole output tensors are compared, with the same bar as every bf16
case: e(X) = max|gpu - ref| / max|ref| <= 2e-2 for X in {O, L, dQ, dK, dV}.
"""
import sys

import pytest

import gen
from parity_util import check

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


SHAPES = [(1, 2, 1), (2, 2, 2), (63, 4, 2), (64, 2, 2), (65, 4, 4), (129, 6, 2), (300, 4, 1), (513, 8, 2)]


@pytest.mark.parametrize("T,Hq,Hkv", SHAPES, ids=lambda x: str(x))
def test_d128_small_shapes(T, Hq, Hkv):
    log("d128 T %d Hq %d Hkv %d" % (T, Hq, Hkv))
    q, k, v, do = gen.small_case(5000 + T, 2, Hq, Hkv, T, 128, "bf16")
    check(q, k, v, do, "bf16", label="d128 T=%d Hq=%d Hkv=%d" % (T, Hq, Hkv))


@pytest.mark.parametrize("theta,scale", [(0.0, None), (10000.0, 0.05)])
def test_d128_rope_off_and_explicit_scale(theta, scale):
    log("d128 theta %s scale %s" % (theta, scale))
    q, k, v, do = gen.small_case(5901, 1, 4, 2, 150, 128, "bf16")
    check(q, k, v, do, "bf16", theta=theta, scale=scale, label="d128 theta=%s" % theta)


def test_d128_workload_full_size():
    w = gen.WORKLOADS[6]
    log("workload %s" % w.name)
    q, k, v, do = gen.layer_inputs(w, 0)
    check(q, k, v, do, w.dtype, theta=w.theta, label=w.name)
