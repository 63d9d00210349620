"""The allocation-free decode (ne_attn_decode_static) against the workspace decode (ne_attn_decode).

ne_attn_decode_static keeps its partial results in the library's own per-device array instead of
a caller workspace.  Each call here goes through the C ABI and is compared, output by output, with
ne_attn_decode on the same inputs, to the bf16 bar e(X) = max|a - b| / max|b| <= 2e-2 (and with the
double-precision oracle to the same bar).  Three calls in a row share the array: the served
workload's shape, then smaller inputs (a ragged batch on the 16-column path, then the 32-column
path), so each call finds the previous call's contents in the array.  The size limit is checked
on the host, before any launch.
"""
import ctypes
import sys

import numpy as np
import pytest
import torch

import causal_gqa_flashattention_ne_amd as ne
import gen
import oracle

TOL = 2e-2


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def bf16(x, dev):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev).to(torch.bfloat16).contiguous()


def rel(a, b):
    return float(np.abs(a - b).max() / np.abs(b).max())


def test_static_decode_rejects_too_large_before_launch():
    # 20000 (sequence, kv head) pairs: more arrival counters than the array reserves; rejected by
    # the host-side size check before anything runs on a device (fake, aligned pointers)
    p = ne.make_decode_params(10000, 4, 2, 1, 64, 64)
    f = ctypes.c_void_p(4096)
    rc = ne.lib().ne_attn_decode_static(ctypes.byref(p), f, f, f, f, f, f, None)
    assert rc == -5, rc                                   # NE_ERR_WORKSPACE
    assert ne.decode_static_max_bytes() == 32 << 20


@pytest.mark.gpu
def test_static_decode_matches_workspace_decode_on_successive_calls():
    dev = torch.device("cuda:0")
    w = gen.DECODE_WORKLOADS[2]
    cases = [
        ("served workload %s" % w.name, (w.seed, w.B, w.Hq, w.Hkv, w.n, w.cache_rows, w.D, None)),
        ("smaller ragged batch", (31, 3, 6, 2, 2, 700, 64, None)),
        ("32-column path", (32, 2, 4, 1, 8, 300, 64, [129, 300])),
    ]
    for name, (seed, B, Hq, Hkv, n, rows, D, lens) in cases:
        log("case %s: B%d Hq%d Hkv%d n%d rows%d D%d" % (name, B, Hq, Hkv, n, rows, D))
        q, k, v, kv_len = gen.decode_case(seed, B, Hq, Hkv, n, rows, D, lens)
        kc = gen.round_bf16(oracle.rope(k, 10000.0).astype(np.float32))
        qd, kd, vd = bf16(q, dev), bf16(kc, dev), bf16(v, dev)
        ld = torch.from_numpy(kv_len).to(dev)
        cs = ne.rope_table(rows, D, 10000.0, dev)
        p = ne.make_decode_params(B, Hq, Hkv, n, D, rows, None, cs)
        o_s = torch.full_like(qd, float("nan"))
        l_s = torch.full((B, Hq, n), float("nan"), dtype=torch.float32, device=dev)
        ne.attn_decode_static_into(p, qd, kd, vd, ld, o_s, l_s)
        o_w = torch.full_like(qd, float("nan"))
        l_w = torch.full((B, Hq, n), float("nan"), dtype=torch.float32, device=dev)
        ws = torch.zeros(max(1, ne.decode_workspace_bytes(p)), dtype=torch.uint8, device=dev)
        ne.attn_decode_into(p, qd, kd, vd, ld, o_w, l_w, ws)
        torch.cuda.synchronize()
        o_s, l_s, o_w, l_w = (t.float().cpu().numpy() for t in (o_s, l_s, o_w, l_w))
        assert np.isfinite(o_s).all() and np.isfinite(l_s).all()
        o_ref, l_ref = oracle.decode(q, kc, v, kv_len, theta=10000.0)
        errs = {"O vs workspace": rel(o_s, o_w), "L vs workspace": rel(l_s, l_w),
                "O vs oracle": rel(o_s, o_ref), "L vs oracle": rel(l_s, l_ref)}
        log("  %s" % {k2: "%.2e" % e for k2, e in errs.items()})
        assert all(e <= TOL for e in errs.values()), errs
