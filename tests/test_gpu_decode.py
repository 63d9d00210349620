"""GPU parity of decode-time attention (ne_attn_decode) against the double-precision oracle.

The cache holds the keys rotated at their positions; both sides read the same bf16 cache
(rotated by the oracle in double, then rounded to bf16).  Whole output tensors are compared with
the bf16 bar: e(X) = max|gpu - ref| / max|ref| <= 2e-2 for X in {O, L}.
"""
import sys

import numpy as np
import pytest
import torch

import causal_gqa_flashattention_ne_amd as ne
import gen
import oracle

pytestmark = pytest.mark.gpu
TOL = 2e-2


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def bf16(x, dev):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev).to(torch.bfloat16).contiguous()


def run_case(seed, B, Hq, Hkv, n, rows, D, kv_len=None, theta=10000.0, scale=None):
    dev = torch.device("cuda:0")
    q, k, v, lens = gen.decode_case(seed, B, Hq, Hkv, n, rows, D, kv_len)
    kc = gen.round_bf16(oracle.rope(k, theta).astype(np.float32)) if theta > 0 else k
    o_ref, L_ref = oracle.decode(q, kc, v, lens, theta=theta, scale=scale)
    o, lse = ne.attn_decode(bf16(q, dev), bf16(kc, dev), bf16(v, dev),
                            torch.from_numpy(lens).to(dev), rope_theta=theta, scale=scale)
    o = o.float().cpu().numpy()
    lse = lse.cpu().numpy()
    e_o = np.abs(o - o_ref).max() / np.abs(o_ref).max()
    e_l = np.abs(lse - L_ref).max() / np.abs(L_ref).max()
    log("  decode B%d Hq%d Hkv%d n%d rows%d D%d lens %s: e(O) %.2e e(L) %.2e"
        % (B, Hq, Hkv, n, rows, D, list(lens)[:6], e_o, e_l))
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    assert e_o <= TOL and e_l <= TOL, (e_o, e_l)
    return e_o, e_l


CASES = [
    # seed, B, Hq, Hkv, n, rows, D, kv_len
    (1, 3, 4, 2, 1, 200, 64, None),            # ragged lengths, one new token
    (2, 2, 12, 4, 1, 512, 64, [512, 1]),       # the 116M-model heads; full cache and a one-row cache
    (3, 2, 12, 4, 5, 300, 64, [5, 300]),       # several new tokens (MTP-style drafts)
    (4, 2, 8, 8, 1, 2048, 64, [2048, 1537]),   # MHA, long cache: many chunks
    (5, 2, 4, 1, 8, 640, 64, [129, 640]),      # G = 4, n = 8: the 32-column maximum
    (6, 2, 2, 2, 32, 96, 64, [32, 96]),        # G = 1, n = 32
    (7, 2, 4, 2, 3, 130, 32, [64, 65]),        # D = 32; lengths at a tile boundary
    (8, 4, 4, 2, 2, 4096, 64, None),           # long ragged caches
    (10, 100, 2, 1, 1, 130, 64, None),         # more sequences than lanes in the length scan
    (11, 1, 3, 1, 1, 8192, 64, [8192]),        # one sequence shared by many waves, merged
    (12, 1, 3, 1, 5, 130, 64, [65]),           # a last piece no column of the first tokens sees
    (13, 3, 16, 1, 1, 700, 64, [700, 1, 333]), # G = 16: the widest 16-column group
    (14, 2, 8, 2, 2, 1000, 64, [100, 200]),    # fewer valid tiles than waves: one-tile shares
    (15, 3, 6, 2, 1, 1000, 128, None),         # head_dim 128 (32-key tiles)
    (16, 2, 4, 1, 4, 300, 128, [300, 9]),      # head_dim 128, 16 columns, short sequence
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "s%d-B%d-H%d-%d-n%d-T%d-D%d" % c[:7])
def test_decode_parity(case):
    seed, B, Hq, Hkv, n, rows, D, kv_len = case
    log("decode case %s" % (case,))
    run_case(seed, B, Hq, Hkv, n, rows, D, kv_len)


@pytest.mark.parametrize("theta,scale", [(0.0, None), (10.0, 0.3)])
def test_decode_rope_off_and_scale(theta, scale):
    log("decode theta %s scale %s" % (theta, scale))
    run_case(9, 2, 6, 2, 2, 257, 64, [257, 70], theta=theta, scale=scale)


def test_decode_matches_forward_last_rows():
    """The library's decode on a cache filled by ne_rope_apply agrees with the library's own forward
    at the last n positions: the same bf16 rotation of the keys.  The decode always carries the
    query as bf16 hi + lo; the forward drops the low part for blocks whose score bound is under
    kLoBound (as here), so the two differ by the query's bf16 rounding in the scores: about 2^-9 of
    a score of a few units, ~1e-4 of L's scale (bar 1e-3), ~1e-3 of O's (bar 1e-2)."""
    dev = torch.device("cuda:0")
    B, Hq, Hkv, T, D, n = 2, 12, 4, 320, 64, 3
    q, k, v, _ = gen.small_case(31, B, Hq, Hkv, T, D, "bf16")
    qd, kd, vd = bf16(q, dev), bf16(k, dev), bf16(v, dev)
    o_f, l_f = ne.attn_fwd(qd, kd, vd, rope_theta=10000.0)
    kc = ne.rope_apply(kd, 10000.0)
    lens = torch.full((B,), T, dtype=torch.int32, device=dev)
    o_d, l_d = ne.attn_decode(qd[:, :, T - n:].contiguous(), kc, vd, lens, rope_theta=10000.0)
    e_o = (o_d.float() - o_f[:, :, T - n:].float()).abs().max().item() / o_f.float().abs().max().item()
    e_l = (l_d - l_f[:, :, T - n:]).abs().max().item() / l_f.abs().max().item()
    log("  decode vs forward: e(O) %.2e e(L) %.2e" % (e_o, e_l))
    assert e_o <= 1e-2 and e_l <= 1e-3


def test_decode_deterministic():
    dev = torch.device("cuda:0")
    q, k, v, lens = gen.decode_case(41, 2, 8, 2, 2, 1000, 64)
    args = (bf16(q, dev), bf16(k, dev), bf16(v, dev), torch.from_numpy(lens).to(dev))
    o1, l1 = ne.attn_decode(*args)
    o2, l2 = ne.attn_decode(*args)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_decode_workspace_reuse():
    """One workspace across calls of different lengths: the per-segment arrival counters of the
    16-column path are left at zero by every call."""
    dev = torch.device("cuda:0")
    B, Hq, Hkv, n, rows, D = 3, 6, 2, 1, 3000, 64
    p = ne.make_decode_params(B, Hq, Hkv, n, D, rows, None, ne.rope_table(rows, D, 10000.0, dev))
    ws = torch.zeros(ne.decode_workspace_bytes(p), dtype=torch.uint8, device=dev)
    for i, lens in enumerate(([3000, 2000, 1000], [17, 2999, 640], [3000, 3000, 3000])):
        q, k, v, lv = gen.decode_case(50 + i, B, Hq, Hkv, n, rows, D, lens)
        kc = gen.round_bf16(oracle.rope(k, 10000.0).astype(np.float32))
        o_ref, L_ref = oracle.decode(q, kc, v, lv, theta=10000.0)
        qd = bf16(q, dev)
        o = torch.empty_like(qd)
        lse = torch.empty(B, Hq, n, dtype=torch.float32, device=dev)
        ne.attn_decode_into(p, qd, bf16(kc, dev), bf16(v, dev), torch.from_numpy(lv).to(dev), o, lse, ws)
        torch.cuda.synchronize()
        e_o = np.abs(o.float().cpu().numpy() - o_ref).max() / np.abs(o_ref).max()
        e_l = np.abs(lse.cpu().numpy() - L_ref).max() / np.abs(L_ref).max()
        log("  reuse call %d lens %s: e(O) %.2e e(L) %.2e" % (i, lens, e_o, e_l))
        assert e_o <= TOL and e_l <= TOL
