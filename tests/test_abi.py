"""C-ABI checks that need no GPU: the library loads, exports every function include/ne_attn.h
declares, and rejects bad arguments with the documented codes before anything is launched.

The pointers passed below are never dereferenced: every call here fails validation, which runs
before any HIP call.
"""
import ctypes
import os
import re

import pytest

import causal_gqa_flashattention_ne_amd as ne

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ne_attn.h")

ALIGNED = 0x10000          # fake, 16-byte aligned, never dereferenced
MISALIGNED = 0x10008


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ne_[a-z_0-9]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(ne.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = ne.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert L.ne_abi_version() == ne.ABI_VERSION
    assert ne.status_string(0) == "ok"
    for code in range(-6, 0):
        assert ne.status_string(code) != "unknown status"
    assert ne.status_string(-99) == "unknown status"


def params(**kw):
    base = dict(B=2, Hq=4, Hkv=2, T=16, D=64, dtype_code=ne.NE_DTYPE_BF16)
    base.update(kw)
    return ne.make_params(**base)


def fwd(p, q=ALIGNED, k=ALIGNED, v=ALIGNED, o=ALIGNED, lse=ALIGNED, ws=ALIGNED, ws_bytes=1 << 30):
    vp = ctypes.c_void_p
    return ne.lib().ne_attn_fwd(ctypes.byref(p), vp(q), vp(k), vp(v), vp(o), vp(lse), vp(ws), ws_bytes, None)


def bwd(p, ws_bytes=1 << 30, ptrs=None):
    vp = ctypes.c_void_p
    ptrs = ptrs or [ALIGNED] * 10
    return ne.lib().ne_attn_bwd(ctypes.byref(p), *[vp(x) for x in ptrs], ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(Hq=3, Hkv=2), -2),
    (dict(B=0), -2),
    (dict(T=-1), -2),
    (dict(Hkv=0), -2),
    (dict(D=48), -3),
    (dict(D=256), -3),
    (dict(D=128, dtype_code=ne.NE_DTYPE_F32), -3),   # head_dim 128 on the bf16 path only
    (dict(dtype_code=7), -3),
    (dict(B=1 << 20, Hq=64, Hkv=1, T=1 << 10), -2),
])
def test_forward_rejects_bad_shapes(kw, code):
    assert fwd(params(**kw)) == code
    assert bwd(params(**kw)) == code
    assert ne.lib().ne_attn_bwd_workspace_bytes(ctypes.byref(params(**kw))) == 0
    assert ne.lib().ne_attn_fwd_workspace_bytes(ctypes.byref(params(**kw))) == 0


def test_causal_must_be_one():
    p = params()
    p.causal = 0
    assert fwd(p) == -3


def test_null_and_misaligned_pointers():
    p = params()
    assert fwd(p, q=0) == -1
    assert fwd(p, lse=0) == -1
    assert fwd(p, v=MISALIGNED) == -4
    ptrs = [ALIGNED] * 10
    ptrs[9] = 0
    assert bwd(p, ptrs=ptrs) == -1
    ptrs[9] = MISALIGNED
    assert bwd(p, ptrs=ptrs) == -4


def test_rope_table_rows_checked():
    p = params()
    p.rope_cs = ALIGNED
    p.rope_rows = 15          # T = 16
    assert fwd(p) == -2
    p.rope_cs = MISALIGNED
    p.rope_rows = 16
    assert fwd(p) == -4


def test_workspace_size_and_check():
    p = params(B=2, Hq=4, Hkv=2, T=16, D=64)
    need = ne.bwd_workspace_bytes(p)
    delta = 2 * 4 * 16 * 4
    rows_padded = 2 * 4 * 64         # bf16: rows of each head padded to whole 64-row tiles
    # bf16: (-l', -delta) per padded row | low-part flag per 128-row query block (256-byte
    # aligned) | max |k| per 64-row key tile (aligned) | scaled rotated Q hi | its lo | rotated K
    # float32: delta | one dQ slice per 128-key tile | one dK and one dV slice per share of a key
    # tile (128 keys; shares: enough for ~1024 workgroups, at most one 32-query step each: here
    # 4 key-tile units and 2 steps per unit, so 2 shares)
    assert need == rows_padded * 2 * 4 + 256 + 256 + 2 * (2 * 4 * 16 * 64 * 2) + 2 * 2 * 16 * 64 * 2
    # the forward's: max |k| per key tile (aligned), then the rotated keys when there is RoPE
    pf = params(B=2, Hq=4, Hkv=2, T=16, D=64, dtype_code=ne.NE_DTYPE_F32)
    shares = 2
    assert ne.bwd_workspace_bytes(pf) == ((delta + 255) // 256) * 256 + (2 * 4 + 2 * shares * 2 * 2) * 16 * 64 * 4
    # long sequences: one share per key tile (the tiles alone are >= 1024 workgroups); 16 dQ slices
    pl = params(B=8, Hq=8, Hkv=8, T=2048, D=64, dtype_code=ne.NE_DTYPE_F32)
    assert ne.bwd_workspace_bytes(pl) == 8 * 8 * 2048 * 4 + (16 * 8 * 8 + 2 * 8 * 8) * 2048 * 64 * 4
    assert bwd(p, ws_bytes=need - 1) == -5
    # with RoPE the training pair's workspace also holds the re-ordered table
    pr = params(B=2, Hq=4, Hkv=2, T=16, D=64)
    pr.rope_cs, pr.rope_rows = ALIGNED, 16
    assert ne.bwd_workspace_bytes(pr) == need + 64 * 64 * 2 * 4


def test_rope_entry_points_validate():
    L = ne.lib()
    vp = ctypes.c_void_p
    assert L.ne_rope_table(0, 64, 10000.0, vp(ALIGNED), None) == -2
    assert L.ne_rope_table(16, 63, 10000.0, vp(ALIGNED), None) == -2
    assert L.ne_rope_table(16, 64, 0.0, vp(ALIGNED), None) == -2
    assert L.ne_rope_table(16, 64, 10000.0, None, None) == -1
    assert L.ne_rope_table(16, 64, 10000.0, vp(MISALIGNED), None) == -4
    rp = ne.RopeParams()
    rp.B, rp.H, rp.T, rp.D, rp.dtype, rp.pos_offset, rp.rope_cs, rp.rope_rows = 1, 2, 8, 64, 1, 4, ALIGNED, 11
    assert L.ne_rope_apply(ctypes.byref(rp), vp(ALIGNED), vp(ALIGNED), 0, None) == -2   # 8 + 4 > 11
    rp.rope_rows = 12
    assert L.ne_rope_apply(ctypes.byref(rp), vp(MISALIGNED), vp(ALIGNED), 0, None) == -4
    rp.D = 16
    assert L.ne_rope_apply(ctypes.byref(rp), vp(ALIGNED), vp(ALIGNED), 0, None) == -3
    rp.D, rp.pos_offset = 64, -1
    assert L.ne_rope_apply(ctypes.byref(rp), vp(ALIGNED), vp(ALIGNED), 0, None) == -2


def test_forward_workspace():
    p = params(B=2, Hq=4, Hkv=2, T=16, D=64)
    assert ne.fwd_workspace_bytes(p) == 256               # no RoPE: max |k| per key tile only
    assert fwd(p, ws=0) == -1
    p.rope_cs, p.rope_rows = ALIGNED, 16
    need = ne.fwd_workspace_bytes(p)
    # and the bf16 rotated keys, rotated once per call, and the RoPE table re-ordered for the query
    # rotation (whole 64-row tiles of D/2 (cos, sin) float32 pairs)
    assert need == 256 + 2 * 2 * 16 * 64 * 2 + 64 * 64 * 2 * 4
    assert fwd(p, ws=0) == -1
    assert fwd(p, ws=MISALIGNED) == -4
    assert fwd(p, ws_bytes=need - 1) == -5
    pf = params(B=2, Hq=4, Hkv=2, T=16, D=64, dtype_code=ne.NE_DTYPE_F32)
    pf.rope_cs, pf.rope_rows = ALIGNED, 16
    assert ne.fwd_workspace_bytes(pf) == 0                # float32 rotates keys in the kernel


def dparams(**kw):
    base = dict(B=2, Hq=4, Hkv=2, n=1, D=64, cache_rows=128)
    base.update(kw)
    return ne.make_decode_params(**base)


def dec(p, ws_bytes=1 << 30, ptrs=None):
    vp = ctypes.c_void_p
    ptrs = ptrs or [ALIGNED] * 7
    return ne.lib().ne_attn_decode(ctypes.byref(p), *[vp(x) for x in ptrs], ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), -2),
    (dict(n=0), -2),
    (dict(Hq=3), -2),
    (dict(n=200), -2),                      # more new tokens than cache rows
    (dict(D=48), -3),
    (dict(n=17), -3),                       # G * n = 34 > 32 query columns
    (dict(D=128, n=9), -3),                 # head_dim 128: at most 16 query columns
    (dict(D=256), -3),
    (dict(cache_rows=1 << 26), -2),
])
def test_decode_rejects_bad_shapes(kw, code):
    p = dparams(**kw)
    assert dec(p) == code
    assert ne.lib().ne_attn_decode_workspace_bytes(ctypes.byref(p)) == 0


def test_head_dim_128_accepted():
    pb = params(D=128, dtype_code=ne.NE_DTYPE_BF16)
    assert ne.lib().ne_attn_bwd_workspace_bytes(ctypes.byref(pb)) > 0
    assert ne.decode_workspace_bytes(dparams(D=128, n=8)) > 0      # G * n = 16
    assert ne.decode_workspace_bytes(dparams(D=64, n=9)) > 0       # 18 columns: the 32-column path


def test_decode_dtype_pointers_workspace():
    p = dparams()
    p.dtype = ne.NE_DTYPE_F32
    assert dec(p) == -3                     # bf16 only
    p = dparams()
    need = ne.decode_workspace_bytes(p)
    assert need > 0 and need % 4 == 0
    assert dec(p, ws_bytes=need - 1) == -5
    ptrs = [ALIGNED] * 7
    ptrs[3] = 0                             # kv_len
    assert dec(p, ptrs=ptrs) == -1
    ptrs[3] = MISALIGNED
    assert dec(p, ptrs=ptrs) == -4
    p.rope_cs, p.rope_rows = ALIGNED, 127   # table shorter than the cache
    assert dec(p) == -2


def qparams(**kw):
    base = dict(B=2, T=16, C=128, Hq=4, Hkv=2, D=64)
    base.update(kw)
    return ne.make_qkv_params(**base)


def qkv(p, ptrs=None):
    vp = ctypes.c_void_p
    ptrs = ptrs or [ALIGNED] * 5
    return ne.lib().ne_qkv_proj(ctypes.byref(p), *[vp(x) for x in ptrs], None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), -2),
    (dict(T=-1), -2),
    (dict(Hkv=0), -2),
    (dict(C=96), -3),                        # C must be a multiple of 64
    (dict(D=48), -3),
    (dict(B=1 << 16, T=1 << 10, C=1 << 6), -2),
])
def test_qkv_rejects_bad_shapes(kw, code):
    assert qkv(qparams(**kw)) == code


def test_qkv_dtype_pointers_table():
    p = qparams()
    p.dtype = ne.NE_DTYPE_F32
    assert qkv(p) == -3                      # bf16 only
    p = qparams()
    ptrs = [ALIGNED] * 5
    ptrs[1] = 0                              # w
    assert qkv(p, ptrs=ptrs) == -1
    ptrs[1] = MISALIGNED
    assert qkv(p, ptrs=ptrs) == -4
    p.rope_cs, p.rope_rows = ALIGNED, 15     # T = 16
    assert qkv(p) == -2
    p.rope_cs, p.rope_rows = MISALIGNED, 16
    assert qkv(p) == -4
