"""Causal grouped-query FlashAttention with RoPE for MI355X (gfx950): thin Python binding.

Every step of the computation runs in the HIP kernels of ``libne_attn.so`` (C ABI declared in
``include/ne_attn.h``).  This module only marshals arguments: it checks tensor shapes/dtypes,
allocates outputs with torch (device memory) and passes raw device pointers plus the current
torch HIP stream through ctypes.  There is no fallback: if the library is missing, every call
raises.

Functions (same names as the C entry points, minus the ``ne_`` prefix):
  rope_table(rows, D, theta, device)             -> float32 [rows, D/2, 2] (cached)
  rope_apply(x, theta, inverse=False, pos_offset=0)
  attn_fwd(q, k, v, rope_theta=10000.0, scale=None)          -> (o, lse)
  attn_bwd(q, k, v, o, lse, do, rope_theta=10000.0, scale=None) -> (dq, dk, dv)
and the allocation-free forms ``attn_fwd_into`` / ``attn_bwd_into`` used by the benchmark.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libne_attn.so")

NE_OK = 0
NE_DTYPE_F32 = 0
NE_DTYPE_BF16 = 1
ABI_VERSION = 9

EXPORTS = ("ne_abi_version", "ne_status_string", "ne_rope_table", "ne_rope_apply", "ne_attn_fwd_workspace_bytes",
           "ne_attn_fwd", "ne_attn_bwd_workspace_bytes", "ne_attn_bwd", "ne_attn_bwd_preprocess", "ne_attn_bwd_main",
           "ne_attn_decode_workspace_bytes", "ne_attn_decode", "ne_qkv_proj", "ne_attn_fwd_train",
           "ne_attn_bwd_train", "ne_attn_bwd_train_preprocess", "ne_attn_decode_static",
           "ne_attn_decode_static_max_bytes")


class AttnParams(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("T", ctypes.c_int32), ("D", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("causal", ctypes.c_int32), ("scale", ctypes.c_float),
                ("rope_cs", ctypes.c_void_p), ("rope_rows", ctypes.c_int32)]


class DecodeParams(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("n", ctypes.c_int32), ("D", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("cache_rows", ctypes.c_int32), ("scale", ctypes.c_float),
                ("rope_cs", ctypes.c_void_p), ("rope_rows", ctypes.c_int32)]


class QkvParams(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("C", ctypes.c_int32),
                ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("rope_cs", ctypes.c_void_p), ("rope_rows", ctypes.c_int32)]


class RopeParams(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("T", ctypes.c_int32),
                ("D", ctypes.c_int32), ("dtype", ctypes.c_int32), ("pos_offset", ctypes.c_int32),
                ("rope_cs", ctypes.c_void_p), ("rope_rows", ctypes.c_int32)]


class NeError(RuntimeError):
    def __init__(self, fn, code, msg):
        super().__init__("%s failed: %s (code %d)" % (fn, msg, code))
        self.code = code


_lib = None


def lib():
    """The loaded C-ABI library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libne_attn.so is not built (%s); run "
                              "`python -m causal_gqa_flashattention_ne_amd.build`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.ne_abi_version.restype = ctypes.c_int
        L.ne_status_string.argtypes = [ctypes.c_int]
        L.ne_status_string.restype = ctypes.c_char_p
        L.ne_rope_table.argtypes = [i32, i32, ctypes.c_double, vp, vp]
        L.ne_rope_apply.argtypes = [ctypes.POINTER(RopeParams), vp, vp, ctypes.c_int, vp]
        L.ne_attn_fwd_workspace_bytes.argtypes = [ctypes.POINTER(AttnParams)]
        L.ne_attn_fwd_workspace_bytes.restype = sz
        L.ne_attn_fwd.argtypes = [ctypes.POINTER(AttnParams), vp, vp, vp, vp, vp, vp, sz, vp]
        L.ne_attn_bwd_workspace_bytes.argtypes = [ctypes.POINTER(AttnParams)]
        L.ne_attn_bwd_workspace_bytes.restype = sz
        L.ne_attn_bwd.argtypes = [ctypes.POINTER(AttnParams)] + [vp] * 9 + [vp, sz, vp]
        L.ne_attn_bwd_preprocess.argtypes = [ctypes.POINTER(AttnParams), vp, vp, vp, vp, vp, vp, sz, vp]
        L.ne_attn_bwd_main.argtypes = [ctypes.POINTER(AttnParams)] + [vp] * 8 + [vp, sz, vp]
        L.ne_attn_decode_workspace_bytes.argtypes = [ctypes.POINTER(DecodeParams)]
        L.ne_attn_decode_workspace_bytes.restype = sz
        L.ne_attn_decode.argtypes = [ctypes.POINTER(DecodeParams)] + [vp] * 7 + [sz, vp]
        L.ne_attn_decode_static.argtypes = [ctypes.POINTER(DecodeParams)] + [vp] * 6 + [vp]
        L.ne_attn_decode_static_max_bytes.argtypes = []
        L.ne_attn_decode_static_max_bytes.restype = sz
        L.ne_qkv_proj.argtypes = [ctypes.POINTER(QkvParams)] + [vp] * 6
        L.ne_attn_fwd_train.argtypes = [ctypes.POINTER(AttnParams), vp, vp, vp, vp, vp, vp, sz, vp]
        L.ne_attn_bwd_train.argtypes = [ctypes.POINTER(AttnParams)] + [vp] * 9 + [vp, sz, vp]
        L.ne_attn_bwd_train_preprocess.argtypes = [ctypes.POINTER(AttnParams), vp, vp, vp, vp, vp, vp, sz, vp]
        for f in ("ne_rope_table", "ne_rope_apply", "ne_attn_fwd", "ne_attn_bwd", "ne_attn_bwd_preprocess",
                  "ne_attn_bwd_main", "ne_attn_decode", "ne_attn_decode_static", "ne_qkv_proj", "ne_attn_fwd_train",
                  "ne_attn_bwd_train", "ne_attn_bwd_train_preprocess"):
            getattr(L, f).restype = ctypes.c_int
        if L.ne_abi_version() != ABI_VERSION:
            raise ImportError("libne_attn.so ABI %d, binding expects %d" % (L.ne_abi_version(), ABI_VERSION))
        _lib = L
    return _lib


def _check(fn, code):
    if code != NE_OK:
        raise NeError(fn, code, lib().ne_status_string(code).decode())


def status_string(code: int) -> str:
    return lib().ne_status_string(code).decode()


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return NE_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return NE_DTYPE_BF16
    raise TypeError("unsupported dtype %s (float32 or bfloat16)" % t.dtype)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _need(t: torch.Tensor, name: str, shape=None, dtype=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be on a GPU device" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous ([B, H, T, D] row-major)" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))


_tables = {}


def rope_table(rows: int, D: int, theta: float, device) -> torch.Tensor:
    """float32 [rows, D/2, 2] (cos, sin) table, computed by the library's fp64 kernel; cached."""
    device = torch.device(device)
    key = (int(rows), int(D), float(theta), str(device))
    t = _tables.get(key)
    if t is None:
        t = torch.empty((rows, D // 2, 2), dtype=torch.float32, device=device)
        _check("ne_rope_table", lib().ne_rope_table(rows, D, float(theta), _ptr(t), _stream(device)))
        _tables[key] = t
    return t


def make_params(B, Hq, Hkv, T, D, dtype_code, scale=None, rope_cs=None) -> AttnParams:
    p = AttnParams()
    p.B, p.Hq, p.Hkv, p.T, p.D = B, Hq, Hkv, T, D
    p.dtype = dtype_code
    p.causal = 1
    p.scale = float(scale) if scale else 0.0
    p.rope_cs = rope_cs.data_ptr() if rope_cs is not None else None
    p.rope_rows = rope_cs.shape[0] if rope_cs is not None else 0
    return p


def _params_for(q, k, rope_theta, scale):
    _need(q, "q")
    B, Hq, T, D = q.shape
    _need(k, "k", dtype=q.dtype, device=q.device)
    if k.dim() != 4 or k.shape[0] != B or k.shape[2] != T or k.shape[3] != D:
        raise ValueError("k has shape %s, incompatible with q %s" % (tuple(k.shape), tuple(q.shape)))
    Hkv = k.shape[1]
    cs = rope_table(T, D, rope_theta, q.device) if rope_theta and rope_theta > 0 else None
    return make_params(B, Hq, Hkv, T, D, _dtype_code(q), scale, cs), cs


def attn_fwd_into(p: AttnParams, q, k, v, o, lse, ws=None, stream=None):
    """Forward into preallocated o/lse with the workspace tensor ws (uint8; allocated here when None
    and fwd_workspace_bytes(p) > 0).  No checks beyond the library's."""
    st = stream if stream is not None else _stream(q.device)
    if ws is None:
        n = fwd_workspace_bytes(p)
        ws = torch.empty(n, dtype=torch.uint8, device=q.device) if n else None
    wp, wn = (_ptr(ws), ws.numel() * ws.element_size()) if ws is not None else (None, 0)
    _check("ne_attn_fwd", lib().ne_attn_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                            wp, wn, st))


def attn_bwd_into(p: AttnParams, q, k, v, o, lse, do, dq, dk, dv, ws, stream=None):
    """Backward into preallocated dq/dk/dv using the workspace tensor ws (uint8)."""
    st = stream if stream is not None else _stream(q.device)
    _check("ne_attn_bwd", lib().ne_attn_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                            _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws),
                                            ws.numel() * ws.element_size(), st))


def attn_bwd_preprocess_into(p: AttnParams, q, k, o, lse, do, ws, stream=None):
    st = stream if stream is not None else _stream(o.device)
    _check("ne_attn_bwd_preprocess", lib().ne_attn_bwd_preprocess(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(o),
                                                                  _ptr(lse), _ptr(do), _ptr(ws),
                                                                  ws.numel() * ws.element_size(), st))


def attn_bwd_main_into(p: AttnParams, q, k, v, lse, do, dq, dk, dv, ws, stream=None):
    st = stream if stream is not None else _stream(q.device)
    _check("ne_attn_bwd_main", lib().ne_attn_bwd_main(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(lse),
                                                      _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws),
                                                      ws.numel() * ws.element_size(), st))


def fwd_workspace_bytes(p: AttnParams) -> int:
    return int(lib().ne_attn_fwd_workspace_bytes(ctypes.byref(p)))


def bwd_workspace_bytes(p: AttnParams) -> int:
    return int(lib().ne_attn_bwd_workspace_bytes(ctypes.byref(p)))


def attn_fwd(q, k, v, rope_theta: float = 10000.0, scale=None):
    """Causal GQA attention forward.  q [B,Hq,T,D], k/v [B,Hkv,T,D] (float32 or bfloat16).

    Returns (o [B,Hq,T,D] in q's dtype, lse [B,Hq,T] float32, natural log).  rope_theta <= 0 or
    None disables RoPE; scale None means 1/sqrt(D).
    """
    p, _ = _params_for(q, k, rope_theta, scale)
    _need(v, "v", shape=k.shape, dtype=q.dtype, device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    attn_fwd_into(p, q, k, v, o, lse)
    return o, lse


def attn_bwd(q, k, v, o, lse, do, rope_theta: float = 10000.0, scale=None):
    """Backward of attn_fwd: returns (dq, dk, dv); dk/dv summed over each kv group's heads."""
    p, _ = _params_for(q, k, rope_theta, scale)
    _need(v, "v", shape=k.shape, dtype=q.dtype, device=q.device)
    _need(o, "o", shape=q.shape, dtype=q.dtype, device=q.device)
    _need(do, "do", shape=q.shape, dtype=q.dtype, device=q.device)
    _need(lse, "lse", shape=q.shape[:3], dtype=torch.float32, device=q.device)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    ws = torch.empty(max(1, bwd_workspace_bytes(p)), dtype=torch.uint8, device=q.device)
    attn_bwd_into(p, q, k, v, o, lse, do, dq, dk, dv, ws)
    return dq, dk, dv


def rope_apply(x, theta: float = 10000.0, inverse: bool = False, pos_offset: int = 0, out=None):
    """y = R x (or R^T x) for x [B, H, T, D]; row t uses position t + pos_offset.  out may be x."""
    _need(x, "x")
    B, H, T, D = x.shape
    y = torch.empty_like(x) if out is None else out
    _need(y, "out", shape=x.shape, dtype=x.dtype, device=x.device)
    cs = rope_table(T + pos_offset, D, theta, x.device)
    rp = RopeParams()
    rp.B, rp.H, rp.T, rp.D = B, H, T, D
    rp.dtype = _dtype_code(x)
    rp.pos_offset = pos_offset
    rp.rope_cs = cs.data_ptr()
    rp.rope_rows = cs.shape[0]
    _check("ne_rope_apply", lib().ne_rope_apply(ctypes.byref(rp), _ptr(x), _ptr(y), int(bool(inverse)),
                                                _stream(x.device)))
    return y


def default_scale(D: int) -> float:
    return 1.0 / math.sqrt(D)


def make_decode_params(B, Hq, Hkv, n, D, cache_rows, scale=None, rope_cs=None) -> DecodeParams:
    p = DecodeParams()
    p.B, p.Hq, p.Hkv, p.n, p.D = B, Hq, Hkv, n, D
    p.dtype = NE_DTYPE_BF16
    p.cache_rows = cache_rows
    p.scale = float(scale) if scale is not None else 0.0
    p.rope_cs = rope_cs.data_ptr() if rope_cs is not None else None
    p.rope_rows = rope_cs.shape[0] if rope_cs is not None else 0
    return p


def decode_workspace_bytes(p: DecodeParams) -> int:
    return int(lib().ne_attn_decode_workspace_bytes(ctypes.byref(p)))


def attn_decode_into(p: DecodeParams, q, k_cache, v_cache, kv_len, o, lse, ws, stream=None):
    """Decode into preallocated o / lse with the workspace tensor ws (uint8, zero-filled before its
    first use: every call leaves it ready for the next; one call at a time per workspace)."""
    st = stream if stream is not None else _stream(q.device)
    _check("ne_attn_decode", lib().ne_attn_decode(ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(kv_len),
                                                  _ptr(o), _ptr(lse), _ptr(ws), ws.numel() * ws.element_size(), st))


def attn_decode_static_into(p: DecodeParams, q, k_cache, v_cache, kv_len, o, lse, stream=None):
    """Decode into preallocated o / lse with no workspace: the partial results live in the library's
    own per-device array (ne_attn_decode_static).  Calls on one GPU must not overlap in time."""
    st = stream if stream is not None else _stream(q.device)
    _check("ne_attn_decode_static", lib().ne_attn_decode_static(ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                                                _ptr(kv_len), _ptr(o), _ptr(lse), st))


def decode_static_max_bytes() -> int:
    """Size of the library's per-device array behind ne_attn_decode_static."""
    return int(lib().ne_attn_decode_static_max_bytes())


def attn_decode(q, k_cache, v_cache, kv_len, rope_theta: float = 10000.0, scale=None):
    """Attention of n new tokens per sequence against a KV cache (bfloat16).

    q [B, Hq, n, D] un-rotated; k_cache / v_cache [B, Hkv, cache_rows, D] with keys already rotated
    at their positions; kv_len [B] int32 on the device (valid rows, the new tokens included).
    Returns (o [B, Hq, n, D], lse [B, Hq, n] float32, natural log).
    """
    _need(q, "q")
    B, Hq, n, D = q.shape
    _need(k_cache, "k_cache", dtype=q.dtype, device=q.device)
    _need(v_cache, "v_cache", shape=k_cache.shape, dtype=q.dtype, device=q.device)
    if k_cache.dim() != 4 or k_cache.shape[0] != B or k_cache.shape[3] != D:
        raise ValueError("k_cache must be [B, Hkv, cache_rows, D]")
    if kv_len.dtype != torch.int32 or kv_len.shape != (B,) or kv_len.device != q.device:
        raise ValueError("kv_len must be an int32 tensor of shape [B] on the queries' device")
    Hkv, rows = k_cache.shape[1], k_cache.shape[2]
    cs = rope_table(rows, D, rope_theta, q.device) if rope_theta and rope_theta > 0 else None
    p = make_decode_params(B, Hq, Hkv, n, D, rows, scale, cs)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, n), dtype=torch.float32, device=q.device)
    ws = torch.zeros(max(1, decode_workspace_bytes(p)), dtype=torch.uint8, device=q.device)
    attn_decode_into(p, q, k_cache, v_cache, kv_len, o, lse, ws)
    return o, lse


def make_qkv_params(B, T, C, Hq, Hkv, D, rope_cs=None) -> QkvParams:
    p = QkvParams()
    p.B, p.T, p.C, p.Hq, p.Hkv, p.D = B, T, C, Hq, Hkv, D
    p.dtype = NE_DTYPE_BF16
    p.rope_cs = rope_cs.data_ptr() if rope_cs is not None else None
    p.rope_rows = rope_cs.shape[0] if rope_cs is not None else 0
    return p


def qkv_proj_into(p: QkvParams, x, w, q, k, v, stream=None):
    """Projection into preallocated q, k, v ([B, H, T, D] bf16)."""
    st = stream if stream is not None else _stream(x.device)
    _check("ne_qkv_proj", lib().ne_qkv_proj(ctypes.byref(p), _ptr(x), _ptr(w), _ptr(q), _ptr(k), _ptr(v), st))


def qkv_proj(x, w, Hq: int, Hkv: int, rope_theta: float = 10000.0):
    """Query, key and value projections with RoPE on queries and keys (bfloat16).

    x [B, T, C]; w [(Hq + 2 Hkv) D, C], features packed [query heads | key heads | value heads].
    Returns (q [B, Hq, T, D] rotated, k [B, Hkv, T, D] rotated, v [B, Hkv, T, D]).
    """
    _need(x, "x")
    _need(w, "w", dtype=x.dtype, device=x.device)
    if x.dim() != 3 or w.dim() != 2 or w.shape[1] != x.shape[2] or w.shape[0] % (Hq + 2 * Hkv):
        raise ValueError("x must be [B, T, C] and w [(Hq + 2 Hkv) D, C]")
    B, T, C = x.shape
    D = w.shape[0] // (Hq + 2 * Hkv)
    cs = rope_table(T, D, rope_theta, x.device) if rope_theta and rope_theta > 0 else None
    p = make_qkv_params(B, T, C, Hq, Hkv, D, cs)
    q = torch.empty((B, Hq, T, D), dtype=x.dtype, device=x.device)
    k = torch.empty((B, Hkv, T, D), dtype=x.dtype, device=x.device)
    v = torch.empty_like(k)
    qkv_proj_into(p, x, w, q, k, v)
    return q, k, v


def attn_fwd_train_into(p: AttnParams, q, k, v, o, lse, ws, stream=None):
    """Training forward into preallocated o / lse, leaving the backward's rotated operands in ws
    (uint8, >= bwd_workspace_bytes(p)); pass the same ws to attn_bwd_train_into."""
    st = stream if stream is not None else _stream(q.device)
    _check("ne_attn_fwd_train", lib().ne_attn_fwd_train(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                                         _ptr(ws), ws.numel() * ws.element_size(), st))


def attn_bwd_train_preprocess_into(p: AttnParams, q, k, o, lse, do, ws, stream=None):
    st = stream if stream is not None else _stream(q.device)
    _check("ne_attn_bwd_train_preprocess",
           lib().ne_attn_bwd_train_preprocess(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(o), _ptr(lse), _ptr(do), _ptr(ws),
                                              ws.numel() * ws.element_size(), st))


def attn_bwd_train_into(p: AttnParams, q, k, v, o, lse, do, dq, dk, dv, ws, stream=None):
    """Training backward (after attn_fwd_train_into with the same ws) into preallocated gradients."""
    st = stream if stream is not None else _stream(q.device)
    _check("ne_attn_bwd_train", lib().ne_attn_bwd_train(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                                         _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws),
                                                         ws.numel() * ws.element_size(), st))


def attn_train(q, k, v, do, rope_theta: float = 10000.0, scale=None):
    """Forward and backward through the training pair.  Returns (o, lse, dq, dk, dv)."""
    p, _ = _params_for(q, k, rope_theta, scale)
    ws = torch.empty(bwd_workspace_bytes(p), dtype=torch.uint8, device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    attn_fwd_train_into(p, q, k, v, o, lse, ws)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    attn_bwd_train_into(p, q, k, v, o, lse, do, dq, dk, dv, ws)
    return o, lse, dq, dk, dv
