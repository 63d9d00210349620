"""Double-precision CPU oracle for causal GQA attention with RoPE.

TEST INFRASTRUCTURE ONLY: the parity reference for the HIP library.  Only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import this package.
The product path never calls it and shares no code with it.

The arithmetic lives in ``ne_oracle.c`` (plain C, double, OpenMP over KV groups); this module
only builds it with gcc, loads it and marshals numpy arrays.  Every function is pinned by the
tests in ``tests/test_oracle_*.py`` (closed forms, finite differences, independent library
routines, invariants).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ne_oracle.c")
_LIB = os.path.join(_HERE, "libne_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, IEEE semantics: no fast-math) into oracle/libne_oracle.so."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
               "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.ora_attn.argtypes = [ctypes.c_int] * 5 + [ctypes.c_double, ctypes.c_double] + [dp] * 9 + [
            ctypes.c_void_p, ctypes.c_int]
        lib.ora_attn.restype = ctypes.c_int
        lib.ora_rope.argtypes = [ctypes.c_int] * 4 + [ctypes.c_double, ctypes.c_int, ctypes.c_int, dp, dp]
        lib.ora_rope.restype = None
        lib.ora_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _d(x):
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(x):
    if x is None:
        return None
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def max_threads() -> int:
    return _load().ora_max_threads()


def rope(x, theta, inverse=False, pos_offset=0):
    """y = R_t x (or R_t^T x) for x of shape [B, H, T, D]; row t uses position t + pos_offset."""
    x = _d(x)
    B, H, T, D = x.shape
    y = np.empty_like(x)
    _load().ora_rope(B, H, T, D, float(theta), int(pos_offset), int(bool(inverse)), _ptr(x), _ptr(y))
    return y


def attention(q, k, v, do=None, theta=10000.0, scale=None, groups=None, nthreads=0):
    """Causal GQA attention with RoPE in double.

    q [B,Hq,T,D], k/v [B,Hkv,T,D], do [B,Hq,T,D] or None.
    Returns (o, L) or (o, L, dq, dk, dv).  ``groups`` is an optional iterable of (b, g) pairs to
    compute (the rest of every output is NaN); ``scale`` None means 1/sqrt(D); theta <= 0 means
    no RoPE.
    """
    q, k, v = _d(q), _d(k), _d(v)
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, T, D) or v.shape != k.shape:
        raise ValueError("shape mismatch")
    o = np.full_like(q, np.nan)
    L = np.full((B, Hq, T), np.nan)
    mask = None
    if groups is not None:
        mask = np.zeros(B * Hkv, dtype=np.uint8)
        for b, g in groups:
            mask[b * Hkv + g] = 1
    dq = dk = dv = None
    if do is not None:
        do = _d(do)
        dq = np.full_like(q, np.nan)
        dk = np.full_like(k, np.nan)
        dv = np.full_like(v, np.nan)
    rc = _load().ora_attn(B, Hq, Hkv, T, D, float(theta), float(scale or 0.0),
                          _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(o), _ptr(L),
                          _ptr(dq), _ptr(dk), _ptr(dv),
                          None if mask is None else mask.ctypes.data_as(ctypes.c_void_p),
                          int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle failed with code %d" % rc)
    if do is None:
        return o, L
    return o, L, dq, dk, dv


def decode(q, k_cache, v_cache, kv_len, theta=10000.0, scale=None):
    """Attention of n new query tokens per sequence against a KV cache, in double.

    q [B, Hq, n, D]: un-rotated queries; token i of sequence b sits at position kv_len[b] - n + i
    and is rotated there (RoPE as in ``rope``; theta <= 0: none).  k_cache / v_cache
    [B, Hkv, Tc, D]: keys already rotated at their own positions, and values; rows at or past
    kv_len[b] are ignored.  Token i sees the keys 0 .. kv_len[b] - n + i (causal), with query head h
    reading kv head h // (Hq / Hkv).  Returns (o [B, Hq, n, D], L [B, Hq, n], natural log).

    This is the definition of the last n rows of ``attention`` written out directly (softmax over
    the visible prefix; one numpy matrix product per head for the scores and one for P V); the
    tests pin it to ``attention`` itself.
    """
    q, kc, vc = _d(q), _d(k_cache), _d(v_cache)
    B, Hq, n, D = q.shape
    Hkv = kc.shape[1]
    G = Hq // Hkv
    s = scale or 1.0 / np.sqrt(D)
    o = np.empty_like(q)
    L = np.empty((B, Hq, n))
    for b in range(B):
        lb = int(kv_len[b])
        p0 = lb - n
        qr = rope(q[b:b + 1], theta, pos_offset=p0)[0] if theta > 0 else q[b]
        for h in range(Hq):
            K = kc[b, h // G, :lb]
            V = vc[b, h // G, :lb]
            S = s * (qr[h] @ K.T)                       # [n, lb]
            for i in range(n):
                S[i, p0 + i + 1:] = -np.inf             # keys after the token's own position
            m = S.max(axis=1, keepdims=True)
            e = np.exp(S - m)
            l = e.sum(axis=1, keepdims=True)
            o[b, h] = (e / l) @ V
            L[b, h] = (m + np.log(l))[:, 0]
    return o, L


def qkv_proj(x, w, Hq, Hkv, theta=10000.0):
    """The query, key and value projections of one attention block, in double, with RoPE on the
    queries and keys (bias-free linear maps: agentlenshq NanoEuler page, "핵심 아키텍처 및 설계";
    RoPE on queries and keys: "기술 사양").

    x [B, T, C]: the (normalised) activations.  w [(Hq + 2 Hkv) D, C]: the packed weights, output
    feature f = x . w[f]; the features are [query heads | key heads | value heads], head-major with
    d fastest inside each head.  Returns (q, k, v) in the attention layout [B, H, T, D]: q and k
    rotated at positions 0 .. T-1 (theta <= 0: not rotated), v as projected.
    """
    x, w = _d(x), _d(w)
    B, T, C = x.shape
    N = w.shape[0]
    if w.shape[1] != C or N % (Hq + 2 * Hkv):
        raise ValueError("shape mismatch")
    D = N // (Hq + 2 * Hkv)
    y = x.reshape(B * T, C) @ w.T                          # [B*T, N]
    y = y.reshape(B, T, Hq + 2 * Hkv, D).transpose(0, 2, 1, 3)
    q, k, v = y[:, :Hq], y[:, Hq:Hq + Hkv], y[:, Hq + Hkv:]
    if theta > 0:
        q, k = rope(q, theta), rope(k, theta)
    return np.ascontiguousarray(q), np.ascontiguousarray(k), np.ascontiguousarray(v)


def rmsnorm(x, g, eps=1e-5):
    """x / sqrt(mean(x^2) + eps) * g over the last axis (bias-free pre-normalisation: agentlenshq
    NanoEuler page, "기술 사양")."""
    x = _d(x)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * _d(g)


def block(x, g, wqkv, wo, dy, Hq, Hkv, theta=10000.0, eps=1e-5):
    """One pre-norm attention block and its gradients, in double:

        xn = rmsnorm(x, g);  q, k, v = qkv_proj(xn, wqkv)  (RoPE on q and k);
        o = causal GQA attention(q, k, v);  y = x + concat_heads(o) wo^T

    (the block order of the agentlenshq NanoEuler page, "기술 사양": RMSNorm pre-normalisation,
    RoPE on queries and keys, GQA; bias-free linear maps).  x [B, T, C], g [C], wqkv
    [(Hq + 2 Hkv) D, C], wo [C, Hq D], dy [B, T, C] the gradient of the loss with respect to y.
    Returns (y, dx, dg, dwqkv, dwo).  The backward is the chain rule written out step by step, the
    attention part through ``attention``'s own backward; the tests pin it to central finite
    differences.
    """
    x, g, wqkv, wo, dy = _d(x), _d(g), _d(wqkv), _d(wo), _d(dy)
    B, T, C = x.shape
    N = wqkv.shape[0]
    D = N // (Hq + 2 * Hkv)
    # forward
    r = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)     # [B, T, 1]
    u = x / r
    xn = u * g
    q, k, v = qkv_proj(xn, wqkv, Hq, Hkv, theta=theta)              # rotated q, k
    o, _ = attention(q, k, v, theta=0.0)
    oc = o.transpose(0, 2, 1, 3).reshape(B, T, Hq * D)              # heads concatenated
    y = x + oc @ wo.T
    # backward
    dwo = np.einsum("btc,btj->cj", dy, oc)
    doc = dy @ wo                                                   # [B, T, Hq D]
    do = doc.reshape(B, T, Hq, D).transpose(0, 2, 1, 3)
    _, _, dq, dk, dv = attention(q, k, v, do, theta=0.0)            # w.r.t. the rotated q, k
    if theta > 0:
        dq, dk = rope(dq, theta, inverse=True), rope(dk, theta, inverse=True)
    dyp = np.concatenate([dq, dk, dv], axis=1).transpose(0, 2, 1, 3).reshape(B, T, N)
    dwqkv = np.einsum("btn,btc->nc", dyp, xn)
    dxn = dyp @ wqkv
    dg = np.einsum("btc,btc->c", dxn, u)
    du = dxn * g
    dx = dy + du / r - x * np.sum(du * x, axis=-1, keepdims=True) / (C * r ** 3)
    return y, dx, dg, dwqkv, dwo
