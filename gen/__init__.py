"""Seeded synthetic inputs for causal GQA attention (shared by the oracle tests and the GPU path).

This module holds no attention arithmetic: it only draws random tensors.  Both sides of every
parity check (the CPU oracle under ``oracle/`` and the HIP library) receive the very same
arrays from here.

Recipe
------
* A counter-based SplitMix64 stream (Steele, Lea, Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014; the finaliser constants are the published ``mix64`` ones).  Element
  ``e`` of a stream with key ``k`` is ``mix64(k + (e + 1) * GAMMA)`` where GAMMA is the golden
  ratio increment 0x9E3779B97F4A7C15.
* The stream key of a tensor is ``mix64(mix64(mix64(seed) ^ layer) ^ tensor_id)`` with tensor ids
  Q=0, K=1, V=2, dO=3, key-row pick=4.
* One standard normal per element by Box-Muller in double: the high and low 32-bit halves of the
  64-bit draw give u1, u2 in (0, 1) as ``(x + 0.5) / 2**32``; ``z = sqrt(-2 ln u1) cos(2 pi u2)``.
* ``z * sigma`` is rounded to float32 (round to nearest even), then to bfloat16 (round to
  nearest even) for bf16 workloads.
* Outlier keys (the byte-level MHA workload): for every (batch, kv head) exactly
  ``round(frac * T)`` distinct positions are picked by a partial Fisher-Yates shuffle driven by
  the key-row-pick stream, and those key rows are multiplied by ``key_scale`` (a power of two,
  so the product is exact in both float32 and bfloat16).
"""
from __future__ import annotations

import dataclasses
import hashlib

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "do": 3, "pick": 4, "len": 5, "x": 6, "w": 7}


def mix64(z):
    """SplitMix64 finaliser on uint64 numpy values (wraps modulo 2**64)."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def stream_key(seed: int, layer: int, tensor: int, extra: int = 0) -> np.uint64:
    k = mix64(np.uint64(seed))
    k = mix64(k ^ np.uint64(layer))
    k = mix64(k ^ np.uint64(tensor))
    if extra:
        k = mix64(k ^ np.uint64(extra))
    return np.uint64(k)


def raw_u64(key: np.uint64, n: int, start: int = 0) -> np.ndarray:
    ctr = np.arange(start + 1, start + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return mix64(key + ctr * GAMMA)


def normals(key: np.uint64, n: int, chunk: int = 1 << 22) -> np.ndarray:
    """n standard normals (float64) from the stream ``key``."""
    out = np.empty(n, dtype=np.float64)
    for s in range(0, n, chunk):
        m = min(chunk, n - s)
        x = raw_u64(key, m, s)
        hi = (x >> np.uint64(32)).astype(np.float64)
        lo = (x & np.uint64(0xFFFFFFFF)).astype(np.float64)
        u1 = (hi + 0.5) * (1.0 / 4294967296.0)
        u2 = (lo + 0.5) * (1.0 / 4294967296.0)
        out[s:s + m] = np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)
    return out


def round_bf16(x32: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 (round to nearest, ties to even), returned widened back to float32."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    return r.astype(np.uint32).view(np.float32).reshape(x32.shape)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already exactly representable in bfloat16."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if np.any(u & np.uint32(0xFFFF)):
        raise ValueError("values are not bfloat16-representable")
    return (u >> np.uint32(16)).astype(np.uint16)


def tensor(seed, layer, name, shape, sigma=1.0, dtype="f32", extra=0) -> np.ndarray:
    """Seeded N(0, sigma^2) tensor, float32 values (bf16-representable when dtype == 'bf16')."""
    n = int(np.prod(shape))
    z = normals(stream_key(seed, layer, TENSOR_IDS[name], extra), n)
    x = (z * sigma).astype(np.float32)
    if dtype == "bf16":
        x = round_bf16(x)
    elif dtype != "f32":
        raise ValueError(dtype)
    return x.reshape(shape)


def pick_positions(seed: int, layer: int, b: int, g: int, T: int, count: int) -> np.ndarray:
    """``count`` distinct positions in [0, T) by a partial Fisher-Yates shuffle (sorted)."""
    key = stream_key(seed, layer, TENSOR_IDS["pick"], extra=1 + b * 65536 + g)
    draws = raw_u64(key, count)
    perm = np.arange(T, dtype=np.int64)
    for i in range(count):
        j = i + int(draws[i] % np.uint64(T - i))
        perm[i], perm[j] = perm[j], perm[i]
    return np.sort(perm[:count])


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    T: int
    D: int
    dtype: str            # "f32" or "bf16"
    layers: int = 1
    theta: float = 10000.0
    sigma_qkv: float = 1.0
    sigma_do: float = 1.0
    outlier_frac: float = 0.0
    outlier_scale: float = 1.0
    seed: int = 0

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def causal_pairs(self) -> int:
        return self.B * self.Hq * self.T * (self.T + 1) // 2


# The five workloads (shapes and value recipes follow the NanoEuler model-config table on the
# agentlenshq page "NanoEuler: C와 CUDA로 밑바닥부터 구축한 GPT-2 규모의 LLM", section
# "모델 구성", and the byte-level GPT page "Tiny hackable CUDA language model implementation").
WORKLOADS = {
    1: Workload("tiny-cpu-model-f32", 1, 4, 2, 128, 32, "f32", seed=1),
    2: Workload("small-model-batch-f32-x4", 16, 4, 2, 128, 32, "f32", layers=4, sigma_do=0.1, seed=2),
    3: Workload("gpt116m-layer-bf16", 16, 12, 4, 512, 64, "bf16", sigma_do=0.1, seed=3),
    4: Workload("gpt116m-stack-bf16-x16", 16, 12, 4, 512, 64, "bf16", layers=16, sigma_do=0.1, seed=4),
    5: Workload("byte-mha-bf16-t2048", 8, 8, 8, 2048, 64, "bf16", outlier_frac=0.01,
                outlier_scale=8.0, seed=5),
    # head_dim 128 variant of the 116M layer: the same width (768) as 6 query heads over 2 kv heads
    6: Workload("gpt116m-width-d128-bf16", 16, 6, 2, 512, 128, "bf16", sigma_do=0.1, seed=6),
}


def layer_inputs(w: Workload, layer: int = 0):
    """(q, k, v, do) float32 numpy arrays in [B, H, T, D] layout for one layer of workload w."""
    q = tensor(w.seed, layer, "q", (w.B, w.Hq, w.T, w.D), w.sigma_qkv, w.dtype)
    k = tensor(w.seed, layer, "k", (w.B, w.Hkv, w.T, w.D), w.sigma_qkv, w.dtype)
    v = tensor(w.seed, layer, "v", (w.B, w.Hkv, w.T, w.D), w.sigma_qkv, w.dtype)
    do = tensor(w.seed, layer, "do", (w.B, w.Hq, w.T, w.D), w.sigma_do, w.dtype)
    if w.outlier_frac > 0.0:
        cnt = int(round(w.outlier_frac * w.T))
        for b in range(w.B):
            for g in range(w.Hkv):
                pos = pick_positions(w.seed, layer, b, g, w.T, cnt)
                k[b, g, pos, :] *= np.float32(w.outlier_scale)
    return q, k, v, do


def small_case(seed, B, Hq, Hkv, T, D, dtype="f32", sigma_do=1.0, layer=0):
    """Inputs for an ad-hoc shape (tests): same recipe as the workloads."""
    w = Workload("adhoc", B, Hq, Hkv, T, D, dtype, sigma_do=sigma_do, seed=seed)
    return layer_inputs(w, layer)


def sha256(x: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(x).tobytes()).hexdigest()


def decode_case(seed, B, Hq, Hkv, n, cache_rows, D, kv_len=None, dtype="bf16"):
    """Inputs of one decode call (tests, benchmark): the new tokens' queries q [B, Hq, n, D], raw
    (un-rotated) keys and values of the whole cache [B, Hkv, cache_rows, D], and the valid lengths
    kv_len [B] (given, or drawn uniformly in [n, cache_rows] per sequence).  The same N(0, 1)
    recipe as the workloads; the caller rotates the keys into the cache."""
    q = tensor(seed, 0, "q", (B, Hq, n, D), 1.0, dtype)
    k = tensor(seed, 0, "k", (B, Hkv, cache_rows, D), 1.0, dtype)
    v = tensor(seed, 0, "v", (B, Hkv, cache_rows, D), 1.0, dtype)
    if kv_len is None:
        draws = raw_u64(stream_key(seed, 0, TENSOR_IDS["len"]), B)
        kv_len = [n + int(d % np.uint64(cache_rows - n + 1)) for d in draws]
    return q, k, v, np.asarray(kv_len, dtype=np.int32)


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    """One decode call: n new tokens per sequence against a cache of cache_rows rows per kv head,
    valid lengths kv_len drawn uniformly in [n, cache_rows] (a ragged serving batch) unless full."""
    name: str
    B: int
    Hq: int
    Hkv: int
    n: int
    cache_rows: int
    D: int
    full: bool = False
    theta: float = 10000.0
    seed: int = 0


# Decode shapes: the 116M model's attention heads (12 query heads over 4 kv heads, d = 64) at its
# own context of 512 positions, and a serving batch over longer caches.
DECODE_WORKLOADS = {
    1: DecodeWorkload("gpt116m-decode-b16-ctx512", 16, 12, 4, 1, 512, 64, full=True, seed=11),
    2: DecodeWorkload("gpt116m-heads-decode-b64-cache4096", 64, 12, 4, 1, 4096, 64, seed=12),
}


def decode_inputs(w: DecodeWorkload):
    """(q, k, v, kv_len) of decode workload w (k un-rotated; the caller rotates it into the cache)."""
    return decode_case(w.seed, w.B, w.Hq, w.Hkv, w.n, w.cache_rows, w.D,
                       [w.cache_rows] * w.B if w.full else None)


def qkv_case(seed, B, T, C, Hq, Hkv, D, dtype="bf16"):
    """Inputs of the query/key/value projection: activations x [B, T, C] ~ N(0, 1) (the unit-RMS
    output of the pre-norm) and packed weights w [(Hq + 2 Hkv) D, C] ~ N(0, 1/C), so that every
    projected feature has unit variance."""
    x = tensor(seed, 0, "x", (B, T, C), 1.0, dtype)
    w = tensor(seed, 0, "w", ((Hq + 2 * Hkv) * D, C), 1.0 / np.sqrt(C), dtype)
    return x, w


@dataclasses.dataclass(frozen=True)
class QkvWorkload:
    name: str
    B: int
    T: int
    C: int
    Hq: int
    Hkv: int
    D: int
    theta: float = 10000.0
    seed: int = 0

    @property
    def flops(self) -> int:
        return 2 * self.B * self.T * self.C * (self.Hq + 2 * self.Hkv) * self.D


# The 116M model's projection: 16 sequences of 512 tokens, width 768, 12 query and 4 kv heads of 64
QKV_WORKLOADS = {
    1: QkvWorkload("gpt116m-qkv-proj-bf16", 16, 512, 768, 12, 4, 64, seed=21),
}


def device_normals(seed: int, shape, device, dtype, sigma: float = 1.0):
    """Normals of standard deviation ``sigma`` drawn on ``device`` by torch's seeded generator
    (Philox4x32-10 on GPUs), in ``dtype``: for tensors too large to draw on the host.  A check that
    uses them reads back the slices it compares, so both sides see the same values."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=dtype)
    if sigma != 1.0:
        x.mul_(sigma)
    return x
