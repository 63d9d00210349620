"""Helpers for the GPU parity tests: upload generated inputs, run the HIP path through the C ABI,
and compare with the double-precision oracle.

Error metric (per output tensor X in {O, L, dQ, dK, dV}):
    e(X) = max |X_gpu - X_oracle| / max |X_oracle|
The bar is 1e-5 for the float32 path and 2e-2 for the bfloat16 path.
"""
import json
import os

import numpy as np
import torch

import causal_gqa_flashattention_ne_amd as ne
import oracle

TOL = {"f32": 1e-5, "bf16": 2e-2}
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def to_dev(x: np.ndarray, dtype: str, device="cuda:0") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(device=device).to(TORCH_DT[dtype]).contiguous()


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    scale = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / scale) if scale > 0 else float(np.max(np.abs(got)))


def run_gpu(q, k, v, do, dtype, theta=10000.0, scale=None):
    """Forward + backward on cuda:0 with NaN-prefilled outputs; returns numpy float64 arrays."""
    qd, kd, vd, dod = (to_dev(x, dtype) for x in (q, k, v, do))
    B, Hq, T, D = q.shape
    cs = ne.rope_table(T, D, theta, qd.device) if theta and theta > 0 else None
    p = ne.make_params(B, Hq, k.shape[1], T, D, ne._dtype_code(qd), scale, cs)
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((B, Hq, T), float("nan"), dtype=torch.float32, device=qd.device)
    ne.attn_fwd_into(p, qd, kd, vd, o, lse)
    dq = torch.full_like(qd, float("nan"))
    dk = torch.full_like(kd, float("nan"))
    dv = torch.full_like(vd, float("nan"))
    ws = torch.full((ne.bwd_workspace_bytes(p),), 0xFF, dtype=torch.uint8, device=qd.device)
    ne.attn_bwd_into(p, qd, kd, vd, o, lse, dod, dq, dk, dv, ws)
    torch.cuda.synchronize()
    return tuple(to_np(t) for t in (o, lse, dq, dk, dv))


def run_gpu_train(q, k, v, do, dtype, theta=10000.0, scale=None):
    """The same through the training pair (ne_attn_fwd_train / ne_attn_bwd_train, one workspace)."""
    qd, kd, vd, dod = (to_dev(x, dtype) for x in (q, k, v, do))
    B, Hq, T, D = q.shape
    cs = ne.rope_table(T, D, theta, qd.device) if theta and theta > 0 else None
    p = ne.make_params(B, Hq, k.shape[1], T, D, ne._dtype_code(qd), scale, cs)
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((B, Hq, T), float("nan"), dtype=torch.float32, device=qd.device)
    ws = torch.full((ne.bwd_workspace_bytes(p),), 0xFF, dtype=torch.uint8, device=qd.device)
    ne.attn_fwd_train_into(p, qd, kd, vd, o, lse, ws)
    dq = torch.full_like(qd, float("nan"))
    dk = torch.full_like(kd, float("nan"))
    dv = torch.full_like(vd, float("nan"))
    ne.attn_bwd_train_into(p, qd, kd, vd, o, lse, dod, dq, dk, dv, ws)
    torch.cuda.synchronize()
    return tuple(to_np(t) for t in (o, lse, dq, dk, dv))


def compare(gpu, ref, dtype, groups=None, Hq=None, Hkv=None):
    """Per-tensor relative errors; restricted to the (b, g) groups when given."""
    names = ("O", "L", "dQ", "dK", "dV")
    errs = {}
    for name, a, b in zip(names, gpu, ref):
        if groups is not None:
            G = Hq // Hkv
            sel_a, sel_b = [], []
            for (bb, gg) in groups:
                if name in ("dK", "dV"):
                    sel_a.append(a[bb, gg]); sel_b.append(b[bb, gg])
                else:
                    sel_a.append(a[bb, gg * G:(gg + 1) * G]); sel_b.append(b[bb, gg * G:(gg + 1) * G])
            a, b = np.stack(sel_a), np.stack(sel_b)
        assert not np.isnan(a).any(), "%s has unwritten (NaN) elements" % name
        errs[name] = rel_err(a, b)
    return errs


def check(q, k, v, do, dtype, theta=10000.0, scale=None, groups=None, label="", train=False):
    gpu = (run_gpu_train if train else run_gpu)(q, k, v, do, dtype, theta, scale)
    ref = oracle.attention(q, k, v, do, theta=theta, scale=scale, groups=groups)
    errs = compare(gpu, ref, dtype, groups, q.shape[1], k.shape[1])
    log_path = os.environ.get("NE_PARITY_LOG")
    if log_path:
        with open(log_path, "a") as f:
            f.write(json.dumps({"case": label, "dtype": dtype, "shape": list(q.shape) + [k.shape[1]],
                                "theta": theta, "errors": errs}) + "\n")
    bad = {n: e for n, e in errs.items() if not e <= TOL[dtype]}
    assert not bad, "%s %s: errors above %g: %s (all: %s)" % (label, dtype, TOL[dtype], bad, errs)
    return errs
