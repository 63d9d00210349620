"""A pre-norm attention block on the GPU, forward and backward, around the library's kernels.

    xn = rmsnorm(x, g);  q, k, v = RoPE-projected xn (ne_qkv_proj);  o = attention(q, k, v)
    (ne_attn_fwd / ne_attn_bwd);  y = x + concat_heads(o) wo^T

the block order of the agentlenshq NanoEuler page ("기술 사양": RMSNorm pre-normalisation, RoPE
on queries and keys, GQA; bias-free linear maps).  The projection, the attention and undoing the
rotation of dq, dk (ne_rope_apply) run in the library's kernels; RMSNorm, the output projection
and the matrix products of the projections' backward are torch float32 operations on the same
device.  Activations between the two parts are bfloat16 (the kernels' dtype).
"""
from __future__ import annotations

import torch

from . import attn_bwd, attn_fwd, qkv_proj, rope_apply


def block_forward_backward(x, g, wqkv, wo, dy, Hq: int, Hkv: int, rope_theta: float = 10000.0, eps: float = 1e-5):
    """x [B, T, C] bf16; g [C]; wqkv [(Hq + 2 Hkv) D, C] bf16 (packed [query | key | value] heads);
    wo [C, Hq D]; dy [B, T, C] the gradient of the loss with respect to y.

    Returns (y, dx, dg, dwqkv, dwo) in float32.
    """
    B, T, C = x.shape
    N = wqkv.shape[0]
    D = N // (Hq + 2 * Hkv)
    xf = x.float()
    gf = g.float()
    wof = wo.float()
    dyf = dy.float()
    # forward
    r = torch.sqrt((xf * xf).mean(dim=-1, keepdim=True) + eps)
    u = xf / r
    xn = (u * gf).to(torch.bfloat16).contiguous()
    q, k, v = qkv_proj(xn, wqkv, Hq, Hkv, rope_theta=rope_theta)          # q, k rotated
    o, lse = attn_fwd(q, k, v, rope_theta=0.0)
    oc = o.float().permute(0, 2, 1, 3).reshape(B, T, Hq * D)
    y = xf + oc @ wof.t()
    # backward
    dwo = torch.einsum("btc,btj->cj", dyf, oc)
    do = (dyf @ wof).reshape(B, T, Hq, D).permute(0, 2, 1, 3).contiguous().to(torch.bfloat16)
    dq, dk, dv = attn_bwd(q, k, v, o, lse, do, rope_theta=0.0)             # w.r.t. the rotated q, k
    if rope_theta and rope_theta > 0:
        dq = rope_apply(dq, rope_theta, inverse=True)
        dk = rope_apply(dk, rope_theta, inverse=True)
    dyp = torch.cat([dq, dk, dv], dim=1).float().permute(0, 2, 1, 3).reshape(B, T, N)
    dwqkv = torch.einsum("btn,btc->nc", dyp, xn.float())
    dxn = dyp @ wqkv.float()
    dg = (dxn * u).sum(dim=(0, 1))
    du = dxn * gf
    dx = dyf + du / r - xf * (du * xf).sum(dim=-1, keepdim=True) / (C * r ** 3)
    return y, dx, dg, dwqkv, dwo
