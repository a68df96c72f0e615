"""An independent fp64 transformer built from torch library routines.

Used only to pin the oracle: ``F.rms_norm``, ``F.linear``,
``F.scaled_dot_product_attention`` and ``F.silu`` carry the arithmetic, and
RoPE is written as complex multiplication (pair (j, j + dh/2) read as the
complex number x_j + i x_{j+dh/2}, multiplied by exp(i * pos * base^(-2j/dh))).
None of it calls the oracle.
"""
from __future__ import annotations

import torch
import torch.nn.functional as F

T64 = torch.float64


def t(a):
    return torch.as_tensor(a, dtype=T64)


def rms(x, g, eps):
    return F.rms_norm(x, (x.shape[-1],), weight=g, eps=eps)


def rope(x, pos, H, dh, base):
    n = x.shape[0]
    half = dh // 2
    xh = x.view(n, H, dh)
    z = torch.complex(xh[..., :half].contiguous(), xh[..., half:].contiguous())
    j = torch.arange(half, dtype=T64)
    theta = t(pos)[:, None] * (float(base) ** (-2.0 * j / dh))[None, :]
    rot = torch.polar(torch.ones_like(theta), theta)[:, None, :]
    zr = z * rot
    return torch.cat([zr.real, zr.imag], dim=-1).reshape(n, H * dh)


def attn(q, K, V, H, dh):
    n, m = q.shape[0], K.shape[0]
    qh = q.view(n, H, dh).transpose(0, 1).unsqueeze(0)
    kh = K.view(m, H, dh).transpose(0, 1).unsqueeze(0)
    vh = V.view(m, H, dh).transpose(0, 1).unsqueeze(0)
    o = F.scaled_dot_product_attention(qh, kh, vh)
    return o.squeeze(0).transpose(0, 1).reshape(n, H * dh)


def qkv(x, pos, lw, dims):
    xn = rms(x, t(lw["attn_norm"]), dims.rms_eps)
    q = rope(F.linear(xn, t(lw["wq"])), pos, dims.n_heads, dims.head_dim, dims.rope_base)
    k = rope(F.linear(xn, t(lw["wk"])), pos, dims.n_heads, dims.head_dim, dims.rope_base)
    v = F.linear(xn, t(lw["wv"]))
    return q, k, v


def finish_layer(x, o, lw, dims):
    h = x + F.linear(o, t(lw["wo"]))
    hn = rms(h, t(lw["ffn_norm"]), dims.rms_eps)
    return h + F.linear(F.silu(F.linear(hn, t(lw["w_gate"]))) * F.linear(hn, t(lw["w_up"])), t(lw["w_down"]))


def full_layer(x, lw, dims):
    """Every row of the sequence through one layer (fresh K/V for all rows)."""
    pos = torch.arange(x.shape[0])
    q, k, v = qkv(x, pos, lw, dims)
    return finish_layer(x, attn(q, k, v, dims.n_heads, dims.head_dim), lw, dims)


def partial_layer(x_rows, rows, lw, K_old, V_old, dims):
    """Rows ``rows`` through one layer against a cache whose other rows are stale.

    Returns (y_rows, K_new, V_new): the cache with the recomputed rows replaced.
    """
    q, k, v = qkv(x_rows, torch.as_tensor(rows), lw, dims)
    K_new, V_new = t(K_old).clone(), t(V_old).clone()
    K_new[rows] = k
    V_new[rows] = v
    return finish_layer(x_rows, attn(q, K_new, V_new, dims.n_heads, dims.head_dim), lw, dims), K_new, V_new


def forward(tokens, model, dims, n_layers=None):
    """Full forward of the first ``n_layers`` layers; returns the residual rows."""
    x = t(model["embed"])[torch.as_tensor(tokens)]
    L = dims.n_layers if n_layers is None else n_layers
    for li in range(L):
        x = full_layer(x, model["layers"][li], dims)
    return x


def logits(x, model, dims):
    return F.linear(rms(x, t(model["final_norm"]), dims.rms_eps), t(model["lm_head"]))
