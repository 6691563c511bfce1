"""Dense whole-sequence forward in float64 torch, used to pin the oracle.

This is a different formulation of the same decoder from the oracle's
incremental one: all positions at once, causal attention through torch's
``scaled_dot_product_attention`` (grouped-query mapping by ``enable_gqa``),
``rms_norm`` and ``silu`` from torch, and RoPE as a complex multiplication.
If the oracle's token-by-token decode with a KV cache agrees with it at every
position, the cache bookkeeping, causal masking and the layer arithmetic are
pinned together.
"""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F


def _w(a) -> torch.Tensor:
    a = np.asarray(a)
    if a.dtype == np.uint16:  # bf16 bits
        return torch.from_numpy(a.astype(np.int16)).view(torch.bfloat16).to(torch.float64)
    return torch.from_numpy(a.astype(np.float64))


def _rope(x: torch.Tensor, pos: torch.Tensor, theta: float) -> torch.Tensor:
    """x [T][heads][D]; pairs (i, i + D/2) rotate as the complex number
    x_i + 1j * x_{i+D/2} times exp(1j * pos * theta**(-2i/D))."""
    d = x.shape[-1]
    half = d // 2
    inv = theta ** (-2.0 * torch.arange(half, dtype=torch.float64) / d)
    ang = pos.to(torch.float64)[:, None] * inv[None, :]  # [T][half]
    rot = torch.polar(torch.ones_like(ang), ang)[:, None, :]
    z = torch.complex(x[..., :half], x[..., half:]) * rot
    return torch.cat([z.real, z.imag], dim=-1)


def dense_logits(cfg, weights, tokens, kv_round) -> torch.Tensor:
    """Logits [T][V] (float64) for tokens [T] at positions 0..T-1.

    kv_round maps a float64 tensor to the values the KV cache stores."""
    t = len(tokens)
    h, d, hq, hkv = cfg.hidden, cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads
    emb = _w(weights["embed"])
    x = emb[torch.as_tensor(np.asarray(tokens, dtype=np.int64))]
    pos = torch.arange(t)
    for lw in weights["layers"]:
        a = F.rms_norm(x, (h,), weight=_w(lw["attn_norm"]), eps=cfg.rms_eps)
        qkv = a @ _w(lw["w_qkv"]).T
        q = qkv[:, : hq * d].reshape(t, hq, d)
        k = qkv[:, hq * d:(hq + hkv) * d].reshape(t, hkv, d)
        v = qkv[:, (hq + hkv) * d:].reshape(t, hkv, d)
        q = _rope(q, pos, cfg.rope_theta)
        k = kv_round(_rope(k, pos, cfg.rope_theta))
        v = kv_round(v)
        att = F.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1), v.transpose(0, 1),
                                             is_causal=True, enable_gqa=True)
        x = x + att.transpose(0, 1).reshape(t, hq * d) @ _w(lw["w_o"]).T
        m = F.rms_norm(x, (h,), weight=_w(lw["mlp_norm"]), eps=cfg.rms_eps)
        x = x + (F.silu(m @ _w(lw["w_gate"]).T) * (m @ _w(lw["w_up"]).T)) @ _w(lw["w_down"]).T
    xf = F.rms_norm(x, (h,), weight=_w(weights["final_norm"]), eps=cfg.rms_eps)
    return xf @ emb.T


def round_f32(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.float32).to(torch.float64)


def round_bf16_via_f32(x: torch.Tensor) -> torch.Tensor:
    """torch's float64 -> bfloat16 goes through float32 (two roundings); the
    oracle rounds once, so the two can differ by one bf16 ulp in rare cases."""
    return x.to(torch.bfloat16).to(torch.float64)
