"""A second, independent CPU implementation in torch float64 with autograd.

Test-only. It shares no code with the oracle or with the HIP path: it uses
library routines where they exist (torch's rms_norm, scaled-dot-product
attention, cross_entropy) and complex multiplication for the rotary step, so
that a mistake in the oracle's hand-written formulas would show as a
disagreement here.
"""
from __future__ import annotations

import math

import torch
import torch.nn.functional as F


def _layout(depth, vocab, d, head_dim, n_kv=1):
    qkv = d + 2 * n_kv * head_dim
    shapes = [("E", vocab, d)]
    for l in range(depth):
        shapes += [(f"h{l}.Wqkv", qkv, d), (f"h{l}.Wo", d, d),
                   (f"h{l}.Wfc", 4 * d, d), (f"h{l}.Wpr", d, 4 * d)]
    shapes.append(("U", vocab, d))
    out, off = [], 0
    for name, r, c in shapes:
        out.append((name, off, r, c))
        off = -(-(off + r * c) // 128) * 128
    return out, off


def loss_and_grads(flat, tokens, targets, depth, vocab, d, head_dim,
                   softcap=15.0, base=10000.0, eps=1e-6):
    """flat: float64 numpy array of parameters. Returns (loss, grad numpy)."""
    lay, total = _layout(depth, vocab, d, head_dim)
    theta = torch.tensor(flat[:total], dtype=torch.float64, requires_grad=True)
    W = {name: theta[off:off + r * c].view(r, c) for name, off, r, c in lay}
    tok = torch.as_tensor(tokens, dtype=torch.long)
    tgt = torch.as_tensor(targets, dtype=torch.long)
    B, T = tok.shape
    H, D = d // head_dim, head_dim

    half = D // 2
    freqs = base ** (-torch.arange(0, D, 2, dtype=torch.float64) / D)     # [D/2]
    ang = torch.arange(T, dtype=torch.float64)[:, None] * freqs[None, :]  # [T, D/2]
    rot = torch.polar(torch.ones_like(ang), ang)                          # e^{i theta}

    def rotary(z):                      # z [..., T, D], pairs (j, j + D/2)
        zc = torch.complex(z[..., :half], z[..., half:]) * rot
        return torch.cat([zc.real, zc.imag], dim=-1)

    def norm(z):
        return F.rms_norm(z, (z.shape[-1],), eps=eps)

    x = norm(F.embedding(tok, W["E"]))                                    # [B, T, d]
    for l in range(depth):
        h = norm(x)
        qkv = h @ W[f"h{l}.Wqkv"].T
        q = qkv[..., :d].view(B, T, H, D).transpose(1, 2)                 # [B, H, T, D]
        k = qkv[..., d:d + D].view(B, 1, T, D)
        v = qkv[..., d + D:].view(B, 1, T, D)
        q = norm(rotary(q))
        k = norm(rotary(k))
        o = F.scaled_dot_product_attention(q, k.expand(B, H, T, D).contiguous(),
                                           v.expand(B, H, T, D).contiguous(),
                                           is_causal=True)
        x = x + o.transpose(1, 2).reshape(B, T, d) @ W[f"h{l}.Wo"].T
        u = norm(x) @ W[f"h{l}.Wfc"].T
        x = x + torch.relu(u).square() @ W[f"h{l}.Wpr"].T
    logits = norm(x) @ W["U"].T
    z = softcap * torch.tanh(logits / softcap)
    loss = F.cross_entropy(z.reshape(-1, vocab), tgt.reshape(-1))
    loss.backward()
    g = torch.zeros(len(flat), dtype=torch.float64)
    g[:total] = theta.grad
    return float(loss.detach()), g.numpy()


def attention_only(qh, kh, v):
    """Causal multi-query attention via torch's SDPA: qh [T,H,D], kh/v [T,D]."""
    q = torch.as_tensor(qh).permute(1, 0, 2)[None]
    T, H, D = qh.shape
    k = torch.as_tensor(kh)[None, None].expand(1, H, T, D).contiguous()
    vv = torch.as_tensor(v)[None, None].expand(1, H, T, D).contiguous()
    o = F.scaled_dot_product_attention(q, k, vv, is_causal=True)
    return o[0].permute(1, 0, 2).numpy()
