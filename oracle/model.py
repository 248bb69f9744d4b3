"""fp64 numpy oracle: forward, loss and hand-derived backward of the dense GPT.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What is computed, and where the pages fix it:
  * dense decoder-only Transformer, Llama-like but simpler
      [release] architecture list (dense, no sparsity; Llama-like)
  * untied token embedding E[V,d] and lm_head U[V,d]
      [release] architecture list (embedding/unembedding not shared)
  * the token-embedding output is RMS-normalised
      [release] architecture list (norm after token embedding)
  * RMSNorm without learnable parameters
      [release] architecture list
  * rotary position embeddings and nothing else for position
      [release] architecture list
  * QK-norm: the query and key vectors are normalised
      [release] architecture list
  * multi-query attention (one K/V head shared by all query heads)
      [release] architecture list; the configs give 1 KV head
  * relu^2 activation in a 4x MLP
      [release] architecture list; [tutorial] section 2.2 (FFN ratio 4)
  * bias-free linear layers
      [release] architecture list
  * tanh logit softcap
      [release] architecture list
  * next-token cross-entropy objective
      [tutorial] section 2.3 (pretraining objective)
  * width = 64 * depth, 128-dim heads (depth 20 -> 1280 wide, 10 heads;
    depth 30 -> 1920 wide, 15 heads)
      [tutorial] section 2.2 table; [harness] "Thiết kế depth-only scaling"

Readings where the pages are silent:
  RMSNorm n(v) = v / sqrt(mean(v^2) + eps), eps = 1e-6; pre-norm residual
  blocks x += f(n(x)); a final norm before lm_head; rotary on half-split pairs
  (j, j + D/2) with angle t * base^(-2j/D), base 10000, positions 0..T-1 in
  each row, rotating by +angle; rotary first, then the QK RMSNorm (the two
  commute exactly); attention scale 1/sqrt(D), causal mask that keeps the
  diagonal; softcap c * tanh(l / c) with c = 15 on every logit; natural-log
  cross-entropy averaged over all B*T positions.

Everything is float64. The backward pass is derived by hand (chain rule,
written out below); finite differences and an independent autograd
implementation check it in the tests.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


# --------------------------------------------------------------------------
# configuration and flat parameter layout
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class OracleConfig:
    """Shape of the model. ``head_dim`` may be overridden for tiny
    finite-difference configs; the product path fixes it at 128."""
    depth: int
    vocab: int
    seq_len: int
    batch: int
    head_dim: int = 128
    n_kv_head: int = 1
    d_model: int | None = None      # default 64 * depth
    softcap: float = 15.0
    rope_base: float = 10000.0
    eps: float = 1e-6

    @property
    def d(self) -> int:
        return self.d_model if self.d_model is not None else 64 * self.depth

    @property
    def n_head(self) -> int:
        return self.d // self.head_dim

    @property
    def d_ff(self) -> int:
        return 4 * self.d

    @property
    def qkv_out(self) -> int:
        return self.d + 2 * self.n_kv_head * self.head_dim

    @property
    def M(self) -> int:
        return self.batch * self.seq_len


def _align128(n: int) -> int:
    return (n + 127) // 128 * 128


def layout(cfg: OracleConfig):
    """Flat parameter order: E, then per layer Wqkv, Wo, Wfc, Wpr, then U.

    Every matrix is [out, in] row-major (y = x W^T); the query rows of Wqkv
    are head 0..H-1 in order, then the key rows, then the value rows. Each
    tensor starts on a multiple of 128 elements. Returns a list of
    (name, offset, rows, cols)."""
    d, L = cfg.d, cfg.depth
    out, off = [], 0

    def add(name, rows, cols):
        nonlocal off
        out.append((name, off, rows, cols))
        off = _align128(off + rows * cols)

    add("E", cfg.vocab, d)
    for l in range(L):
        add(f"h{l}.Wqkv", cfg.qkv_out, d)
        add(f"h{l}.Wo", d, d)
        add(f"h{l}.Wfc", cfg.d_ff, d)
        add(f"h{l}.Wpr", d, cfg.d_ff)
    add("U", cfg.vocab, d)
    return out


def param_count(cfg: OracleConfig, padded: bool = False) -> int:
    lay = layout(cfg)
    if padded:
        name, off, r, c = lay[-1]
        return _align128(off + r * c)
    return sum(r * c for _, _, r, c in lay)


def unpack(cfg: OracleConfig, flat: np.ndarray) -> dict:
    """Views of a flat float64 buffer as named matrices."""
    return {name: flat[off:off + r * c].reshape(r, c)
            for name, off, r, c in layout(cfg)}


# --------------------------------------------------------------------------
# building blocks
# --------------------------------------------------------------------------

def rmsnorm(v: np.ndarray, eps: float):
    """Parameter-free RMSNorm over the last axis.
    Returns (y, rinv) with rinv = 1 / sqrt(mean(v^2) + eps)."""
    rinv = 1.0 / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps)
    return v * rinv, rinv


def rmsnorm_bwd(dy: np.ndarray, y: np.ndarray, rinv: np.ndarray) -> np.ndarray:
    """Gradient through y = v * rinv(v), n = len(v):
    d rinv / d v_j = -rinv^3 v_j / n, hence
    dv = rinv * (dy - y * mean(dy * y))."""
    return rinv * (dy - y * np.mean(dy * y, axis=-1, keepdims=True))


def rope_tables(cfg: OracleConfig, T: int | None = None):
    """cos and sin of theta[t, j] = t * base^(-2j/D), t = 0..T-1, j < D/2."""
    T = cfg.seq_len if T is None else T
    half = cfg.head_dim // 2
    inv_freq = cfg.rope_base ** (-2.0 * np.arange(half, dtype=np.float64)
                                 / cfg.head_dim)
    theta = np.arange(T, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.cos(theta), np.sin(theta)


def rope(z: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate pairs (z_j, z_{j+D/2}) by +theta. z is [T, ..., D]; cos/sin are
    [T, D/2] and broadcast over the middle axes."""
    half = z.shape[-1] // 2
    shape = (cos.shape[0],) + (1,) * (z.ndim - 2) + (half,)
    c, s = cos.reshape(shape), sin.reshape(shape)
    a, b = z[..., :half], z[..., half:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def rope_bwd(g: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Transpose of the rotation: rotate the gradient by -theta."""
    return rope(g, cos, -sin)


def causal_mqa(qh: np.ndarray, kh: np.ndarray, v: np.ndarray):
    """Textbook causal softmax attention with one K/V head shared by every
    query head. qh [T,H,D], kh [T,D], v [T,D] -> (o [T,H,D], P [H,T,T]).
    The contractions are plain matrix products (every head against the one
    key / value matrix)."""
    T, H, D = qh.shape
    qt = np.ascontiguousarray(qh.transpose(1, 0, 2))          # [H, T, D]
    s = np.matmul(qt, kh.T) / math.sqrt(D)                    # [H, T, T]: s[h,t,u] = q_t . k_u
    mask = np.triu(np.ones((T, T), dtype=bool), k=1)          # u > t
    s = np.where(mask[None], -np.inf, s)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)                                             # exact 0 where masked
    p /= p.sum(axis=-1, keepdims=True)
    o = np.matmul(p, v).transpose(1, 0, 2)                    # o[t,h] = sum_u p[h,t,u] v_u
    return o, p


# --------------------------------------------------------------------------
# forward for one batch row
# --------------------------------------------------------------------------

def row_forward(cfg: OracleConfig, P: dict, tok: np.ndarray, keep: bool):
    """Forward pass for one row of T tokens. Returns (logits_capped z [T,V],
    cache or None). ``keep`` saves what the backward pass needs."""
    T = tok.shape[0]
    d, H, D, L = cfg.d, cfg.n_head, cfg.head_dim, cfg.depth
    cos, sin = rope_tables(cfg, T)
    cache = {"layers": []} if keep else None

    e = P["E"][tok]                                   # gather [T, d]
    x, r0 = rmsnorm(e, cfg.eps)                       # norm after the embedding
    if keep:
        cache["x0"], cache["r0"] = x.copy(), r0
    for l in range(L):
        Wqkv, Wo = P[f"h{l}.Wqkv"], P[f"h{l}.Wo"]
        Wfc, Wpr = P[f"h{l}.Wfc"], P[f"h{l}.Wpr"]
        # attention sub-block
        h, r1 = rmsnorm(x, cfg.eps)
        qkv = h @ Wqkv.T
        q = qkv[:, :d].reshape(T, H, D)
        k = qkv[:, d:d + D]
        v = qkv[:, d + D:d + 2 * D]
        qh, rq = rmsnorm(rope(q, cos, sin), cfg.eps)   # per head vector
        kh, rk = rmsnorm(rope(k, cos, sin), cfg.eps)
        o, p = causal_mqa(qh, kh, v)
        of = o.reshape(T, d)
        x = x + of @ Wo.T
        # MLP sub-block
        h2, r2 = rmsnorm(x, cfg.eps)
        pre = h2 @ Wfc.T
        a = np.maximum(pre, 0.0) ** 2
        x = x + a @ Wpr.T
        if keep:
            cache["layers"].append(dict(h=h, r1=r1, qh=qh, rq=rq, kh=kh, rk=rk,
                                        v=v, o=of, h2=h2, r2=r2, pre=pre, a=a))
    xf, rf = rmsnorm(x, cfg.eps)
    logits = xf @ P["U"].T
    z = cfg.softcap * np.tanh(logits / cfg.softcap)
    if keep:
        cache.update(xf=xf, rf=rf, cos=cos, sin=sin)
    return z, cache


def causal_mqa_bwd(qh, kh, v, o, do):
    """Gradients of causal_mqa: with P the attention weights,
    dv_u = sum_h sum_{t>=u} P dO, dP = dO v^T, delta = rowsum(dO * O),
    dS = P (dP - delta), dq = dS k / sqrt(D), dk = sum_h dS^T q / sqrt(D).
    Returns (dqh [T,H,D], dkh [T,D], dv [T,D])."""
    T, H, D = qh.shape
    _, p = causal_mqa(qh, kh, v)                           # recompute P [H,T,T]
    dot = np.ascontiguousarray(do.transpose(1, 0, 2))      # [H, T, D]
    qt = np.ascontiguousarray(qh.transpose(1, 0, 2))
    dv = sum(p[h].T @ dot[h] for h in range(H))          # summed over heads and queries
    dp = np.matmul(dot, v.T)                               # [H, T, T]
    delta = (do * o).sum(axis=-1).T                        # [H, T] = rowsum(P * dP)
    ds = p * (dp - delta[:, :, None])
    dqh = np.matmul(ds, kh).transpose(1, 0, 2) / math.sqrt(D)
    dkh = sum(ds[h].T @ qt[h] for h in range(H)) / math.sqrt(D)
    return dqh, dkh, dv


def softcap_ce_grad(z, lse, tgt, c, w):
    """Gradient of w * sum_t (lse_t - z[t, tgt_t]) with respect to the raw
    logits l, where z = c tanh(l / c): w (softmax(z) - onehot) (1 - (z/c)^2)."""
    T = z.shape[0]
    dz = np.exp(z - lse[:, None])
    dz[np.arange(T), tgt] -= 1.0
    dz *= w
    return dz * (1.0 - (z / c) ** 2)


def softcap_ce_rows(logits, tgt, c, w):
    """Per-row loss and logit gradient of the capped cross-entropy for raw
    logits [R, V] (the lm_head output). Returns (loss [R], dlogits [R, V])."""
    z = c * np.tanh(np.asarray(logits, dtype=np.float64) / c)
    lt, lse = _token_losses(z, tgt)
    return lt, softcap_ce_grad(z, lse, tgt, c, w)


def _token_losses(z: np.ndarray, tgt: np.ndarray):
    zmax = z.max(axis=-1, keepdims=True)
    lse = (zmax + np.log(np.exp(z - zmax).sum(axis=-1, keepdims=True)))[:, 0]
    return lse - z[np.arange(z.shape[0]), tgt], lse


# --------------------------------------------------------------------------
# public entry points
# --------------------------------------------------------------------------

def _as_params(cfg, params):
    flat = np.asarray(params, dtype=np.float64)
    return unpack(cfg, flat)


def forward_loss(cfg: OracleConfig, params: np.ndarray, tokens: np.ndarray,
                 targets: np.ndarray, return_token_losses: bool = False):
    """Mean next-token cross-entropy over all B*T positions (natural log).
    ``params`` is the flat buffer (any float dtype, upcast to float64);
    tokens/targets are int [B, T]."""
    P = _as_params(cfg, params)
    tokens = np.asarray(tokens).reshape(-1, cfg.seq_len)
    targets = np.asarray(targets).reshape(-1, cfg.seq_len)
    per_tok = []
    for b in range(tokens.shape[0]):
        z, _ = row_forward(cfg, P, tokens[b], keep=False)
        lt, _ = _token_losses(z, targets[b])
        per_tok.append(lt)
    per_tok = np.stack(per_tok)
    loss = per_tok.sum() / per_tok.size
    return (loss, per_tok) if return_token_losses else loss


def forward_backward(cfg: OracleConfig, params: np.ndarray, tokens: np.ndarray,
                     targets: np.ndarray, rows=None, M: int | None = None):
    """Loss and gradient of the mean loss with respect to every parameter.

    Processes one batch row at a time and accumulates into a flat float64
    gradient with the same layout as ``params``. ``rows`` restricts the work
    to a subset of rows while keeping the 1/M normalisation (M defaults to
    the number of rows processed times T), which lets the tests and the
    timing leg run a bounded sample of a large batch.
    Returns (loss_over_processed_rows, grads_flat, per_token_losses)."""
    P = _as_params(cfg, params)
    tokens = np.asarray(tokens).reshape(-1, cfg.seq_len)
    targets = np.asarray(targets).reshape(-1, cfg.seq_len)
    rows = list(range(tokens.shape[0])) if rows is None else list(rows)
    T = cfg.seq_len
    M = len(rows) * T if M is None else M
    grads = np.zeros(param_count(cfg, padded=True), dtype=np.float64)
    G = unpack(cfg, grads)
    total, per_tok = 0.0, []
    for b in rows:
        z, cache = row_forward(cfg, P, tokens[b], keep=True)
        lt, lse = _token_losses(z, targets[b])
        total += lt.sum()
        per_tok.append(lt)
        _row_backward(cfg, P, G, tokens[b], targets[b], z, lse, cache, 1.0 / M)
    return total / M, grads, np.stack(per_tok)


def _row_backward(cfg, P, G, tok, tgt, z, lse, cache, w):
    """Hand-derived backward for one row; adds into the gradient views G."""
    T = tok.shape[0]
    d, H, D, L, c = cfg.d, cfg.n_head, cfg.head_dim, cfg.depth, cfg.softcap
    cos, sin = cache["cos"], cache["sin"]

    dl = softcap_ce_grad(z, lse, tgt, c, w)
    # lm_head: l = xf U^T
    G["U"] += dl.T @ cache["xf"]
    dxf = dl @ P["U"]
    dx = rmsnorm_bwd(dxf, cache["xf"], cache["rf"])

    for l in reversed(range(L)):
        Wqkv, Wo = P[f"h{l}.Wqkv"], P[f"h{l}.Wo"]
        Wfc, Wpr = P[f"h{l}.Wfc"], P[f"h{l}.Wpr"]
        a_ = cache["layers"][l]
        # MLP: x_out = x_mid + relu(h2 Wfc^T)^2 Wpr^T, h2 = n(x_mid)
        G[f"h{l}.Wpr"] += dx.T @ a_["a"]
        da = dx @ Wpr
        dpre = da * 2.0 * np.maximum(a_["pre"], 0.0)
        G[f"h{l}.Wfc"] += dpre.T @ a_["h2"]
        dh2 = dpre @ Wfc
        dx = dx + rmsnorm_bwd(dh2, a_["h2"], a_["r2"])
        # attention: x_mid = x_in + o Wo^T
        G[f"h{l}.Wo"] += dx.T @ a_["o"]
        do = (dx @ Wo).reshape(T, H, D)
        qh, kh, v = a_["qh"], a_["kh"], a_["v"]
        dqh, dkh, dv = causal_mqa_bwd(qh, kh, v, a_["o"].reshape(T, H, D), do)
        # QK-norm, then the transposed rotation
        dq = rope_bwd(rmsnorm_bwd(dqh, qh, a_["rq"]), cos, sin)
        dk = rope_bwd(rmsnorm_bwd(dkh, kh, a_["rk"]), cos, sin)
        dqkv = np.concatenate([dq.reshape(T, d), dk, dv], axis=1)
        G[f"h{l}.Wqkv"] += dqkv.T @ a_["h"]
        dh = dqkv @ Wqkv
        dx = dx + rmsnorm_bwd(dh, a_["h"], a_["r1"])

    # embedding norm, then scatter-add into the gathered rows
    de = rmsnorm_bwd(dx, cache["x0"], cache["r0"])
    np.add.at(G["E"], tok, de)
