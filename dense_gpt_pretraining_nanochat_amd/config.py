"""Model configuration and the exact work calculators (parameters, FLOPs, bytes).

The model is fixed by its depth alone: width = 64 * depth, 128-dim heads,
4x MLP (wmrh.cn tutorial, section 2.2 table: depth 20 gives 1280 wide and
10 heads; depth 30 gives 1920 wide and 15 heads; vnrom.net "nanochat: khung
thử nghiệm đơn giản nhất…", section "Thiết kế depth-only scaling": depth is
the only knob). Multi-query attention with one K/V head (followin.io release
article, architecture list). Vocabulary 65,536 (wmrh.cn tutorial, section
2.1).

This module is host-side bookkeeping for the binding, the tests and the
bench. The C library validates and lays out configs on its own.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

HEAD_DIM = 128
MI355X_BF16_DENSE_FLOPS = 2.5166e15    # 256 CU x 2.4 GHz x 4096 FLOP/clk/CU
MI355X_HBM_BYTES_PER_S = 8.0e12


@dataclass(frozen=True)
class Config:
    depth: int
    vocab_size: int
    seq_len: int
    batch: int
    dtype: str = "bf16"            # 'f32' or 'bf16' (params and activations)
    softcap: float = 15.0
    rope_base: float = 10000.0
    rms_eps: float = 1e-6
    init_std: float = 0.02
    n_kv_head: int = 1
    head_dim: int = HEAD_DIM

    @property
    def d_model(self) -> int:
        return 64 * self.depth

    @property
    def n_head(self) -> int:
        return self.d_model // self.head_dim

    @property
    def d_ff(self) -> int:
        return 4 * self.d_model

    @property
    def qkv_out(self) -> int:
        return self.d_model + 2 * self.n_kv_head * self.head_dim

    @property
    def tokens(self) -> int:
        return self.batch * self.seq_len

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


# The five workloads: tiny fp32, small, mid, depth-20 speedrun shape, depth-26.
PRESETS = {
    "C1": Config(depth=2, vocab_size=512, seq_len=64, batch=2, dtype="f32"),
    "C2": Config(depth=4, vocab_size=8192, seq_len=512, batch=8),
    "C3": Config(depth=12, vocab_size=65536, seq_len=2048, batch=8),
    "C4": Config(depth=20, vocab_size=65536, seq_len=2048, batch=32),
    "C5": Config(depth=26, vocab_size=65536, seq_len=2048, batch=16),
}
# seeds: params 1000 + index, data 2000 + index; token law per workload
SEEDS = {name: (1000 + i + 1, 2000 + i + 1) for i, name in enumerate(PRESETS)}
TOKEN_LAW = {"C1": "uniform", "C2": "zipf", "C3": "zipf", "C4": "zipf", "C5": "zipf"}


def tensor_shapes(cfg: Config, n_kv_head: int | None = None):
    kv = cfg.n_kv_head if n_kv_head is None else n_kv_head
    d, F, V = cfg.d_model, cfg.d_ff, cfg.vocab_size
    shapes = [("E", V, d)]
    for l in range(cfg.depth):
        shapes += [(f"h{l}.Wqkv", d + 2 * kv * cfg.head_dim, d), (f"h{l}.Wo", d, d),
                   (f"h{l}.Wfc", F, d), (f"h{l}.Wpr", d, F)]
    shapes.append(("U", V, d))
    return shapes


def param_count(cfg: Config, n_kv_head: int | None = None) -> int:
    return sum(r * c for _, r, c in tensor_shapes(cfg, n_kv_head))


def matmul_param_count(cfg: Config) -> int:
    """Every parameter that takes part in a matrix product: all but the
    embedding table, whose forward is a row gather."""
    return param_count(cfg) - cfg.vocab_size * cfg.d_model


def flops_per_token(cfg: Config) -> float:
    """6 * N_matmul + the exact causal attention count 6 * L * d * (T + 1)
    (forward QK^T and PV: 4 d (t + 1) per token at position t, averaged over
    t, times 3 for forward + backward)."""
    L, d, T = cfg.depth, cfg.d_model, cfg.seq_len
    return 6.0 * matmul_param_count(cfg) + 6.0 * L * d * (T + 1)


def flops_per_step(cfg: Config) -> float:
    return flops_per_token(cfg) * cfg.tokens


def flops_variants(cfg: Config) -> dict:
    L, d, T = cfg.depth, cfg.d_model, cfg.seq_len
    return {
        "causal_exact": flops_per_step(cfg),
        "noncausal_12LdT": (6.0 * matmul_param_count(cfg) + 12.0 * L * d * T) * cfg.tokens,
        "all_params_6N": 6.0 * param_count(cfg) * cfg.tokens,
    }


def mfu(cfg: Config, seconds_per_step: float) -> float:
    return flops_per_step(cfg) / seconds_per_step / MI355X_BF16_DENSE_FLOPS
