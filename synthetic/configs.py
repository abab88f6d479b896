"""Workload shapes for the MILO hot path.

The pages evaluate Qwen2.5-3B and Qwen2.5-7B with 512-shot prompts on one GPU
(evolve.pub review of arXiv 2609.29913, Summary and Scope).  Neither the
weights nor the six task datasets are available, so every KV block is a seeded
planted-spectrum matrix with the shapes below (the attention geometry of those
two models: head_dim 128, GQA groups of 8 and 7 query heads per KV head).

Budgets are per pool; a pool is one (sequence, layer, KV head, K-or-V) stream of
blocks, and R = budget_frac * blocks_per_seq * head_dim.
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class Config:
    idx: int
    workload: str
    storage: str            # "f32" or "bf16" for the cache; factors use the same by default
    layers: int
    n_kv_heads: int
    n_q_heads: int
    head_dim: int
    block_len: int
    blocks_per_seq: int
    batch: int
    tau_k: tuple
    tau_v: tuple
    budget_fracs: tuple = (0.5,)
    factor_storages: tuple = ()  # empty -> same as storage
    sel_blocks: int = 0          # 0 -> every block attended
    tail_len: int = 0
    eps2: float = 1e-4
    noise_std: float = 1e-3
    rope_base: float = 1e6

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def context_len(self) -> int:
        return self.block_len * self.blocks_per_seq

    @property
    def blocks_per_layer(self) -> int:
        """K blocks (= V blocks) of one layer over the whole batch."""
        return self.batch * self.n_kv_heads * self.blocks_per_seq

    @property
    def pools_per_layer(self) -> int:
        return self.batch * self.n_kv_heads

    def budget(self, frac: float | None = None) -> int:
        frac = self.budget_fracs[0] if frac is None else frac
        return int(round(frac * self.blocks_per_seq * self.head_dim))

    @property
    def attended_blocks(self) -> int:
        return self.sel_blocks if self.sel_blocks else self.blocks_per_seq

    @property
    def context_tokens_per_step(self) -> int:
        """Sum over sequences of attended tokens (selected blocks + tail)."""
        return self.batch * (self.attended_blocks * self.block_len + self.tail_len)

    def storages(self):
        return self.factor_storages or (self.storage,)


CONFIGS = {
    0: Config(0, "tiny-fp32: 1 layer, 1 KV head, 1 q head, 8 blocks x 256 tokens",
              "f32", layers=1, n_kv_heads=1, n_q_heads=1, head_dim=128, block_len=256,
              blocks_per_seq=8, batch=1, tau_k=(4.0, 32.0), tau_v=(4.0, 32.0)),
    1: Config(1, "qwen2.5-3b-shaped layer: 2 KV heads, 16 q heads, 32 blocks x 1024 tokens",
              "bf16", layers=1, n_kv_heads=2, n_q_heads=16, head_dim=128, block_len=1024,
              blocks_per_seq=32, batch=1, tau_k=(4.0, 24.0), tau_v=(16.0, 64.0)),
    2: Config(2, "qwen2.5-7b-shaped stack: 28 layers, 4 KV heads, 28 q heads, batch 8, "
                 "8 of 64 blocks x 1024 tokens + 256-token tail",
              "bf16", layers=28, n_kv_heads=4, n_q_heads=28, head_dim=128, block_len=1024,
              blocks_per_seq=64, batch=8, tau_k=(4.0, 24.0), tau_v=(16.0, 64.0),
              sel_blocks=8, tail_len=256),
    3: Config(3, "budget/precision sweep on the 3b-shaped layer: 25/50/75% x {bf16, int8}",
              "bf16", layers=1, n_kv_heads=2, n_q_heads=16, head_dim=128, block_len=1024,
              blocks_per_seq=32, batch=1, tau_k=(4.0, 24.0), tau_v=(16.0, 64.0),
              budget_fracs=(0.25, 0.5, 0.75), factor_storages=("bf16", "i8")),
    4: Config(4, "qwen2.5-3b-shaped long context: 36 layers, 2 KV heads, 16 q heads, "
                 "batch 16, 64 blocks x 2048 tokens",
              "bf16", layers=36, n_kv_heads=2, n_q_heads=16, head_dim=128, block_len=2048,
              blocks_per_seq=64, batch=16, tau_k=(4.0, 24.0), tau_v=(16.0, 64.0)),
}


def pool_layout(cfg: Config, frac: float | None = None):
    """Pool CSR and budgets for one layer's K (or V) blocks.

    Block id within a layer = (s * n_kv_heads + h) * blocks_per_seq + b, so each
    (s, h) pool is a contiguous run of blocks_per_seq blocks.
    """
    n_pools = cfg.pools_per_layer
    ptr = [p * cfg.blocks_per_seq for p in range(n_pools + 1)]
    budgets = [cfg.budget(frac)] * n_pools
    return ptr, budgets
