"""The five synthetic workloads.

Shapes follow the model families the TwinKV pages evaluate on (Llama-3.2-1B:
16 layers x 8 KV heads, head_dim 64; Qwen3-4B: 36 layers x 8 KV heads,
head_dim 128), stretched to longer prefixes.  Parameters a workload does not
restate are inherited from the one before it (tau 0.9, window 64, 4 sinks,
64 recent positions, noise sigma 0.05, clusters of 2..8, RoPE base 1e4).
"""
from __future__ import annotations

import dataclasses


@dataclasses.dataclass(frozen=True)
class Config:
    cfg_id: int
    name: str
    G: int  # independent heads = batch * layers * kv_heads
    N: int  # prefix length
    d: int  # head dim
    rope_base: float
    twin_frac: float  # fraction of positions that are planted copies
    twin_mode: str  # "tree": copies of random earlier keys; "cluster": clusters of 2..8
    sigma: float  # standard deviation of the noise added to each copy
    tau: float
    window: int
    sink: int
    recent: int
    mode: str  # "score+select", "repair", "score+select+repair"
    removal: float | None  # uniform removal ratio r (capacity = floor(N(1-r)))
    budget_frac: float | None = None  # Dirichlet workload: fraction of slots kept
    group: int = 8  # heads per (batch, layer) sharing one Dirichlet split
    seed: int = 0

    @property
    def keys(self) -> int:
        return self.G * self.N

    def with_(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    1: Config(1, "tiny", G=1, N=512, d=64, rope_base=1e4, twin_frac=0.20,
              twin_mode="tree", sigma=0.05, tau=0.9, window=32, sink=4, recent=32,
              mode="score+select", removal=0.5),
    2: Config(2, "llama-3.2-1b-32k", G=16 * 8, N=32768, d=64, rope_base=1e4,
              twin_frac=0.10, twin_mode="cluster", sigma=0.05, tau=0.9, window=64,
              sink=4, recent=64, mode="score+select", removal=0.5),
    3: Config(3, "qwen3-4b-32k-repair", G=36 * 8, N=32768, d=128, rope_base=1e6,
              twin_frac=0.15, twin_mode="cluster", sigma=0.05, tau=0.9, window=64,
              sink=4, recent=64, mode="repair", removal=0.5),
    4: Config(4, "long-131k", G=32 * 8, N=131072, d=128, rope_base=5e5,
              twin_frac=0.05, twin_mode="cluster", sigma=0.1, tau=0.85, window=128,
              sink=4, recent=64, mode="score+select", removal=0.75),
    5: Config(5, "batched-8k-dirichlet", G=16 * 16 * 8, N=8192, d=64, rope_base=1e4,
              twin_frac=0.25, twin_mode="cluster", sigma=0.05, tau=0.9, window=64,
              sink=4, recent=64, mode="score+select+repair", removal=None,
              budget_frac=0.3),
}


def get_config(cfg_id: int, **overrides) -> Config:
    cfg = CONFIGS[int(cfg_id)]
    return cfg.with_(**overrides) if overrides else cfg
