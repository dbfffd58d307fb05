"""Seeded synthetic inputs shared by the oracle-side tests and the GPU path.

This package builds inputs only: post-RoPE keys with planted near-duplicate
clusters, value vectors, post-RoPE queries of the last prefix positions,
per-head capacities, random retained sets and count permutations.  It
holds none of the scoring, selection or repair arithmetic; both the oracle
and the HIP library consume what it produces.
"""
from .configs import CONFIGS, Config, get_config
from .generator import (
    bf16_bits_to_f32,
    count_permutation,
    dirichlet_capacities,
    f64_to_bf16_bits,
    gumbel_retained,
    make_head,
    make_heads,
    make_queries,
    rope_tables,
)

__all__ = [
    "CONFIGS",
    "Config",
    "get_config",
    "bf16_bits_to_f32",
    "count_permutation",
    "f64_to_bf16_bits",
    "dirichlet_capacities",
    "gumbel_retained",
    "make_head",
    "make_heads",
    "make_queries",
    "rope_tables",
]
