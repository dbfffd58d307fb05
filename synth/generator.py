"""Seeded synthetic keys, values, capacities and retained sets.

Every head is generated from its own numpy stream,
``PCG64(SeedSequence([seed, cfg_id, g]))``, so any single head can be
regenerated on its own, bit for bit, without generating the others.

Per head (N positions, head dim d):

1. raw keys X ~ N(0, 1), drawn in float32 and widened to float64;
2. rotary position embedding with base theta applied in float64, rotating the
   half-split pairs (p, p + d/2) of position i by the angle i * theta^(-2p/d);
   the pages compute redundancy on keys as the cache stores them, after RoPE
   (TwinKV arXiv page, section 3.2), so copies are planted after the rotation;
3. planted near-duplicates, post-RoPE:
   * ``tree``: round(frac*N) positions t >= 1 are drawn without replacement and
     visited in increasing order; each becomes K[src] + noise with src uniform
     in [0, t), so copies of copies form trees;
   * ``cluster``: clusters are added until round(frac*N) copies exist; a cluster
     draws its size s uniformly from 2..8, an unused source p, and s-1 unused
     positions after p, each set to K[p] + noise (the last cluster is cut to hit
     the exact count);
   noise is i.i.d. N(0, sigma^2) per component;
4. values V = N(0, 1) * f_i with one LogNormal(0, 0.5) factor f_i per position;
5. keys and values are rounded to float32 and then to bfloat16 (round to
   nearest even); the arrays hold the raw bf16 bit patterns as uint16.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os

import numpy as np

from .configs import Config

# Offsets that keep the auxiliary streams apart from the per-head key streams.
_CAPACITY_STREAM = 1_000_003
_GUMBEL_STREAM = 2
_QUERY_STREAM = 3
_PERM_STREAM = 4


def _head_rng(cfg: Config, g: int, *extra: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.seed, cfg.cfg_id, int(g), *extra])))


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round to float32, then to bfloat16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 exactly."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


_ROPE_CACHE: dict = {}


def rope_tables(N: int, d: int, base: float):
    """cos/sin of i * base^(-2p/d) for i < N, p < d/2, in float64."""
    key = (int(N), int(d), float(base))
    hit = _ROPE_CACHE.get(key)
    if hit is not None:
        return hit
    half = d // 2
    inv_freq = base ** (-2.0 * np.arange(half, dtype=np.float64) / d)
    ang = np.arange(N, dtype=np.float64)[:, None] * inv_freq[None, :]
    tab = (np.cos(ang), np.sin(ang))
    if len(_ROPE_CACHE) > 4:
        _ROPE_CACHE.clear()
    _ROPE_CACHE[key] = tab
    return tab


def _apply_rope(X: np.ndarray, base: float) -> np.ndarray:
    N, d = X.shape
    cos, sin = rope_tables(N, d, base)
    half = d // 2
    a, b = X[:, :half], X[:, half:]
    out = np.empty_like(X)
    out[:, :half] = a * cos - b * sin
    out[:, half:] = a * sin + b * cos
    return out


def _plant_tree(rng, X, n_copies, sigma):
    N, d = X.shape
    parent = np.full(N, -1, dtype=np.int64)
    if n_copies == 0 or N < 2:
        return parent
    targets = np.sort(rng.choice(np.arange(1, N), size=n_copies, replace=False))
    for t in targets:
        src = int(rng.integers(0, t))
        X[t] = X[src] + sigma * rng.standard_normal(d)
        parent[t] = src
    return parent


def _plant_clusters(rng, X, n_copies, sigma):
    N, d = X.shape
    cluster = np.full(N, -1, dtype=np.int64)
    used = np.zeros(N, dtype=bool)
    placed = 0
    cid = 0
    while placed < n_copies:
        size = int(rng.integers(2, 9))
        k = min(size - 1, n_copies - placed)
        members: list[int] = []
        for _ in range(10000):
            p = int(rng.integers(0, N))
            if used[p] or N - 1 - p < k:
                continue
            members = []
            seen = set()
            for _ in range(64):
                for c in rng.integers(p + 1, N, size=2 * k + 2):
                    c = int(c)
                    if not used[c] and c not in seen:
                        seen.add(c)
                        members.append(c)
                        if len(members) == k:
                            break
                if len(members) == k:
                    break
            if len(members) == k:
                break
        else:
            raise RuntimeError("could not place a twin cluster; twin fraction too high for N")
        m = np.sort(np.asarray(members, dtype=np.int64))
        X[m] = X[p][None, :] + sigma * rng.standard_normal((k, d))
        used[p] = True
        used[m] = True
        cluster[p] = cid
        cluster[m] = cid
        cid += 1
        placed += k
    return cluster


def make_head(cfg: Config, g: int, N: int | None = None, d: int | None = None):
    """Generate head ``g`` of a workload.

    Returns a dict with ``K`` and ``V`` (uint16 bf16 bits, [N][d]) and the planted
    structure: ``cluster`` (cluster id per position, -1 if none) for clustered
    workloads, ``parent`` (source of each copy, -1 if none) for copy trees.
    """
    N = cfg.N if N is None else int(N)
    d = cfg.d if d is None else int(d)
    rng = _head_rng(cfg, g)
    X = rng.standard_normal((N, d), dtype=np.float32).astype(np.float64)
    X = _apply_rope(X, cfg.rope_base)
    n_copies = int(round(cfg.twin_frac * N))
    out = {}
    if cfg.twin_mode == "tree":
        out["parent"] = _plant_tree(rng, X, n_copies, cfg.sigma)
        out["cluster"] = _tree_components(out["parent"])
    elif cfg.twin_mode == "cluster":
        out["cluster"] = _plant_clusters(rng, X, n_copies, cfg.sigma)
    elif cfg.twin_mode == "none":
        out["cluster"] = np.full(N, -1, dtype=np.int64)
    else:
        raise ValueError(cfg.twin_mode)
    V = rng.standard_normal((N, d), dtype=np.float32)
    f = rng.lognormal(0.0, 0.5, size=N).astype(np.float32)
    V = V * f[:, None]
    out["K"] = f64_to_bf16_bits(X)
    out["V"] = f64_to_bf16_bits(V)
    return out


def _tree_components(parent: np.ndarray) -> np.ndarray:
    """Component id of every node that takes part in a copy tree, -1 otherwise."""
    N = parent.shape[0]
    root = np.arange(N)
    for t in range(N):  # parents precede children, so one forward pass suffices
        if parent[t] >= 0:
            root[t] = root[parent[t]]
    involved = parent >= 0
    involved[parent[parent >= 0]] = True
    comp = np.where(involved, root, -1)
    return comp.astype(np.int64)


def _default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def make_heads(cfg: Config, heads=None, N: int | None = None, d: int | None = None,
               threads: int | None = None, with_values: bool = True, out_K=None, out_V=None):
    """Generate several heads in parallel threads.

    Returns ``(K, V, clusters)`` with K, V uint16 [len(heads)][N][d] (V is None when
    ``with_values`` is false) and clusters int64 [len(heads)][N].
    """
    heads = list(range(cfg.G)) if heads is None else [int(h) for h in heads]
    N = cfg.N if N is None else int(N)
    d = cfg.d if d is None else int(d)
    H = len(heads)
    K = out_K if out_K is not None else np.empty((H, N, d), dtype=np.uint16)
    V = None
    if with_values:
        V = out_V if out_V is not None else np.empty((H, N, d), dtype=np.uint16)
    clusters = np.empty((H, N), dtype=np.int64)
    rope_tables(N, d, cfg.rope_base)  # build the shared table once, outside the workers

    def work(slot):
        h = make_head(cfg, heads[slot], N=N, d=d)
        K[slot] = h["K"]
        if V is not None:
            V[slot] = h["V"]
        clusters[slot] = h["cluster"]

    nt = threads or _default_threads()
    if nt <= 1 or H <= 1:
        for s in range(H):
            work(s)
    else:
        with _cf.ThreadPoolExecutor(nt) as ex:
            list(ex.map(work, range(H)))
    return K, V, clusters


def dirichlet_capacities(cfg: Config, G: int | None = None, N: int | None = None) -> np.ndarray:
    """Per-head capacities from a Dirichlet(1) split of a shared slot budget.

    Heads are grouped ``cfg.group`` at a time (one group per batch element and
    layer).  A group owns T = group * floor(budget_frac * N) slots.  Each head
    gets floor(p_h * T); the leftover slots go one each to the heads with the
    largest fractional parts (ties to the lowest head).  A head above N is cut to
    N and its excess is handed to the uncut heads in proportion to p_h, by the
    same floor-plus-largest-remainder rule, until no head exceeds N.
    """
    G = cfg.G if G is None else int(G)
    N = cfg.N if N is None else int(N)
    grp = int(cfg.group)
    if G % grp:
        raise ValueError("G must be a multiple of the group size")
    per_head = int(np.floor(cfg.budget_frac * N))
    T = grp * per_head
    caps = np.empty(G, dtype=np.int64)
    for q in range(G // grp):
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.seed, cfg.cfg_id, _CAPACITY_STREAM, q])))
        p = rng.dirichlet(np.ones(grp))
        b = _largest_remainder(p, T)
        while np.any(b > N):
            over = b > N
            excess = int((b[over] - N).sum())
            b[over] = N
            free = b < N
            share = np.where(free, p, 0.0)
            if share.sum() <= 0:
                raise ValueError("budget exceeds group capacity")
            b = b + _largest_remainder(share / share.sum(), excess)
        assert int(b.sum()) == T
        caps[q * grp:(q + 1) * grp] = b
    return caps.astype(np.int32)


def _largest_remainder(p: np.ndarray, total: int) -> np.ndarray:
    raw = p * total
    b = np.floor(raw).astype(np.int64)
    rem = raw - b
    left = int(total - b.sum())
    order = np.argsort(-rem, kind="stable")
    b[order[:left]] += 1
    return b


def gumbel_retained(cfg: Config, g: int, N: int | None = None, keep: int | None = None) -> np.ndarray:
    """A random retained mask: the top ``keep`` positions (default N/2) by an
    i.i.d. Gumbel(0, 1) draw per position, ties to the lowest position."""
    N = cfg.N if N is None else int(N)
    keep = N // 2 if keep is None else int(keep)
    rng = _head_rng(cfg, g, _GUMBEL_STREAM)
    z = rng.gumbel(size=N)
    idx = np.argsort(-z, kind="stable")[:keep]
    m = np.zeros(N, dtype=np.uint8)
    m[idx] = 1
    return m


def make_queries(cfg: Config, g: int, Gq: int = 4, W: int = 32, N: int | None = None, d: int | None = None):
    """Post-RoPE queries of the last W prefix positions for the Gq query heads
    that share KV head ``g`` ([Gq][W][d] bf16 bits).

    Raw queries are N(0, s_g^2) with one sharpness s_g per KV head, drawn
    log-uniformly from [0.25, 2]: heads differ in how concentrated their
    attention over the prefix is, which is what capacity allocation reacts
    to.  Query t is rotated with the workload's base at position N - W + t.
    """
    N = cfg.N if N is None else int(N)
    d = cfg.d if d is None else int(d)
    W = min(int(W), N)
    rng = _head_rng(cfg, g, _QUERY_STREAM)
    s_g = float(np.exp(rng.uniform(np.log(0.25), np.log(2.0))))
    X = rng.standard_normal((Gq, W, d), dtype=np.float32).astype(np.float64) * s_g
    cos, sin = rope_tables(N, d, cfg.rope_base)
    cos, sin = cos[N - W:], sin[N - W:]
    half = d // 2
    a, b = X[..., :half], X[..., half:]
    out = np.empty_like(X)
    out[..., :half] = a * cos - b * sin
    out[..., half:] = a * sin + b * cos
    return f64_to_bf16_bits(out)


def count_permutation(cfg: Config, g: int, capacity: int, seed: int, N: int | None = None) -> np.ndarray:
    """A seeded permutation of head ``g``'s unprotected positions (int32 [N]):
    position i takes the count of position perm[i].  Protected positions (the
    first min(sink, b) and the last min(recent, b - s) for capacity b) map to
    themselves.  ``seed`` picks one of the fixed permutations (the pages use
    three fixed seeds: 11, 29 and 47)."""
    N = cfg.N if N is None else int(N)
    b = int(min(max(int(capacity), 0), N))
    s = min(cfg.sink, b)
    r = min(cfg.recent, b - s)
    perm = np.arange(N, dtype=np.int64)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), cfg.cfg_id, int(g), _PERM_STREAM])))
    free = np.arange(s, N - r)
    perm[free] = rng.permutation(free)
    return perm.astype(np.int32)
