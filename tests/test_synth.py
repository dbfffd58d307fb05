"""The seeded generator: determinism, per-head independence and its planted
structure.  (The generator is input construction, not part of the method;
these checks are self-consistency only.)"""
import numpy as np

from synth import (CONFIGS, bf16_bits_to_f32, dirichlet_capacities, f64_to_bf16_bits, get_config,
                   gumbel_retained, make_head, make_heads)


def test_bf16_rounding_nearest_even():
    x = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -2.5, 1 + 2 ** -8 + 2 ** -20, 0.0])
    bits = f64_to_bf16_bits(x)
    assert bits.tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x3F81, 0x0000]
    assert bf16_bits_to_f32(bits).tolist() == [1.0, 1.0, 1.015625, -2.5, 1.0078125, 0.0]


def test_heads_are_deterministic_and_independent():
    cfg = get_config(2)
    a = make_head(cfg, 7, N=2048)
    b = make_head(cfg, 7, N=2048)
    assert np.array_equal(a["K"], b["K"]) and np.array_equal(a["V"], b["V"])
    K, V, cl = make_heads(cfg, heads=[3, 7], N=2048, threads=2)
    assert np.array_equal(K[1], a["K"]) and np.array_equal(V[1], a["V"])
    assert np.array_equal(cl[1], a["cluster"])
    assert not np.array_equal(K[0], K[1])


def test_planted_fraction_and_twin_cosine():
    for cfg_id in (2, 3, 4, 5):
        cfg = get_config(cfg_id)
        N = 4096
        h = make_head(cfg, 0, N=N)
        cl = h["cluster"]
        n_clusters = len(set(cl[cl >= 0].tolist()))
        assert (cl >= 0).sum() == round(cfg.twin_frac * N) + n_clusters
        sizes = np.bincount(cl[cl >= 0])
        assert sizes.min() >= 2 and sizes.max() <= 8
        K = bf16_bits_to_f32(h["K"]).astype(np.float64)
        cos = []
        for c in range(min(n_clusters, 50)):
            m = np.flatnonzero(cl == c)
            src = m[0]
            for j in m[1:]:
                cos.append(K[src] @ K[j] / np.linalg.norm(K[src]) / np.linalg.norm(K[j]))
        expect = 1 / np.sqrt(1 + cfg.sigma ** 2)
        assert abs(np.mean(cos) - expect) < 2e-3


def test_copy_trees_tiny_config():
    cfg = get_config(1)
    h = make_head(cfg, 0)
    par = h["parent"]
    assert (par >= 0).sum() == round(0.2 * cfg.N)
    t = np.flatnonzero(par >= 0)
    assert np.all(par[t] < t)


def test_dirichlet_capacities():
    cfg = get_config(5)
    caps = dirichlet_capacities(cfg)
    assert caps.shape == (cfg.G,)
    T = cfg.group * int(np.floor(cfg.budget_frac * cfg.N))
    assert T == 19656
    assert np.all(caps.reshape(-1, cfg.group).sum(1) == T)
    assert caps.min() >= 0 and caps.max() <= cfg.N
    assert np.array_equal(caps, dirichlet_capacities(cfg))


def test_gumbel_retained_half():
    cfg = get_config(3)
    m = gumbel_retained(cfg, 5, N=1000)
    assert m.sum() == 500 and set(np.unique(m).tolist()) <= {0, 1}
    assert np.array_equal(m, gumbel_retained(cfg, 5, N=1000))


def test_config_table():
    assert [CONFIGS[i].G * CONFIGS[i].N for i in range(1, 6)] == [512, 128 * 32768, 288 * 32768,
                                                                 256 * 131072, 2048 * 8192]
