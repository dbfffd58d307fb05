"""GPU parity of the count statistics (twinkv_count_stats) against the
oracle's count_stats: every integer count exactly, the discount sum to fp64
summation order and the value-only cut exactly, on oracle-computed counts,
energies and selections (uniform and Dirichlet capacities, with and without
selections); plus the invariants on the GPU's own full-size outputs.
"""
import numpy as np
import pytest
import torch

import key_redundancy_scoring_amd as krs
from oracle import twinkv_oracle as O
from synth import dirichlet_capacities, get_config, make_heads

pytestmark = pytest.mark.gpu


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch.device("cuda:0")


def _flat(st):
    return [st["n"], st["twin"], *st["hist"], st["kept"], st["added"], st["removed"], *st["margins_added"],
            *st["margins_removed"], *st["margins_pool"]]


@pytest.mark.parametrize("cfg_id,G,N,dirichlet", [(2, 3, 1500, False), (5, 8, 900, True), (4, 2, 700, False)])
def test_count_stats_on_oracle_inputs(cfg_id, G, N, dirichlet):
    cfg = get_config(cfg_id)
    K, V, _ = make_heads(cfg, heads=range(G), N=N)
    r = cfg.removal if cfg.removal is not None else 0.5
    caps = dirichlet_capacities(cfg, G=G, N=N) if dirichlet else np.array([O.uniform_budget(N, r)] * G)
    refs = [O.score_head(K[g], V[g], cfg.tau, cfg.window) for g in range(G)]
    count = np.stack([x["count"] for x in refs]).astype(np.int32)
    energy = np.stack([x["energy"] for x in refs])
    kt = np.stack([O.select_head(x["score"], x["energy"], int(caps[g]), cfg.sink, cfg.recent)[0]
                   for g, x in enumerate(refs)])
    kv = np.stack([O.select_head(x["energy"], x["energy"], int(caps[g]), cfg.sink, cfg.recent)[0]
                   for g, x in enumerate(refs)])
    d = _dev()
    for with_sel in (True, False):
        res = krs.count_stats(torch.from_numpy(count).to(d), torch.from_numpy(energy).to(d),
                              torch.from_numpy(caps.astype(np.int32)).to(d), cfg.sink, cfg.recent,
                              keep_twin=torch.from_numpy(kt).to(d) if with_sel else None,
                              keep_value=torch.from_numpy(kv).to(d) if with_sel else None)
        torch.cuda.synchronize()
        st, fs = res["stats"].cpu().numpy(), res["fstats"].cpu().numpy()
        for g in range(G):
            ref = O.count_stats(count[g], energy[g], kt[g] if with_sel else np.zeros(N, np.uint8),
                                kv[g] if with_sel else np.zeros(N, np.uint8), int(caps[g]), cfg.sink, cfg.recent)
            assert st[g].tolist() == _flat(ref), f"head {g} selections {with_sel}"
            np.testing.assert_allclose(fs[g, 0], ref["omega_sum"], rtol=1e-12)
            assert fs[g, 1] == ref["e_cut"]


def test_count_stats_fullsize_invariants():
    cfg = get_config(2)
    G, N = cfg.G, cfg.N
    K, V, _ = make_heads(cfg)
    d = _dev()
    tk = torch.from_numpy(K.view(np.int16)).to(d)
    tv = torch.from_numpy(V.view(np.int16)).to(d)
    cap = O.uniform_budget(N, cfg.removal)
    caps = torch.full((G,), cap, dtype=torch.int32, device=d)
    res = krs.score(tk, tv, cfg.tau, cfg.window, cfg.sink, cfg.recent)
    st = krs.select(res["score"], res["energy"], caps, cfg.sink, cfg.recent)
    sv = krs.select(res["energy"], res["energy"], caps, cfg.sink, cfg.recent)
    out = krs.count_stats(res["count"], res["energy"], caps, cfg.sink, cfg.recent, keep_twin=st["keep"],
                          keep_value=sv["keep"])
    torch.cuda.synchronize()
    s = out["stats"].cpu().numpy()
    P = cfg.sink + cfg.recent
    assert np.all(s[:, 0] == N - P)
    assert np.all(s[:, 2:8].sum(1) == N - P)
    assert np.all(s[:, 8] == cap - P)
    assert np.all(s[:, 9] == s[:, 10])
    assert np.all(s[:, 21:26].sum(1) == N - P)
    frac_twin = s[:, 1].sum() / s[:, 0].sum()
    change = s[:, 9].sum() / s[:, 8].sum()
    print(f"[stats 32k] twin fraction {frac_twin:.4f}, selection change vs value-only {change:.4f}", flush=True)
    assert 0.05 < frac_twin < 0.2  # 10% planted copies plus their sources
