"""GPU parity of the score variants (twinkv_variant_score + twinkv_select)
against the oracle's variant_scores + select_head: value-only, rarity-only
(also with the standalone count score's ceil budget) and the within-head
count permutation with the three fixed seeds.  The variant keys are checked
on oracle-computed counts and energies; the whole chain (GPU score ->
variant -> select) is checked against the oracle chain with the usual
exclusions.
"""
import numpy as np
import pytest
import torch

import key_redundancy_scoring_amd as krs
from oracle import twinkv_oracle as O
from synth import count_permutation, get_config, make_heads
from tests import parity as PR

pytestmark = pytest.mark.gpu

SEEDS = (11, 29, 47)


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch.device("cuda:0")


def _up(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(_dev())


def _oracle_counts(cfg, G, N):
    K, V, _ = make_heads(cfg, heads=range(G), N=N)
    refs = [O.score_head(K[g], V[g], cfg.tau, cfg.window) for g in range(G)]
    return K, V, refs


def _variants(cfg, G, N, caps):
    out = [("value", None), ("rarity", None), ("twin", None)]
    for seed in SEEDS:
        out.append(("twin", np.stack([count_permutation(cfg, g, caps[g], seed, N=N) for g in range(G)])))
    return out


@pytest.mark.parametrize("cfg_id,G,N", [(2, 3, 1200), (5, 8, 700)])
def test_variant_keys_and_selection_on_oracle_counts(cfg_id, G, N):
    cfg = get_config(cfg_id)
    _, _, refs = _oracle_counts(cfg, G, N)
    count = np.stack([r["count"] for r in refs]).astype(np.int32)
    energy = np.stack([r["energy"] for r in refs])
    caps = [O.uniform_budget(N, 0.5)] * G
    tc = torch.from_numpy(count).to(_dev())
    te = torch.from_numpy(energy).to(_dev())
    inexact = 0
    for name, perm in _variants(cfg, G, N, caps):
        tp = torch.from_numpy(perm).to(_dev()) if perm is not None else None
        v = krs.variant_score(tc, te, name, perm=tp)
        sel = krs.select(v["score"], v["tie"], caps, cfg.sink, cfg.recent)
        torch.cuda.synchronize()
        sc, tie = v["score"].cpu().numpy(), v["tie"].cpu().numpy()
        keep = sel["keep"].cpu().numpy()
        for g in range(G):
            rs, rt = O.variant_scores(energy[g], count[g], N, name, perm=None if perm is None else perm[g])
            np.testing.assert_allclose(sc[g], rs, rtol=1e-13, atol=0, err_msg=f"{name} score head {g}")
            np.testing.assert_array_equal(tie[g], rt, err_msg=f"{name} tie head {g}")
            okeep, _ = O.select_head(rs, rt, caps[g], cfg.sink, cfg.recent)
            if PR.boundary_gap(rs, rt, caps[g], cfg.sink, cfg.recent) >= PR.BOUNDARY_GAP:
                np.testing.assert_array_equal(keep[g], okeep, err_msg=f"{name} keep head {g}")
            else:
                inexact += 1
    print(f"[variants cfg{cfg_id}] selections checked by properties only: {inexact}", flush=True)
    assert inexact == 0


def test_twin_variant_reproduces_score_bitwise():
    cfg = get_config(2)
    G, N = 2, 900
    K, V, _ = make_heads(cfg, heads=range(G), N=N)
    res = krs.score(_up(K), _up(V), cfg.tau, cfg.window, cfg.sink, cfg.recent, omega=True)
    v = krs.variant_score(res["count"], res["energy"], "twin")
    r = krs.variant_score(res["count"], res["energy"], "rarity")
    torch.cuda.synchronize()
    assert torch.equal(v["score"], res["score"])
    assert torch.equal(r["score"], res["omega"])


@pytest.mark.parametrize("cfg_id,G,N", [(2, 3, 1500), (4, 2, 1100)])
def test_variant_chain_against_oracle(cfg_id, G, N):
    """GPU score -> variant -> select against the oracle chain; heads with a
    tau-band row or a near-tied boundary are checked by the selection
    properties only."""
    cfg = get_config(cfg_id)
    K, V, _ = make_heads(cfg, heads=range(G), N=N)
    r = cfg.removal if cfg.removal is not None else 0.5
    res = krs.score(_up(K), _up(V), cfg.tau, cfg.window, cfg.sink, cfg.recent)
    torch.cuda.synchronize()
    refs = [PR.score_reference(K[g], V[g], cfg.tau, cfg.window) for g in range(G)]
    chains = [("value", None, O.uniform_budget(N, r)), ("rarity", None, O.ceil_budget(N, r))]
    chains += [("twin", seed, O.uniform_budget(N, r)) for seed in SEEDS]
    inexact = 0
    for name, seed, cap in chains:
        caps = [cap] * G
        perm = None
        if seed is not None:
            perm = np.stack([count_permutation(cfg, g, cap, seed, N=N) for g in range(G)])
        v = krs.variant_score(res["count"], res["energy"], name,
                              perm=torch.from_numpy(perm).to(_dev()) if perm is not None else None)
        sel = krs.select(v["score"], v["tie"], caps, cfg.sink, cfg.recent)
        torch.cuda.synchronize()
        keep = sel["keep"].cpu().numpy()
        kept = sel["kept_idx"].cpu().numpy()
        off = sel["offsets"].cpu().numpy()
        gsc, gtie = v["score"].cpu().numpy(), v["tie"].cpu().numpy()
        for g in range(G):
            ref = refs[g]
            rs, rt = O.variant_scores(ref["energy"], ref["count"], N, name, perm=None if perm is None else perm[g])
            PR.check_select_properties(keep[g], kept[off[g]:off[g + 1]], gsc[g], gtie[g], cap, cfg.sink, cfg.recent,
                                       tag=f"{name} head {g}")
            exact = ref["band"].sum() == 0 and PR.boundary_gap(rs, rt, cap, cfg.sink, cfg.recent) >= PR.BOUNDARY_GAP
            if exact:
                okeep, _o = O.select_head(rs, rt, cap, cfg.sink, cfg.recent)
                np.testing.assert_array_equal(keep[g], okeep, err_msg=f"{name} chain keep head {g}")
            else:
                inexact += 1
    print(f"[variant chain cfg{cfg_id}] selections checked by properties only: {inexact}", flush=True)
    assert inexact == 0
