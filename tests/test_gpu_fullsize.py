"""GPU parity at the full workload sizes, launched as the benchmark launches
them (one call over every head of the workload).

The oracle cannot score whole workloads in test time, so each size is checked
three ways:

* element by element against the oracle on sampled outputs: whole heads
  (first and last head of the batch, plus one in the middle where the oracle
  is cheap) and seeded row samples of further heads that include the sink /
  recent boundaries and the last row block;
* value energy against the oracle for every head;
* the packed cache of host-drawn retained sets of the workload's quotas,
  bit for bit against the oracle for every head;
* properties that hold at any size for every head: planted near-duplicate
  clusters lower-bound the counts, every best twin is a valid nonlocal
  position, the selection keeps exactly its capacity with protection and a
  clean rank separation, and the repair's orphans, donors, pairs and S1 are
  the ones its own b(S0) implies.

The long-context workload (N = 131072, d = 128) runs 16 of its 256 heads at
full N: the per-head launch shape is the same and host-side generation of all
256 heads would take minutes.
"""
import numpy as np
import pytest
import torch

import key_redundancy_scoring_amd as krs
from oracle import twinkv_oracle as O
from synth import dirichlet_capacities, get_config, gumbel_retained, make_heads
from tests import parity as PR
from tests.test_gpu_gather import check_gather

pytestmark = pytest.mark.gpu


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch.device("cuda:0")


def _say(*a):
    print(*a, flush=True)


def _up(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(_dev())


def _sample_rows(N, g, n_random=384, edge=96):
    rng = np.random.default_rng([7, N, g])
    rows = np.concatenate([np.arange(edge), np.arange(N - edge, N), rng.choice(N, n_random, replace=False)])
    return np.unique(rows)


def _score_rows(res, g, rows):
    out = {k: res[k][g].cpu().numpy()[rows] for k in ("count", "energy", "score")}
    out["best"] = res["best_sim"][g].cpu().numpy()[rows]
    out["arg"] = res["best_idx"][g].cpu().numpy()[rows]
    if "omega" in res:
        out["omega"] = res["omega"][g].cpu().numpy()[rows]
    return out


def _check_energy_all(res, V):
    e = res["energy"].cpu().numpy()
    for g in range(V.shape[0]):
        np.testing.assert_allclose(e[g], O.value_energy(O.widen_bf16(V[g])), rtol=PR.ENERGY_RTOL, atol=0,
                                   err_msg=f"energy head {g}")


def _check_best_valid(best, arg, N, w, allowed=None, tag=""):
    """Every reported twin is a nonlocal (and, in repair, retained) position;
    -1 only when no such position exists."""
    i = np.arange(N)
    has_any = (i - w - 1 >= 0) | (i + w + 1 <= N - 1)
    if allowed is not None:
        cols = np.flatnonzero(allowed)
        if cols.size == 0:
            has_any = np.zeros(N, bool)
        else:
            # a retained column exists at distance > w from i
            has_any = (cols[0] < i - w) | (cols[-1] > i + w)
    assert np.all((arg >= 0) == has_any), f"{tag} best twin presence"
    ok = arg >= 0
    assert np.all(np.abs(i[ok] - arg[ok]) > w), f"{tag} best twin inside the window"
    if allowed is not None:
        assert np.all(allowed[arg[ok]] != 0), f"{tag} best twin not retained"
    assert np.all((best[ok] >= -1.0 - 1e-12) & (best[ok] <= 1.0 + 1e-12)), f"{tag} similarity out of range"
    assert np.all(best[~ok] == -1.0), f"{tag} empty best twin must be -1"


def _check_cluster_counts(count, cluster, w, tag=""):
    """A planted copy and its cluster mates are near-duplicates (cosine ~0.99
    against tau <= 0.9), so each row counts at least its mates outside the
    window; random pairs rarely pass tau, so most rows count exactly that."""
    N = count.shape[0]
    members = np.flatnonzero(cluster >= 0)
    lower = np.zeros(N, np.int64)
    order = np.argsort(cluster[members], kind="stable")
    m = members[order]
    cid = cluster[m]
    starts = np.flatnonzero(np.r_[True, cid[1:] != cid[:-1]])
    ends = np.r_[starts[1:], m.size]
    for s, e in zip(starts, ends):
        pos = m[s:e]
        far = np.abs(pos[:, None] - pos[None, :]) > w
        lower[pos] = far.sum(1)
    assert np.all(count >= lower), f"{tag} count below the planted cluster mates"
    assert np.mean(count == lower) > 0.98, f"{tag} counts far from the planted structure"


def _check_select_all(keep, kept, off, score, energy, caps, sink, recent, tag=""):
    G, N = keep.shape
    for g in range(G):
        cap = int(min(max(int(caps[g]), 0), N))
        prot = O.protected_mask(N, cap, sink, recent)
        k = keep[g].astype(bool)
        assert int(k.sum()) == cap, f"{tag} head {g}: |keep| {k.sum()} != {cap}"
        assert np.all(k[prot]), f"{tag} head {g}: protected position dropped"
        assert np.array_equal(np.flatnonzero(k), kept[off[g]:off[g + 1]]), f"{tag} head {g}: kept_idx"
        s, e = score[g], energy[g]
        ku = np.flatnonzero(k & ~prot)
        du = np.flatnonzero(~k & ~prot)
        if ku.size and du.size:
            wk = ku[np.lexsort((-ku, e[ku], s[ku]))[0]]  # the lowest-ranked kept position
            bd = du[np.lexsort((-du, e[du], s[du]))[-1]]  # the highest-ranked evicted one
            assert (s[wk], e[wk], -wk) > (s[bd], e[bd], -bd), f"{tag} head {g}: an evicted position outranks a kept one"


def _check_repair_all(S0, res, tau, w, sink, recent, tag=""):
    G, N = S0.shape
    S1 = res["keep"].cpu().numpy()
    b = res["best_sim"].cpu().numpy()
    a = res["best_idx"].cpu().numpy()
    no, nd, ns = (res[k].cpu().numpy() for k in ("n_orphans", "n_donors", "n_swaps"))
    pairs = res["pairs"].cpu().numpy()
    for g in range(G):
        s0 = S0[g] != 0
        K = int(s0.sum())
        _check_best_valid(b[g], a[g], N, w, allowed=S0[g], tag=f"{tag} head {g}")
        prot = O.protected_mask(N, K, sink, recent)
        orph = np.flatnonzero(~s0 & (b[g] < tau))
        don = np.flatnonzero(s0 & ~prot & (b[g] >= tau))
        assert no[g] == orph.size and nd[g] == don.size, f"{tag} head {g}: |O|, |D|"
        m = min(orph.size, don.size)
        assert ns[g] == m, f"{tag} head {g}: m"
        o_rank = orph[np.lexsort((orph, b[g][orph]))][:m]
        d_rank = don[np.lexsort((don, -b[g][don]))][:m]
        np.testing.assert_array_equal(pairs[g][:m, 0], o_rank, err_msg=f"{tag} head {g}: orphans")
        np.testing.assert_array_equal(pairs[g][:m, 1], d_rank, err_msg=f"{tag} head {g}: donors")
        assert np.all(pairs[g][m:] == -1), f"{tag} head {g}: pair padding"
        want = s0.copy()
        want[d_rank] = False
        want[o_rank] = True
        np.testing.assert_array_equal(S1[g].astype(bool), want, err_msg=f"{tag} head {g}: S1")


def _oracle_head_checks(K, V, g, cfg, res, sel, rep, cap, tag, tally):
    """Whole-head parity of score, select and (when given) repair of the
    selection against the oracle."""
    ref = PR.score_reference(K, V, cfg.tau, cfg.window)
    gpu = _score_rows(res, g, np.arange(cfg.N))
    r = PR.compare_score(gpu, ref, tag=f"{tag} head {g}")
    okeep, oidx = O.select_head(ref["score"], ref["energy"], cap, cfg.sink, cfg.recent)
    exact = PR.select_exact(r, ref, cap, cfg.sink, cfg.recent)
    if exact:
        keep = sel["keep"][g].cpu().numpy()
        np.testing.assert_array_equal(keep, okeep, err_msg=f"{tag} head {g} keep")
    r["select_heads"] = 1
    r["select_inexact_heads"] = 0 if exact else 1
    if rep is not None and exact:
        rref = PR.repair_reference(K, okeep, cfg.tau, cfg.window, cfg.sink, cfg.recent)
        rg = {k: rep[k][g].cpu().numpy() for k in ("keep", "n_orphans", "n_donors", "n_swaps", "pairs")}
        rg["best"] = rep["best_sim"][g].cpu().numpy()
        rg["arg"] = rep["best_idx"][g].cpu().numpy()
        r["repair"] = PR.compare_repair(rg, rref, okeep, cfg.tau, tag=f"{tag} head {g} repair")
    r["variants"] = _variant_checks(ref, cfg, cap, tag=f"{tag} head {g}")
    tally.add(r)
    _say(f"[{tag}] head {g} whole-head parity ok: {r}")


def _variant_checks(ref, cfg, cap, tag):
    """Score variants of one whole head at full size: the oracle's counts and
    energies go through the GPU's variant keys and selection; the keys match
    the oracle's variant_scores and the kept sets its select_head (rarity
    also with the standalone score's ceil budget)."""
    N = cfg.N
    c = torch.from_numpy(ref["count"].astype(np.int32)[None]).to(_dev())
    e = torch.from_numpy(np.ascontiguousarray(ref["energy"])[None]).to(_dev())
    r = cfg.removal if cfg.removal is not None else 0.5
    out = {}
    for name, cp in (("value", cap), ("rarity", cap), ("rarity", O.ceil_budget(N, r))):
        v = krs.variant_score(c, e, name)
        sel = krs.select(v["score"], v["tie"], [cp], cfg.sink, cfg.recent)
        torch.cuda.synchronize()
        rs, rt = O.variant_scores(ref["energy"], ref["count"], N, name)
        np.testing.assert_allclose(v["score"][0].cpu().numpy(), rs, rtol=1e-13, atol=0, err_msg=f"{tag} {name}")
        np.testing.assert_array_equal(v["tie"][0].cpu().numpy(), rt, err_msg=f"{tag} {name} tie")
        okeep, _ = O.select_head(rs, rt, cp, cfg.sink, cfg.recent)
        if PR.boundary_gap(rs, rt, cp, cfg.sink, cfg.recent) >= PR.BOUNDARY_GAP:
            np.testing.assert_array_equal(sel["keep"][0].cpu().numpy(), okeep, err_msg=f"{tag} {name} keep")
            out[f"{name}@{cp}"] = "exact"
        else:
            out[f"{name}@{cp}"] = "boundary near-tie"
    return out


def _row_checks(K, V, g, cfg, res, tag, tally):
    rows = _sample_rows(cfg.N, g)
    ref = PR.score_reference(K, V, cfg.tau, cfg.window, rows=rows)
    r = PR.compare_score(_score_rows(res, g, rows), ref, tag=f"{tag} head {g} rows")
    tally.add(r)
    _say(f"[{tag}] head {g} sampled rows ok: {r}")


def _score_select(cfg, K, V, caps, repair_selected):
    tk, tv = _up(K), _up(V)
    res = krs.score(tk, tv, cfg.tau, cfg.window, cfg.sink, cfg.recent, omega=True)
    off = krs.capacity_offsets(caps, cfg.N)
    sel = krs.select(res["score"], res["energy"], torch.tensor(caps, dtype=torch.int32, device=_dev()), cfg.sink,
                     cfg.recent, offsets=off)
    # the repair of the selection reuses the score pass's best twins, as a
    # score -> select -> repair step does
    rep = krs.repair(tk, sel["keep"], cfg.tau, cfg.window, cfg.sink, cfg.recent,
                     prior=res) if repair_selected else None
    torch.cuda.synchronize()
    return res, sel, rep


def _score_select_suite(cfg, caps, whole_heads, row_heads, repair_selected, tag):
    _say(f"[{tag}] generating G={cfg.G} N={cfg.N} d={cfg.d}")
    K, V, clusters = make_heads(cfg)
    _say(f"[{tag}] score + select{' + repair' if repair_selected else ''} on the GPU")
    res, sel, rep = _score_select(cfg, K, V, caps, repair_selected)
    count = res["count"].cpu().numpy()
    best = res["best_sim"].cpu().numpy()
    arg = res["best_idx"].cpu().numpy()
    for g in range(cfg.G):
        _check_best_valid(best[g], arg[g], cfg.N, cfg.window, tag=f"{tag} head {g}")
        _check_cluster_counts(count[g], clusters[g], cfg.window, tag=f"{tag} head {g}")
    _check_energy_all(res, V)
    _say(f"[{tag}] all-head score properties ok")
    _check_select_all(sel["keep"].cpu().numpy(), sel["kept_idx"].cpu().numpy(), sel["offsets"].cpu().numpy(),
                      res["score"].cpu().numpy(), res["energy"].cpu().numpy(), caps, cfg.sink, cfg.recent, tag)
    _say(f"[{tag}] all-head select properties ok")
    if rep is not None:
        _check_repair_all(sel["keep"].cpu().numpy(), rep, cfg.tau, cfg.window, cfg.sink, cfg.recent, tag)
        _say(f"[{tag}] all-head repair properties ok, swaps {int(rep['n_swaps'].sum())}")
    tally = PR.Tally(tag)
    for g in row_heads:
        _row_checks(K[g], V[g], g, cfg, res, tag, tally)
    for g in whole_heads:
        _oracle_head_checks(K[g], V[g], g, cfg, res, sel, rep, int(caps[g]), tag, tally)
    tally.check()
    # packed cache of host-drawn retained sets of the same quotas, every head
    kept = [np.flatnonzero(gumbel_retained(cfg, g, keep=int(caps[g]))) for g in range(cfg.G)]
    total = check_gather(K, V, kept, tag=tag)
    _say(f"[{tag}] packed cache of {total} rows bit-exact")


def test_fullsize_llama32_1b_32k():
    cfg = get_config(2)
    caps = [O.uniform_budget(cfg.N, cfg.removal)] * cfg.G
    _score_select_suite(cfg, caps, whole_heads=[0], row_heads=[cfg.G // 2, cfg.G - 1], repair_selected=True,
                        tag="llama 32k")


def test_fullsize_batched_8k_dirichlet():
    cfg = get_config(5)
    caps = dirichlet_capacities(cfg)
    _score_select_suite(cfg, caps, whole_heads=[0, 1029, cfg.G - 1], row_heads=[517, 1500],
                        repair_selected=True, tag="batched 8k")


def test_fullsize_long_131k_head_subset():
    cfg = get_config(4).with_(G=16)
    caps = [O.uniform_budget(cfg.N, cfg.removal)] * cfg.G
    _score_select_suite(cfg, caps, whole_heads=[], row_heads=[0, 9, cfg.G - 1], repair_selected=False,
                        tag="long 131k")


def test_fullsize_qwen3_4b_repair():
    cfg = get_config(3)
    _say(f"[qwen repair] generating G={cfg.G} N={cfg.N} d={cfg.d}")
    K, _, _ = make_heads(cfg, with_values=False)
    S0 = np.stack([gumbel_retained(cfg, g) for g in range(cfg.G)])
    _say("[qwen repair] repair on the GPU")
    rep = krs.repair(_up(K), torch.from_numpy(S0).to(_dev()), cfg.tau, cfg.window, cfg.sink, cfg.recent)
    torch.cuda.synchronize()
    _check_repair_all(S0, rep, cfg.tau, cfg.window, cfg.sink, cfg.recent, "qwen repair")
    _say(f"[qwen repair] all-head repair properties ok, swaps {int(rep['n_swaps'].sum())}")
    tally = PR.Tally("qwen repair")
    for g in (0, cfg.G - 1):
        rref = PR.repair_reference(K[g], S0[g], cfg.tau, cfg.window, cfg.sink, cfg.recent)
        rg = {k: rep[k][g].cpu().numpy() for k in ("keep", "n_orphans", "n_donors", "n_swaps", "pairs")}
        rg["best"] = rep["best_sim"][g].cpu().numpy()
        rg["arg"] = rep["best_idx"][g].cpu().numpy()
        r = PR.compare_repair(rg, rref, S0[g], cfg.tau, tag=f"qwen repair head {g}")
        assert rref["m"] > 0
        tally.add(r)
        _say(f"[qwen repair] head {g} whole-head parity ok: {r}")
    tally.check()
