"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle on
the same seeded inputs, element by element, at sizes the oracle finishes in
seconds that still span several workgroups, LDS stages and ragged tails;
plus the degenerate cases.  Full-size workloads live in test_gpu_fullsize.py.
"""
import numpy as np
import pytest
import torch

import key_redundancy_scoring_amd as krs
from oracle import twinkv_oracle as O
from synth import dirichlet_capacities, get_config, gumbel_retained, make_heads
from tests import parity as PR

pytestmark = pytest.mark.gpu


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch.device("cuda:0")


def _up(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(_dev())


def _say(*a):
    print(*a, flush=True)


def _score_numpy(res, g):
    return {k: res[k][g].cpu().numpy() for k in ("count", "best_sim", "best_idx", "energy", "score", "omega")
            if k in res} | {"best": res["best_sim"][g].cpu().numpy(), "arg": res["best_idx"][g].cpu().numpy()}


def _run_score_select_repair(K, V, cfg, caps, do_repair_on_select=False, tag=""):
    """Score + select (+ repair of the select output) on the GPU and check every
    head against the oracle."""
    G, N, d = K.shape
    _say(f"[{tag}] score G={G} N={N} d={d}")
    tk, tv = _up(K), _up(V)
    res = krs.score(tk, tv, cfg.tau, cfg.window, cfg.sink, cfg.recent, omega=True)
    sel = krs.select(res["score"], res["energy"], torch.tensor(caps, dtype=torch.int32, device=_dev()),
                     cfg.sink, cfg.recent)
    rep_res = rep_pr = None
    if do_repair_on_select:
        rep_res = krs.repair(tk, sel["keep"], cfg.tau, cfg.window, cfg.sink, cfg.recent)
        # the same repair, reusing the score pass's unrestricted best twins
        rep_pr = krs.repair(tk, sel["keep"], cfg.tau, cfg.window, cfg.sink, cfg.recent, prior=res)
    torch.cuda.synchronize()
    keep = sel["keep"].cpu().numpy()
    kept = sel["kept_idx"].cpu().numpy()
    off = sel["offsets"].cpu().numpy()
    reports = []
    tally = PR.Tally(tag)
    for g in range(G):
        ref = PR.score_reference(K[g], V[g], cfg.tau, cfg.window)
        gpu = _score_numpy(res, g)
        r = PR.compare_score(gpu, ref, tag=f"{tag} head {g}")
        cap = int(caps[g])
        okeep, oidx = O.select_head(ref["score"], ref["energy"], cap, cfg.sink, cfg.recent)
        exact = PR.select_exact(r, ref, cap, cfg.sink, cfg.recent)
        PR.check_select_properties(keep[g], kept[off[g]:off[g + 1]], gpu["score"], gpu["energy"], cap, cfg.sink,
                                   cfg.recent, tag=f"{tag} head {g}")
        if exact:
            np.testing.assert_array_equal(keep[g], okeep, err_msg=f"{tag} head {g} keep")
            np.testing.assert_array_equal(kept[off[g]:off[g + 1]], oidx, err_msg=f"{tag} head {g} kept_idx")
        r["select_heads"] = 1
        r["select_inexact_heads"] = 0 if exact else 1
        if rep_res is not None and exact:
            rref = PR.repair_reference(K[g], okeep, cfg.tau, cfg.window, cfg.sink, cfg.recent)
            for name, rr in (("repair", rep_res), ("repair with prior", rep_pr)):
                rg = {k: rr[k][g].cpu().numpy() for k in ("keep", "n_orphans", "n_donors", "n_swaps", "pairs")}
                rg["best"] = rr["best_sim"][g].cpu().numpy()
                rg["arg"] = rr["best_idx"][g].cpu().numpy()
                r[name] = PR.compare_repair(rg, rref, okeep, cfg.tau, tag=f"{tag} head {g} {name}")
        reports.append(r)
        tally.add(r)
    _say(f"[{tag}] ok", reports[:2])
    tally.check()
    return res, sel, reports


def test_tiny_config_full():
    cfg = get_config(1)
    K, V, _ = make_heads(cfg)
    caps = [O.uniform_budget(cfg.N, cfg.removal)] * cfg.G
    _run_score_select_repair(K, V, cfg, caps, do_repair_on_select=True, tag="cfg1")


@pytest.mark.parametrize("cfg_id,G,N", [(2, 3, 1500), (2, 2, 513), (2, 1, 65), (4, 2, 1100), (3, 2, 700), (2, 1, 8300)])
def test_score_select_ragged(cfg_id, G, N):
    cfg = get_config(cfg_id)
    K, V, _ = make_heads(cfg, heads=range(G), N=N)
    r = cfg.removal if cfg.removal is not None else 0.5
    caps = [O.uniform_budget(N, r)] * G
    _run_score_select_repair(K, V, cfg, caps, do_repair_on_select=True, tag=f"cfg{cfg_id} G{G} N{N}")


def test_dirichlet_capacities_small():
    cfg = get_config(5)
    G, N = 16, 900
    K, V, _ = make_heads(cfg, heads=range(G), N=N)
    caps = dirichlet_capacities(cfg, G=G, N=N)
    _run_score_select_repair(K, V, cfg, caps, do_repair_on_select=True, tag="cfg5 small")


@pytest.mark.parametrize("N", [1300, 257])
def test_repair_gumbel_small(N):
    cfg = get_config(3)
    G = 3
    _say(f"[repair gumbel N={N}]")
    K, _, _ = make_heads(cfg, heads=range(G), N=N, with_values=False)
    S0 = np.stack([gumbel_retained(cfg, g, N=N) for g in range(G)])
    res = krs.repair(_up(K), torch.from_numpy(S0).to(_dev()), cfg.tau, cfg.window, cfg.sink, cfg.recent)
    torch.cuda.synchronize()
    tally = PR.Tally(f"repair gumbel N={N}")
    for g in range(G):
        rref = PR.repair_reference(K[g], S0[g], cfg.tau, cfg.window, cfg.sink, cfg.recent)
        rg = {k: res[k][g].cpu().numpy() for k in ("keep", "n_orphans", "n_donors", "n_swaps", "pairs")}
        rg["best"] = res["best_sim"][g].cpu().numpy()
        rg["arg"] = res["best_idx"][g].cpu().numpy()
        tally.add(PR.compare_repair(rg, rref, S0[g], cfg.tau, tag=f"gumbel head {g}"))
        assert rref["m"] > 0  # the case exercises real swaps
    tally.check()


# ---------------------------------------------------------------------------
# degenerate cases


def _bf16(x):
    from synth import f64_to_bf16_bits
    return f64_to_bf16_bits(np.asarray(x, dtype=np.float64))


def _score_one(K, V, tau, window, sink=4, recent=8):
    res = krs.score(_up(K), _up(V), tau, window, sink, recent, omega=True)
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("N,w", [(1, 0), (2, 1), (33, 32), (34, 32), (5, 0), (40, 39), (40, 2 ** 31 - 1)])
def test_few_positions(N, w):
    rng = np.random.default_rng(N)
    K = _bf16(rng.standard_normal((2, N, 64)))
    V = _bf16(rng.standard_normal((2, N, 64)))
    _say(f"[few N={N} w={w}]")
    res = _score_one(K, V, 0.5, w)
    for g in range(2):
        ref = PR.score_reference(K[g], V[g], 0.5, w)
        PR.compare_score(_score_numpy(res, g), ref, tag=f"few N={N} head {g}")
    for cap in (0, N // 2, N):
        sel = krs.select(res["score"], res["energy"], [cap, cap], 1, 1)
        torch.cuda.synchronize()
        for g in range(2):
            ok, oi = O.select_head(res["score"][g].cpu().numpy(), res["energy"][g].cpu().numpy(), cap, 1, 1)
            np.testing.assert_array_equal(sel["keep"][g].cpu().numpy(), ok)


def test_identical_and_zero_keys_tie_rules():
    N, d = 700, 64
    rng = np.random.default_rng(1)
    Kf = rng.standard_normal((1, N, d))
    Kf[0, 100:700:50] = Kf[0, 50]  # exact copies of key 50 at 100, 150, ...: sim exactly 1, exact ties
    Kf[0, 300] = 0.0  # a zero key
    Kf[0, 301] = 0.0
    K = _bf16(Kf)
    V = _bf16(np.ones((1, N, d)))  # equal energies: the tie rule falls through to positions
    _say("[identical keys]")
    for tau in (0.9, -0.5):
        res = _score_one(K, V, tau, 16)
        ref = PR.score_reference(K[0], V[0], tau, 16)
        PR.compare_score(_score_numpy(res, 0), ref, tag=f"identical tau={tau}")
        a = res["best_idx"][0].cpu().numpy()
        assert a[50] == 100 and a[650] == 50
        sel = krs.select(res["score"], res["energy"], [350], 4, 8)
        torch.cuda.synchronize()
        ok, oi = O.select_head(ref["score"], ref["energy"], 350, 4, 8)
        np.testing.assert_array_equal(sel["keep"][0].cpu().numpy(), ok)


def test_all_zero_values_select_by_position():
    N = 300
    rng = np.random.default_rng(2)
    K = _bf16(rng.standard_normal((1, N, 128)))
    V = np.zeros((1, N, 128), np.uint16)
    res = _score_one(K, V, 0.9, 8)
    sel = krs.select(res["score"], res["energy"], [100], 4, 8)
    torch.cuda.synchronize()
    idx = sel["kept_idx"].cpu().numpy()
    assert idx.tolist() == list(range(4 + 88)) + list(range(N - 8, N))


def test_capacity_edges_and_clamping():
    cfg = get_config(2)
    G, N = 6, 400
    K, V, _ = make_heads(cfg, heads=range(G), N=N)
    res = krs.score(_up(K), _up(V), cfg.tau, cfg.window, 4, 64)
    caps = [0, 3, 40, 67, 68, N]
    sel = krs.select(res["score"], res["energy"], caps, 4, 64)
    torch.cuda.synchronize()
    keep = sel["keep"].cpu().numpy()
    off = sel["offsets"].cpu().numpy()
    for g in range(G):
        ok, oi = O.select_head(res["score"][g].cpu().numpy(), res["energy"][g].cpu().numpy(), caps[g], 4, 64)
        np.testing.assert_array_equal(keep[g], ok)
        np.testing.assert_array_equal(sel["kept_idx"].cpu().numpy()[off[g]:off[g + 1]], oi)


def test_capacity_offsets_device_clamps_and_spans_chunks():
    """twinkv_capacity_offsets against the host prefix sums of the clamped
    capacities, over more heads than one workgroup's chunk of 1024."""
    rng = np.random.default_rng(5)
    N = 777
    for G in (1, 1024, 2500):
        caps = rng.integers(-5, N + 6, size=G).astype(np.int32)
        got = krs.capacity_offsets_device(torch.from_numpy(caps).to(_dev()), N)
        torch.cuda.synchronize()
        want = np.concatenate([[0], np.cumsum(np.clip(caps.astype(np.int64), 0, N))])
        np.testing.assert_array_equal(got.cpu().numpy(), want, err_msg=f"G={G}")


def test_repair_noop_and_extremes():
    cfg = get_config(3)
    G, N = 4, 600
    K, _, _ = make_heads(cfg, heads=range(G), N=N, with_values=False)
    masks = np.zeros((G, N), np.uint8)
    masks[1] = 1  # keep everything: no orphans
    masks[2, ::2] = 1
    masks[3, :5] = 1
    res = krs.repair(_up(K), torch.from_numpy(masks).to(_dev()), cfg.tau, cfg.window, cfg.sink, cfg.recent)
    torch.cuda.synchronize()
    tally = PR.Tally("repair extremes")
    for g in range(G):
        rref = PR.repair_reference(K[g], masks[g], cfg.tau, cfg.window, cfg.sink, cfg.recent)
        rg = {k: res[k][g].cpu().numpy() for k in ("keep", "n_orphans", "n_donors", "n_swaps", "pairs")}
        rg["best"] = res["best_sim"][g].cpu().numpy()
        rg["arg"] = res["best_idx"][g].cpu().numpy()
        tally.add(PR.compare_repair(rg, rref, masks[g], cfg.tau, tag=f"extreme head {g}"))
    tally.check()
    assert int(res["n_swaps"][0]) == 0 and int(res["n_swaps"][1]) == 0


def test_repair_short_retained_sets():
    """Retained sets shorter than a tile, a tile, a stage of the d = 64
    restricted sweep (128 columns) and one more, at random positions, with and
    without the score pass's twins as the prior, against the oracle."""
    cfg = get_config(2)
    sizes = [1, 3, 31, 32, 33, 127, 128, 129]
    G, N = len(sizes), 700
    K, V, _ = make_heads(cfg, heads=range(G), N=N)
    rng = np.random.default_rng(20261203)
    masks = np.zeros((G, N), np.uint8)
    for g, k in enumerate(sizes):
        masks[g, rng.choice(N, size=k, replace=False)] = 1
    tk = _up(K)
    prior = krs.score(tk, _up(V), cfg.tau, cfg.window, cfg.sink, cfg.recent)
    keep_in = torch.from_numpy(masks).to(_dev())
    plain = krs.repair(tk, keep_in, cfg.tau, cfg.window, cfg.sink, cfg.recent)
    with_prior = krs.repair(tk, keep_in, cfg.tau, cfg.window, cfg.sink, cfg.recent, prior=prior)
    torch.cuda.synchronize()
    tally = PR.Tally("short retained sets")
    for g in range(G):
        rref = PR.repair_reference(K[g], masks[g], cfg.tau, cfg.window, cfg.sink, cfg.recent)
        for name, res in (("repair", plain), ("repair with prior", with_prior)):
            rg = {k: res[k][g].cpu().numpy() for k in ("keep", "n_orphans", "n_donors", "n_swaps", "pairs")}
            rg["best"] = res["best_sim"][g].cpu().numpy()
            rg["arg"] = res["best_idx"][g].cpu().numpy()
            tally.add(PR.compare_repair(rg, rref, masks[g], cfg.tau, tag=f"short retained set K={sizes[g]} {name}"))
    tally.check()


def test_deterministic_repeat():
    cfg = get_config(2)
    K, V, _ = make_heads(cfg, heads=range(4), N=2000)
    tk, tv = _up(K), _up(V)
    a = krs.score(tk, tv, cfg.tau, cfg.window, omega=True)
    b = krs.score(tk, tv, cfg.tau, cfg.window, omega=True)
    torch.cuda.synchronize()
    for k in ("count", "best_sim", "best_idx", "energy", "score", "omega"):
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("cfg_id,G,N,removal", [(2, 4, 2500, 0.5), (3, 3, 1700, 0.3), (2, 2, 900, 0.9)])
def test_repair_prior_matches_full_sweep(cfg_id, G, N, removal):
    """Repair with the score pass's best twins as the prior against the full
    restricted sweep, on the GPU: the same b(S0) and position wherever the
    two sweeps' fp32 screens are not within rounding of a tie, and then the
    same orphans, donors, pairs and S1.  Heads with a random retained set and
    with the score-ranked one."""
    cfg = get_config(cfg_id)
    K, V, _ = make_heads(cfg, heads=range(G), N=N)
    tk, tv = _up(K), _up(V)
    res = krs.score(tk, tv, cfg.tau, cfg.window, cfg.sink, cfg.recent)
    cap = O.uniform_budget(N, removal)
    sel = krs.select(res["score"], res["energy"], torch.full((G,), cap, dtype=torch.int32, device=_dev()),
                     cfg.sink, cfg.recent)
    rnd = torch.from_numpy(np.stack([gumbel_retained(cfg, g, N=N, keep=cap) for g in range(G)])).to(_dev())
    for name, keep in (("selected", sel["keep"]), ("random", rnd)):
        full = krs.repair(tk, keep, cfg.tau, cfg.window, cfg.sink, cfg.recent)
        pr = krs.repair(tk, keep, cfg.tau, cfg.window, cfg.sink, cfg.recent, prior=res)
        torch.cuda.synchronize()
        fa, pa = full["best_idx"].cpu().numpy(), pr["best_idx"].cpu().numpy()
        fb, pb = full["best_sim"].cpu().numpy(), pr["best_sim"].cpu().numpy()
        diff = fa != pa
        # a different choice only between positions whose similarities agree
        # to within the fp32 screen's rounding
        np.testing.assert_allclose(pb[diff], fb[diff], rtol=0, atol=1e-5, err_msg=f"{name} near-tie rows")
        np.testing.assert_array_equal(pb[~diff], fb[~diff], err_msg=f"{name} b(S0)")
        if not diff.any():
            for k in ("keep", "n_orphans", "n_donors", "n_swaps", "pairs"):
                assert torch.equal(full[k], pr[k]), f"{name} {k}"
        reused = (pa >= 0) & np.take_along_axis(keep.cpu().numpy(), np.maximum(res["best_idx"].cpu().numpy(), 0),
                                                1).astype(bool)
        _say(f"[prior {name} cfg{cfg_id}] rows reused {reused.mean():.3f}, differing choices {int(diff.sum())}")


def test_repair_prior_out_of_range_indices_are_swept():
    """Prior indices outside [0, N) other than -1 (N + 5, INT32_MAX, -2,
    INT32_MIN) count as not retained: those rows are swept, so the result
    equals the full restricted sweep."""
    cfg = get_config(2)
    G, N = 2, 1200
    K, V, _ = make_heads(cfg, heads=range(G), N=N)
    tk, tv = _up(K), _up(V)
    res = krs.score(tk, tv, cfg.tau, cfg.window, cfg.sink, cfg.recent)
    keep = torch.from_numpy(np.stack([gumbel_retained(cfg, g, N=N) for g in range(G)])).to(_dev())
    bad = {"best_sim": res["best_sim"].clone(), "best_idx": res["best_idx"].clone()}
    bad["best_idx"][:, ::3] = N + 5
    bad["best_idx"][:, 1::7] = 2 ** 31 - 1
    bad["best_idx"][:, 2::11] = -2
    bad["best_idx"][:, 5::13] = -2 ** 31
    full = krs.repair(tk, keep, cfg.tau, cfg.window, cfg.sink, cfg.recent)
    pr = krs.repair(tk, keep, cfg.tau, cfg.window, cfg.sink, cfg.recent, prior=bad)
    torch.cuda.synchronize()
    rows = np.zeros((G, N), bool)
    rows[:, ::3] = True
    rows[:, 1::7] = True
    rows[:, 2::11] = True
    rows[:, 5::13] = True
    fa, pa = full["best_idx"].cpu().numpy(), pr["best_idx"].cpu().numpy()
    np.testing.assert_array_equal(pa[rows], fa[rows])
    np.testing.assert_array_equal(pr["best_sim"].cpu().numpy()[rows], full["best_sim"].cpu().numpy()[rows])


def _plant_near_tie(rng, d, lo=1e-9, hi=3e-6):
    """A row key and two candidate keys whose exact cosines with it differ by
    lo < gap < hi, below the fp32 error of the sweep: the second candidate is
    the first with one small bf16 component moved by one unit in the last
    place.  Returns bf16 bits (row, first, second) and the two cosines."""
    while True:
        base = rng.standard_normal(d)
        row = _bf16(base + 0.05 * rng.standard_normal(d))
        a = _bf16(base)
        r64 = O.widen_bf16(row)
        for c in np.argsort(np.abs(O.widen_bf16(a)))[:16]:
            b = a.copy()
            b[c] = np.uint16(int(b[c]) + 1)
            K = O.widen_bf16(np.stack([row, a, b]))
            n = O.squared_norms(K)
            s = O.cosine_rows(K, n, np.array([0]), np.array([1, 2]))[0]
            if lo < abs(s[1] - s[0]) < hi:
                return row, a, b, s


@pytest.mark.parametrize("d", [64, 128])
def test_cross_tile_near_ties_resolve_exactly(d):
    """Rows whose two best candidates sit in different tiles of the same
    half-row (positions = 0 mod 8) with exact cosines closer than the fp32
    error: the score pass and the repair sweep must both return the exact
    maximum.  Planted on both sides of the row (later columns: the row side
    of the single-order sweep; earlier ones: its column side)."""
    rng = np.random.default_rng(77 + d)
    N, w = 1600, 8
    K = _bf16(rng.standard_normal((N, d)))
    planted = {}
    for k in range(12):
        row, a, b, s = _plant_near_tie(rng, d)
        if k % 2:  # the larger cosine at the earlier position half of the time
            a, b, s = b, a, s[::-1]
        if k < 6:  # candidates after the row
            i, j1, j2 = 40 + k, 296 + 40 * k, 704 + 48 * k
        else:      # candidates before the row
            i, j1, j2 = 1500 + k, 96 + 24 * (k - 6), 520 + 40 * (k - 6)
        K[i], K[j1], K[j2] = row, a, b
        planted[i] = j1 if s[0] > s[1] else j2
    V = _bf16(rng.standard_normal((N, d)))
    _say(f"[cross-tile near-ties d={d}]")
    res = _score_one(K[None], V[None], 0.9, w)
    ref = PR.score_reference(K, V, 0.9, w)
    got = res["best_idx"][0].cpu().numpy()
    for i, j in planted.items():
        assert ref["arg"][i] == j, f"planted row {i}: oracle picks {ref['arg'][i]}, expected {j}"
        assert got[i] == j, f"score pass, row {i}: picks {got[i]}, exact best {j}"
    tally = PR.Tally("cross-tile near-ties")
    tally.add(PR.compare_score(_score_numpy(res, 0), ref, tag="cross-tile score"))
    # the repair sweep over every retained column but a few, without a prior
    keep = np.ones((1, N), np.uint8)
    keep[0, 1:N:97] = 0
    rep = krs.repair(_up(K[None]), torch.from_numpy(keep).to(_dev()), 0.9, w, 4, 8)
    torch.cuda.synchronize()
    rref = PR.repair_reference(K, keep[0], 0.9, w, 4, 8)
    rb = rep["best_idx"][0].cpu().numpy()
    for i in planted:
        assert rb[i] == rref["arg"][i], f"repair sweep, row {i}: picks {rb[i]}, exact best {rref['arg'][i]}"
    rg = {k: rep[k][0].cpu().numpy() for k in ("keep", "n_orphans", "n_donors", "n_swaps", "pairs")}
    rg["best"] = rep["best_sim"][0].cpu().numpy()
    rg["arg"] = rb
    tally.add(PR.compare_repair(rg, rref, keep[0], 0.9, tag="cross-tile repair"))
    tally.check()


def test_all_identical_keys_overflow_the_candidate_lists():
    """Every key the same: every cosine is exactly 1, every row is queued for
    the exact resolve and each has far more candidates than its list holds,
    so the rows go to the exhaustive pass.  The best twin is the lowest
    eligible position, with cosine 1, in the score pass and in the repair
    sweep alike."""
    rng = np.random.default_rng(9)
    N, d, w = 2100, 64, 16
    K = np.repeat(_bf16(rng.standard_normal((1, 1, d))), N, axis=1)
    V = _bf16(rng.standard_normal((1, N, d)))
    want = np.where(np.arange(N) > w, 0, np.arange(N) + w + 1)  # the lowest j with |i - j| > w
    _say("[identical keys, overflow]")
    res = _score_one(K, V, 0.5, w)
    np.testing.assert_array_equal(res["best_idx"][0].cpu().numpy(), want)
    assert np.all(res["best_sim"][0].cpu().numpy() == 1.0)
    keep = np.ones((1, N), np.uint8)
    keep[0, :5] = 0  # the lowest positions evicted: the answer moves
    rep = krs.repair(_up(K), torch.from_numpy(keep).to(_dev()), 0.5, w, 4, 8)
    torch.cuda.synchronize()
    rref = PR.repair_reference(K[0], keep[0], 0.5, w, 4, 8)
    np.testing.assert_array_equal(rep["best_idx"][0].cpu().numpy(), rref["arg"])
    assert np.all(rep["best_sim"][0].cpu().numpy() == 1.0)
