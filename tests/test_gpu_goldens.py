"""Every workload's retained sets, repair swaps, counts and best twins on the
GPU against the fp64 oracle's, on the seeded head subsets that
tests/golden/make_oracle_goldens.py computed on the CPU (the whole batch of
the Llama-3.2-1B 32k workload, 32 heads of the Qwen3-4B repair workload, 8
heads of the long 131k workload at full N, 128 heads of the batched 8k
workload, the tiny workload).

The GPU runs the step the benchmark times: score -> select -> repair of the
selection with the score pass's twins as the prior (repair of the Gumbel
retained set, no prior, for the repair workload), over the checked heads in
one launch each (the per-head work and launch shape are those of the full
batch: heads are independent).  Per head it checks:

* the regenerated inputs hash to the oracle run's;
* counts bit for bit (rows with a pair in the tau band: within the band);
* best-twin positions bit for bit, except at the oracle's near-tie rows,
  where the GPU's pick must be one of the stored candidates and not an
  exact-tie loser; best_sim against the exact cosine of the reported pair,
  which is the oracle's pair wherever the positions match;
* energy against the oracle's, score against the oracle's formula on the
  oracle's energy and the counts just certified equal to the oracle's;
* the keep mask bit for bit when no count is band-affected and the
  selection boundary is not a near-tie;
* |O|, |D|, m, b(S0)'s positions, S1 and the swap pairs bit for bit, with
  the same near-tie rule.

Every exclusion is counted, printed and bounded, and a results record per
workload (parameters, checked heads, input digests, exclusion counts,
verdict) is written to $TWINKV_RESULTS_DIR (default gpurun_out/results).
"""
import json
import os

import numpy as np
import pytest
import torch

import key_redundancy_scoring_amd as krs
from oracle import twinkv_oracle as O
from synth import dirichlet_capacities, get_config, gumbel_retained, make_heads
from tests import parity as PR
from tests.golden import make_oracle_goldens as MG

pytestmark = pytest.mark.gpu
RESULTS = os.environ.get("TWINKV_RESULTS_DIR", os.path.join(os.path.dirname(os.path.dirname(__file__)),
                                                            "gpurun_out", "results"))


def _say(*a):
    print(*a, flush=True)


def _up(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda:0")


def _chunks_equal(got, want, what, tag):
    bad = [k for k, (a, b) in enumerate(zip(got, want)) if a != b]
    assert len(got) == len(want) and not bad, \
        f"{tag}: {what} differs from the oracle in {MG.CHUNK}-row chunks {bad[:8]}"


def _pairs_sim(K, n, rows, cols):
    """Exact cosine of each (row, col) pair by the oracle's definition."""
    out = np.full(rows.shape[0], -1.0)
    ok = cols >= 0
    for s in range(0, rows.shape[0], 1 << 15):
        r, c, m = rows[s:s + (1 << 15)], cols[s:s + (1 << 15)], ok[s:s + (1 << 15)]
        if m.any():
            dots = np.einsum("nd,nd->n", K[r[m]], K[c[m]])
            den = np.sqrt(n[r[m]] * n[c[m]])
            with np.errstate(invalid="ignore", divide="ignore"):
                sim = np.where(den > 0, dots / np.where(den > 0, den, 1.0), 0.0) + 0.0
            part = out[s:s + (1 << 15)]
            part[m] = sim
            out[s:s + (1 << 15)] = part
    return out


def _check_picks(gpu_arg, near, K, n, best_sim_gpu, tag, allowed=None):
    """Near-tie rows: the GPU's pick is a stored candidate (eligible and within
    NEAR_TIE of the maximum), within TIE_RTOL of the maximum, and not an
    exact tie of the maximum other than the lowest position.  Returns the arg
    array with those rows masked and the oracle's maximum at each row whose
    pick differs from the oracle's."""
    masked = gpu_arg.astype(np.int64).copy()
    differs = {}
    for key, cand in near.items():
        r = int(key)
        cand = cand["cand"] if isinstance(cand, dict) else cand
        j = int(gpu_arg[r])
        assert j in cand, f"{tag} row {r}: near-tie pick {j} is not among the oracle's candidates {cand[:8]}"
        if allowed is not None:
            assert allowed[j], f"{tag} row {r}: pick {j} is not retained"
        sims = _pairs_sim(K, n, np.full(len(cand), r), np.asarray(cand))
        top = sims.max()
        lowest_top = min(c for c, s in zip(cand, sims) if s == top)
        pick_sim = sims[cand.index(j)]
        assert pick_sim < top or j == lowest_top, f"{tag} row {r}: pick {j} ties the maximum but is not the lowest"
        tol = max(PR.TIE_RTOL, 2 * PR.EXACT_SIM_RTOL) * max(abs(top), 1e-300)
        assert pick_sim >= top - tol, f"{tag} row {r}: pick {j} at {pick_sim} is not the maximum {top}"
        assert abs(best_sim_gpu[r] - pick_sim) <= PR.EXACT_SIM_RTOL * abs(pick_sim), f"{tag} row {r}: reported sim"
        if j != lowest_top:  # the oracle's pick: the lowest position attaining the maximum
            differs[r] = float(top)
        masked[r] = -2
    return masked, differs


def _check_repair(gold, rep, g_local, K, n, S0, tag, tally, tau, sink, recent):
    gr = gold
    arg = rep["best_idx"][g_local].cpu().numpy()
    best = rep["best_sim"][g_local].cpu().numpy()
    masked, differs = _check_picks(arg, gr["near_tie"], K, n, best, tag + " b(S0)", allowed=S0)
    rows = np.arange(arg.shape[0])
    np.testing.assert_allclose(best, _pairs_sim(K, n, rows, arg.astype(np.int64)), rtol=PR.EXACT_SIM_RTOL, atol=0,
                               err_msg=f"{tag} b(S0) against the exact cosine of the reported pair")
    _chunks_equal(MG.chunk_digests(masked), gr["arg_chunks"], "b(S0) positions", tag)
    # a near-tie pick changes the swap only if the swap rule, applied to the
    # GPU's b with the oracle's maxima put back at those rows, gives another
    # result; otherwise |O|, |D|, m, S1 and the pairs must be the oracle's
    effect = PR.near_tie_effect(best, differs, S0, tau, sink, recent)
    rep_c = {"repair_heads": 1, "repair_near_tie_differs": len(differs),
             "repair_class_ambiguous": effect["class_changes"], "repair_rank_affected": int(effect["swap_changes"])}
    if not effect["swap_changes"]:
        got = [int(rep[k][g_local]) for k in ("n_orphans", "n_donors", "n_swaps")]
        assert got == [gr["n_orphans"], gr["n_donors"], gr["m"]], f"{tag}: |O|, |D|, m {got} vs oracle"
        m = gr["m"]
        pairs = rep["pairs"][g_local].cpu().numpy()
        assert MG.digest(np.packbits(rep["keep"][g_local].cpu().numpy())) == gr["keep"], f"{tag}: S1"
        assert MG.digest(np.ascontiguousarray(pairs[:m], dtype="<i4")) == gr["pairs"], f"{tag}: swap pairs"
        assert np.all(pairs[m:] == -1), f"{tag}: pair padding"
    else:
        _say(f"[{tag}] a near-tie pick of b(S0) changes the swap; checking it follows from the GPU's own b")
        gpu = {k: rep[k][g_local].cpu().numpy() for k in ("keep", "n_orphans", "n_donors", "n_swaps", "pairs")}
        gpu["best"] = best
        PR.check_swap_follows(gpu, S0, tau, sink, recent, tag)
    tally.add(rep_c)
    return rep_c


def _run_workload(cfg_id):
    gold = json.load(open(MG.golden_path(cfg_id)))
    cfg = get_config(cfg_id)
    assert gold["near_tie"] == PR.NEAR_TIE and gold["band"] == PR.BAND and gold["chunk"] == MG.CHUNK
    heads = [h["head"] for h in gold["heads"]]
    assert heads == MG.checked_heads(cfg_id), "the stored subset is not the seeded one"
    _say(f"[golden {cfg.name}] generating {len(heads)} of {cfg.G} heads, N={cfg.N}, d={cfg.d}")
    K, V, _ = make_heads(cfg, heads=heads)
    tk = _up(K)
    tally = PR.Tally(f"golden {cfg.name}")
    record = {"workload": cfg.name, "G": cfg.G, "N": cfg.N, "d": cfg.d, "tau": cfg.tau, "window": cfg.window,
              "sink": cfg.sink, "recent": cfg.recent, "mode": cfg.mode, "removal": cfg.removal,
              "checked_heads": heads, "heads": {}}
    if cfg.mode == "repair":
        S0 = np.stack([gumbel_retained(cfg, g) for g in heads])
        rep = krs.repair(tk, torch.from_numpy(S0).to("cuda:0"), cfg.tau, cfg.window, cfg.sink, cfg.recent)
        torch.cuda.synchronize()
    else:
        caps_all = MG.capacities(cfg_id)
        caps = [int(caps_all[g]) for g in heads]
        res = krs.score(tk, _up(V), cfg.tau, cfg.window, cfg.sink, cfg.recent, omega=True)
        sel = krs.select(res["score"], res["energy"], caps, cfg.sink, cfg.recent)
        rep = krs.repair(tk, sel["keep"], cfg.tau, cfg.window, cfg.sink, cfg.recent, prior=res)
        torch.cuda.synchronize()
    for gl, h in enumerate(gold["heads"]):
        g = h["head"]
        tag = f"{cfg.name} head {g}"
        assert MG.input_digest(K[gl], V[gl]) == h["inputs"], f"{tag}: regenerated inputs differ from the oracle run's"
        Kf = O.widen_bf16(K[gl])
        n = O.squared_norms(Kf)
        hrec = {"inputs": h["inputs"][:16]}
        if cfg.mode == "repair":
            hrec.update(_check_repair(h["repair"], rep, gl, Kf, n, S0[gl] != 0, tag, tally,
                                      cfg.tau, cfg.sink, cfg.recent))
        else:
            count = res["count"][gl].cpu().numpy()
            arg = res["best_idx"][gl].cpu().numpy()
            best = res["best_sim"][gl].cpu().numpy()
            band = {int(r): v for r, v in h["band"].items()}
            for r, (c_lo, nb) in band.items():
                assert c_lo <= count[r] <= c_lo + nb, f"{tag} row {r}: count {count[r]} outside its band"
            _chunks_equal(MG.chunk_digests(MG.mask_rows(count, list(band), -1)), h["count_chunks"], "counts", tag)
            masked, differs = _check_picks(arg, h["near_tie"], Kf, n, best, tag)
            _chunks_equal(MG.chunk_digests(masked), h["arg_chunks"], "best-twin positions", tag)
            rows = np.arange(cfg.N)
            np.testing.assert_allclose(best, _pairs_sim(Kf, n, rows, arg.astype(np.int64)), rtol=PR.EXACT_SIM_RTOL,
                                       atol=0, err_msg=f"{tag} best_sim against the exact cosine of the pair")
            e = O.value_energy(O.widen_bf16(V[gl]))
            np.testing.assert_allclose(res["energy"][gl].cpu().numpy(), e, rtol=PR.ENERGY_RTOL, atol=0,
                                       err_msg=f"{tag} energy")
            ok = np.ones(cfg.N, bool)
            ok[list(band)] = False
            s_ref, w_ref = O.frequency_score(e, count, cfg.N)  # counts certified equal outside the band
            np.testing.assert_allclose(res["score"][gl].cpu().numpy()[ok], s_ref[ok], rtol=1e-13, atol=0,
                                       err_msg=f"{tag} score")
            np.testing.assert_allclose(res["omega"][gl].cpu().numpy()[ok], w_ref[ok], rtol=1e-13, atol=0,
                                       err_msg=f"{tag} omega")
            gap = h["boundary_gap"]
            exact = not band and (gap == "inf" or gap >= PR.BOUNDARY_GAP)
            if exact:
                keep = sel["keep"][gl].cpu().numpy()
                assert MG.digest(np.packbits(keep)) == h["keep"], f"{tag}: keep mask differs from the oracle's"
            rc = {"rows": cfg.N, "band_rows": len(band), "near_tie_rows": len(h["near_tie"]),
                  "near_tie_differs": len(differs), "select_heads": 1, "select_inexact_heads": 0 if exact else 1}
            tally.add(rc)
            hrec.update(rc)
            if exact:
                keep_o = sel["keep"][gl].cpu().numpy() != 0  # certified equal to the oracle's selection
                hrec.update(_check_repair(h["repair"], rep, gl, Kf, n, keep_o, tag + " repair", tally,
                                          cfg.tau, cfg.sink, cfg.recent))
        record["heads"][str(g)] = hrec
    totals = tally.check()
    record["exclusions"] = totals
    record["verdict"] = "pass"
    os.makedirs(RESULTS, exist_ok=True)
    with open(os.path.join(RESULTS, f"{cfg.name}.parity.json"), "w") as f:
        json.dump(record, f, indent=1)
    _say(f"[golden {cfg.name}] {len(heads)} heads match the oracle; exclusions {totals}")


@pytest.mark.parametrize("cfg_id", [1, 2, 3, 4, 5])
def test_workload_against_oracle_goldens(cfg_id):
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    _run_workload(cfg_id)
