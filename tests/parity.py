"""Parity rules between the HIP library and the fp64 oracle.

Matching rules (stated in the problem: similarities and scores within relative
tolerance 1e-3; counts, argmax and retained index sets bit-exact; ties to the
lowest index), with the exclusions the fp32 sweep makes necessary.  None of
them is silent: every compare_* call returns the count of each kind, a
``Tally`` adds them up per test, and each test asserts its totals against a
stated bound (zero for everything but validated near-ties on the synthetic
workloads).

* tau band: a pair with |sim - tau| < 1e-3 may fall on either side of tau in
  fp32; the GPU count must lie in [c_lo, c_lo + band], where c_lo counts the
  nonlocal pairs with sim >= tau + 1e-3 and band counts those inside the band.
* argmax near-ties: both sweeps settle every candidate within twice the fp32
  error of a row's maximum in fp64 (a row where another tile comes that
  close goes to the exact resolve), so the GPU's best twin is the exact
  maximum at its lowest position, up to two limits: the two sides' fp64
  cosines of one pair agree to EXACT_SIM_RTOL, and the score pass merges its
  row and column sides through a 64-bit key that keeps the cosine's bits
  above the lowest ceil(log2 N) (2^-34 relative at N <= 2^18).  A row where
  the GPU's position differs from the oracle's must therefore be a near-tie
  whose pick lies within TIE_RTOL of the maximum (strictly below it: exact
  ties resolve to the lowest position), and the GPU must report the pick's
  exact cosine.  Rows with an eligible similarity strictly below the
  maximum by less than NEAR_TIE = 2e-5 are counted as near-tie rows (the
  stored oracle results list their candidates).
* selection: heads with a band-affected row, or whose kept/evicted boundary
  ranks differ by a relative score gap below 1e-12, are checked by the
  properties a top-k selection must have instead of bit for bit (the oracle
  never takes a GPU value as input).
* repair: when a row's best surviving twin differs at a validated near-tie,
  the swap rule decides exactly whether that changes |O|, |D|, m, the pairs
  or S1 (it is applied to the GPU's b and to the GPU's b with the oracle's
  maxima put back); if not, they are compared bit for bit.
"""
from __future__ import annotations

import numpy as np

from oracle import twinkv_oracle as O

BAND = 1e-3
# near-tie rows, counted and listed (see above)
NEAR_TIE = 2e-5
# how far below the oracle's maximum a differing pick may lie, relative: the
# packed merge of the score pass (2^-34 at N <= 2^18) or fp64 rounding
TIE_RTOL = 2.0 ** -34
BOUNDARY_GAP = 1e-12
# Energies and squared norms are fp64 sums of d exact products (bf16 squares
# are exact).  Both sides add the same non-negative terms in different orders,
# so each is within (d-1) * 2^-53 of the exact sum relative to it: the two
# agree to 2 * 127 * 2^-53 at d <= 128 (usually bit for bit).
ENERGY_RTOL = 2 * 127 * 2.0 ** -53
# The exact-path cosine dot / sqrt(n_i n_j) of one pair: the dot and each
# squared norm are such sums (<= 127 roundings each), plus the product,
# sqrt and division; the two sides agree to twice the bound of one.
EXACT_SIM_RTOL = 2 * (2 * 127 + 3) * 2.0 ** -53

# the kinds of exclusion a Tally counts
KINDS = ("rows", "band_rows", "near_tie_rows", "near_tie_differs", "select_heads", "select_inexact_heads",
         "repair_heads", "repair_near_tie_differs", "repair_class_ambiguous", "repair_rank_affected")


class Tally:
    """Sum of the exclusion counts of one test, printed and bounded."""

    def __init__(self, tag: str):
        self.tag = tag
        self.c = {k: 0 for k in KINDS}

    def add(self, rep: dict):
        for k in KINDS:
            self.c[k] += int(rep.get(k, 0))
        for sub in ("repair", "repair with prior"):
            if sub in rep:
                self.add(rep[sub])

    def check(self, near_tie_frac: float = 1e-6, **bounds):
        """Print the totals; assert every bounded kind (default bound 0 for
        band rows, inexact selections and swaps changed by a near-tie pick)
        and the fraction of rows whose argmax took another candidate within
        TIE_RTOL of the maximum."""
        print(f"[{self.tag}] exclusions: {self.c}", flush=True)
        lim = {"band_rows": 0, "select_inexact_heads": 0, "repair_class_ambiguous": 0, "repair_rank_affected": 0}
        lim.update(bounds)
        for k, v in lim.items():
            assert self.c[k] <= v, f"{self.tag}: {self.c[k]} {k} (bound {v}); all counts {self.c}"
        assert self.c["near_tie_differs"] <= max(1.0, near_tie_frac * self.c["rows"]), \
            f"{self.tag}: {self.c['near_tie_differs']} near-tie argmax picks differ over {self.c['rows']} rows"
        return self.c


def score_reference(Kbits, Vbits, tau, window, rows=None):
    K = O.widen_bf16(Kbits)
    V = O.widen_bf16(Vbits)
    N = K.shape[0]
    n = O.squared_norms(K)
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    c, b, a = O.twin_count_and_best(K, tau, window, rows=rows, n=n)
    e = O.value_energy(V[rows])
    s, w = O.frequency_score(e, c, N)
    band, c_lo, gap = _exclusion_stats(K, n, rows, np.arange(N), tau, window)
    return {"rows": rows, "count": c, "best": b, "arg": a, "energy": e, "score": s, "omega": w, "band": band,
            "c_lo": c_lo, "gap": gap, "K": K, "n": n, "window": int(window), "cols": None}


def _exclusion_stats(K, n, rows, cols, tau, window):
    band = np.zeros(rows.size, np.int64)
    c_lo = np.zeros(rows.size, np.int64)
    gap = np.full(rows.size, np.inf)
    step = max(1, (1 << 24) // max(1, cols.size))
    for s in range(0, rows.size, step):
        grp = rows[s:s + step]
        sims = O.cosine_rows(K, n, grp, cols)
        ok = O.nonlocal_mask(grp, cols, window)
        if tau is not None:
            inb = ok & (np.abs(sims - tau) < BAND)
            band[s:s + step] = inb.sum(1)
            c_lo[s:s + step] = (ok & (sims > tau) & ~inb).sum(1)
        if cols.size >= 2:
            # gap to the largest eligible similarity strictly below the
            # maximum (exact ties do not make a near-tie: they must resolve
            # to the lowest position)
            masked = np.where(ok, sims, -np.inf)
            best = masked.max(1)
            below = np.where(masked < best[:, None], masked, -np.inf).max(1)
            with np.errstate(invalid="ignore"):
                gap[s:s + step] = np.where(np.isfinite(below) & np.isfinite(best), best - below, np.inf)
    return band, c_lo, gap


def validate_near_tie_picks(ref, rows, ga, gb, allowed=None, tag=""):
    """Rows where the GPU's best twin differs from the oracle's: each must be
    a near-tie row, the GPU's position must be eligible (nonlocal, retained
    when ``allowed`` is given) with an exact cosine within NEAR_TIE of the
    oracle's maximum, and the GPU must report that cosine.  Returns the
    number of such rows."""
    near = (ref["gap"] > 0) & (ref["gap"] < NEAR_TIE)
    diff = ga != ref["arg"]
    bad = diff & ~near
    assert not bad.any(), (f"{tag} argmax mismatch at rows {rows[bad][:10]}: gpu {ga[bad][:10]} "
                           f"oracle {ref['arg'][bad][:10]} best gpu {gb[bad][:5]} oracle {ref['best'][bad][:5]}")
    K, n, w = ref["K"], ref["n"], ref["window"]
    N = K.shape[0]
    for t in np.flatnonzero(diff):
        i, j = int(rows[t]), int(ga[t])
        assert 0 <= j < N and abs(i - j) > w, f"{tag} row {i}: near-tie pick {j} is not an eligible position"
        if allowed is not None:
            assert allowed[j] != 0, f"{tag} row {i}: near-tie pick {j} is not retained"
        sim = float(O.cosine_rows(K, n, np.array([i]), np.array([j]))[0, 0])
        top = float(ref["best"][t])
        tol = max(TIE_RTOL, 2 * EXACT_SIM_RTOL) * max(abs(top), 1e-300)
        assert sim >= top - tol, f"{tag} row {i}: pick {j} at {sim} is not the maximum {top} (tolerance {tol:.3g})"
        # an exact tie with the maximum must go to the lowest position, the oracle's
        assert sim < ref["best"][t], f"{tag} row {i}: pick {j} ties the maximum but is not the lowest position"
        assert abs(gb[t] - sim) <= EXACT_SIM_RTOL * abs(sim), f"{tag} row {i}: reported {gb[t]} for {sim}"
    return int(diff.sum())


def compare_score(gpu, ref, tag=""):
    """gpu: dict of numpy arrays for the same rows.  Asserts the rules, returns a report."""
    rows = ref["rows"]
    rep = {"rows": int(rows.size)}
    band_rows = ref["band"] > 0
    rep["band_rows"] = int(band_rows.sum())
    gc = gpu["count"].astype(np.int64)
    bad = ~band_rows & (gc != ref["count"])
    assert not bad.any(), f"{tag} count mismatch at rows {rows[bad][:10]}: gpu {gc[bad][:10]} oracle {ref['count'][bad][:10]}"
    lo, hi = ref["c_lo"][band_rows], ref["c_lo"][band_rows] + ref["band"][band_rows]
    assert np.all((gc[band_rows] >= lo) & (gc[band_rows] <= hi)), f"{tag} band-row count outside its band"
    near = (ref["gap"] > 0) & (ref["gap"] < NEAR_TIE)
    rep["near_tie_rows"] = int(near.sum())
    ga = gpu["arg"].astype(np.int64)
    rep["near_tie_differs"] = validate_near_tie_picks(ref, rows, ga, gpu["best"], tag=tag)
    np.testing.assert_allclose(gpu["best"], ref["best"], rtol=1e-3, atol=1e-12, err_msg=f"{tag} best_sim")
    same = ga == ref["arg"]
    # the fixup recomputes the chosen pair exactly in fp64: same pair, same value
    np.testing.assert_allclose(gpu["best"][same], ref["best"][same], rtol=EXACT_SIM_RTOL, atol=0,
                               err_msg=f"{tag} exact best")
    rep["best_bitwise"] = float(np.mean(gpu["best"] == ref["best"]))
    np.testing.assert_allclose(gpu["energy"], ref["energy"], rtol=ENERGY_RTOL, atol=0, err_msg=f"{tag} energy")
    eq = gc == ref["count"]
    np.testing.assert_allclose(gpu["score"][eq], ref["score"][eq], rtol=1e-13, atol=0, err_msg=f"{tag} score")
    np.testing.assert_allclose(gpu["score"], ref["score"], rtol=1e-3, atol=0, err_msg=f"{tag} score (band rows)")
    if gpu.get("omega") is not None:
        np.testing.assert_allclose(gpu["omega"][eq], ref["omega"][eq], rtol=1e-13, atol=0, err_msg=f"{tag} omega")
    rep["score_bitwise"] = float(np.mean(gpu["score"] == ref["score"]))
    return rep


def boundary_gap(score, energy, capacity, sink, recent):
    """Relative score gap between the last kept and the first evicted
    unprotected position in the oracle's ranking (inf if nothing is cut)."""
    N = score.shape[0]
    s_cnt, r_cnt = O.protected_counts(capacity, sink, recent)
    u = capacity - s_cnt - r_cnt
    cand = np.arange(s_cnt, N - r_cnt)
    if u <= 0 or u >= cand.size:
        return np.inf
    order = np.lexsort((cand, -energy[cand], -score[cand]))
    a, b = score[cand[order[u - 1]]], score[cand[order[u]]]
    if a == b:
        return np.inf  # an exact score tie: energy, then position decide, both exact on both sides
    return abs(a - b) / max(abs(a), abs(b), 1e-300)


def select_exact(score_rep, ref, capacity, sink, recent):
    """Whether a head's selection must match the oracle bit for bit."""
    return score_rep["band_rows"] == 0 and boundary_gap(ref["score"], ref["energy"], capacity, sink,
                                                        recent) >= BOUNDARY_GAP


def check_select_properties(keep, kept_idx, score, energy, capacity, sink, recent, tag=""):
    """What any correct selection must satisfy, given the scores it ranked."""
    N = keep.shape[0]
    cap = int(min(max(capacity, 0), N))
    prot = O.protected_mask(N, cap, sink, recent)
    assert int(keep.sum()) == cap, f"{tag} |keep| {keep.sum()} != {cap}"
    assert np.all(keep[prot] == 1), f"{tag} protected position dropped"
    assert np.array_equal(np.flatnonzero(keep), kept_idx), f"{tag} kept_idx is not the ascending keep list"
    ku = np.flatnonzero((keep == 1) & ~prot)
    du = np.flatnonzero((keep == 0) & ~prot)
    if ku.size and du.size:
        worst_kept = min(ku, key=lambda i: (score[i], energy[i], -i))
        best_drop = max(du, key=lambda i: (score[i], energy[i], -i))
        assert (score[worst_kept], energy[worst_kept], -worst_kept) > (score[best_drop], energy[best_drop], -best_drop), \
            f"{tag} an evicted position outranks a kept one"


def compare_repair(gpu, ref, keep_in, tau, tag=""):
    """gpu: numpy dict (keep, best, arg, n_orphans, n_donors, n_swaps, pairs) for one head;
    ref: repair_reference output.  Returns a report."""
    N = ref["best"].shape[0]
    rows = np.arange(N)
    rep = {"repair_heads": 1}
    ga = gpu["arg"].astype(np.int64)
    mism = ga != ref["arg"]
    rep["repair_near_tie_differs"] = validate_near_tie_picks(ref, rows, ga, gpu["best"], allowed=keep_in,
                                                             tag=f"{tag} b(S0)")
    np.testing.assert_allclose(gpu["best"], ref["best"], rtol=1e-3, atol=1e-12, err_msg=f"{tag} b(S0)")
    np.testing.assert_allclose(gpu["best"][~mism], ref["best"][~mism], rtol=EXACT_SIM_RTOL, atol=0,
                               err_msg=f"{tag} exact b")
    # A differing row is a near-tie: the GPU's b is the exact cosine of a pair
    # within NEAR_TIE of the maximum.  Whether that changes the swap is
    # decided exactly: the swap rule is applied to the GPU's b and to the GPU's
    # b with the oracle's values put back at the differing rows.
    diff_rows = np.flatnonzero(mism)
    effect = near_tie_effect(gpu["best"], {int(r): float(ref["best"][r]) for r in diff_rows}, keep_in, tau,
                             ref["sink"], ref["recent"])
    rep["repair_class_ambiguous"] = effect["class_changes"]
    rep["repair_rank_affected"] = int(effect["swap_changes"])
    if not effect["swap_changes"]:
        assert int(gpu["n_orphans"]) == ref["n_orphans"], f"{tag} |O|"
        assert int(gpu["n_donors"]) == ref["n_donors"], f"{tag} |D|"
        assert int(gpu["n_swaps"]) == ref["m"], f"{tag} m"
        np.testing.assert_array_equal(gpu["keep"], ref["keep"], err_msg=f"{tag} S1")
        m = ref["m"]
        np.testing.assert_array_equal(gpu["pairs"][:m], ref["pairs"], err_msg=f"{tag} swap pairs")
        assert np.all(gpu["pairs"][m:] == -1)
    else:
        check_swap_follows(gpu, keep_in, tau, ref["sink"], ref["recent"], tag)
    # properties that hold regardless
    assert int(gpu["keep"].sum()) == int(np.asarray(keep_in).sum()), f"{tag} budget changed"
    return rep


def repair_reference(Kbits, keep_in, tau, window, sink, recent):
    K = O.widen_bf16(Kbits)
    ref = O.repair_head(K, keep_in, tau, window, sink, recent)
    n = O.squared_norms(K)
    cols = np.flatnonzero(np.asarray(keep_in) != 0)
    _, _, gap = _exclusion_stats(K, n, np.arange(K.shape[0]), cols, None, window)
    ref.update({"gap": gap, "K": K, "n": n, "window": int(window), "sink": int(sink), "recent": int(recent)})
    return ref


def swap_rule(b, keep_in, tau, sink, recent):
    """The one-shot swap of "TwinKV: A Composable Repair Pass ..." section 3.4
    applied to given b(S0): orphans (evicted, b < tau) by ascending b, donors
    (retained, unprotected against K = |S0|, b >= tau) by descending b, ties
    to the lower position; the m = min(|O|, |D|) leading pairs swap."""
    b = np.asarray(b, dtype=np.float64)
    s0 = np.asarray(keep_in) != 0
    N = b.shape[0]
    prot = O.protected_mask(N, int(s0.sum()), sink, recent)
    idx = np.arange(N)
    o = idx[~s0 & (b < tau)]
    d = idx[s0 & ~prot & (b >= tau)]
    o = o[np.lexsort((o, b[o]))]
    d = d[np.lexsort((d, -b[d]))]
    m = min(o.size, d.size)
    s1 = s0.copy()
    s1[d[:m]] = False
    s1[o[:m]] = True
    return {"n_orphans": int(o.size), "n_donors": int(d.size), "m": int(m),
            "pairs": np.stack([o[:m], d[:m]], axis=1), "keep": s1}


def check_swap_follows(gpu, keep_in, tau, sink, recent, tag=""):
    """The GPU's |O|, |D|, m, pairs and S1 are the swap rule applied to its
    own b(S0) (for a head whose swap a near-tie pick changed)."""
    want = swap_rule(gpu["best"], keep_in, tau, sink, recent)
    got = [int(gpu[k]) for k in ("n_orphans", "n_donors", "n_swaps")]
    assert got == [want["n_orphans"], want["n_donors"], want["m"]], f"{tag}: |O|, |D|, m from its own b"
    m = want["m"]
    np.testing.assert_array_equal(np.asarray(gpu["pairs"])[:m], want["pairs"], err_msg=f"{tag}: pairs from its own b")
    assert np.all(np.asarray(gpu["pairs"])[m:] == -1), f"{tag}: pair padding"
    np.testing.assert_array_equal(np.asarray(gpu["keep"]) != 0, want["keep"], err_msg=f"{tag}: S1 from its own b")


def near_tie_effect(b_gpu, b_ref_rows: dict, keep_in, tau, sink, recent):
    """Whether putting the oracle's b back at the near-tie rows where the GPU
    picked another candidate changes the swap (counts, pairs or S1), and how
    many of those rows change class (b on the other side of tau)."""
    if not b_ref_rows:
        return {"swap_changes": False, "class_changes": 0}
    b_gpu = np.asarray(b_gpu, dtype=np.float64)
    alt = b_gpu.copy()
    rows = np.fromiter(b_ref_rows.keys(), dtype=np.int64)
    alt[rows] = np.fromiter(b_ref_rows.values(), dtype=np.float64)
    base = swap_rule(b_gpu, keep_in, tau, sink, recent)
    other = swap_rule(alt, keep_in, tau, sink, recent)
    same = all(base[k] == other[k] for k in ("n_orphans", "n_donors", "m")) and \
        np.array_equal(base["pairs"], other["pairs"]) and np.array_equal(base["keep"], other["keep"])
    return {"swap_changes": not same, "class_changes": int(np.sum((b_gpu[rows] < tau) != (alt[rows] < tau)))}
