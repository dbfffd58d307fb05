"""Pins for the fp64 oracle: worked examples printed on the pages, closed forms,
invariants, exhaustive search and brute force on tiny inputs.

Each test is chosen so that a plausible slip in the oracle (a dropped +1, >=
for >, a window off by one, a missing normalisation, a wrong tie order, a swap
ranked the wrong way) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import brute
from oracle import twinkv_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# score: the Figure 3 example and the reversal condition


def test_figure3_normalised_scores():
    g = _golden("figure3_example.json")
    N = g["N"]
    e = np.array([g["A"]["energy"], g["B"]["energy"]])
    c = np.array([2, 0])  # A carries a count-2 key, B a count-0 key
    s, w = O.frequency_score(e, c, N)
    tol = 0.5 * 10 ** -g["printed_decimals"]
    assert abs(e[0] * w[0] - g["A"]["normalized_score"]) <= tol
    assert abs(e[1] * w[1] - g["B"]["normalized_score"]) <= tol
    # the rank reversal: A has more energy, B ranks higher after weighting
    assert e[0] > e[1] and s[1] > s[0]
    # the other assignment of the printed counts cannot reproduce the numbers
    s2, w2 = O.frequency_score(e, np.array([0, 2]), N)
    assert abs(e[0] * w2[0] - g["A"]["normalized_score"]) > tol


def _bf16_exact(rows):
    """bf16 bit patterns of values that bf16 holds exactly (asserted)."""
    x = np.asarray(rows, dtype=np.float32)
    u = x.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exact in bf16"
    return (u >> 16).astype(np.uint16)


def test_value_energy_closed_forms():
    """e = ||v||^2 ([P2] section 3.2) on bf16-exact rows whose squared norm is
    known in closed form: a 3-4-5 row gives 25 (||v|| would give 5), a row of
    d halves gives d/4 (||v|| = sqrt(d)/2), a unit basis row 1, a zero row 0,
    and a row mixing 2^10, 2^-10 and -2 the exact 2^20 + 4 + 2^-20 (which
    fp64 holds; any dropped or doubled term changes it)."""
    for d in (64, 128):
        rows = np.zeros((5, d), np.float32)
        rows[0, :2] = (3.0, 4.0)
        rows[1, :] = 0.5
        rows[2, d - 1] = 1.0
        rows[4, [0, 7, d // 2]] = (2.0 ** 10, 2.0 ** -10, -2.0)
        e = O.value_energy(O.widen_bf16(_bf16_exact(rows)))
        assert e.tolist() == [25.0, d / 4.0, 1.0, 0.0, 2.0 ** 20 + 4.0 + 2.0 ** -20]


def test_value_energy_reads_values_not_keys():
    """Through the whole-head score: with keys and values that differ, the
    energy and the score follow the values.  Keys are orthonormal basis rows
    (no twins, count 0, score = e * ln(N+1)); values are 3-4 rows scaled by
    the position, so e_i = 25 (i+1)^2 exactly."""
    N, d = 16, 64
    Kf = np.zeros((N, d), np.float32)
    Kf[np.arange(N), np.arange(N)] = 1.0
    Vf = np.zeros((N, d), np.float32)
    Vf[:, 0] = 3.0 * (np.arange(N) + 1)
    Vf[:, 1] = 4.0 * (np.arange(N) + 1)
    r = O.score_head(_bf16_exact(Kf), _bf16_exact(Vf), 0.5, 2)
    want = 25.0 * (np.arange(N) + 1.0) ** 2
    assert r["energy"].tolist() == want.tolist()
    assert np.all(r["count"] == 0)
    np.testing.assert_allclose(r["score"], want * math.log(N + 1.0), rtol=1e-15, atol=0)
    # the energy is not a function of the keys: swapping in other keys keeps it
    r2 = O.score_head(_bf16_exact(Kf[::-1].copy()), _bf16_exact(Vf), 0.5, 2)
    assert r2["energy"].tolist() == want.tolist()


def test_discount_closed_forms():
    N = 1000
    c = np.arange(N)
    s, w = O.frequency_score(np.ones(N), c, N)
    assert w[0] == 1.0  # a key with no twin keeps its full energy
    assert s[0] == pytest.approx(math.log(N + 1))
    assert np.all(np.diff(s) < 0)  # more twins, smaller score
    assert np.all(w > 0) and np.all(w <= 1)
    # c = N would make the discount log(1) = 0; one below keeps it positive
    assert s[-1] == pytest.approx(math.log((N + 1) / N))
    # energy scales the score linearly
    s3, _ = O.frequency_score(np.full(N, 3.0), c, N)
    np.testing.assert_allclose(s3, 3 * s, rtol=0, atol=0)


def test_reversal_condition():
    """For e_i > e_j > 0, weighting reverses their order iff
    1 < e_i/e_j < d_j/d_i (section 3.2 of the frequency-correction page)."""
    rng = np.random.default_rng(5)
    N = 4096
    for _ in range(2000):
        ei, ej = sorted(rng.uniform(0.1, 2.0, 2), reverse=True)
        if ei == ej:
            continue
        ci, cj = rng.integers(0, 20, 2)
        s, _ = O.frequency_score(np.array([ei, ej]), np.array([ci, cj]), N)
        di, dj = math.log((N + 1) / (ci + 1)), math.log((N + 1) / (cj + 1))
        assert (s[0] < s[1]) == (1 < ei / ej < dj / di)


# ---------------------------------------------------------------------------
# budget and protection: the printed boundary examples


def test_short_prefix_clipping_example():
    g = _golden("short_prefix_example.json")
    B = O.uniform_budget(g["N"], g["removal"])
    assert B == g["budget"]
    s, r = O.protected_counts(B, g["sink_param"], g["recent_param"])
    assert (s, r, B - s - r) == (g["sinks"], g["recent"], g["unprotected"])
    rng = np.random.default_rng(0)
    keep, idx = O.select_head(rng.random(g["N"]), rng.random(g["N"]), B, g["sink_param"], g["recent_param"])
    expect = list(range(4)) + list(range(g["N"] - 39, g["N"]))
    assert idx.tolist() == expect


def test_two_head_budget_example():
    g = _golden("budget_conservation.json")
    B = O.uniform_budget(g["N"], g["removal"])
    s, r = O.protected_counts(B, 4, 64)
    assert (B, s + r, B - s - r) == (g["B"], g["P"], g["U"])
    assert sum(g["capacities"]) == 2 * B
    assert min(g["capacities"]) >= g["P"] + g["U"] // 2 == g["min_capacity"]
    rng = np.random.default_rng(1)
    for cap in g["capacities"]:
        keep, idx = O.select_head(rng.random(g["N"]), rng.random(g["N"]), cap, 4, 64)
        assert keep.sum() == cap and idx.size == cap


def test_budget_floor():
    assert O.uniform_budget(10, 0.35) == 6  # 6.5 -> 6: floor, not ceil or round
    assert O.uniform_budget(8192, 0.7) == 2457
    assert O.uniform_budget(32768, 0.5) == 16384
    assert O.uniform_budget(131072, 0.75) == 32768
    assert O.uniform_budget(7, 0.0) == 7


def test_protection_clipping_small_capacities():
    assert O.protected_counts(0, 4, 64) == (0, 0)
    assert O.protected_counts(3, 4, 64) == (3, 0)  # sinks take priority
    assert O.protected_counts(10, 4, 64) == (4, 6)
    assert O.protected_counts(100, 4, 64) == (4, 64)


# ---------------------------------------------------------------------------
# similarity, count and best twin: closed forms


def _rows(N, idx_vec):
    return np.array(idx_vec, dtype=np.float64)


def test_strict_threshold_at_exact_cosine():
    # (1,0) and (3,4): cosine exactly 3/5
    d, N, w = 4, 8, 2
    K = np.zeros((N, d))
    K[:, 2] = 1.0  # filler orthogonal to both
    K[0] = [1, 0, 0, 0]
    K[5] = [3, 4, 0, 0]
    c, b, a = O.twin_count_and_best(K, 0.6, w)
    assert b[0] == 0.6 and a[0] == 5 and c[0] == 0 and c[5] == 0  # sim == tau is not a twin
    c, _, _ = O.twin_count_and_best(K, 0.5999, w)
    assert c[0] == 1 and c[5] == 1


def test_window_boundary():
    d, N, w = 4, 12, 3
    K = np.zeros((N, d))
    K[:, 3] = 1.0
    K[2] = [1, 1, 0, 0]
    K[2 + w] = [2, 2, 0, 0]  # |i-j| = w: local, excluded
    K[2 + w + 1] = [0.5, 0.5, 0, 0]  # |i-j| = w+1: counted
    c, b, a = O.twin_count_and_best(K, 0.9, w)
    assert c[2] == 1 and a[2] == 2 + w + 1 and b[2] == 1.0
    assert c[2 + w] == 0  # its only copies are within the window
    assert c[2 + w + 1] == 1 and a[2 + w + 1] == 2


def test_orthogonal_keys_zero_count():
    d = 32
    N = d
    K = np.diag(np.arange(1, N + 1, dtype=np.float64))  # orthogonal, different norms
    w = 4
    c, b, a = O.twin_count_and_best(K, 0.5, w)
    assert np.all(c == 0)
    assert np.all(b == 0.0)
    for i in range(N):
        assert a[i] == (0 if i > w else i + w + 1)  # lowest eligible position


def test_planted_exact_duplicates_scale_invariant():
    rng = np.random.default_rng(2)
    d, N, w = 16, 64, 4
    K = rng.integers(-8, 9, size=(N, d)).astype(np.float64)
    base = K[10].copy()
    for p, scale in [(20, 2.0), (40, 0.5), (12, 4.0), (63, 1.0)]:
        K[p] = scale * base  # exact multiples: cosine exactly 1
    c, b, a = O.twin_count_and_best(K, 0.99, w)
    # 10's nonlocal copies: 20, 40, 63 (12 is inside the window)
    assert c[10] == 3 and b[10] == 1.0 and a[10] == 20
    assert c[12] == 3 and a[12] == 20  # 12 sees 20, 40, 63 (10 is local)
    assert c[20] == 4 and a[20] == 10


def test_no_eligible_positions():
    rng = np.random.default_rng(3)
    for N, w in [(1, 0), (5, 4), (33, 32), (2, 1)]:
        K = rng.standard_normal((N, 8))
        c, b, a = O.twin_count_and_best(K, 0.1, w)
        assert np.all(c == 0) and np.all(b == -1.0) and np.all(a == -1)


def test_antiparallel_and_zero_keys():
    d, N, w = 4, 6, 1
    K = np.zeros((N, d))
    K[0] = [1, 2, 0, 0]
    K[3] = [-1, -2, 0, 0]
    # positions 1, 2, 4, 5 are zero keys: similarity 0 with everything
    c, b, a = O.twin_count_and_best(K, 0.5, w)
    assert c[0] == 0
    assert b[0] == 0.0 and a[0] == 2  # zero keys (sim 0) beat the antiparallel one (-1)
    K2 = np.zeros((3, d))
    K2[0] = [1, 2, 0, 0]
    K2[2] = [-1, -2, 0, 0]
    c, b, a = O.twin_count_and_best(K2, 0.5, 1)
    assert b[0] == -1.0 and a[0] == 2  # a real maximum of -1, told apart by a >= 0
    assert b[1] == -1.0 and a[1] == -1  # nothing eligible


def test_count_invariants_random():
    rng = np.random.default_rng(4)
    d, N, w = 8, 200, 5
    K = rng.standard_normal((N, d))
    for _ in range(30):  # plant some near-duplicates
        i, j = rng.integers(0, N, 2)
        K[j] = K[i] + 0.01 * rng.standard_normal(d)
    tau = 0.8
    c, b, a = O.twin_count_and_best(K, tau, w)
    n = O.squared_norms(K)
    S = O.cosine_rows(K, n, np.arange(N))
    ok = O.nonlocal_mask(np.arange(N), np.arange(N), w)
    T = (S > tau) & ok
    assert np.array_equal(T, T.T)  # the twin relation is symmetric
    assert c.sum() % 2 == 0
    assert np.array_equal(c, T.sum(1))
    assert np.all(b[:, None] >= np.where(ok, S, -np.inf))
    assert np.all((b >= -1) & (b <= 1 + 1e-15))
    for i in range(N):
        assert ok[i, a[i]] and S[i, a[i]] == b[i]
        assert not np.any(S[i, : a[i]][ok[i, : a[i]]] == b[i])  # lowest index on ties


def test_oracle_matches_brute_force_tiny():
    rng = np.random.default_rng(6)
    for trial in range(6):
        N, d = int(rng.integers(20, 70)), int(rng.choice([4, 8]))
        w = int(rng.integers(0, 6))
        K = np.round(rng.standard_normal((N, d)) * 4) / 4  # coarse grid: many exact ties
        for _ in range(6):
            i, j = rng.integers(0, N, 2)
            K[j] = K[i] * rng.choice([1.0, 2.0, 0.5])
        tau = float(rng.choice([0.3, 0.6, 0.9]))
        c, b, a = O.twin_count_and_best(K, tau, w)
        bf = brute.twin_stats(K.tolist(), tau, w)
        assert [x[0] for x in bf] == c.tolist()
        assert [x[2] for x in bf] == a.tolist()
        np.testing.assert_allclose([x[1] for x in bf], b, rtol=0, atol=1e-15)


def test_best_surviving_twin_restricted_columns():
    rng = np.random.default_rng(7)
    N, d, w = 60, 8, 3
    K = np.round(rng.standard_normal((N, d)) * 4) / 4
    S0 = (rng.random(N) < 0.5).astype(np.uint8)
    b, a = O.best_surviving_twin(K, S0, w)
    bf = brute.twin_stats(K.tolist(), 0.5, w, allowed=S0.tolist())
    assert [x[2] for x in bf] == a.tolist()
    np.testing.assert_allclose([x[1] for x in bf], b, rtol=0, atol=1e-15)
    assert np.all(S0[a[a >= 0]] == 1)
    # empty retained set: every b is -1
    b0, a0 = O.best_surviving_twin(K, np.zeros(N, np.uint8), w)
    assert np.all(b0 == -1) and np.all(a0 == -1)


# ---------------------------------------------------------------------------
# the synthetic generator's planted structure predicts the oracle's counts


@pytest.mark.parametrize("cfg_id,N", [(2, 3000), (4, 3000), (5, 2500)])
def test_planted_clusters_predict_counts(cfg_id, N):
    from synth import get_config, make_head

    cfg = get_config(cfg_id)
    h = make_head(cfg, 3, N=N)
    K = O.widen_bf16(h["K"])
    c, b, _ = O.twin_count_and_best(K, cfg.tau, cfg.window)
    cl = h["cluster"]
    pos = np.arange(N)
    expect = np.zeros(N, dtype=np.int64)
    for i in np.flatnonzero(cl >= 0):
        mates = pos[(cl == cl[i]) & (np.abs(pos - i) > cfg.window)]
        expect[i] = mates.size
    assert np.array_equal(c, expect)
    assert np.all(b[expect > 0] > 0.97)


# ---------------------------------------------------------------------------
# selection


def test_select_matches_exhaustive_search():
    rng = np.random.default_rng(8)
    for trial in range(40):
        N = int(rng.integers(6, 12))
        cap = int(rng.integers(0, N + 1))
        sink, recent = int(rng.integers(0, 3)), int(rng.integers(0, 3))
        # coarse values so that exact score and energy ties occur
        s = rng.integers(0, 3, N).astype(float)
        e = rng.integers(0, 3, N).astype(float)
        keep, idx = O.select_head(s, e, cap, sink, recent)
        assert idx.tolist() == brute.select_exhaustive(s.tolist(), e.tolist(), cap, sink, recent)


def test_select_tie_rule_explicit():
    # equal scores: higher energy wins; equal score and energy: lower position wins
    s = np.array([0, 5, 5, 5, 5, 0.0])
    e = np.array([0, 1, 2, 2, 1, 0.0])
    keep, idx = O.select_head(s, e, 4, 1, 1)  # 1 sink + 1 recent + 2 chosen
    assert idx.tolist() == [0, 2, 3, 5]
    keep, idx = O.select_head(s, e, 3, 1, 1)
    assert idx.tolist() == [0, 2, 5]
    keep, idx = O.select_head(s, e, 5, 1, 1)
    assert idx.tolist() == [0, 1, 2, 3, 5]


def test_select_invariants_random():
    rng = np.random.default_rng(9)
    for _ in range(20):
        N = int(rng.integers(50, 400))
        cap = int(rng.integers(0, N + 1))
        s, e = rng.random(N), rng.random(N)
        keep, idx = O.select_head(s, e, cap, 4, 32)
        prot = O.protected_mask(N, cap, 4, 32)
        assert keep.sum() == cap and np.all(keep[prot] == 1)
        assert np.all(np.diff(idx) > 0)
        kept_u = np.flatnonzero((keep == 1) & ~prot)
        drop_u = np.flatnonzero((keep == 0) & ~prot)
        if kept_u.size and drop_u.size:
            assert s[kept_u].min() >= s[drop_u].max()


# ---------------------------------------------------------------------------
# repair


def _hand_keys():
    u1, u2, u3, u4 = np.eye(4)
    K = np.array([u4, u1, u2, u1, u3, u2, u1 + u2, u3, u3 + u4, u1, u2 + u3, u4])
    return K


def test_repair_hand_example():
    """Twelve positions, window 1, tau 0.9, one sink and one recent slot.
    S0 = {0, 1, 3, 6, 9, 11}.  Derived by hand:
    b(S0) = [1, 1, 1/sqrt2, 1, 0, 0, 1/sqrt2, 0, 1/sqrt2, 1, 1/2, 1];
    orphans by (b asc, i asc) = 4, 5, 7, 10, 2, 8;
    donors by (b desc, j asc) = 1, 3, 9 (6 has b < tau; 0 and 11 are protected);
    m = 3, pairs (4,1), (5,3), (7,9); S1 = {0, 4, 5, 6, 7, 11}."""
    K = _hand_keys()
    S0 = np.zeros(12, np.uint8)
    S0[[0, 1, 3, 6, 9, 11]] = 1
    r = O.repair_head(K, S0, 0.9, 1, 1, 1)
    h = 1 / math.sqrt(2)
    np.testing.assert_allclose(r["best"], [1, 1, h, 1, 0, 0, h, 0, h, 1, 0.5, 1], rtol=0, atol=1e-15)
    assert r["arg"].tolist() == [11, 3, 6, 1, 0, 0, 1, 0, 0, 1, 6, 0]
    assert r["orphans"].tolist() == [4, 5, 7, 10, 2, 8]
    assert r["donors"].tolist() == [1, 3, 9]
    assert r["m"] == 3
    assert r["pairs"].tolist() == [[4, 1], [5, 3], [7, 9]]
    assert np.flatnonzero(r["keep"]).tolist() == [0, 4, 5, 6, 7, 11]
    # the one-shot pass is not idempotent: all copies of u1 left together
    r2 = O.repair_head(K, r["keep"], 0.9, 1, 1, 1)
    assert r2["m"] > 0 and 1 in r2["orphans"].tolist()


def test_repair_donor_at_exact_tau():
    # b == tau makes a donor (>=) but a pair with sim == tau is not an orphan's twin (<)
    K = np.zeros((8, 4))
    K[:, 2] = 1.0
    K[1] = [1, 0, 0, 0]
    K[4] = [3, 4, 0, 0]
    S0 = np.zeros(8, np.uint8)
    S0[[1, 4]] = 1
    r = O.repair_head(K, S0, 0.6, 1, 0, 0)
    assert r["best"][1] == 0.6 and r["best"][4] == 0.6
    assert r["donors"].tolist() == [1, 4]  # tie in b: lower position first
    # evicted filler keys: cos with (1,0,0,0) is 0 and with (3,4,0,0) is 0 -> orphans
    assert r["n_orphans"] == 6 and r["m"] == 2


def test_repair_noop_when_redundancy_consistent():
    rng = np.random.default_rng(10)
    for _ in range(20):
        N, d, w = 80, 16, 2
        K = rng.standard_normal((N, d))
        K[40:] = K[:40] * 1.0  # every key has an exact twin 40 positions away
        S0 = np.zeros(N, np.uint8)
        S0[rng.permutation(40)[:20]] = 1  # keep one copy of 20 pairs, none of the others
        r = O.repair_head(K, S0, 0.95, w, 0, 0)
        # every evicted key with a retained twin is covered; evicted keys whose twin was
        # also evicted are orphans, but no retained key duplicates another: no donors
        assert r["n_donors"] == 0 and r["m"] == 0
        assert np.array_equal(r["keep"], S0)
        # symmetric case: every evicted key has a surviving twin -> no orphans
        S0b = np.zeros(N, np.uint8)
        S0b[:40] = 1
        rb = O.repair_head(K, S0b, 0.95, w, 0, 0)
        assert rb["n_orphans"] == 0 and np.array_equal(rb["keep"], S0b)


def test_repair_budget_and_pairs_random():
    rng = np.random.default_rng(11)
    for _ in range(25):
        N, d = int(rng.integers(30, 120)), 8
        w = int(rng.integers(0, 4))
        K = np.round(rng.standard_normal((N, d)) * 2) / 2
        for _ in range(N // 4):
            i, j = rng.integers(0, N, 2)
            K[j] = K[i]
        S0 = (rng.random(N) < rng.uniform(0.2, 0.8)).astype(np.uint8)
        sink, recent = int(rng.integers(0, 3)), int(rng.integers(0, 5))
        r = O.repair_head(K, S0, 0.9, w, sink, recent)
        assert r["keep"].sum() == S0.sum()
        prot = O.protected_mask(N, int(S0.sum()), sink, recent)
        for o, dn in r["pairs"]:
            assert S0[o] == 0 and r["keep"][o] == 1
            assert S0[dn] == 1 and r["keep"][dn] == 0 and not prot[dn]
        bf = brute.repair(K.tolist(), S0.tolist(), 0.9, w, sink, recent)
        assert bf["orphans"] == r["orphans"].tolist()
        assert bf["donors"] == r["donors"].tolist()
        assert bf["pairs"] == [tuple(p) for p in r["pairs"].tolist()]


def test_repair_idempotent_when_twins_touch_protected_positions():
    """If every twin relation joins a protected position to an unprotected one,
    and S0 keeps the protected positions, a second pass changes nothing."""
    rng = np.random.default_rng(12)
    for _ in range(20):
        N, d, w = 60, 32, 1
        sink, recent = 3, 3
        K = rng.standard_normal((N, d))
        prot_pos = list(range(sink)) + list(range(N - recent, N))
        free = np.arange(sink, N - recent)
        twins = rng.choice(free, size=10, replace=False)
        for t in twins:
            K[t] = K[rng.choice(prot_pos)] * 2.0
        S0 = np.zeros(N, np.uint8)
        S0[prot_pos] = 1
        S0[rng.choice(free, size=20, replace=False)] = 1
        r1 = O.repair_head(K, S0, 0.9, w, sink, recent)
        r2 = O.repair_head(K, r1["keep"], 0.9, w, sink, recent)
        assert r2["m"] == 0 and np.array_equal(r2["keep"], r1["keep"])


# ---------------------------------------------------------------------------
# physical cache layout (section 3.4 of the frequency-correction page)


def test_pack_retained_hand_example():
    """Two heads, five positions, d = 2: head 0 keeps {0, 3}, head 1 keeps
    {1, 2, 4}; rows come out in sequence order, head 0 first, no padding."""
    K = np.arange(2 * 5 * 2, dtype=np.uint16).reshape(2, 5, 2)
    V = (1000 + np.arange(2 * 5 * 2)).astype(np.uint16).reshape(2, 5, 2)
    Kp, Vp, off = O.pack_retained(K, V, [[0, 3], [1, 2, 4]])
    assert off.tolist() == [0, 2, 5]
    assert Kp.tolist() == [[0, 1], [6, 7], [12, 13], [14, 15], [18, 19]]
    assert Vp.tolist() == [[1000, 1001], [1006, 1007], [1012, 1013], [1014, 1015], [1018, 1019]]


def test_pack_retained_payload_matches_budget_example():
    """The payload is exactly 2*d*sum(b_h) elements; with the two-head example
    capacities (202, 310) that is 2*d*H*B for H = 2, B = 256 (budget
    conservation), and each packed row equals its source row bit for bit."""
    g = _golden("budget_conservation.json")
    rng = np.random.default_rng(5)
    N, d = g["N"], 64
    K = rng.integers(0, 1 << 16, size=(2, N, d), dtype=np.uint16)
    V = rng.integers(0, 1 << 16, size=(2, N, d), dtype=np.uint16)
    kept = [np.sort(rng.choice(N, c, replace=False)) for c in g["capacities"]]
    Kp, Vp, off = O.pack_retained(K, V, kept)
    assert Kp.size + Vp.size == 2 * d * sum(g["capacities"]) == 2 * d * 2 * g["B"]
    for h in range(2):
        rows = slice(off[h], off[h + 1])
        assert np.array_equal(Kp[rows], K[h][kept[h]]) and np.array_equal(Vp[rows], V[h][kept[h]])


def test_pack_retained_rejects_unordered_and_handles_empty():
    K = np.zeros((2, 4, 8), np.uint16)
    with pytest.raises(ValueError):
        O.pack_retained(K, None, [[2, 1], []])
    Kp, Vp, off = O.pack_retained(K, None, [[], []])
    assert Kp.shape == (0, 8) and Vp is None and off.tolist() == [0, 0, 0]


# ---------------------------------------------------------------------------
# head allocation (section 3.3 and appendices A.1-A.3 of the frequency-correction page)


def _layer_scores(H, N, lo, hi, high_counts):
    """Scores 2.0 on the first high_counts[h] unprotected positions of head h, 1.0 elsewhere."""
    z = np.ones((H, N), np.float32)
    for h, c in enumerate(high_counts):
        z[h, lo:lo + c] = 2.0
    return z


def test_allocation_two_head_example():
    """A.1's constructed example: N = 512, r = 0.5 gives B = 256, P = 68,
    U = 188; g = (80, 296) must give b = (202, 310)."""
    g = _golden("budget_conservation.json")
    N, B = g["N"], g["B"]
    z = _layer_scores(2, N, 4, N - 64, [80, 296])
    r = O.allocate_heads(z, N, B, 4, 64)
    assert r["P"] == g["P"] and r["U"] == g["U"]
    assert r["g"].tolist() == [80, 296]
    assert r["b"].tolist() == g["capacities"]


def test_allocation_conservation_and_floor_random():
    rng = np.random.default_rng(11)
    for trial in range(30):
        H = int(rng.integers(1, 9))
        N = int(rng.integers(80, 400))
        B = int(rng.integers(0, N + 1))
        z = rng.random((H, N)).astype(np.float32) ** 4
        r = O.allocate_heads(z, N, B, 4, 64)
        assert int(r["b"].sum()) == H * B
        assert np.all(r["b"] >= r["P"] + r["U"] // 2)
        assert np.all(r["b"] <= N)
        if r["U"] > 0:
            assert int(r["g"].sum()) == H * r["U"]


def test_allocation_half_remainders_go_to_first_heads():
    """U = 3, g = (2, 4): u~ = (2.5, 3.5), one slot of rounding goes to head 0."""
    N, B = 40, 5  # sink 1, recent 1 -> P = 2, U = 3
    z = _layer_scores(2, N, 1, N - 1, [2, 4])
    r = O.allocate_heads(z, N, B, 1, 1)
    assert r["g"].tolist() == [2, 4]
    assert r["b"].tolist() == [2 + 3, 2 + 3]
    z = _layer_scores(3, N, 1, N - 1, [2, 4, 3])  # u~ = (2.5, 3.5, 3): R = 1 -> head 0
    r = O.allocate_heads(z, N, B, 1, 1)
    assert r["g"].tolist() == [2, 4, 3] and r["b"].tolist() == [5, 5, 5]


def test_allocation_ties_and_degenerate_cases():
    N, B = 20, 10  # sink 1, recent 1 -> P = 2, U = 8, 18 unprotected per head
    z = np.ones((2, N), np.float32)
    r = O.allocate_heads(z, N, B, 1, 1)  # all equal: head 0's positions come first
    assert r["g"].tolist() == [16, 0] and r["b"].tolist() == [2 + 12, 2 + 4]
    z = np.zeros((3, N), np.float32)
    z[:, 0] = 5.0  # only protected positions carry attention: the pool is all zero
    r = O.allocate_heads(z, N, B, 1, 1)
    assert r["g"].tolist() == [8, 8, 8] and r["b"].tolist() == [B, B, B]
    sp = _golden("short_prefix_example.json")  # U = 0: allocation skipped
    r = O.allocate_heads(np.random.default_rng(0).random((4, sp["N"])).astype(np.float32), sp["N"], sp["budget"],
                         sp["sink_param"], sp["recent_param"])
    assert r["U"] == 0 and r["b"].tolist() == [sp["budget"]] * 4


def _attention_brute(K, Q, pool):
    N, d = len(K), len(K[0])
    Gq, W = len(Q), len(Q[0])
    agg = [0.0] * N
    for g in range(Gq):
        for w in range(W):
            t = N - W + w
            logit = [math.fsum(Q[g][w][c] * K[j][c] for c in range(d)) / math.sqrt(d) for j in range(t + 1)]
            m = max(logit)
            den = math.fsum(math.exp(x - m) for x in logit)
            for j in range(t + 1):
                agg[j] += math.exp(logit[j] - m) / den / Gq
    half = pool // 2
    return [max(agg[max(0, i - half):min(N, i + half + 1)]) for i in range(N)]


def test_prefix_attention_matches_brute_force():
    rng = np.random.default_rng(4)
    for N, d, Gq, W, pool in [(9, 4, 2, 3, 7), (12, 8, 4, 5, 3), (6, 4, 1, 6, 1)]:
        K = rng.standard_normal((N, d)) * 2
        Q = rng.standard_normal((Gq, W, d)) * 2
        z = O.prefix_attention_scores(K, Q, pool)
        ref = _attention_brute(K.tolist(), Q.tolist(), pool)
        np.testing.assert_allclose(z, ref, rtol=1e-12, atol=0)


def test_prefix_attention_closed_forms():
    """Equal keys give the uniform causal softmax: query t puts 1/(t+1) on every
    i <= t.  Without pooling the scores sum to W (each query's weights sum
    to one); the width-7 pool takes the maximum of the 7 surrounding sums."""
    N, d, Gq, W = 50, 8, 4, 32
    K = np.ones((N, d))
    Q = np.random.default_rng(2).standard_normal((Gq, W, d))
    z1 = O.prefix_attention_scores(K, Q, pool=1)
    t = np.arange(N - W, N)
    expect = np.array([np.sum(1.0 / (t[t >= i] + 1)) for i in range(N)])
    np.testing.assert_allclose(z1, expect, rtol=1e-13)
    assert abs(z1.sum() - W) < 1e-12
    z7 = O.prefix_attention_scores(K, Q, pool=7)
    np.testing.assert_allclose(z7, [expect[max(0, i - 3):i + 4].max() for i in range(N)], rtol=1e-13)


# ---------------------------------------------------------------------------
# score variants: the standalone count score of the TwinKV page (Eq. 3) and
# the ablations of the frequency-correction page (sections 5.3 and 5.5)


def test_variant_value_only_is_energy_topk():
    rng = np.random.default_rng(21)
    for trial in range(20):
        N = int(rng.integers(8, 14))
        cap = int(rng.integers(0, N + 1))
        e = np.round(rng.random(N) * 4, 1)  # coarse: ties happen
        c = rng.integers(0, 4, N)
        sc, tie = O.variant_scores(e, c, N, "value")
        _, idx = O.select_head(sc, tie, cap, 1, 2)
        assert idx.tolist() == brute.select_exhaustive(e, e, cap, 1, 2)


def test_variant_rarity_ranks_counts_then_position():
    """Removing value: lowest counts first, equal counts to the lower position;
    the same order as the TwinKV page's s = -r/n."""
    N = 12
    c = np.array([0, 5, 1, 1, 0, 3, 2, 0, 1, 4, 0, 0])
    e = np.arange(N, dtype=float)[::-1] + 1  # energies must not matter
    sc, tie = O.variant_scores(e, c, N, "rarity")
    keep, idx = O.select_head(sc, tie, 7, 1, 2)  # protected {0, 10, 11}; 4 more by (count, position)
    assert idx.tolist() == [0, 2, 3, 4, 7, 10, 11]
    neg = -c / N  # Eq. 3 directly, with the lower position on ties
    cand = np.arange(1, 10)
    order = cand[np.lexsort((cand, -neg[cand]))]
    assert sorted(order[:4].tolist()) == [2, 3, 4, 7]


def test_variant_twin_matches_score_and_permutation_keeps_multiset():
    from synth import count_permutation, get_config
    cfg = get_config(2).with_(N=300)
    rng = np.random.default_rng(3)
    N = 300
    e = rng.random(N) * 10
    c = rng.integers(0, 9, N)
    sc, tie = O.variant_scores(e, c, N, "twin")
    assert np.array_equal(sc, O.frequency_score(e, c, N)[0]) and np.array_equal(tie, e)
    sc_id, _ = O.variant_scores(e, c, N, "twin", perm=np.arange(N))
    assert np.array_equal(sc_id, sc)
    cap = 150
    perms = [count_permutation(cfg, 5, cap, seed) for seed in (11, 29, 47)]
    s_cnt, r_cnt = O.protected_counts(cap, cfg.sink, cfg.recent)
    for p in perms:
        assert np.array_equal(np.sort(p), np.arange(N))
        assert np.array_equal(p[:s_cnt], np.arange(s_cnt)) and np.array_equal(p[N - r_cnt:], np.arange(N - r_cnt, N))
        cp = c[p]
        assert np.array_equal(np.sort(cp[s_cnt:N - r_cnt]), np.sort(c[s_cnt:N - r_cnt]))
    assert not np.array_equal(perms[0], perms[1])


def test_ceil_budget_differs_from_floor():
    """The TwinKV page keeps ceil((1-rho) n), the frequency page floor(N(1-r))."""
    assert O.ceil_budget(10, 0.55) == 5 and O.uniform_budget(10, 0.55) == 4
    assert O.ceil_budget(32768, 0.5) == O.uniform_budget(32768, 0.5) == 16384
    assert O.ceil_budget(7, 0.0) == 7 and O.ceil_budget(7, 1.0) == 0


# ---------------------------------------------------------------------------
# count statistics (Figure 1(b) of the TwinKV page; section 2.1, 5.5 and B.2
# of the frequency-correction page)


def test_count_stats_hand_example():
    """Capacity 8 with one sink and two recent slots protects {0, 12, 13};
    the 11 unprotected positions 1..11 have counts 0,1,2,3,4,5,8,9,30,0,1."""
    N = 14
    c = np.array([7, 0, 1, 2, 3, 4, 5, 8, 9, 30, 0, 1, 6, 0])
    e = np.array([1, 10, 9, 8, 7, 6, 5, 4, 3, 2, 1.2, 1.1, 1, 1], dtype=float)
    kv = np.zeros(N, np.uint8)
    kv[[0, 1, 2, 3, 4, 12, 13]] = 1  # value-only keeps energies 10, 9, 8, 7: the cut is 7
    kt = kv.copy()
    kt[4] = 0
    kt[10] = 1  # Twin drops position 4 (e 7) for position 10 (e 1.2)
    st = O.count_stats(c, e, kt, kv, 8, 1, 2)
    assert st["n"] == 11 and st["twin"] == 9
    assert st["hist"] == [2, 2, 1, 2, 2, 2]
    cu = np.array([0, 1, 2, 3, 4, 5, 8, 9, 30, 0, 1])
    assert abs(st["omega_sum"] - sum(math.log(15 / (x + 1)) / math.log(15) for x in cu)) < 1e-12
    assert (st["kept"], st["added"], st["removed"], st["e_cut"]) == (4, 1, 1, 7.0)
    assert st["margins_added"] == [0, 0, 0, 0, 1]     # |1.2/7 - 1| = 0.83
    assert st["margins_removed"] == [1, 0, 0, 0, 0]   # the cut itself
    assert st["margins_pool"] == [1, 0, 2, 4, 4]


def test_count_stats_planted_fraction():
    """On a synthetic head the twin fraction is the share of planted cluster
    members with a mate outside the window (the planted structure predicts
    every count, see the cluster pin above)."""
    from synth import get_config, make_head
    cfg = get_config(2)
    N = 2000
    h = make_head(cfg, 1, N=N)
    r = O.score_head(h["K"], h["V"], cfg.tau, cfg.window)
    cap = O.uniform_budget(N, 0.5)
    kt, _ = O.select_head(r["score"], r["energy"], cap, cfg.sink, cfg.recent)
    kv, _ = O.select_head(r["energy"], r["energy"], cap, cfg.sink, cfg.recent)
    st = O.count_stats(r["count"], r["energy"], kt, kv, cap, cfg.sink, cfg.recent)
    prot = O.protected_mask(N, cap, cfg.sink, cfg.recent)
    cl = h["cluster"]
    pos = np.arange(N)
    has_mate = np.array([cl[i] >= 0 and np.any((cl == cl[i]) & (np.abs(pos - i) > cfg.window)) for i in range(N)])
    assert st["twin"] == int((has_mate & ~prot).sum())
    assert sum(st["hist"]) == st["n"] == int((~prot).sum())
    assert st["kept"] == cap - int(prot.sum())
    assert st["added"] == st["removed"]  # both selections keep the same number


def test_restricted_twin_is_the_unrestricted_one_when_retained():
    """[P1] section 3.4, Eq. 4: b_i(S0) is a maximum over the retained nonlocal
    positions.  When the lowest position attaining the maximum over all
    nonlocal positions is retained, it is also b_i(S0)'s position, with the
    same value; otherwise b_i(S0) is no larger; with no nonlocal position at
    all both are -1.  Checked with the pure-Python brute force (exact ties
    planted by duplicated keys) and against the oracle's restricted twin."""
    rng = np.random.default_rng(41)
    reused = 0
    for trial in range(24):
        N = int(rng.integers(2, 40))
        w = int(rng.integers(0, 4))
        K = rng.integers(-3, 4, size=(N, 4)).astype(float)
        if N > 4:
            K[rng.integers(0, N, 3)] = K[rng.integers(0, N)]  # exact ties
        S0 = rng.random(N) < 0.5
        allr = brute.twin_stats(K.tolist(), 0.9, w)
        subr = brute.twin_stats(K.tolist(), 0.9, w, allowed=S0.tolist())
        ob, oa = O.best_surviving_twin(K, S0.astype(np.uint8), w)
        for i in range(N):
            _, fb, fa = allr[i]
            _, sb, sa = subr[i]
            assert (sb, sa) == (ob[i], oa[i]) or (math.isclose(sb, ob[i], rel_tol=1e-15) and sa == oa[i])
            if fa < 0:
                assert sa < 0 and sb == -1.0
            elif S0[fa]:
                assert (sa, sb) == (fa, fb)
                reused += 1
            else:
                assert sb <= fb
    assert reused > 50
