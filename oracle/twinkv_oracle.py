"""Plain fp64 CPU oracle for the TwinKV key-redundancy hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library and imports nothing from it.

Sources (cited by page title and section / equation; no line numbers):

* [P1] "TwinKV: A Composable Repair Pass for KV Cache Eviction via Pairwise
  Key Redundancy" (arXiv HTML page): section 3.1 problem setup, section 3.2
  redundancy scoring (Eq. 1 cosine similarity, Eq. 2 redundancy count, the
  protected sink / recent regions), section 3.4 composable repair (Eq. 4 best
  surviving twin, orphans, donors, severity ranking, swap), section 3.5.
* [P2] "Small Frequency Corrections Can Change What Survives KV Cache
  Compression" (paperpeel page): section 3.1 exact budget and protected
  positions, section 3.2 value-weighted nonlocal key rarity (count, value
  energy, discounted score, tie rule), section 3.3 head allocation from prefix
  attention (Equation 5), section 3.4 selection in sequence order and the
  packed, unpadded cache layout, appendix A.2 prefix-attention statistics,
  appendix A.3 budget conservation, appendix B.2 measured count statistics,
  appendix A.1 boundary handling and the Figure 3 example.

Every quantity is evaluated straight from its definition in float64.  Keys and
values arrive as bf16 bit patterns and are widened exactly.  Matrix products
(numpy/BLAS) serve as the one library primitive; evaluating the per-row
definitions for a group of rows at once changes no value's definition.

Readings where the pages are silent or disagree (each is listed in the
design notes of the repository as well):

* log in the score is the natural log (any base rescales all scores by one
  positive constant, so no selection changes);
* the normalised discount is omega = log((N+1)/(c+1)) / log(N+1), which gives a
  zero-count key a weight of exactly 1 and reproduces the Figure 3 numbers;
* a zero-norm key has cosine similarity 0 with every key;
* the per-head budget is an input capacity; the uniform capacity is P2's
  floor(N(1-r)) (P1's ceil is not used);
* protection is clipped per head against its own capacity: s = min(sink, b),
  recent = min(recent, b - s) (P2 section 3.1 and appendix A.1 applied per head);
* repair protects the same clipped regions computed with K = |S0|; protected
  positions that S0 evicted may still be orphans; only donors exclude them;
* all ties go to the lowest position;
* head allocation (P2 section 3.3, A.2): the W = 32 queries are those of the
  last W prefix positions; the attention of the Gq query heads sharing a KV
  head is averaged and that of the W queries summed (a sum and a mean differ
  by W = 32, a power of two, so no float32 score or ranking changes); the
  max-pool window of 7 is centred and cut at the ends of the prefix, and
  pooling comes before protected positions are excluded; the scores are
  evaluated in float64 and rounded once to float32, the precision the page
  names, and the global ranking compares those float32 values;
* count statistics (P2 B.2): the six histogram bins are {0}, {1}, {2}, {3,4},
  {5..8}, {9+} and the five margin bins have edges 5%, 10%, 25%, 50% (the
  page prints neither); every position is counted where the page samples
  at most 16 per group.
"""
from __future__ import annotations

import math

import numpy as np

NONE = -1  # index returned when no eligible position exists


# ----------------------------------------------------------------------------
# inputs


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# [P1] section 3.2 and [P2] section 3.2: norms and value energy


def squared_norms(X: np.ndarray) -> np.ndarray:
    """n_i = ||x_i||_2^2 in float64 (the squared l2 norm used to normalise keys,
    [P1] section 3.2, and the value energy e_i = ||v_i||^2, [P2] section 3.2)."""
    X = np.asarray(X, dtype=np.float64)
    return np.einsum("nd,nd->n", X, X)


def value_energy(V: np.ndarray) -> np.ndarray:
    """e_{h,i} = ||v_{h,i}||_2^2 ([P2] section 3.2)."""
    return squared_norms(V)


# ----------------------------------------------------------------------------
# [P1] Eq. 1: cosine similarity


def cosine_rows(K: np.ndarray, n: np.ndarray, rows: np.ndarray, cols: np.ndarray | None = None) -> np.ndarray:
    """sim(i, j) = k_i . k_j / sqrt(n_i * n_j) for i in ``rows``, j in ``cols``.

    [P1] Eq. 1 defines sim(i, j) as the dot product of the l2-normalised keys.
    A zero-norm key has no direction; its similarity is taken as 0.
    """
    cols = np.arange(K.shape[0]) if cols is None else np.asarray(cols)
    dots = K[rows] @ K[cols].T
    denom = np.sqrt(n[rows][:, None] * n[cols][None, :])
    with np.errstate(invalid="ignore", divide="ignore"):
        sims = dots / denom
    sims[denom == 0.0] = 0.0
    return sims + 0.0  # canonicalise -0.0


def nonlocal_mask(rows: np.ndarray, cols: np.ndarray, window: int) -> np.ndarray:
    """True where |i - j| > w ([P1] section 3.2: j lies outside the local window
    of i; with w >= 0 this also excludes j = i)."""
    return np.abs(rows[:, None].astype(np.int64) - cols[None, :].astype(np.int64)) > int(window)


# ----------------------------------------------------------------------------
# [P1] Eq. 2 / [P2] section 3.2 count, and the best nonlocal twin


def _row_groups(rows: np.ndarray, n_cols: int, budget_elems: int = 1 << 24):
    step = max(1, budget_elems // max(1, n_cols))
    for s in range(0, rows.shape[0], step):
        yield rows[s:s + step]


def twin_count_and_best(K: np.ndarray, tau: float, window: int, rows=None, n: np.ndarray | None = None):
    """Per row i (all rows by default):

    * count c_i = #{ j : |i - j| > w and sim(i, j) > tau }  ([P1] Eq. 2,
      [P2] section 3.2; both inequalities strict; protected positions count);
    * best b_i = max over the same nonlocal j of sim(i, j) (reported whether or
      not it exceeds tau), and a_i = the lowest j attaining it;
      b_i = -1 and a_i = -1 when no j satisfies |i - j| > w.

    ``K`` is one head's keys as float64 [N][d].
    """
    K = np.asarray(K, dtype=np.float64)
    N = K.shape[0]
    n = squared_norms(K) if n is None else n
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    cols = np.arange(N)
    count = np.zeros(rows.shape[0], dtype=np.int64)
    best = np.full(rows.shape[0], -1.0)
    arg = np.full(rows.shape[0], NONE, dtype=np.int64)
    pos = 0
    for grp in _row_groups(rows, N):
        sims = cosine_rows(K, n, grp, cols)
        ok = nonlocal_mask(grp, cols, window)
        count[pos:pos + grp.size] = np.count_nonzero((sims > tau) & ok, axis=1)
        b, a = _masked_max_first(sims, ok)
        best[pos:pos + grp.size] = b
        arg[pos:pos + grp.size] = a
        pos += grp.size
    return count, best, arg


def _masked_max_first(sims: np.ndarray, ok: np.ndarray, col_ids: np.ndarray | None = None):
    """Max over allowed entries of each row and the first (lowest) column
    attaining it; (-1, -1) for rows with nothing allowed."""
    masked = np.where(ok, sims, -np.inf)
    a = np.argmax(masked, axis=1)  # first occurrence of the maximum
    b = masked[np.arange(masked.shape[0]), a]
    has = ok.any(axis=1)
    b = np.where(has, b, -1.0)
    if col_ids is not None:
        a = col_ids[a]
    a = np.where(has, a, NONE)
    return b, a.astype(np.int64)


def best_surviving_twin(K: np.ndarray, retained: np.ndarray, window: int, rows=None, n: np.ndarray | None = None):
    """[P1] Eq. 4: b_i(S0) = max over j in S0 with |i - j| > w, j != i of
    sim(i, j), and -1 if no such j; a_i(S0) is the lowest such j attaining it
    (-1 if none)."""
    K = np.asarray(K, dtype=np.float64)
    N = K.shape[0]
    n = squared_norms(K) if n is None else n
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    cols = np.flatnonzero(np.asarray(retained) != 0)
    best = np.full(rows.shape[0], -1.0)
    arg = np.full(rows.shape[0], NONE, dtype=np.int64)
    if cols.size == 0:
        return best, arg
    pos = 0
    for grp in _row_groups(rows, cols.size):
        sims = cosine_rows(K, n, grp, cols)
        ok = nonlocal_mask(grp, cols, window)
        b, a = _masked_max_first(sims, ok, cols)
        best[pos:pos + grp.size] = b
        arg[pos:pos + grp.size] = a
        pos += grp.size
    return best, arg


# ----------------------------------------------------------------------------
# [P2] section 3.2: frequency-discounted score


def frequency_score(energy: np.ndarray, count: np.ndarray, N: int):
    """s_{h,i} = e_{h,i} * log((N + 1) / (c_{h,i} + 1)) with the natural log, and
    the normalised discount omega = log((N+1)/(c+1)) / log(N+1) in (0, 1]
    ([P2] section 3.2 and the Figure 3 example)."""
    e = np.asarray(energy, dtype=np.float64)
    c = np.asarray(count, dtype=np.float64)
    disc = np.log((N + 1.0) / (c + 1.0))
    return e * disc, disc / math.log(N + 1.0)


# ----------------------------------------------------------------------------
# [P2] section 3.1: exact budget and protected positions


def uniform_budget(N: int, removal: float) -> int:
    """B = floor(N (1 - r)) ([P2] section 3.1, Equation 1)."""
    return int(math.floor(N * (1.0 - removal)))


def protected_counts(capacity: int, sink: int, recent: int):
    """Sinks first, then recent positions, both clipped to the capacity:
    s = min(sink, b), recent = min(recent, b - s) ([P2] section 3.1 and
    appendix A.1, where a 43-slot budget holds 4 sinks and 39 recent)."""
    s = min(int(sink), int(capacity))
    r = min(int(recent), int(capacity) - s)
    return s, r


def protected_mask(N: int, capacity: int, sink: int, recent: int) -> np.ndarray:
    s, r = protected_counts(capacity, sink, recent)
    m = np.zeros(N, dtype=bool)
    m[:s] = True
    if r > 0:
        m[N - r:] = True
    return m


# ----------------------------------------------------------------------------
# score variants: [P1] section 3.2 (Eq. 3) and the ablations of [P2]
# sections 5.3 and 5.5


def ceil_budget(N: int, removal: float) -> int:
    """[P1] section 3.1: |S| = ceil((1 - rho) n), evaluated in float64."""
    return int(math.ceil(N * (1.0 - removal)))


def variant_scores(energy: np.ndarray, count: np.ndarray, N: int, variant: str, perm=None):
    """Selection keys (score, tie) of one head for select_head, whose order is
    (score desc, tie desc, position asc):

    * "twin":   e * ln((N+1)/(c+1)), tie e ([P2] section 3.2);
    * "value":  e, tie e (frequency removed, [P2] section 5.3);
    * "rarity": the normalised discount ln((N+1)/(c+1)) / ln(N+1), tie 0, so
      equal counts fall to the lower position (value removed, [P2] section
      5.3); the same order as [P1]'s s = -r/n (Eq. 3), whose ties the page
      leaves open (read: lower position first).

    ``perm`` (optional, int [N]): position i takes the count of position
    perm[i] (the within-head count permutation of [P2] section 5.5; the
    caller permutes the unprotected positions among themselves)."""
    e = np.asarray(energy, dtype=np.float64)
    c = np.asarray(count, dtype=np.int64)
    if perm is not None:
        c = c[np.asarray(perm, dtype=np.int64)]
    score, omega = frequency_score(e, c, N)
    if variant == "twin":
        return score, e
    if variant == "value":
        return e.copy(), e
    if variant == "rarity":
        return omega, np.zeros_like(e)
    raise ValueError(variant)


# ----------------------------------------------------------------------------
# [P2] section 3.4: per-head selection


def select_head(score: np.ndarray, energy: np.ndarray, capacity: int, sink: int, recent: int):
    """Retain the protected positions and the top (b_h - P) unprotected
    positions by score; exact score ties go to higher value energy, then to the
    lower position ([P2] sections 3.2 and 3.4).  Returns the keep mask (uint8)
    and the retained positions in ascending (sequence) order."""
    N = score.shape[0]
    cap = int(capacity)
    if not 0 <= cap <= N:
        raise ValueError("capacity out of range")
    prot = protected_mask(N, cap, sink, recent)
    s_cnt, r_cnt = protected_counts(cap, sink, recent)
    u = cap - s_cnt - r_cnt
    cand = np.flatnonzero(~prot)
    order = np.lexsort((cand, -energy[cand], -score[cand]))  # last key is primary
    keep = prot.copy()
    keep[cand[order[:u]]] = True
    assert int(keep.sum()) == cap
    return keep.astype(np.uint8), np.flatnonzero(keep).astype(np.int64)


# ----------------------------------------------------------------------------
# [P1] section 3.4: composable repair


def repair_head(K: np.ndarray, retained: np.ndarray, tau: float, window: int, sink: int, recent: int):
    """One-shot repair of a retained set S0 at a fixed budget ([P1] section 3.4).

    * b_i = b_i(S0) for every position (Eq. 4), computed once against S0;
    * orphans O: i not in S0 with b_i < tau, ranked by ascending b (ties: lower i);
    * donors D: j in S0, outside the protected sink / recent regions, with
      b_j >= tau, ranked by descending b (ties: lower j);
    * m = min(|O|, |D|); the m most severe pairs (O[k], D[k]) are swapped, so
      S1 = S0 - D[:m] + O[:m] and |S1| = |S0|.
    """
    K = np.asarray(K, dtype=np.float64)
    N = K.shape[0]
    S0 = np.asarray(retained) != 0
    Kb = int(S0.sum())
    best, arg = best_surviving_twin(K, S0, window)
    prot = protected_mask(N, Kb, sink, recent)
    idx = np.arange(N)
    o = idx[(~S0) & (best < tau)]
    dn = idx[S0 & (~prot) & (best >= tau)]
    o = o[np.lexsort((o, best[o]))]
    dn = dn[np.lexsort((dn, -best[dn]))]
    m = min(o.size, dn.size)
    S1 = S0.copy()
    S1[dn[:m]] = False
    S1[o[:m]] = True
    assert int(S1.sum()) == Kb
    pairs = np.stack([o[:m], dn[:m]], axis=1) if m else np.zeros((0, 2), dtype=np.int64)
    return {
        "keep": S1.astype(np.uint8),
        "best": best,
        "arg": arg,
        "orphans": o,
        "donors": dn,
        "n_orphans": int(o.size),
        "n_donors": int(dn.size),
        "m": int(m),
        "pairs": pairs.astype(np.int64),
    }


# ----------------------------------------------------------------------------
# count statistics: [P1] section 2 / Figure 1(b), [P2] sections 2.1, 5.5 and
# appendix B.2

COUNT_BINS = ((0, 0), (1, 1), (2, 2), (3, 4), (5, 8), (9, None))  # six-bin histogram
MARGIN_EDGES = (0.05, 0.10, 0.25, 0.50)                           # five margin bins


def count_stats(count: np.ndarray, energy: np.ndarray, keep_twin: np.ndarray, keep_value: np.ndarray,
                capacity: int, sink: int, recent: int) -> dict:
    """Statistics of one head over its unprotected positions (protection
    clipped against ``capacity`` as in the selection):

    * n: unprotected positions; twin: those with at least one nonlocal twin
      (c >= 1, the fraction of [P1] Figure 1(b) and [P2] section 2.1);
    * hist: the six-bin count histogram of [P2] Figure 1 / B.2, bins
      {0}, {1}, {2}, {3,4}, {5..8}, {9+} (the page does not print its edges);
    * omega_sum: sum of the normalised discounts ln((N+1)/(c+1))/ln(N+1)
      (the mean of [P2] section 5.5 is omega_sum / n);
    * kept, added, removed: unprotected positions retained by the Twin
      selection, retained by Twin but not by value-only, and the reverse
      (selection change = added / kept, [P2] B.2);
    * e_cut: the lowest unprotected energy value-only retains (0 if none);
      margins_added / _removed / _pool: |e/e_cut - 1| of the Twin-added, the
      Twin-removed and all unprotected positions in five bins with edges
      5%, 10%, 25%, 50% ([P2] B.2 counts every position, where the page
      samples at most 16 per group; its edges are not printed)."""
    c = np.asarray(count, dtype=np.int64)
    e = np.asarray(energy, dtype=np.float64)
    N = c.shape[0]
    prot = protected_mask(N, int(capacity), sink, recent)
    u = ~prot
    kt = (np.asarray(keep_twin) != 0) & u
    kv = (np.asarray(keep_value) != 0) & u
    cu = c[u]
    hist = []
    for lo, hi in COUNT_BINS:
        m = cu >= lo if hi is None else (cu >= lo) & (cu <= hi)
        hist.append(int(m.sum()))
    omega = np.log((N + 1.0) / (cu + 1.0)) / math.log(N + 1.0)
    e_cut = float(e[kv].min()) if kv.any() else 0.0

    def margins(mask):
        out = [0] * (len(MARGIN_EDGES) + 1)
        if e_cut <= 0.0:
            return out
        dev = np.abs(e[mask] / e_cut - 1.0)
        for x in dev:
            out[int(np.searchsorted(MARGIN_EDGES, x, side="right"))] += 1
        return out

    added = kt & ~kv
    removed = kv & ~kt
    return {"n": int(u.sum()), "twin": int((cu >= 1).sum()), "hist": hist, "omega_sum": float(omega.sum()),
            "kept": int(kt.sum()), "added": int(added.sum()), "removed": int(removed.sum()), "e_cut": e_cut,
            "margins_added": margins(added), "margins_removed": margins(removed), "margins_pool": margins(u)}


# ----------------------------------------------------------------------------
# [P2] section 3.3 and appendix A.2: head capacities from prefix attention


def prefix_attention_scores(K: np.ndarray, Q: np.ndarray, pool: int = 7) -> np.ndarray:
    """Capacity statistics of one KV head ([P2] section 3.3, appendix A.2).

    ``K``: the head's keys [N][d]; ``Q``: the queries of its Gq query heads at
    the last W prefix positions t = N-W .. N-1, [Gq][W][d] (all float64).
    a[g,t,i] = exp(q_{g,t}.k_i / sqrt(d)) / sum_{j<=t} exp(q_{g,t}.k_j / sqrt(d))
    for i <= t and 0 for i > t (the causal softmax of A.2).  The Gq query
    heads are averaged, the W queries summed, and the result max-pooled over
    positions with a centred window of ``pool`` positions cut at the ends of
    the prefix.  Returns the pooled score of every position (float64)."""
    K = np.asarray(K, dtype=np.float64)
    Q = np.asarray(Q, dtype=np.float64)
    N, d = K.shape
    Gq, W, _ = Q.shape
    t_pos = np.arange(N - W, N)
    logits = np.einsum("gtd,nd->gtn", Q, K) / math.sqrt(d)
    causal = np.arange(N)[None, None, :] <= t_pos[None, :, None]
    logits = np.where(causal, logits, -np.inf)
    m = logits.max(axis=2, keepdims=True)
    ex = np.where(causal, np.exp(logits - m), 0.0)
    a = ex / ex.sum(axis=2, keepdims=True)
    agg = a.mean(axis=0).sum(axis=0)
    half = pool // 2
    z = np.empty(N)
    for i in range(N):
        z[i] = agg[max(0, i - half):min(N, i + half + 1)].max()
    return z


def allocate_heads(z: np.ndarray, N: int, B: int, sink: int, recent: int) -> dict:
    """Equation 5 of [P2] section 3.3 for one layer's H KV heads sharing the
    per-head budget B ([P2] appendices A.2, A.3).

    ``z``: float32 [H][N] capacity scores.  With s = min(sink, B), w =
    min(recent, B - s), P = s + w, U = B - P: g_h counts head h's positions
    among the H*U largest unprotected scores of the layer (ties to the lower
    head, then the lower position; all scores zero gives g_h = U);
    u~_h = (g_h + U)/2, u_h = floor(u~_h) + delta_h where the first
    R = H*U - sum floor(u~_h) heads with fractional part 1/2 get delta = 1;
    b_h = P + u_h.  U = 0 skips the allocation (b_h = B)."""
    z = np.asarray(z, dtype=np.float32)
    H = z.shape[0]
    s_cnt, r_cnt = protected_counts(B, sink, recent)
    P = s_cnt + r_cnt
    U = B - P
    if U == 0:
        return {"b": np.full(H, B, np.int64), "g": np.zeros(H, np.int64), "P": P, "U": U}
    lo, hi = s_cnt, N - r_cnt
    vals = z[:, lo:hi].astype(np.float64)
    if not np.any(vals != 0.0):
        g = np.full(H, U, np.int64)
    else:
        flat = vals.reshape(-1)
        order = np.lexsort((np.arange(flat.size), -flat))  # score desc, then head, then position
        pick = order[:H * U]
        g = np.bincount(pick // vals.shape[1], minlength=H).astype(np.int64)
    twice = g + U                       # 2 * u~_h, an integer
    fl = twice // 2
    R = H * U - int(fl.sum())
    half = np.flatnonzero(twice % 2 == 1)
    delta = np.zeros(H, np.int64)
    delta[half[:R]] = 1
    b = P + fl + delta
    assert int(b.sum()) == H * B
    return {"b": b, "g": g, "P": P, "U": U}


# ----------------------------------------------------------------------------
# [P2] section 3.4: physical cache layout of a selection


def pack_retained(K: np.ndarray, V: np.ndarray | None, kept: list):
    """The retained keys (and values) of every head in sequence order, heads
    one after another with no padding ([P2] section 3.4): head g contributes
    rows K[g][kept[g]] (kept[g] ascending), copied unchanged.  ``K``, ``V``:
    [G][N][d] arrays (bf16 bit patterns or any dtype; copied as they are).
    Returns (K_packed [total][d], V_packed or None, offsets int64 [G+1])."""
    G = K.shape[0]
    if len(kept) != G:
        raise ValueError("one retained list per head")
    offsets = np.zeros(G + 1, dtype=np.int64)
    kp, vp = [], []
    for g in range(G):
        idx = np.asarray(kept[g], dtype=np.int64)
        if idx.size and (np.any(np.diff(idx) <= 0) or idx[0] < 0 or idx[-1] >= K.shape[1]):
            raise ValueError("retained positions must be ascending and within the prefix")
        offsets[g + 1] = offsets[g] + idx.size
        kp.append(K[g][idx])
        if V is not None:
            vp.append(V[g][idx])
    d = K.shape[2]
    Kp = np.concatenate(kp, axis=0) if kp else np.zeros((0, d), K.dtype)
    Vp = (np.concatenate(vp, axis=0) if vp else np.zeros((0, d), V.dtype)) if V is not None else None
    return Kp, Vp, offsets


# ----------------------------------------------------------------------------
# whole-head pipelines


def score_head(Kbits: np.ndarray, Vbits: np.ndarray, tau: float, window: int, rows=None):
    """Count, best nonlocal twin, energy and score for one head (bf16 bits in)."""
    K = widen_bf16(Kbits)
    V = widen_bf16(Vbits)
    N = K.shape[0]
    c, b, a = twin_count_and_best(K, tau, window, rows=rows)
    e = value_energy(V if rows is None else V[np.asarray(rows)])
    s, w = frequency_score(e, c, N)
    return {"count": c, "best": b, "arg": a, "energy": e, "score": s, "omega": w}
