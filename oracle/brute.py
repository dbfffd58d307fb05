"""Pure-Python brute force for tiny heads.

TEST INFRASTRUCTURE ONLY (same rule as ``twinkv_oracle``).  It evaluates the
same definitions element by element with ``math.fsum`` and explicit loops, and
checks selections by exhaustive search over subsets, so the vectorised oracle
can be compared against an evaluation that shares none of its array code.

Sources: [P1] "TwinKV: A Composable Repair Pass for KV Cache Eviction via
Pairwise Key Redundancy", section 3.2 (Eq. 1, Eq. 2) and section 3.4 (Eq. 4);
[P2] "Small Frequency Corrections Can Change What Survives KV Cache
Compression", sections 3.1, 3.2 and 3.4.
"""
from __future__ import annotations

import itertools
import math


def _sim(ki, kj):
    ni = math.fsum(x * x for x in ki)
    nj = math.fsum(x * x for x in kj)
    if ni * nj == 0.0:
        return 0.0
    return math.fsum(a * b for a, b in zip(ki, kj)) / math.sqrt(ni * nj)


def twin_stats(keys, tau, window, allowed=None):
    """keys: list of lists of floats.  Returns per-row (count, best, arg) where
    count uses every nonlocal j, and best/arg range over nonlocal j that are
    also in ``allowed`` (all positions when None)."""
    N = len(keys)
    out = []
    for i in range(N):
        c = 0
        best, arg = -1.0, -1
        for j in range(N):
            if abs(i - j) <= window:
                continue
            s = _sim(keys[i], keys[j])
            if s > tau:
                c += 1
            if allowed is not None and not allowed[j]:
                continue
            if arg < 0 or s > best:
                best, arg = s, j
        out.append((c, best, arg))
    return out


def score(e, c, N):
    return e * math.log((N + 1.0) / (c + 1.0))


def select_exhaustive(scores, energies, capacity, sink, recent):
    """Keep set by exhaustive search: among all subsets of the unprotected
    positions with the right size, the retained one is the subset whose
    members, listed best-first by (score desc, energy desc, position asc), form
    the lexicographically greatest sequence.  Only for tiny N."""
    N = len(scores)
    s = min(sink, capacity)
    r = min(recent, capacity - s)
    prot = set(range(s)) | set(range(N - r, N))
    cand = [i for i in range(N) if i not in prot]
    u = capacity - s - r

    def key(i):
        return (scores[i], energies[i], -i)

    best = None
    for sub in itertools.combinations(cand, u):
        seq = sorted((key(i) for i in sub), reverse=True)
        if best is None or seq > best[0]:
            best = (seq, sub)
    keep = sorted(prot | set(best[1] if best else ()))
    return keep


def repair(keys, retained, tau, window, sink, recent):
    """Loop form of the one-shot repair pass."""
    N = len(keys)
    S0 = [bool(x) for x in retained]
    K = sum(S0)
    stats = twin_stats(keys, tau, window, allowed=S0)
    b = [st[1] for st in stats]
    s = min(sink, K)
    r = min(recent, K - s)
    prot = set(range(s)) | set(range(N - r, N))
    orphans = sorted((i for i in range(N) if not S0[i] and b[i] < tau), key=lambda i: (b[i], i))
    donors = sorted((j for j in range(N) if S0[j] and j not in prot and b[j] >= tau), key=lambda j: (-b[j], j))
    m = min(len(orphans), len(donors))
    S1 = list(S0)
    for k in range(m):
        S1[donors[k]] = False
        S1[orphans[k]] = True
    return {"keep": S1, "best": b, "orphans": orphans, "donors": donors, "m": m,
            "pairs": [(orphans[k], donors[k]) for k in range(m)]}
