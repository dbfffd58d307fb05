"""Oracle results of the five synthetic workloads on seeded head subsets,
stored for the GPU tests (tests/test_gpu_goldens.py).

    python tests/golden/make_oracle_goldens.py [--configs 1 2 3 4 5] [--procs 8]

Writes tests/golden/oracle_<workload>.json.  TEST INFRASTRUCTURE: this script
calls only ``oracle/`` (the fp64 CPU oracle) and ``synth/`` (the seeded input
generator); no value in its output comes from the HIP library.  It runs on
the CPU, one head per process with one BLAS thread each.

Per checked head it records, for the workload's path (score -> select ->
repair of the selection, or repair of the Gumbel retained set for the
Qwen3-4B workload):

* the sha256 of the head's keys and values (bf16 bits), so a test confirms
  it regenerated the same inputs;
* counts and best-twin positions as sha256 digests of 8192-row chunks (int32
  little-endian), with the rows that the parity rules exclude masked on both
  sides: a count whose row has a pair inside the tau band is replaced by -1
  (the band itself is stored), a best-twin position whose row has a
  near-tie is replaced by -2 (its candidates are stored);
* the keep mask (np.packbits) digest, the capacity and the relative score gap
  at the selection boundary;
* for the repair: |O|, |D|, m, the digests of b(S0)'s positions (masked the
  same way), of S1 and of the swap pairs, and per near-tie row whether it is
  an orphan or donor and whether its b is within 2 * NEAR_TIE of tau;
* a few sampled rows in plain numbers, for diagnostics.

Exclusion rules (the same as tests/parity.py): a pair with |sim - tau| <
BAND is in the tau band; a row is a near-tie when some eligible position's
similarity lies strictly below its maximum by less than NEAR_TIE, and its
candidates are all eligible positions within NEAR_TIE of the maximum.
Workloads, head subsets (seeded; always the first and the last head):
tiny 1 of 1, Llama-3.2-1B 32k all 128, Qwen3-4B 32 of 288, long 131k 8 of 256,
batched 8k 128 of 2048.
"""
from __future__ import annotations

import os

if __name__ == "__main__":  # one BLAS thread per worker process (set before numpy loads)
    for _v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[_v] = "1"

import argparse  # noqa: E402
import concurrent.futures as cf  # noqa: E402
import hashlib  # noqa: E402
import json  # noqa: E402
import sys  # noqa: E402
import time  # noqa: E402

import numpy as np  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from oracle import twinkv_oracle as O  # noqa: E402
from synth import dirichlet_capacities, get_config, gumbel_retained, make_head  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))
BAND = 1e-3
NEAR_TIE = 2e-5
CHUNK = 8192
SUBSET = {1: 1, 2: 128, 3: 32, 4: 8, 5: 128}
SAMPLES = 24


def golden_path(cfg_id: int) -> str:
    return os.path.join(HERE, f"oracle_{get_config(cfg_id).name}.json")


def checked_heads(cfg_id: int) -> list:
    """The seeded head subset of a workload (first and last head included)."""
    cfg = get_config(cfg_id)
    k = min(SUBSET[cfg_id], cfg.G)
    if k >= cfg.G:
        return list(range(cfg.G))
    rng = np.random.default_rng([cfg.seed, cfg_id, 7919])
    mid = rng.choice(np.arange(1, cfg.G - 1), size=k - 2, replace=False)
    return sorted({0, cfg.G - 1, *[int(x) for x in mid]})


def digest(a) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()[:32]


def chunk_digests(a) -> list:
    a = np.ascontiguousarray(np.asarray(a), dtype="<i4")
    return [digest(a[s:s + CHUNK]) for s in range(0, a.shape[0], CHUNK)]


def mask_rows(a, rows, fill):
    out = np.array(a, dtype=np.int64, copy=True)
    if len(rows):
        out[np.asarray(rows, dtype=np.int64)] = fill
    return out


def input_digest(Kbits, Vbits) -> str:
    return hashlib.sha256(np.ascontiguousarray(Kbits).tobytes() + np.ascontiguousarray(Vbits).tobytes()).hexdigest()


def exclusions(K, n, cols, tau, window, budget_elems=1 << 24):
    """Tau-band rows {row: [c_lo, band]} (when tau is given) and near-tie rows
    {row: [candidates]} of every row against the columns ``cols``."""
    N = K.shape[0]
    band, near = {}, {}
    if cols.size == 0:
        return band, near
    step = max(1, budget_elems // cols.size)
    for s in range(0, N, step):
        grp = np.arange(s, min(N, s + step))
        sims = O.cosine_rows(K, n, grp, cols)
        ok = O.nonlocal_mask(grp, cols, window)
        if tau is not None:
            inb = ok & (np.abs(sims - tau) < BAND)
            nb = inb.sum(1)
            for r in np.flatnonzero(nb):
                c_lo = int((ok[r] & (sims[r] > tau) & ~inb[r]).sum())
                band[int(grp[r])] = [c_lo, int(nb[r])]
        masked = np.where(ok, sims, -np.inf)
        best = masked.max(1)
        close = ok & (masked >= best[:, None] - NEAR_TIE) & (masked < best[:, None])
        for r in np.flatnonzero(close.any(1)):
            cand = ok[r] & (masked[r] >= best[r] - NEAR_TIE)
            near[int(grp[r])] = [int(j) for j in cols[cand]]
    return band, near


def repair_record(K, n, S0, cfg):
    rr = O.repair_head(K, S0, cfg.tau, cfg.window, cfg.sink, cfg.recent)
    cols = np.flatnonzero(np.asarray(S0) != 0)
    _, near = exclusions(K, n, cols, None, cfg.window)
    in_od = np.zeros(K.shape[0], bool)
    in_od[rr["orphans"]] = True
    in_od[rr["donors"]] = True
    near_info = {str(r): {"cand": c, "in_od": bool(in_od[r]),
                          "near_tau": bool(abs(rr["best"][r] - cfg.tau) < 2 * NEAR_TIE)} for r, c in near.items()}
    return {
        "K": int(cols.size), "n_orphans": rr["n_orphans"], "n_donors": rr["n_donors"], "m": rr["m"],
        "arg_chunks": chunk_digests(mask_rows(rr["arg"], list(near), -2)),
        "keep": digest(np.packbits(rr["keep"].astype(np.uint8))),
        "pairs": digest(np.ascontiguousarray(rr["pairs"], dtype="<i4")),
        "near_tie": near_info,
    }


def head_record(cfg_id: int, g: int, capacity: int | None):
    cfg = get_config(cfg_id)
    t0 = time.perf_counter()
    h = make_head(cfg, g)
    K = O.widen_bf16(h["K"])
    n = O.squared_norms(K)
    rec = {"head": g, "inputs": input_digest(h["K"], h["V"])}
    rng = np.random.default_rng([cfg_id, g, 31])
    rows = np.unique(np.concatenate([[0, cfg.N - 1], rng.choice(cfg.N, SAMPLES, replace=False)]))
    if cfg.mode == "repair":
        S0 = gumbel_retained(cfg, g)
        rec["repair"] = repair_record(K, n, S0, cfg)
    else:
        c, b, a = O.twin_count_and_best(K, cfg.tau, cfg.window, n=n)
        e = O.value_energy(O.widen_bf16(h["V"]))
        s, _ = O.frequency_score(e, c, cfg.N)
        band, near = exclusions(K, n, np.arange(cfg.N), cfg.tau, cfg.window)
        keep, _ = O.select_head(s, e, capacity, cfg.sink, cfg.recent)
        rec.update({
            "capacity": int(capacity),
            "count_chunks": chunk_digests(mask_rows(c, list(band), -1)),
            "arg_chunks": chunk_digests(mask_rows(a, list(near), -2)),
            "band": {str(r): v for r, v in band.items()},
            "near_tie": {str(r): v for r, v in near.items()},
            "keep": digest(np.packbits(keep)),
            "boundary_gap": _boundary_gap(s, e, capacity, cfg.sink, cfg.recent),
            "samples": [[int(r), int(c[r]), int(a[r]), float(b[r])] for r in rows],
        })
        rec["repair"] = repair_record(K, n, keep, cfg)
    rec["seconds"] = round(time.perf_counter() - t0, 1)
    return rec


def _boundary_gap(score, energy, capacity, sink, recent):
    """Relative score gap at the kept/evicted boundary of the oracle's ranking
    (a string "inf" when nothing is cut or the boundary is an exact tie)."""
    N = score.shape[0]
    s_cnt, r_cnt = O.protected_counts(capacity, sink, recent)
    u = capacity - s_cnt - r_cnt
    cand = np.arange(s_cnt, N - r_cnt)
    if u <= 0 or u >= cand.size:
        return "inf"
    order = np.lexsort((cand, -energy[cand], -score[cand]))
    a, b = score[cand[order[u - 1]]], score[cand[order[u]]]
    if a == b:
        return "inf"
    return float(abs(a - b) / max(abs(a), abs(b), 1e-300))


def capacities(cfg_id: int):
    cfg = get_config(cfg_id)
    if cfg.mode == "repair":
        return [None] * cfg.G
    if cfg.removal is not None:
        return [O.uniform_budget(cfg.N, cfg.removal)] * cfg.G
    return [int(x) for x in dirichlet_capacities(cfg)]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--configs", type=int, nargs="*", default=[1, 2, 3, 4, 5])
    ap.add_argument("--procs", type=int, default=8)
    args = ap.parse_args()
    jobs = []
    for cfg_id in args.configs:
        caps = capacities(cfg_id)
        jobs += [(cfg_id, g, caps[g]) for g in checked_heads(cfg_id)]
    # the longest heads first, so the pool drains evenly
    jobs.sort(key=lambda j: -get_config(j[0]).N * get_config(j[0]).d)
    results = {c: [] for c in args.configs}
    t0 = time.perf_counter()
    with cf.ProcessPoolExecutor(max_workers=args.procs) as ex:
        futs = {ex.submit(head_record, *j): j for j in jobs}
        for k, f in enumerate(cf.as_completed(futs), 1):
            cfg_id, g, _ = futs[f]
            rec = f.result()
            results[cfg_id].append(rec)
            print(f"[{k}/{len(jobs)}] workload {cfg_id} head {g}: {rec['seconds']} s "
                  f"(elapsed {time.perf_counter() - t0:.0f} s)", flush=True)
    for cfg_id, recs in results.items():
        cfg = get_config(cfg_id)
        out = {
            "workload": cfg.name, "cfg_id": cfg_id, "G": cfg.G, "N": cfg.N, "d": cfg.d, "tau": cfg.tau,
            "window": cfg.window, "sink": cfg.sink, "recent": cfg.recent, "mode": cfg.mode,
            "removal": cfg.removal, "band": BAND, "near_tie": NEAR_TIE, "chunk": CHUNK,
            "heads": sorted(recs, key=lambda r: r["head"]),
        }
        with open(golden_path(cfg_id), "w") as f:
            json.dump(out, f, separators=(",", ":"))
        print(f"wrote {golden_path(cfg_id)}", flush=True)


if __name__ == "__main__":
    main()
