"""Benchmark of the key-redundancy hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2] [--no-cpu-baseline]
                    [--results-dir DIR]
    python bench.py --calibrate-copy        # plain device copy, for counter calibration

One step = one pass of the workload's whole path over one batch of synthetic
heads that is already resident in HBM:

* score workloads (tiny, Llama-3.2-1B 32k -- the default --, long 131k,
  batched 8k): score (norms/energy pass + single-order Gram sweep that takes
  each unordered nonlocal pair once, for both its row and its column, then
  the resolve of column maxima with the fp64 best-twin fixup and the
  discounted score) -> exact-budget select -> repair
  of the selected set (compaction of the retained keys, restricted Gram over
  them for the rows whose unrestricted twin was evicted, orphan/donor
  ranking and swap);
* the Qwen3-4B repair workload (--config 3): repair of a given retained set,
  the top half of each head by an i.i.d. Gumbel score, with no score pass
  and no prior: every row is swept against the K = N/2 retained columns.

Prints one JSON line.  `value` is keys (head positions) through the whole
path per second.  `roofline` is for the dominant kernel (the single-order
score sweep; the restricted repair sweep in the repair workload), timed with
HIP events that the library records around its launch on the stream it runs
on.  Its `achieved` counts the algorithmic work: one d-length dot product
(2d flop) per unordered nonlocal pair in score mode, per (row, retained
column) pair in repair mode; `gram` also gives the rate as if the full N x N
product had been formed (the work a two-sided sweep would execute).
`traffic` is the HBM traffic per launch measured with rocprofv3 counters for
the current kernel source (null when the source has changed since).  The
score phases are `norms_energy`, `score_sweep` and `score_resolve` (column
maxima, exact re-evaluation of near-maximum column candidates, fp64
fixup).  Outside the timed step, `gather_kv` times the packed cache of the
last step's retained set, and in score workloads `variant_score` the keys of
the permuted-count variant, `count_stats` the per-head count statistics
against value-only selection and `allocate` the per-head capacities from the
attention of the last 32 synthetic prefix queries of each KV head (8 KV
heads per layer).

`cpu_baseline` runs before the GPU is touched: the fp64 oracle's whole step
on whole heads (one seeded head per host core, first and last head
included), one head per process with one BLAS thread each, on
min(16, len(os.sched_getaffinity(0))) processes; its value is the keys of
those heads over the pool's wall time.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "keys scored/sec + Gram TFLOP/s (MFMA % of peak) at N=32k, 1 MI355X"
PEAK_BF16_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 dense bf16 flop/clk/CU (published: 2.5 PFLOP/s)
PEAK_HBM_GBS = 8000.0
PEAK_FP64_TFLOPS = 78.6
# the oracle's whole step costs O(N^2 d) fp64 work per head (15-20 s of one
# host core at N = 32768); longer heads get no CPU baseline
CPU_BASELINE_MAX_N = 32768
_CSRC = os.path.join(ROOT, "key_redundancy_scoring_amd", "csrc")
# the sources of each mode's dominant kernel (its HBM counters are kept only
# while these are unchanged)
SOURCES = {"score": [os.path.join(_CSRC, "tri.hip"), os.path.join(_CSRC, "sweep.h")],
           "repair": [os.path.join(_CSRC, "gram.hip"), os.path.join(_CSRC, "sweep.h")]}
# the dominant kernel of each mode per head dim, as the kernel trace names it
SCORE_KERNEL = {64: "tri_sweep_kernel<GramShape<64, 3, 4, 256, 2>>",
                128: "tri_sweep_kernel<GramShape<128, 2, 4, 128, 2>>"}
REPAIR_KERNEL = {64: "gram_kernel<GramShape<64, 2, 4, 128, 3>>",
                 128: "gram_kernel<GramShape<128, 3, 4, 128, 2>>"}

# HBM traffic of one launch of the dominant kernel, from rocprofv3 FETCH_SIZE /
# WRITE_SIZE (KiB per dispatch) scaled by the counters' reading for a plain
# device copy of known size; keyed by the sha256 of the kernel's sources
# (source_hash) at the time the counters were taken, so a changed kernel
# reports null.
MEASURED_TRAFFIC: dict = {
    "eca10f4a3b77fd4116c736015e513f98ad93eba8c54fa33d626df447b9ff6848": {
        "workload": (128, 32768, 64),
        "kernel": "tri_sweep_kernel<GramShape<64, 3, 4, 256, 2>>",
        # FETCH_SIZE 2289442.1 KiB x 1.99994 (a 1 GiB copy reads 524302.7 KiB),
        # WRITE_SIZE 1510389.3 KiB x 1.0 (the same copy writes 1048576 KiB)
        "fetch_bytes": 4688645900,
        "write_bytes": 1546638624,
        "bytes_per_launch": 6235284524,
    },
}


def source_hash(paths) -> str:
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def algorithmic_gram_flops(N: int, d: int, window: int, G: int) -> float:
    """One dot product (2d flop) per unordered pair (i, j) with j - i > w."""
    pairs = max(0, N - window - 1) * max(0, N - window) // 2
    return float(G) * pairs * 2.0 * d


def restricted_gram_flops(N: int, K: int, d: int, G: int) -> float:
    """Repair: every position against the K retained columns (2d flop each)."""
    return float(G) * N * K * 2.0 * d


def _oracle_step(job):
    """The oracle's whole step on one head (runs in a pool worker)."""
    cfg_id, overrides, g, capacity = job
    from threadpoolctl import threadpool_limits

    from oracle import twinkv_oracle as O
    from synth import get_config, gumbel_retained, make_head

    cfg = get_config(cfg_id, **overrides)
    h = make_head(cfg, g)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        if cfg.mode == "repair":
            O.repair_head(O.widen_bf16(h["K"]), gumbel_retained(cfg, g), cfg.tau, cfg.window, cfg.sink, cfg.recent)
        else:
            ref = O.score_head(h["K"], h["V"], cfg.tau, cfg.window)
            keep, _ = O.select_head(ref["score"], ref["energy"], int(capacity), cfg.sink, cfg.recent)
            O.repair_head(O.widen_bf16(h["K"]), keep, cfg.tau, cfg.window, cfg.sink, cfg.recent)
        return time.perf_counter() - t0


def baseline_heads(G: int, count: int, cfg_id: int) -> list:
    """A seeded sample of `count` heads that includes the first and the last."""
    if count >= G:
        return list(range(G))
    rng = np.random.default_rng([cfg_id, 4242])
    mid = rng.choice(np.arange(1, G - 1), size=max(0, count - 2), replace=False)
    return sorted({0, G - 1, *[int(x) for x in mid]})


def cpu_baseline(cfg, overrides: dict, capacities, cores: int | None = None):
    """The fp64 oracle's whole step (as the GPU step: score, select and repair
    of the selection; repair of the Gumbel set in the repair workload) on
    whole heads, one head per host core in a process pool, one BLAS thread
    per process.  Must run before the GPU is initialised (the pool forks)."""
    import concurrent.futures as cf
    import multiprocessing as mp

    affinity = len(os.sched_getaffinity(0))
    cores = min(16, affinity) if cores is None else cores
    heads = baseline_heads(cfg.G, cores, cfg.cfg_id)
    jobs = [(cfg.cfg_id, overrides, g, capacities[g] if capacities is not None else 0) for g in heads]
    t0 = time.perf_counter()
    with cf.ProcessPoolExecutor(max_workers=len(jobs), mp_context=mp.get_context("fork")) as ex:
        per_head = list(ex.map(_oracle_step, jobs))
    wall = time.perf_counter() - t0
    what = "repair of the Gumbel retained set" if cfg.mode == "repair" else \
        "score, select, repair of the selection"
    return {"value": len(heads) * cfg.N / wall, "unit": "keys/s", "cores": len(jobs), "kind": "oracle",
            "sample": f"the oracle's whole step ({what}) of {len(heads)} whole heads at N={cfg.N} "
                      f"(heads {heads[0]}..{heads[-1]}, seeded), one head per process, one BLAS thread each, "
                      f"fp64 numpy; pool wall {wall:.1f} s, per head {min(per_head):.1f}-{max(per_head):.1f} s; "
                      f"{affinity} cores in the affinity mask",
            "heads": heads, "wall_s": wall}


def calibrate_copy():
    """A plain device-to-device copy of 1 GiB, five times, for scaling the
    FETCH_SIZE / WRITE_SIZE counters; the same copies timed (bytes read plus
    written per second: the practical ceiling of a streaming kernel)."""
    import torch

    n = 1 << 30
    a = torch.ones(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    ev[0].record()
    for k in range(5):
        b.copy_(a)
        ev[k + 1].record()
    torch.cuda.synchronize()
    ms = [ev[k].elapsed_time(ev[k + 1]) for k in range(5)]
    best = min(ms[1:])  # the first copy also pages in
    print(json.dumps({"copy_bytes_per_launch": n, "copy_ms": ms,
                      "copy_GBs": 2 * n / (best * 1e-3) / 1e9,
                      "copy_frac_hbm": 2 * n / (best * 1e-3) / 1e9 / PEAK_HBM_GBS}), flush=True)


def _upload_heads(cfg, torch, dev):
    G, N, d = cfg.G, cfg.N, cfg.d
    from synth import make_heads

    K = torch.empty((G, N, d), dtype=torch.int16, device=dev)
    V = torch.empty((G, N, d), dtype=torch.int16, device=dev) if cfg.mode != "repair" else None
    chunk = 32
    for h0 in range(0, G, chunk):
        hs = list(range(h0, min(G, h0 + chunk)))
        k, v, _ = make_heads(cfg, heads=hs, with_values=V is not None)
        K[h0:h0 + len(hs)].copy_(torch.from_numpy(k.view(np.int16)))
        if V is not None:
            V[h0:h0 + len(hs)].copy_(torch.from_numpy(v.view(np.int16)))
    return K, V


def _timed(fn, steps, nev, krs):
    """Run fn(events) `steps` times after one untimed call; average the phase
    times the events bracket."""
    evs = [krs.Events(nev) for _ in range(steps)]
    out = None
    for k in range(steps + 1):
        out = fn(evs[k - 1] if k else None)
    import torch
    torch.cuda.synchronize()
    ms = [float(np.mean([e.elapsed_ms(a, a + 1) for e in evs])) for a in range(nev - 1)]
    for e in evs:
        e.close()
    return out, ms


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--heads", type=int, default=None, help="override the head count (default: the workload's)")
    ap.add_argument("--results-dir", default=None, help="also write the line to DIR/<workload>.bench.json")
    ap.add_argument("--calibrate-copy", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU: every (batch, layer, KV head) is independent, so N GPUs would each run "
              "this same path on G/N of the heads with no communication. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return

    from synth import dirichlet_capacities, get_config, gumbel_retained

    overrides = {"G": args.heads} if args.heads else {}
    cfg = get_config(args.config, **overrides)
    G, N, d = cfg.G, cfg.N, cfg.d
    repair_mode = cfg.mode == "repair"
    if repair_mode:
        cap_list = None
    elif cfg.removal is not None:
        cap_list = [int(np.floor(N * (1.0 - cfg.removal)))] * G
    else:
        cap_list = [int(c) for c in dirichlet_capacities(cfg)]

    # the oracle on the host cores first, before anything initialises the GPU
    cpu = None
    cpu_note = None
    if not args.no_cpu_baseline:
        if N > CPU_BASELINE_MAX_N:
            cpu_note = (f"not run: the oracle's step is O(N^2 d) fp64 work per head, so one whole head at N={N} "
                        f"costs {(N / CPU_BASELINE_MAX_N) ** 2:.0f}x an N={CPU_BASELINE_MAX_N} head (15-20 s on one "
                        f"host core), several minutes")
        else:
            cpu = cpu_baseline(cfg, overrides, cap_list)
            print(f"# cpu baseline: {cpu['sample']}", file=sys.stderr, flush=True)

    import torch

    import key_redundancy_scoring_amd as krs

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a ROCm GPU")
    dev = torch.device("cuda:0")

    t0 = time.perf_counter()
    K, V = _upload_heads(cfg, torch, dev)
    S0 = None
    if repair_mode:
        S0 = torch.from_numpy(np.stack([gumbel_retained(cfg, g) for g in range(G)])).to(dev)
    torch.cuda.synchronize()
    gen_s = time.perf_counter() - t0
    print(f"# generated and uploaded {G} heads in {gen_s:.1f} s", file=sys.stderr, flush=True)

    s_out, sel_out, rep_out = {}, {}, {}
    s_ws = r_ws = None
    if not repair_mode:
        caps = torch.tensor(cap_list, dtype=torch.int32, device=dev)
        offsets = krs.capacity_offsets(cap_list, N)
        offsets_dev = krs.capacity_offsets_device(caps, N)

    def step(ev_s=None, ev_sel=None, ev_r=None):
        nonlocal s_ws, r_ws
        if repair_mode:
            rp = krs.repair(K, S0, cfg.tau, cfg.window, cfg.sink, cfg.recent, out=rep_out, ws=r_ws, events=ev_r)
        else:
            r = krs.score(K, V, cfg.tau, cfg.window, cfg.sink, cfg.recent, out=s_out, ws=s_ws, events=ev_s)
            s_ws = r["ws"]
            s_out.update({k: r[k] for k in ("count", "best_sim", "best_idx", "energy", "score")})
            sl = krs.select(r["score"], r["energy"], caps, cfg.sink, cfg.recent, out=sel_out, events=ev_sel,
                            offsets=offsets_dev, total=int(offsets[-1]))
            sel_out.update({"keep": sl["keep"], "kept_idx": sl["kept_idx"]})
            rp = krs.repair(K, sl["keep"], cfg.tau, cfg.window, cfg.sink, cfg.recent, prior=r, out=rep_out,
                            ws=r_ws, events=ev_r)
        r_ws = rp["ws"]
        rep_out.update({k: rp[k] for k in ("keep", "best_sim", "best_idx", "n_orphans", "n_donors", "n_swaps",
                                           "pairs")})

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [(krs.Events(4), krs.Events(2), krs.Events(5)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        if repair_mode:
            step(ev_r=evs[k][2])
        else:
            step(*evs[k])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps

    def avg(fn):
        return float(np.mean([fn(e) for e in evs]))

    phases = {}
    if not repair_mode:
        phases["norms_energy"] = avg(lambda e: e[0].elapsed_ms(0, 1))
        phases["score_sweep"] = avg(lambda e: e[0].elapsed_ms(1, 2))
        phases["score_resolve"] = avg(lambda e: e[0].elapsed_ms(2, 3))
        phases["select"] = avg(lambda e: e[1].elapsed_ms(0, 1))
    phases["repair_norms"] = avg(lambda e: e[2].elapsed_ms(0, 1))
    phases["repair_compact"] = avg(lambda e: e[2].elapsed_ms(1, 2))
    phases["repair_gram"] = avg(lambda e: e[2].elapsed_ms(2, 3))
    phases["repair_swap"] = avg(lambda e: e[2].elapsed_ms(3, 4))
    for e in evs:
        for x in e:
            x.close()

    # retained-set sizes of the repair's input, and the rows its sweep visits
    if repair_mode:
        kept_in = S0.sum(1, dtype=torch.int64).cpu().numpy()
        swept_frac = 1.0
    else:
        kept_in = np.asarray(cap_list, dtype=np.int64)
        bi = s_out["best_idx"].long()
        reused = (bi < 0) | torch.gather(sel_out["keep"], 1, bi.clamp(min=0)).bool()
        swept_frac = 1.0 - reused.float().mean().item()
    rgram = float(sum(2.0 * N * int(k) * d for k in kept_in))  # every row against the retained columns

    # packed cache of the last step's retained set S1 (not part of the timed step)
    s1_counts = rep_out["keep"].sum(1, dtype=torch.int32)
    s1_total = int(kept_in.sum())  # repair keeps each head's budget
    s1_off = krs.capacity_offsets_device(s1_counts, N)
    s1_sel = krs.select(rep_out["keep"].double(), rep_out["keep"].double(), s1_counts, 0, 0, offsets=s1_off,
                        total=s1_total)  # S1's positions in order: every kept entry scores 1, the rest 0
    gout = {}

    def gather(ev):
        nonlocal gout
        r = krs.gather_kv(K, V, s1_sel["kept_idx"], s1_off, total=s1_total, out=gout, events=ev)
        gout = {"keys": r["keys"], "values": r["values"]}
        return r

    gres, (gather_ms,) = _timed(gather, args.steps, 2, krs)
    gather_bytes = gres["total"] * ((8 if V is not None else 4) * d + 4)
    del s1_sel, gout

    extras = {}
    if not repair_mode:
        extras = _score_extras(cfg, args, krs, torch, dev, K, s_out, sel_out, caps, cap_list, offsets_dev, offsets)

    if repair_mode:
        dom_ms = phases["repair_gram"]
        alg = rgram
        kernel = REPAIR_KERNEL[d]
    else:
        dom_ms = phases["score_sweep"]
        alg = algorithmic_gram_flops(N, d, cfg.window, G)
        kernel = SCORE_KERNEL[d]
    achieved = alg / (dom_ms * 1e-3) / 1e12

    traffic = None
    meas = MEASURED_TRAFFIC.get(source_hash(SOURCES["repair" if repair_mode else "score"]))
    if meas is not None and meas.get("workload") == (G, N, d) and meas.get("kernel") == kernel:
        traffic = meas["bytes_per_launch"]

    twin = int(round(cfg.twin_frac * 100))
    if repair_mode:
        budget = "repair of the top half by a random per-token Gumbel score (no score pass, no prior)"
    elif cfg.removal is not None:
        budget = f"{int(round(cfg.removal * 100))}% removal; score + select + repair of the selected set"
    else:
        budget = (f"Dirichlet(1) split of a {int(round(cfg.budget_frac * 100))}% budget per group of {cfg.group} "
                  f"heads; score + select + repair of the selected set")
    line = {
        "metric": METRIC,
        "value": G * N / (ms_per_step * 1e-3),
        "unit": "keys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {G} heads x N={N} x d={d}, {twin}% planted twins, tau {cfg.tau}, "
                               f"window {cfg.window}, {budget}",
                   "G": G, "N": N, "d": d, "tau": cfg.tau, "window": cfg.window, "sink": cfg.sink,
                   "recent": cfg.recent, "mean_retained": float(np.mean(kept_in)), "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic, "kernel": kernel,
                     "algorithmic_flop_per_launch": alg, "avg_launch_ms": dom_ms},
        "phases_ms": phases,
        "phase_rates": {"repair_gram_tflops_on_swept_rows": rgram * swept_frac / (phases["repair_gram"] * 1e-3) / 1e12,
                        "repair_rows_swept_frac": swept_frac},
        "gather_kv": {"ms": gather_ms, "rows": gres["total"], "algorithmic_bytes": gather_bytes,
                      "GBs": gather_bytes / (gather_ms * 1e-3) / 1e9,
                      "frac_hbm": gather_bytes / (gather_ms * 1e-3) / 1e9 / PEAK_HBM_GBS},
        "swaps_total": int(rep_out["n_swaps"].sum().item()),
        "generation_s": gen_s,
    }
    if not repair_mode:
        dense = 2.0 * G * N * N * d
        line["gram"] = {"dense_equiv_tflops": dense / (dom_ms * 1e-3) / 1e12,
                        "mfma_frac_dense_equiv": dense / (dom_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                        "keys_per_s": G * N / (dom_ms * 1e-3), "ms": dom_ms}
        norms_bytes = G * N * (4 * d + 20)
        line["phase_rates"]["norms_energy_GBs"] = norms_bytes / (phases["norms_energy"] * 1e-3) / 1e9
        line.update(extras)
    if cpu is not None:
        line["cpu_baseline"] = {k: cpu[k] for k in ("value", "unit", "cores", "kind", "sample")}
    elif cpu_note is not None:
        line["cpu_baseline"] = None
        line["cpu_baseline_note"] = cpu_note
    print(json.dumps(line), flush=True)
    if args.results_dir:
        os.makedirs(args.results_dir, exist_ok=True)
        with open(os.path.join(args.results_dir, f"{cfg.name}.bench.json"), "w") as f:
            json.dump(line, f, indent=1)


def _score_extras(cfg, args, krs, torch, dev, K, s_out, sel_out, caps, cap_list, offsets_dev, offsets):
    """Untimed-step extras of the score workloads: permuted-count variant
    keys, count statistics, head allocation."""
    G, N, d = cfg.G, cfg.N, cfg.d
    from synth import count_permutation, make_queries

    permd = torch.from_numpy(np.stack([count_permutation(cfg, g, cap_list[g], 11) for g in range(G)])).to(dev)
    vout = {}

    def variant(ev):
        nonlocal vout
        vout = krs.variant_score(s_out["count"], s_out["energy"], "twin", perm=permd, out=vout, events=ev)
        return vout

    _, (variant_ms,) = _timed(variant, args.steps, 2, krs)
    variant_bytes = G * N * (4 + 8 + 4 + 4 + 16)  # perm, energy, own and permuted count, score and tie
    del permd, vout

    vsel = krs.select(s_out["energy"], s_out["energy"], caps, cfg.sink, cfg.recent, offsets=offsets_dev,
                      total=int(offsets[-1]))

    def stats(ev):
        return krs.count_stats(s_out["count"], s_out["energy"], caps, cfg.sink, cfg.recent,
                               keep_twin=sel_out["keep"], keep_value=vsel["keep"], events=ev)

    sres, (stats_ms,) = _timed(stats, args.steps, 2, krs)
    st_np = sres["stats"].cpu().numpy()
    stats_bytes = G * N * (4 + 8 + 1 + 1) * 2  # count, energy and both masks, read twice
    del vsel

    Qh = torch.from_numpy(np.stack([make_queries(cfg, g) for g in range(G)]).view(np.int16)).to(dev)
    Hkv = 8 if G % 8 == 0 else 1
    B_alloc = krs.uniform_capacity(N, cfg.removal if cfg.removal is not None else 0.5)
    aout, aws = {}, None

    def alloc(ev):
        nonlocal aout, aws
        r = krs.allocate(K, Qh, Hkv, B_alloc, cfg.sink, cfg.recent, out=aout, ws=aws, events=ev)
        aws = r["ws"]
        aout = {kk: r[kk] for kk in ("capacity", "g_count", "z")}
        return r

    _, alloc_ms = _timed(alloc, args.steps, 4, krs)
    nq = Qh.shape[1] * Qh.shape[2]
    logit_flops = 2.0 * G * nq * N * d  # one fp64 dot product per (query, key)
    del Qh, aws
    return {
        "variant_score": {"ms": variant_ms, "variant": "twin with permuted counts (seed 11)",
                          "GBs": variant_bytes / (variant_ms * 1e-3) / 1e9,
                          "frac_hbm": variant_bytes / (variant_ms * 1e-3) / 1e9 / PEAK_HBM_GBS},
        "count_stats": {"ms": stats_ms, "GBs": stats_bytes / (stats_ms * 1e-3) / 1e9,
                        "twin_fraction": float(st_np[:, 1].sum() / st_np[:, 0].sum()),
                        "selection_change_vs_value_only": float(st_np[:, 9].sum() / max(1, st_np[:, 8].sum()))},
        "allocate": {"ms": sum(alloc_ms), "stats_ms": alloc_ms[0], "aggregate_pool_ms": alloc_ms[1],
                     "rank_eq5_ms": alloc_ms[2], "heads_per_layer": Hkv, "queries_per_head": nq,
                     "logit_fp64_tflops": logit_flops / (alloc_ms[0] * 1e-3) / 1e12,
                     "frac_fp64_peak": logit_flops / (alloc_ms[0] * 1e-3) / 1e12 / PEAK_FP64_TFLOPS},
    }


if __name__ == "__main__":
    main()
