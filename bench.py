"""Benchmark of the key-redundancy hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2] [--no-cpu-baseline]
    python bench.py --calibrate-copy        # plain device copy, for counter calibration

One step = one pass of the whole path over one batch of synthetic heads that
is already resident in HBM: score (norms/energy pass + fused Gram sweep with
the fp64 best-twin fixup and the discounted score) -> exact-budget select ->
repair of the selected set (compaction of the retained keys, restricted Gram
over them, orphan/donor ranking and swap).  The default workload is the
Llama-3.2-1B shape: 16 layers x 8 KV heads = 128 heads, N = 32768, head dim
64, 10% planted near-duplicates, tau 0.9, window 64, 4 sinks, 64 recent, 50%
removal.

Prints one JSON line.  `value` is keys (head positions) through the whole path
per second.  `gather_kv` times, outside the step, the packed cache of the
last step's selection (retained keys and values in sequence order),
`variant_score` the keys of the permuted-count variant, `count_stats` the
per-head count statistics against value-only selection, and `allocate` the per-head capacities from the attention of the last 32
synthetic prefix queries of each KV head (8 KV heads per layer).  `roofline` is for the dominant kernel, the score-mode Gram
sweep, timed with HIP events that the library records around its launch on
the stream it runs on; its `achieved` counts the algorithmic work, one
d-length dot product (2d flop) per unordered nonlocal pair, while `gram`
also gives the dense-equivalent rate (both orders of every pair, the work the
sweep executes).  `traffic` is the HBM traffic per launch measured with
rocprofv3 counters for the current Gram source (null when the source has
changed since).  `cpu_baseline` times the fp64 oracle's whole step (score,
select, repair of the selection) on whole heads of the same workload, on the
host, for about `--cpu-seconds` (at least one head).
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
GRAM_SOURCE = os.path.join(ROOT, "key_redundancy_scoring_amd", "csrc", "gram.hip")
# launch shape of the score-mode sweep per head dim, as the kernel trace names it
SCORE_SHAPE = {64: "GramShape<64, 4, 4, 256, 2>", 128: "GramShape<128, 2, 4, 128, 2>"}

# HBM traffic of one score-mode Gram launch on the default workload, from
# rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB per dispatch) scaled by the counters'
# reading for a plain device copy of known size; keyed by the sha256 of the
# Gram source the counters were taken on.
MEASURED_TRAFFIC: dict = {
    "8e228c205b2f4f0945eb331799a250fe6168612366bc8425fb4467f59077fa47": {
        "workload": (128, 32768, 64),
        # FETCH_SIZE 1875232.2 KiB x 1.99994 (a 1 GiB copy reads 524302.6 KiB),
        # WRITE_SIZE 114688.0 KiB x 1.0 (the same copy writes 1048576 KiB)
        "fetch_bytes": 3840368895,
        "write_bytes": 117440512,
        "bytes_per_launch": 3957809407,
    },
}


def source_hash(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def algorithmic_gram_flops(N: int, d: int, window: int, G: int) -> float:
    """One dot product (2d flop) per unordered pair (i, j) with j - i > w."""
    pairs = max(0, N - window - 1) * max(0, N - window) // 2
    return float(G) * pairs * 2.0 * d


def restricted_gram_flops(N: int, K: int, d: int, G: int) -> float:
    """Repair: every position against the K retained columns (2d flop each)."""
    return float(G) * N * K * 2.0 * d


def cpu_baseline(cfg, seconds: float, capacities):
    """The oracle's whole step (score, select and repair of the selection:
    count, best nonlocal twin, energy and score of every row against all N
    positions, the exact-budget selection, then the best surviving twin of
    every row against the retained set and the swap) on whole heads 0, 1, ...
    until about `seconds` of host time are spent (at least one head); timed
    on the host.  The same work per key as the GPU step."""
    from threadpoolctl import threadpool_info

    from oracle import twinkv_oracle as O
    from synth import make_head

    done, spent, g = 0, 0.0, 0
    while (spent < seconds or g == 0) and g < cfg.G:
        h = make_head(cfg, g)
        t0 = time.perf_counter()
        ref = O.score_head(h["K"], h["V"], cfg.tau, cfg.window)
        keep, _ = O.select_head(ref["score"], ref["energy"], int(capacities[g]), cfg.sink, cfg.recent)
        O.repair_head(O.widen_bf16(h["K"]), keep, cfg.tau, cfg.window, cfg.sink, cfg.recent)
        spent += time.perf_counter() - t0
        done += cfg.N
        g += 1
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": done / spent, "unit": "keys/s", "cores": int(threads), "kind": "oracle",
            "sample": f"the whole step (score, select, repair of the selection) of head{'s 0..' if g > 1 else ' '}"
                      f"{g - 1} at N={cfg.N}, fp64 numpy/BLAS, {spent:.1f} s"}


def calibrate_copy():
    """A plain device-to-device copy of 1 GiB, five times, for scaling the
    FETCH_SIZE / WRITE_SIZE counters."""
    import torch

    n = 1 << 30
    a = torch.ones(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=8.0)
    ap.add_argument("--heads", type=int, default=None, help="override the head count (default: the workload's)")
    ap.add_argument("--calibrate-copy", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU: every (batch, layer, KV head) is independent, so N GPUs would each run "
              "this same path on G/N of the heads with no communication. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return

    import torch

    import key_redundancy_scoring_amd as krs
    from synth import dirichlet_capacities, get_config, make_heads

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a ROCm GPU")
    dev = torch.device("cuda:0")
    cfg = get_config(args.config)
    if args.heads:
        cfg = cfg.with_(G=args.heads)
    G, N, d = cfg.G, cfg.N, cfg.d

    t0 = time.perf_counter()
    K = torch.empty((G, N, d), dtype=torch.int16, device=dev)
    V = torch.empty((G, N, d), dtype=torch.int16, device=dev)
    chunk = 32
    for h0 in range(0, G, chunk):
        hs = list(range(h0, min(G, h0 + chunk)))
        k, v, _ = make_heads(cfg, heads=hs)
        K[h0:h0 + len(hs)].copy_(torch.from_numpy(k.view(np.int16)))
        V[h0:h0 + len(hs)].copy_(torch.from_numpy(v.view(np.int16)))
    torch.cuda.synchronize()
    gen_s = time.perf_counter() - t0
    print(f"# generated and uploaded {G} heads in {gen_s:.1f} s", file=sys.stderr, flush=True)

    if cfg.removal is not None:
        cap_list = [krs.uniform_capacity(N, cfg.removal)] * G
    else:
        cap_list = [int(c) for c in dirichlet_capacities(cfg)]
    caps = torch.tensor(cap_list, dtype=torch.int32, device=dev)
    offsets = krs.capacity_offsets(cap_list, N)
    offsets_dev = krs.capacity_offsets_device(caps, N)
    s_out, sel_out, rep_out = {}, {}, {}
    s_ws = r_ws = None

    def step(ev_s=None, ev_sel=None, ev_r=None):
        nonlocal s_ws, r_ws
        r = krs.score(K, V, cfg.tau, cfg.window, cfg.sink, cfg.recent, out=s_out, ws=s_ws, events=ev_s)
        s_ws = r["ws"]
        s_out.update({k: r[k] for k in ("count", "best_sim", "best_idx", "energy", "score")})
        sl = krs.select(r["score"], r["energy"], caps, cfg.sink, cfg.recent, out=sel_out, events=ev_sel,
                        offsets=offsets_dev, total=int(offsets[-1]))
        sel_out.update({"keep": sl["keep"], "kept_idx": sl["kept_idx"]})
        rp = krs.repair(K, sl["keep"], cfg.tau, cfg.window, cfg.sink, cfg.recent, prior=r, out=rep_out, ws=r_ws,
                        events=ev_r)
        r_ws = rp["ws"]
        rep_out.update({k: rp[k] for k in ("keep", "best_sim", "best_idx", "n_orphans", "n_donors", "n_swaps",
                                           "pairs")})

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [(krs.Events(3), krs.Events(2), krs.Events(5)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(*evs[k])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps

    def avg(fn):
        return float(np.mean([fn(e) for e in evs]))

    norms_ms = avg(lambda e: e[0].elapsed_ms(0, 1))
    gram_ms = avg(lambda e: e[0].elapsed_ms(1, 2))
    select_ms = avg(lambda e: e[1].elapsed_ms(0, 1))
    r_norms_ms = avg(lambda e: e[2].elapsed_ms(0, 1))
    r_compact_ms = avg(lambda e: e[2].elapsed_ms(1, 2))
    r_gram_ms = avg(lambda e: e[2].elapsed_ms(2, 3))
    r_swap_ms = avg(lambda e: e[2].elapsed_ms(3, 4))
    for e in evs:
        for x in e:
            x.close()

    # packed cache of the last step's selection (not part of the timed step)
    gev = [krs.Events(2) for _ in range(args.steps)]
    gout = {}
    for k in range(args.steps + 1):
        gres = krs.gather_kv(K, V, sel_out["kept_idx"], offsets_dev, total=int(offsets[-1]), out=gout,
                             events=gev[k - 1] if k else None)
        gout = {"keys": gres["keys"], "values": gres["values"]}
    torch.cuda.synchronize()
    gather_ms = float(np.mean([e.elapsed_ms(0, 1) for e in gev]))
    for e in gev:
        e.close()
    gather_rows = gres["total"]
    gather_bytes = gather_rows * (8 * d + 4)

    # score-variant keys (permuted counts, seed 11) for the last step's counts
    from synth import count_permutation
    permd = torch.from_numpy(np.stack([count_permutation(cfg, g, cap_list[g], 11) for g in range(G)])).to(dev)
    vev = [krs.Events(2) for _ in range(args.steps)]
    vout = {}
    for k in range(args.steps + 1):
        vres = krs.variant_score(s_out["count"], s_out["energy"], "twin", perm=permd, out=vout,
                                 events=vev[k - 1] if k else None)
        vout = vres
    torch.cuda.synchronize()
    variant_ms = float(np.mean([e.elapsed_ms(0, 1) for e in vev]))
    for e in vev:
        e.close()
    variant_bytes = G * N * (4 + 8 + 4 + 4 + 16)  # perm, energy, own and permuted count, score and tie
    del permd, vout, vres

    # count statistics of the last step (Twin selection vs value-only selection)
    vsel = krs.select(s_out["energy"], s_out["energy"], caps, cfg.sink, cfg.recent, offsets=offsets)
    sev = [krs.Events(2) for _ in range(args.steps)]
    for k in range(args.steps + 1):
        sres = krs.count_stats(s_out["count"], s_out["energy"], caps, cfg.sink, cfg.recent,
                               keep_twin=sel_out["keep"], keep_value=vsel["keep"], events=sev[k - 1] if k else None)
    torch.cuda.synchronize()
    stats_ms = float(np.mean([e.elapsed_ms(0, 1) for e in sev]))
    for e in sev:
        e.close()
    st_np = sres["stats"].cpu().numpy()
    stats_bytes = G * N * (4 + 8 + 1 + 1) * 2  # count, energy and both masks, read twice
    del vsel

    # per-head capacities from prefix attention, 8 KV heads per layer
    # (not part of the timed step)
    from synth import make_queries
    Qh = torch.from_numpy(np.stack([make_queries(cfg, g) for g in range(G)]).view(np.int16)).to(dev)
    Hkv = 8 if G % 8 == 0 else 1
    B_alloc = krs.uniform_capacity(N, cfg.removal if cfg.removal is not None else 0.5)
    aev = [krs.Events(4) for _ in range(args.steps)]
    aout, aws = {}, None
    for k in range(args.steps + 1):
        ares = krs.allocate(K, Qh, Hkv, B_alloc, cfg.sink, cfg.recent, out=aout, ws=aws,
                            events=aev[k - 1] if k else None)
        aws = ares["ws"]
        aout = {kk: ares[kk] for kk in ("capacity", "g_count", "z")}
    torch.cuda.synchronize()
    alloc_ms = [float(np.mean([e.elapsed_ms(a, a + 1) for e in aev])) for a in range(3)]
    for e in aev:
        e.close()
    nq = Qh.shape[1] * Qh.shape[2]
    logit_flops = 2.0 * G * nq * N * d  # one fp64 dot product per (query, key)
    del Qh

    alg = algorithmic_gram_flops(N, d, cfg.window, G)
    dense = 2.0 * G * N * N * d
    achieved = alg / (gram_ms * 1e-3) / 1e12
    exec_tflops = dense / (gram_ms * 1e-3) / 1e12
    mean_cap = float(np.mean(cap_list))
    rgram = restricted_gram_flops(N, mean_cap, d, G)
    # rows the restricted sweep visits: those whose unrestricted best twin
    # (the prior from the score pass) was not retained
    bi = s_out["best_idx"].long()
    reused = (bi < 0) | torch.gather(sel_out["keep"], 1, bi.clamp(min=0)).bool()
    swept_frac = 1.0 - reused.float().mean().item()
    norms_bytes = G * N * (4 * d + 20)

    traffic = None
    meas = MEASURED_TRAFFIC.get(source_hash(GRAM_SOURCE))
    if meas is not None and meas.get("workload") == (G, N, d):
        traffic = meas["bytes_per_launch"]

    twin = int(round(cfg.twin_frac * 100))
    budget = (f"{int(round(cfg.removal * 100))}% removal" if cfg.removal is not None
              else f"Dirichlet(1) split of a {int(round(cfg.budget_frac * 100))}% budget per group of {cfg.group} heads")
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
                               f"window {cfg.window}, {budget}; score + select + repair of the selected set",
                   "G": G, "N": N, "d": d, "tau": cfg.tau, "window": cfg.window, "sink": cfg.sink,
                   "recent": cfg.recent, "mean_capacity": mean_cap, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic,
                     "kernel": f"gram_kernel<{SCORE_SHAPE[d]}, score>", "algorithmic_flop_per_launch": alg,
                     "avg_launch_ms": gram_ms},
        "gram": {"dense_equiv_tflops": exec_tflops, "mfma_frac_dense_equiv": exec_tflops / PEAK_BF16_TFLOPS,
                 "keys_per_s": G * N / (gram_ms * 1e-3), "ms": gram_ms},
        "phases_ms": {"norms_energy": norms_ms, "gram_score": gram_ms, "select": select_ms,
                      "repair_norms": r_norms_ms, "repair_compact": r_compact_ms, "repair_gram": r_gram_ms,
                      "repair_swap": r_swap_ms},
        "phase_rates": {"norms_energy_GBs": norms_bytes / (norms_ms * 1e-3) / 1e9,
                        "repair_gram_dense_tflops": rgram * swept_frac / (r_gram_ms * 1e-3) / 1e12,
                        "repair_rows_swept_frac": swept_frac},
        "gather_kv": {"ms": gather_ms, "rows": gather_rows, "algorithmic_bytes": gather_bytes,
                      "GBs": gather_bytes / (gather_ms * 1e-3) / 1e9,
                      "frac_hbm": gather_bytes / (gather_ms * 1e-3) / 1e9 / PEAK_HBM_GBS},
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
        "swaps_total": int(rep_out["n_swaps"].sum().item()),
        "generation_s": gen_s,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds, cap_list)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
