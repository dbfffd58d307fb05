"""Benchmark of the key-redundancy hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2] [--no-cpu-baseline]

One step = one pass of the whole path over one batch of synthetic heads that
is already resident in HBM: score (norms/energy pass + fused Gram sweep with
the fp64 best-twin fixup and the discounted score) -> exact-budget select ->
repair of the selected set (restricted Gram over the retained columns,
orphan/donor ranking and swap).  The default workload is the Llama-3.2-1B
shape: 16 layers x 8 KV heads = 128 heads, N = 32768, head dim 64, 10%
planted near-duplicates, tau 0.9, window 64, 4 sinks, 64 recent, 50% removal.

Prints one JSON line.  `value` is keys (head positions) through the whole path
per second.  `roofline` is for the dominant kernel, the score-mode Gram
sweep, timed with HIP events recorded by the library around its launch on
the stream it runs on; its `achieved` counts the algorithmic work, one
d-length dot product (2d flop) per unordered nonlocal pair.  `cpu_baseline`
times the fp64 oracle on a bounded sample of the same workload on the host.
"""
from __future__ import annotations

import argparse
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


def algorithmic_gram_flops(N: int, d: int, window: int, G: int) -> float:
    """One dot product (2d flop) per unordered pair (i, j) with j - i > w."""
    pairs = max(0, N - window - 1) * max(0, N - window) // 2
    return float(G) * pairs * 2.0 * d


def restricted_gram_flops(N: int, K: int, d: int, G: int) -> float:
    """Repair: every position against the K retained columns (2d flop each)."""
    return float(G) * N * K * 2.0 * d


def cpu_baseline(cfg, rows: int, seed_head: int = 0):
    from threadpoolctl import threadpool_info

    from oracle import twinkv_oracle as O
    from synth import make_head

    h = make_head(cfg, seed_head)
    sel = np.arange(rows)
    t0 = time.perf_counter()
    O.score_head(h["K"], h["V"], cfg.tau, cfg.window, rows=sel)
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": rows / dt, "unit": "keys/s", "cores": int(threads), "kind": "oracle",
            "sample": f"score (count, best twin, energy, score) of rows 0..{rows - 1} of head {seed_head} "
                      f"(each row against all N={cfg.N} positions), fp64 numpy/BLAS, {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=4096)
    ap.add_argument("--heads", type=int, default=None, help="override the head count (default: the workload's)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU: every (layer, KV head) is independent, so more GPUs would each run "
              "this same kernel on their share of heads with no communication; run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import key_redundancy_scoring_amd as krs
    from synth import get_config, make_heads

    assert torch.cuda.is_available(), "bench.py needs a ROCm GPU"
    dev = torch.device("cuda:0")
    cfg = get_config(args.config)
    if args.heads:
        cfg = cfg.with_(G=args.heads)
    G, N, d = cfg.G, cfg.N, cfg.d
    removal = cfg.removal if cfg.removal is not None else 0.5

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

    cap = krs.uniform_capacity(N, removal)
    caps = torch.full((G,), cap, dtype=torch.int32, device=dev)
    s_out, sel_out, rep_out = {}, {}, {}
    s_ws = r_ws = None

    def step(ev_s=None, ev_sel=None, ev_r=None):
        nonlocal s_ws, r_ws
        r = krs.score(K, V, cfg.tau, cfg.window, cfg.sink, cfg.recent, out=s_out, ws=s_ws, events=ev_s)
        s_ws = r["ws"]
        s_out.update({k: r[k] for k in ("count", "best_sim", "best_idx", "energy", "score")})
        sl = krs.select(r["score"], r["energy"], caps, cfg.sink, cfg.recent, out=sel_out, events=ev_sel)
        sel_out.update({"keep": sl["keep"], "kept_idx": sl["kept_idx"]})
        rp = krs.repair(K, sl["keep"], cfg.tau, cfg.window, cfg.sink, cfg.recent, out=rep_out, ws=r_ws, events=ev_r)
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

    alg = algorithmic_gram_flops(N, d, cfg.window, G)
    dense = 2.0 * G * N * N * d
    achieved = alg / (gram_ms * 1e-3) / 1e12
    exec_tflops = dense / (gram_ms * 1e-3) / 1e12
    rgram = restricted_gram_flops(N, cap, d, G)
    norms_bytes = G * N * (4 * d + 20)

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
        "config": {"workload": f"{cfg.name}: {G} heads x N={N} x d={d}, {int(cfg.twin_frac * 100)}% planted twins, "
                               f"score+select+repair (repair of the selected set)",
                   "G": G, "N": N, "d": d, "tau": cfg.tau, "window": cfg.window, "sink": cfg.sink,
                   "recent": cfg.recent, "removal": removal, "capacity": cap, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None,
                     "kernel": "gram_kernel<64,score>", "algorithmic_flop_per_launch": alg,
                     "avg_launch_ms": gram_ms},
        "gram": {"dense_equiv_tflops": exec_tflops, "mfma_frac_executed": exec_tflops / PEAK_BF16_TFLOPS,
                 "keys_per_s": G * N / (gram_ms * 1e-3), "ms": gram_ms},
        "phases_ms": {"norms_energy": norms_ms, "gram_score": gram_ms, "select": select_ms,
                      "repair_norms": r_norms_ms, "repair_compact": r_compact_ms, "repair_gram": r_gram_ms,
                      "repair_swap": r_swap_ms},
        "phase_rates": {"norms_energy_GBs": norms_bytes / (norms_ms * 1e-3) / 1e9,
                        "repair_gram_dense_tflops": rgram / (r_gram_ms * 1e-3) / 1e12},
        "swaps_total": int(rep_out["n_swaps"].sum().item()),
        "generation_s": gen_s,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, args.cpu_rows)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
