"""The step (score -> select -> repair with the score pass's twins) captured
once into a HIP graph and replayed: the entry points only launch kernels on
the caller's stream into caller-provided buffers (no allocation, no memset,
no synchronisation), so a replay must reproduce the eager results bit for
bit.  Between replays the outputs are overwritten by eager work, and every
replay is compared with the eager run.
"""
import numpy as np
import pytest
import torch

import key_redundancy_scoring_amd as krs
from oracle import twinkv_oracle as O
from synth import get_config, make_heads

pytestmark = pytest.mark.gpu

SCORE_KEYS = ("count", "best_sim", "best_idx", "energy", "score")
REPAIR_KEYS = ("keep", "best_sim", "best_idx", "n_orphans", "n_donors", "n_swaps", "pairs")


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch.device("cuda:0")


def test_step_graph_replays_match_eager():
    cfg = get_config(2)
    G, N = 4, 3000
    dev = _dev()
    K, V, _ = make_heads(cfg, heads=range(G), N=N)
    tk = torch.from_numpy(K.view(np.int16)).to(dev)
    tv = torch.from_numpy(V.view(np.int16)).to(dev)
    cap = O.uniform_budget(N, cfg.removal)
    caps = torch.full((G,), cap, dtype=torch.int32, device=dev)
    off = krs.capacity_offsets_device(caps, N)
    torch.cuda.synchronize()
    assert torch.equal(off.cpu(), krs.capacity_offsets([cap] * G, N))

    # eager run: the reference, and the buffers the graph will write
    r = krs.score(tk, tv, cfg.tau, cfg.window, cfg.sink, cfg.recent)
    sl = krs.select(r["score"], r["energy"], caps, cfg.sink, cfg.recent, offsets=off, total=G * cap)
    rp = krs.repair(tk, sl["keep"], cfg.tau, cfg.window, cfg.sink, cfg.recent, prior=r)
    torch.cuda.synchronize()
    ref = {("s", k): r[k].clone() for k in SCORE_KEYS}
    ref.update({("sel", "keep"): sl["keep"].clone(), ("sel", "kept_idx"): sl["kept_idx"].clone()})
    ref.update({("r", k): rp[k].clone() for k in REPAIR_KEYS})

    s_out = {k: r[k] for k in SCORE_KEYS}
    sel_out = {"keep": sl["keep"], "kept_idx": sl["kept_idx"]}
    rep_out = {k: rp[k] for k in REPAIR_KEYS}
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            r2 = krs.score(tk, tv, cfg.tau, cfg.window, cfg.sink, cfg.recent, out=s_out, ws=r["ws"])
            sl2 = krs.select(r2["score"], r2["energy"], caps, cfg.sink, cfg.recent, out=sel_out, offsets=off,
                             total=G * cap)
            krs.repair(tk, sl2["keep"], cfg.tau, cfg.window, cfg.sink, cfg.recent, prior=r2, out=rep_out,
                       ws=rp["ws"])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    outs = {("s", k): s_out[k] for k in SCORE_KEYS}
    outs.update({("sel", "keep"): sel_out["keep"], ("sel", "kept_idx"): sel_out["kept_idx"]})
    outs.update({("r", k): rep_out[k] for k in REPAIR_KEYS})
    for replay in range(3):
        for t in outs.values():  # eager work between replays
            t.fill_(-3 if t.dtype != torch.uint8 else 7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for key, t in outs.items():
            assert torch.equal(t, ref[key]), f"replay {replay}: {key} differs from the eager run"
    print(f"[graph] 3 replays of score -> select -> repair bit-exact, swaps {int(ref[('r', 'n_swaps')].sum())}",
          flush=True)
