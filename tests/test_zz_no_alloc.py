"""twinkv_score_noalloc, the allocation-free variant of twinkv_score, through
the C ABI against twinkv_score itself on the same inputs: two calls in a
row, the second on a smaller input (so the static scratch holds the first
call's larger contents when the second starts), each bit for bit equal to
the workspace entry point, whose outputs the parity tests check against the
oracle.  Sizes beyond the scratch are refused before any launch."""
import numpy as np
import pytest
import torch

import key_redundancy_scoring_amd as krs
from key_redundancy_scoring_amd import _lib as L
from synth import get_config, make_heads

pytestmark = pytest.mark.gpu

KEYS = ("count", "best_sim", "best_idx", "energy", "score", "omega")


def _up(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda:0")


def test_score_noalloc_matches_score_on_two_calls():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    cases = [(2, 4, 3000), (4, 3, 1100)]  # (workload, heads, N): the second call is smaller
    for cfg_id, G, N in cases:
        cfg = get_config(cfg_id)
        print(f"[noalloc] workload {cfg_id} G={G} N={N} d={cfg.d}", flush=True)
        K, V, _ = make_heads(cfg, heads=range(G), N=N)
        tk, tv = _up(K), _up(V)
        ref = krs.score(tk, tv, cfg.tau, cfg.window, cfg.sink, cfg.recent, omega=True)
        torch.cuda.synchronize()
        got = krs.score_noalloc(tk, tv, cfg.tau, cfg.window, cfg.sink, cfg.recent, omega=True)
        torch.cuda.synchronize()
        for k in KEYS:
            assert torch.equal(got[k], ref[k]), f"workload {cfg_id} G={G} N={N}: {k} differs"
        p = krs.params(G, N, cfg.d, cfg.tau, cfg.window)
        assert krs.workspace_bytes(L.OP_SCORE, p) <= L.NOALLOC_SCRATCH_BYTES
        print(f"[noalloc] G={G} N={N}: all outputs bit-equal, twins {int((got['count'] > 0).sum())}", flush=True)


def test_score_noalloc_refuses_sizes_beyond_the_scratch():
    lib = krs.load()
    fake = torch.empty(16, dtype=torch.float64, device="cuda:0")
    ptr = L._ptr(fake)
    for G, N, d in ((1, 1 << 21, 64), (64, 32768, 64), (32, 32768, 128)):
        p = krs.params(G, N, d, 0.9, 8)
        assert krs.workspace_bytes(L.OP_SCORE, p) > L.NOALLOC_SCRATCH_BYTES
        st = lib.twinkv_score_noalloc(__import__("ctypes").byref(p), ptr, ptr, ptr, ptr, ptr, ptr, ptr, None, None,
                                      None)
        assert st == L.ERR_TOO_LARGE, st
    assert "scratch" in krs.status_string(L.ERR_TOO_LARGE)
