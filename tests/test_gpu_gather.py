"""GPU parity of the packed cache layout (twinkv_gather_kv) against the
oracle's pack_retained: bit-for-bit equality of every packed row, on
retained sets drawn on the host (seeded Gumbel top-b per head), including
per-head Dirichlet quotas, both head dims and the degenerate cases.
Full-size workloads are covered in test_gpu_fullsize.py.
"""
import numpy as np
import pytest
import torch

import key_redundancy_scoring_amd as krs
from oracle import twinkv_oracle as O
from synth import dirichlet_capacities, get_config, gumbel_retained, make_heads

pytestmark = pytest.mark.gpu


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch.device("cuda:0")


def _up(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(_dev())


def _kept_lists(cfg, caps, N):
    return [np.flatnonzero(gumbel_retained(cfg, g, N=N, keep=int(c))) for g, c in enumerate(caps)]


def check_gather(K, V, kept, tag=""):
    """Run the GPU gather on host-drawn retained lists and compare bit for bit."""
    Kp, Vp, off = O.pack_retained(K, V, kept)
    idx = np.concatenate([np.asarray(k, np.int32) for k in kept]) if kept else np.zeros(0, np.int32)
    kt = torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).to(_dev())
    if kt.numel() == 0:
        kt = torch.zeros(1, dtype=torch.int32, device=_dev())
    res = krs.gather_kv(_up(K), _up(V) if V is not None else None, kt, torch.from_numpy(off))
    torch.cuda.synchronize()
    assert res["total"] == int(off[-1])
    np.testing.assert_array_equal(res["keys"].cpu().numpy().view(np.uint16), Kp, err_msg=f"{tag} keys")
    if V is not None:
        np.testing.assert_array_equal(res["values"].cpu().numpy().view(np.uint16), Vp, err_msg=f"{tag} values")
    else:
        assert res["values"] is None
    return int(off[-1])


@pytest.mark.parametrize("cfg_id,G,N", [(5, 16, 900), (3, 3, 700), (2, 2, 1500)])
def test_gather_quotas(cfg_id, G, N):
    cfg = get_config(cfg_id)
    K, V, _ = make_heads(cfg, heads=range(G), N=N)
    if cfg.removal is None:
        caps = dirichlet_capacities(cfg, G=G, N=N)
    else:
        caps = [O.uniform_budget(N, cfg.removal)] * G
    total = check_gather(K, V, _kept_lists(cfg, caps, N), tag=f"cfg{cfg_id}")
    assert total == int(np.sum(caps))


def test_gather_keys_only_and_extremes():
    cfg = get_config(2)
    G, N = 4, 333
    K, V, _ = make_heads(cfg, heads=range(G), N=N)
    caps = [0, N, 1, 170]  # an empty head, a full head, a single row
    kept = _kept_lists(cfg, caps, N)
    check_gather(K, None, kept, tag="keys only")
    check_gather(K, V, kept, tag="extremes")


def test_gather_empty_and_tiny():
    cfg = get_config(1)
    K, V, _ = make_heads(cfg, heads=[0, 1], N=1)
    assert check_gather(K, V, [[], []], tag="empty") == 0
    assert check_gather(K, V, [[0], [0]], tag="one row") == 2


def test_gather_validation():
    K = torch.zeros((2, 8, 64), dtype=torch.int16, device=_dev())
    kt = torch.zeros(4, dtype=torch.int32, device=_dev())
    with pytest.raises(ValueError):
        krs.gather_kv(K, None, kt, [0, 2])  # wrong offsets length
    with pytest.raises(ValueError):
        krs.gather_kv(K, None, kt, [0, 3, 6])  # kept_idx shorter than total
    with pytest.raises(krs.TwinKVError):
        krs.gather_kv(torch.zeros((2, 8, 32), dtype=torch.int16, device=_dev()), None, kt, [0, 2, 4])
