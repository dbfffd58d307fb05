"""The stored oracle results (tests/golden/oracle_<workload>.json) against
their generator: every file covers exactly the seeded head subset, with the
parity constants the tests use, and records of the tiny workload and of one
short-prefix head of the batched workload recomputed here from oracle/ and
synth/ equal the stored ones field by field.  Runs on the CPU."""
import json
import os

import pytest

from synth import get_config
from tests import parity as PR
from tests.golden import make_oracle_goldens as MG


def _load(cfg_id):
    path = MG.golden_path(cfg_id)
    if not os.path.exists(path):
        pytest.fail(f"missing {path}: run tests/golden/make_oracle_goldens.py")
    return json.load(open(path))


@pytest.mark.parametrize("cfg_id", [1, 2, 3, 4, 5])
def test_golden_file_covers_the_seeded_subset(cfg_id):
    gold = _load(cfg_id)
    cfg = get_config(cfg_id)
    assert gold["near_tie"] == PR.NEAR_TIE and gold["band"] == PR.BAND and gold["chunk"] == MG.CHUNK
    assert (gold["G"], gold["N"], gold["d"], gold["tau"], gold["window"]) == (cfg.G, cfg.N, cfg.d, cfg.tau, cfg.window)
    heads = [h["head"] for h in gold["heads"]]
    assert heads == MG.checked_heads(cfg_id)
    assert 0 in heads and cfg.G - 1 in heads
    nchunks = (cfg.N + MG.CHUNK - 1) // MG.CHUNK
    for h in gold["heads"]:
        rep = h["repair"]
        assert len(rep["arg_chunks"]) == nchunks
        assert 0 <= rep["m"] <= min(rep["n_orphans"], rep["n_donors"])
        if cfg.mode != "repair":
            assert len(h["count_chunks"]) == nchunks and len(h["arg_chunks"]) == nchunks
            assert rep["K"] == h["capacity"]


@pytest.mark.parametrize("cfg_id,head", [(1, 0), (5, 0)])
def test_golden_records_recompute(cfg_id, head):
    gold = _load(cfg_id)
    stored = next(h for h in gold["heads"] if h["head"] == head)
    caps = MG.capacities(cfg_id)
    rec = MG.head_record(cfg_id, head, caps[head])
    rec.pop("seconds")
    stored = dict(stored)
    stored.pop("seconds")
    assert json.loads(json.dumps(rec)) == stored


def test_swap_rule_matches_the_oracle_repair():
    """The swap rule the GPU tests use to judge a near-tie pick gives the
    oracle's repair when fed the oracle's own b(S0); a substituted b that
    crosses tau or reorders a ranking is reported as a change."""
    import numpy as np

    from oracle import twinkv_oracle as O
    from synth import gumbel_retained, make_head

    cfg = get_config(1)
    h = make_head(cfg, 0)
    K = O.widen_bf16(h["K"])
    S0 = gumbel_retained(cfg, 0)
    ref = O.repair_head(K, S0, cfg.tau, cfg.window, cfg.sink, cfg.recent)
    got = PR.swap_rule(ref["best"], S0, cfg.tau, cfg.sink, cfg.recent)
    assert (got["n_orphans"], got["n_donors"], got["m"]) == (ref["n_orphans"], ref["n_donors"], ref["m"])
    assert np.array_equal(got["pairs"], ref["pairs"]) and np.array_equal(got["keep"], ref["keep"] != 0)
    b = ref["best"]
    assert not PR.near_tie_effect(b, {}, S0, cfg.tau, cfg.sink, cfg.recent)["swap_changes"]
    assert not PR.near_tie_effect(b, {0: float(b[0])}, S0, cfg.tau, cfg.sink, cfg.recent)["swap_changes"]
    orphans = ref["orphans"]
    assert ref["m"] >= 2
    first, second = int(orphans[0]), int(orphans[1])
    # the first-ranked orphan pushed past the second reorders the pairs
    eff = PR.near_tie_effect(b, {first: float(b[second]) + 1e-12}, S0, cfg.tau, cfg.sink, cfg.recent)
    assert eff["swap_changes"] and eff["class_changes"] == 0
    # an orphan lifted over tau leaves O
    eff = PR.near_tie_effect(b, {first: cfg.tau}, S0, cfg.tau, cfg.sink, cfg.recent)
    assert eff["swap_changes"] and eff["class_changes"] == 1
