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
