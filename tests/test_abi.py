"""The C-ABI library: it loads, exports every function the header declares,
and its host-side checks reject bad arguments before any launch.  No call in
this file reaches a kernel launch, so it runs without a GPU."""
import ctypes
import subprocess

import pytest

import key_redundancy_scoring_amd as krs
from key_redundancy_scoring_amd import _lib as L
from oracle import twinkv_oracle as O

FAKE = ctypes.c_void_p(0x100000)  # aligned, never dereferenced: every call below fails validation first


def test_library_exports_every_header_symbol():
    lib = krs.load()
    declared = krs.header_symbols()
    assert declared == ["twinkv_allocate", "twinkv_allocate_workspace_bytes", "twinkv_capacity_offsets",
                        "twinkv_count_stats",
                        "twinkv_gather_kv", "twinkv_repair",
                        "twinkv_score", "twinkv_score_noalloc", "twinkv_select", "twinkv_status_string", "twinkv_uniform_capacity",
                        "twinkv_uniform_capacity_ceil", "twinkv_variant_score", "twinkv_workspace_bytes"]
    for name in declared:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert set(declared) <= exported


def test_status_strings():
    for st in (L.OK, L.ERR_ARG, L.ERR_UNSUPPORTED, L.ERR_WORKSPACE, L.ERR_HIP):
        assert krs.status_string(st) != "unknown status"
    assert krs.status_string(12345) == "unknown status"


@pytest.mark.parametrize("N,r", [(172, 0.75), (512, 0.5), (8192, 0.7), (32768, 0.5), (131072, 0.75), (10, 0.35),
                                 (7, 0.0), (7, 1.0), (1000, 0.3)])
def test_uniform_capacity_matches_oracle(N, r):
    assert krs.uniform_capacity(N, r) == O.uniform_budget(N, r)


def test_uniform_capacity_rejects():
    assert krs.uniform_capacity(-1, 0.5) == -1
    assert krs.uniform_capacity(10, 1.5) == -1
    assert krs.uniform_capacity(10, float("nan")) == -1


def test_workspace_sizes():
    p = krs.params(128, 32768, 64, 0.9, 64)
    n = 128 * 32768
    assert krs.workspace_bytes(L.OP_SCORE, p) >= n * 12
    assert krs.workspace_bytes(L.OP_SELECT, p) == 0
    assert krs.workspace_bytes(L.OP_REPAIR, p) >= n * 40
    assert krs.workspace_bytes(L.OP_SCORE, krs.params(1, 10, 96, 0.9, 4)) == 0  # unsupported d
    assert krs.workspace_bytes(7, p) == 0


def _score_call(p, ws_bytes=1 << 30, keys=FAKE, values=FAKE, ws=FAKE):
    lib = krs.load()
    return lib.twinkv_score(ctypes.byref(p) if p is not None else None, keys, values, FAKE, FAKE, FAKE, FAKE, FAKE,
                            None, ws, ws_bytes, None, None)


def test_score_validation():
    good = krs.params(2, 100, 64, 0.9, 8)
    assert _score_call(None) == L.ERR_ARG
    assert _score_call(krs.params(2, 100, 96, 0.9, 8)) == L.ERR_UNSUPPORTED
    assert _score_call(krs.params(0, 100, 64, 0.9, 8)) == L.ERR_ARG
    assert _score_call(krs.params(2, 0, 64, 0.9, 8)) == L.ERR_ARG
    assert _score_call(krs.params(2, (1 << 30) + 1, 64, 0.9, 8)) == L.ERR_ARG
    assert _score_call(krs.params(2, 100, 64, 1.0, 8)) == L.ERR_ARG
    assert _score_call(krs.params(2, 100, 64, -1.0, 8)) == L.ERR_ARG
    assert _score_call(krs.params(2, 100, 64, float("nan"), 8)) == L.ERR_ARG
    assert _score_call(krs.params(2, 100, 64, 0.9, -1)) == L.ERR_ARG
    assert _score_call(krs.params(2, 100, 64, 0.9, 8, sink=-1)) == L.ERR_ARG
    assert _score_call(good, keys=None) == L.ERR_ARG
    assert _score_call(good, keys=ctypes.c_void_p(0x100002)) == L.ERR_ARG  # misaligned
    assert _score_call(good, ws_bytes=16) == L.ERR_WORKSPACE
    assert _score_call(good, ws=None) == L.ERR_WORKSPACE
    assert _score_call(good, ws=ctypes.c_void_p(0x100010)) == L.ERR_ARG  # workspace not 256-byte aligned


def test_select_validation():
    lib = krs.load()
    p = krs.params(2, 100, 0, 0.0, 0)  # select ignores d, tau and window
    call = lambda p, kept=FAKE, off=FAKE, keep=FAKE: lib.twinkv_select(  # noqa: E731
        ctypes.byref(p) if p is not None else None, FAKE, FAKE, FAKE, off, keep, kept, None, 0, None, None)
    assert call(None) == L.ERR_ARG
    assert call(krs.params(2, 0, 0, 0.0, 0)) == L.ERR_ARG
    assert call(p, keep=None) == L.ERR_ARG
    assert call(p, kept=None) == L.ERR_ARG
    assert call(p, off=None) == L.ERR_ARG
    offs = lib.twinkv_capacity_offsets
    assert offs(None, 2, 100, FAKE, None) == L.ERR_ARG
    assert offs(FAKE, 2, 100, None, None) == L.ERR_ARG
    assert offs(FAKE, 0, 100, FAKE, None) == L.ERR_ARG
    assert offs(FAKE, 2, 0, FAKE, None) == L.ERR_ARG
    assert offs(FAKE, 2, (1 << 30) + 1, FAKE, None) == L.ERR_ARG


def test_repair_validation():
    lib = krs.load()
    call = lambda p, keep_out=FAKE, pairs=FAKE, ws=FAKE, nb=1 << 30, ps=None, pi=None: lib.twinkv_repair(  # noqa: E731
        ctypes.byref(p), FAKE, FAKE, ps, pi, keep_out, FAKE, FAKE, FAKE, FAKE, FAKE, pairs, ws, nb, None, None)
    good = krs.params(2, 100, 128, 0.9, 8)
    assert call(krs.params(2, 100, 32, 0.9, 8)) == L.ERR_UNSUPPORTED
    assert call(good, keep_out=None) == L.ERR_ARG
    assert call(good, keep_out=FAKE) == L.ERR_ARG  # keep_out aliases keep_in
    assert call(good, keep_out=ctypes.c_void_p(0x200000), pairs=None) == L.ERR_ARG
    assert call(good, keep_out=ctypes.c_void_p(0x200000), nb=100) == L.ERR_WORKSPACE
    # a prior needs both its similarity and its index
    assert call(good, keep_out=ctypes.c_void_p(0x200000), ps=FAKE) == L.ERR_ARG
    assert call(good, keep_out=ctypes.c_void_p(0x200000), pi=FAKE) == L.ERR_ARG


def test_params_struct_layout():
    assert ctypes.sizeof(L.Params) == 40
    assert [L.Params.G.offset, L.Params.N.offset, L.Params.d.offset, L.Params.window.offset, L.Params.tau.offset,
            L.Params.sink.offset, L.Params.recent.offset] == [0, 8, 16, 20, 24, 32, 36]


def test_gather_validation():
    lib = krs.load()
    p = L.params(2, 8, 64, 0.0, 0)
    # only refusals are exercised: each fails validation before any launch
    bad = [
        (L.params(2, 8, 32, 0.0, 0), FAKE, None, FAKE, FAKE, 4, FAKE, None, L.ERR_UNSUPPORTED),
        (p, None, None, FAKE, FAKE, 4, FAKE, None, L.ERR_ARG),          # no keys
        (p, FAKE, None, FAKE, None, 4, FAKE, None, L.ERR_ARG),          # no offsets
        (p, FAKE, None, FAKE, FAKE, -1, FAKE, None, L.ERR_ARG),         # negative total
        (p, FAKE, None, FAKE, FAKE, 17, FAKE, None, L.ERR_ARG),         # total above G*N
        (p, FAKE, None, None, FAKE, 4, FAKE, None, L.ERR_ARG),          # no kept_idx
        (p, FAKE, None, FAKE, FAKE, 4, None, None, L.ERR_ARG),          # no output
        (p, FAKE, FAKE, FAKE, FAKE, 4, FAKE, None, L.ERR_ARG),          # values without their output
        (p, FAKE, None, FAKE, FAKE, 4, FAKE, FAKE, L.ERR_ARG),          # output without values
        (p, ctypes.c_void_p(0x100008), None, FAKE, FAKE, 4, FAKE, None, L.ERR_ARG),  # misaligned
        (L.params(0, 8, 64, 0.0, 0), FAKE, None, FAKE, FAKE, 0, FAKE, None, L.ERR_ARG),
    ]
    for pp, k, v, idx, off, total, ok_, ov, want in bad:
        assert lib.twinkv_gather_kv(ctypes.byref(pp), k, v, idx, off, total, ok_, ov, None, None) == want


def test_allocate_validation():
    lib = krs.load()
    p = L.params(16, 1000, 64, 0.0, 0, 4, 64)
    nb = lib.twinkv_allocate_workspace_bytes(ctypes.byref(p), 8, 4, 32, 7, 500)
    assert nb > 16 * 1000 * (8 + 4 + 8)  # agg, z and pool at least
    bad_shapes = [(3, 4, 32, 7, 500),     # H does not divide G
                  (8, 4, 33, 7, 500),     # Gq * W above 128
                  (8, 4, 0, 7, 500),      # no queries
                  (8, 4, 32, 6, 500),     # even pool
                  (8, 4, 32, 7, 1001),    # budget above N
                  (8, 4, 32, 7, -1)]
    for H, Gq, W, pool, B in bad_shapes:
        assert lib.twinkv_allocate_workspace_bytes(ctypes.byref(p), H, Gq, W, pool, B) == 0
        assert lib.twinkv_allocate(ctypes.byref(p), H, Gq, W, pool, B, FAKE, FAKE, FAKE, None, None, FAKE, 1 << 40,
                                   None, None) == L.ERR_ARG
    assert lib.twinkv_allocate(ctypes.byref(L.params(16, 1000, 32, 0.0, 0)), 8, 4, 32, 7, 500, FAKE, FAKE, FAKE, None,
                               None, FAKE, 1 << 40, None, None) == L.ERR_UNSUPPORTED
    assert lib.twinkv_allocate(ctypes.byref(p), 8, 4, 32, 7, 500, FAKE, FAKE, None, None, None, FAKE, 1 << 40, None,
                               None) == L.ERR_ARG  # no capacity output
    assert lib.twinkv_allocate(ctypes.byref(p), 8, 4, 32, 7, 500, FAKE, FAKE, FAKE, None, None, FAKE, nb - 1, None,
                               None) == L.ERR_WORKSPACE


@pytest.mark.parametrize("N,r", [(10, 0.55), (172, 0.75), (32768, 0.5), (131072, 0.75), (7, 0.0), (7, 1.0), (0, 0.3)])
def test_ceil_capacity_matches_oracle(N, r):
    assert krs.uniform_capacity_ceil(N, r) == O.ceil_budget(N, r)


def test_variant_validation():
    lib = krs.load()
    p = L.params(2, 8, 0, 0.0, 0)
    other = ctypes.c_void_p(0x200000)
    third = ctypes.c_void_p(0x300000)
    cases = [
        (5, FAKE, FAKE, other, third),       # unknown variant
        (-1, FAKE, FAKE, other, third),
        (0, None, FAKE, other, third),       # no counts
        (0, FAKE, None, other, third),       # no energies
        (0, FAKE, FAKE, None, third),        # no score output
        (0, FAKE, FAKE, other, other),       # score and tie alias
        (0, FAKE, other, other, third),      # score overwrites the energies
    ]
    for variant, cnt, en, sc, tie in cases:
        assert lib.twinkv_variant_score(ctypes.byref(p), variant, cnt, en, None, sc, tie, None, None) == L.ERR_ARG
    assert lib.twinkv_variant_score(ctypes.byref(L.params(0, 8, 0, 0.0, 0)), 0, FAKE, other, None, third,
                                    ctypes.c_void_p(0x400000), None, None) == L.ERR_ARG
    assert krs.uniform_capacity_ceil(-1, 0.5) == -1 and krs.uniform_capacity_ceil(5, 1.5) == -1


def test_count_stats_validation():
    lib = krs.load()
    p = L.params(2, 8, 0, 0.0, 0)
    A, B_, C, D, E, F = (ctypes.c_void_p(x) for x in (0x100000, 0x200000, 0x300000, 0x400000, 0x500000, 0x600000))
    ok_args = [A, B_, None, None, C, D, E]
    for k in (0, 1, 4, 5, 6):  # count, energy, capacity, stats, fstats are required
        args = list(ok_args)
        args[k] = None
        assert lib.twinkv_count_stats(ctypes.byref(p), *args, None, None) == L.ERR_ARG
    assert lib.twinkv_count_stats(ctypes.byref(p), A, B_, F, None, C, D, E, None, None) == L.ERR_ARG  # one selection
    assert lib.twinkv_count_stats(ctypes.byref(L.params(2, 0, 0, 0.0, 0)), *ok_args, None, None) == L.ERR_ARG
