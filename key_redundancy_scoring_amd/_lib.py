"""ctypes binding over libtwinkv.so (the C ABI in include/twinkv.h).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, their data pointers and torch's current HIP stream are handed to
the library, and every step of the computation runs in the library's HIP
kernels.  PyTorch provides device memory and the stream; the library never
allocates.  If the shared library is missing this module raises on use:
there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtwinkv.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "twinkv.h")

OK, ERR_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP, ERR_TOO_LARGE = 0, -1, -2, -3, -4, -5
NOALLOC_SCRATCH_BYTES = 64 << 20
OP_SCORE, OP_SELECT, OP_REPAIR = 0, 1, 2
SCORE_PHASES, SELECT_PHASES, REPAIR_PHASES, GATHER_PHASES, ALLOC_PHASES, VARIANT_PHASES = 3, 1, 4, 1, 3, 1
VARIANTS = {"twin": 0, "value": 1, "rarity": 2}
STAT_INTS = 26
STATS_PHASES = 1


class Params(ctypes.Structure):
    _fields_ = [
        ("G", ctypes.c_int64),
        ("N", ctypes.c_int64),
        ("d", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("tau", ctypes.c_double),
        ("sink", ctypes.c_int32),
        ("recent", ctypes.c_int32),
    ]


class TwinKVError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} (status {status})")
        self.status = status


_lib = None


def load():
    """Load libtwinkv.so (built in-tree by ``key_redundancy_scoring_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m key_redundancy_scoring_amd.build` "
                           "(or __graft_entry__.build()); there is no fallback implementation")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(Params)
    vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    lib.twinkv_workspace_bytes.argtypes = [ctypes.c_int, P]
    lib.twinkv_workspace_bytes.restype = sz
    lib.twinkv_uniform_capacity.argtypes = [i64, ctypes.c_double]
    lib.twinkv_uniform_capacity.restype = i64
    lib.twinkv_status_string.argtypes = [ctypes.c_int]
    lib.twinkv_status_string.restype = ctypes.c_char_p
    lib.twinkv_score.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp]
    lib.twinkv_score.restype = ctypes.c_int
    lib.twinkv_score_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.twinkv_score_noalloc.restype = ctypes.c_int
    lib.twinkv_select.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp]
    lib.twinkv_select.restype = ctypes.c_int
    lib.twinkv_capacity_offsets.argtypes = [vp, i64, i64, vp, vp]
    lib.twinkv_capacity_offsets.restype = ctypes.c_int
    lib.twinkv_repair.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp]
    lib.twinkv_repair.restype = ctypes.c_int
    lib.twinkv_gather_kv.argtypes = [P, vp, vp, vp, vp, i64, vp, vp, vp, vp]
    lib.twinkv_gather_kv.restype = ctypes.c_int
    i32 = ctypes.c_int32
    lib.twinkv_allocate_workspace_bytes.argtypes = [P, i32, i32, i32, i32, i64]
    lib.twinkv_allocate_workspace_bytes.restype = sz
    lib.twinkv_allocate.argtypes = [P, i32, i32, i32, i32, i64, vp, vp, vp, vp, vp, vp, sz, vp, vp]
    lib.twinkv_allocate.restype = ctypes.c_int
    lib.twinkv_uniform_capacity_ceil.argtypes = [i64, ctypes.c_double]
    lib.twinkv_uniform_capacity_ceil.restype = i64
    lib.twinkv_variant_score.argtypes = [P, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp]
    lib.twinkv_variant_score.restype = ctypes.c_int
    lib.twinkv_count_stats.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.twinkv_count_stats.restype = ctypes.c_int
    _lib = lib
    return lib


def header_symbols() -> list[str]:
    """Names of the functions include/twinkv.h declares."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(twinkv_[a-z_]+)\s*\(", text)))


def status_string(status: int) -> str:
    return load().twinkv_status_string(int(status)).decode()


def params(G, N, d, tau, window, sink=4, recent=64) -> Params:
    return Params(int(G), int(N), int(d), int(window), float(tau), int(sink), int(recent))


def workspace_bytes(op: int, p: Params) -> int:
    return int(load().twinkv_workspace_bytes(int(op), ctypes.byref(p)))


def uniform_capacity(N: int, removal: float) -> int:
    return int(load().twinkv_uniform_capacity(int(N), float(removal)))


def uniform_capacity_ceil(N: int, removal: float) -> int:
    return int(load().twinkv_uniform_capacity_ceil(int(N), float(removal)))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(status, where):
    if status != OK:
        raise TwinKVError(status, where)


def _as_bf16_bits(x, name):
    if x.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{name} must hold bf16 values (torch.bfloat16, or raw bits as int16/uint16)")
    if not x.is_cuda or not x.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    if x.dim() != 3:
        raise ValueError(f"{name} must be [G][N][d]")
    return x


def _need(t, shape, dtype, device, name):
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != device or not t.is_contiguous():
        raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)} on {device}")
    return t


def _workspace(ws, nbytes, device):
    if nbytes == 0:
        return ws
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    return ws


def _ws_ptr(ws):
    if ws is None:
        return ctypes.c_void_p(0), 0
    p = ws.data_ptr()
    aligned = (p + 255) & ~255
    return ctypes.c_void_p(aligned), ws.numel() - (aligned - p)


class Events:
    """hipEvents created through the HIP runtime, for the optional ``marks``
    argument (phase timing)."""

    def __init__(self, n: int):
        hip = ctypes.CDLL("libamdhip64.so")
        self._hip = hip
        hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.arr = (ctypes.c_void_p * n)()
        for k in range(n):
            e = ctypes.c_void_p()
            if hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.arr[k] = e.value
        self.n = n

    def elapsed_ms(self, a: int, b: int) -> float:
        self._hip.hipEventSynchronize(self.arr[b])
        out = ctypes.c_float()
        if self._hip.hipEventElapsedTime(ctypes.byref(out), self.arr[a], self.arr[b]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(out.value)

    def close(self):
        for k in range(self.n):
            self._hip.hipEventDestroy(self.arr[k])
        self.n = 0


def _marks(ev: Events | None, phases: int):
    if ev is None:
        return ctypes.c_void_p(0)
    if ev.n < phases + 1:
        raise ValueError(f"need {phases + 1} events")
    return ctypes.cast(ev.arr, ctypes.c_void_p)


def score(keys, values, tau, window, sink=4, recent=64, omega=False, out=None, ws=None, events=None):
    """Counts, best nonlocal twin, energy and score for every head.

    keys, values: bf16 [G][N][d] device tensors.  Returns a dict of device
    tensors: count (int32), best_sim (f64), best_idx (int32), energy (f64),
    score (f64) and optionally omega (f64), each [G][N], plus the workspace
    under "ws" for reuse.
    """
    lib = load()
    keys = _as_bf16_bits(keys, "keys")
    values = _as_bf16_bits(values, "values")
    if values.shape != keys.shape:
        raise ValueError("keys and values must have the same shape")
    G, N, d = keys.shape
    dev = keys.device
    p = params(G, N, d, tau, window, sink, recent)
    out = {} if out is None else out
    o = {
        "count": _need(out.get("count"), (G, N), torch.int32, dev, "count"),
        "best_sim": _need(out.get("best_sim"), (G, N), torch.float64, dev, "best_sim"),
        "best_idx": _need(out.get("best_idx"), (G, N), torch.int32, dev, "best_idx"),
        "energy": _need(out.get("energy"), (G, N), torch.float64, dev, "energy"),
        "score": _need(out.get("score"), (G, N), torch.float64, dev, "score"),
    }
    if omega or out.get("omega") is not None:
        o["omega"] = _need(out.get("omega"), (G, N), torch.float64, dev, "omega")
    nb = workspace_bytes(OP_SCORE, p)
    ws = _workspace(ws, nb, dev)
    wp, wn = _ws_ptr(ws)
    st = lib.twinkv_score(ctypes.byref(p), _ptr(keys), _ptr(values), _ptr(o["count"]), _ptr(o["best_sim"]),
                          _ptr(o["best_idx"]), _ptr(o["energy"]), _ptr(o["score"]), _ptr(o.get("omega")), wp, wn,
                          _stream(), _marks(events, SCORE_PHASES))
    _check(st, "twinkv_score")
    o["ws"] = ws
    return o


def score_noalloc(keys, values, tau, window, sink=4, recent=64, omega=False, out=None, events=None):
    """score() through twinkv_score_noalloc: the library's static per-device
    scratch instead of a workspace (whose size must not exceed
    NOALLOC_SCRATCH_BYTES).  Output
    tensors are allocated here unless given in ``out``; the library call
    itself allocates nothing.  Calls that overlap on one device race."""
    lib = load()
    keys = _as_bf16_bits(keys, "keys")
    values = _as_bf16_bits(values, "values")
    if values.shape != keys.shape:
        raise ValueError("keys and values must have the same shape")
    G, N, d = keys.shape
    dev = keys.device
    p = params(G, N, d, tau, window, sink, recent)
    out = {} if out is None else out
    o = {
        "count": _need(out.get("count"), (G, N), torch.int32, dev, "count"),
        "best_sim": _need(out.get("best_sim"), (G, N), torch.float64, dev, "best_sim"),
        "best_idx": _need(out.get("best_idx"), (G, N), torch.int32, dev, "best_idx"),
        "energy": _need(out.get("energy"), (G, N), torch.float64, dev, "energy"),
        "score": _need(out.get("score"), (G, N), torch.float64, dev, "score"),
    }
    if omega or out.get("omega") is not None:
        o["omega"] = _need(out.get("omega"), (G, N), torch.float64, dev, "omega")
    with torch.cuda.device(dev):
        st = lib.twinkv_score_noalloc(ctypes.byref(p), _ptr(keys), _ptr(values), _ptr(o["count"]),
                                      _ptr(o["best_sim"]), _ptr(o["best_idx"]), _ptr(o["energy"]), _ptr(o["score"]),
                                      _ptr(o.get("omega")), _stream(), _marks(events, SCORE_PHASES))
    _check(st, "twinkv_score_noalloc")
    return o


def capacity_offsets(capacity, N):
    """Start of each head's run in ``kept_idx`` for host capacities, on the
    host (clamped capacities), to size buffers before a call."""
    c = torch.as_tensor(capacity).to("cpu", torch.int64).clamp(0, int(N))
    off = torch.zeros(c.numel() + 1, dtype=torch.int64)
    off[1:] = torch.cumsum(c, 0)
    return off


def capacity_offsets_device(capacity, N, out=None):
    """The same offsets computed by the library on the capacities' device
    (twinkv_capacity_offsets), asynchronously on the current stream."""
    lib = load()
    if capacity.dtype != torch.int32 or not capacity.is_cuda or not capacity.is_contiguous():
        raise ValueError("capacity must be a contiguous int32 device tensor")
    G = capacity.numel()
    off = _need(out, (G + 1,), torch.int64, capacity.device, "offsets")
    _check(lib.twinkv_capacity_offsets(_ptr(capacity), G, int(N), _ptr(off), _stream()), "twinkv_capacity_offsets")
    return off


def select(score_t, energy_t, capacity, sink=4, recent=64, out=None, events=None, offsets=None, total=None):
    """Exact-budget selection.  ``capacity``: int32 device tensor [G] or a
    host sequence (copied to the device).  ``offsets`` (optional): int64
    [G+1] prefix sums of the clamped capacities, on the host or the device.
    Without them the library computes them on the device; the kept list is
    then sized from the host capacities when they are on the host, else G*N
    entries, so no device value is read back; ``total`` (the sum of the
    clamped capacities, when the caller knows it) sizes it exactly.  Returns
    keep (uint8 [G][N]),
    kept_idx (int32, heads concatenated, ascending within a head), the device
    offsets of each head's run and the device capacities."""
    lib = load()
    G, N = score_t.shape
    dev = score_t.device
    for t, nm in ((score_t, "score"), (energy_t, "energy")):
        if t.dtype != torch.float64 or not t.is_contiguous() or t.device != dev or tuple(t.shape) != (G, N):
            raise ValueError(f"{nm} must be contiguous float64 [G][N] on {dev}")
    cap_host = None
    if not torch.is_tensor(capacity) or capacity.device != dev:
        cap_host = torch.as_tensor(capacity, dtype=torch.int32)
        capacity = cap_host.to(dev)
    if capacity.dtype != torch.int32 or capacity.numel() != G or not capacity.is_contiguous():
        raise ValueError("capacity must be int32 [G]")
    out = {} if out is None else out
    if offsets is not None:
        off = torch.as_tensor(offsets, dtype=torch.int64)
        if off.numel() != G + 1:
            raise ValueError("offsets must have G + 1 entries")
        if off.device.type == "cpu" and total is None:
            total = int(off[-1])
        off_dev = off if off.device == dev else off.to(dev)
    else:
        off_dev = capacity_offsets_device(capacity, N, out=out.get("offsets"))
        if cap_host is not None and total is None:
            total = int(capacity_offsets(cap_host, N)[-1])
    if total is None:
        total = G * N
    keep = _need(out.get("keep"), (G, N), torch.uint8, dev, "keep")
    kept = out.get("kept_idx")
    if kept is None or kept.numel() < total:
        kept = torch.empty(max(total, 1), dtype=torch.int32, device=dev)
    p = params(G, N, 0, 0.0, 0, sink, recent)  # select reads only G, N, sink, recent
    st = lib.twinkv_select(ctypes.byref(p), _ptr(score_t), _ptr(energy_t), _ptr(capacity), _ptr(off_dev), _ptr(keep),
                           _ptr(kept), ctypes.c_void_p(0), 0, _stream(), _marks(events, SELECT_PHASES))
    _check(st, "twinkv_select")
    return {"keep": keep, "kept_idx": kept, "offsets": off_dev, "capacity": capacity}


def repair(keys, keep_in, tau, window, sink=4, recent=64, prior=None, out=None, ws=None, events=None):
    """One-shot orphan/donor repair of the retained masks ``keep_in`` (uint8
    [G][N]).  ``prior``: optionally the result of ``score`` on the same keys,
    window and tau (its best_sim and best_idx); rows whose unrestricted best
    twin is retained then take it instead of being swept again.  Returns keep
    (S1), best_sim, best_idx, n_orphans, n_donors, n_swaps and pairs
    ([G][N//2][2], -1 padded)."""
    lib = load()
    keys = _as_bf16_bits(keys, "keys")
    G, N, d = keys.shape
    dev = keys.device
    if keep_in.dtype != torch.uint8 or tuple(keep_in.shape) != (G, N) or not keep_in.is_contiguous() \
            or keep_in.device != dev:
        raise ValueError("keep_in must be contiguous uint8 [G][N] on the keys' device")
    p = params(G, N, d, tau, window, sink, recent)
    ps = pi = ctypes.c_void_p(0)
    if prior is not None:
        psim, pidx = prior["best_sim"], prior["best_idx"]
        for t, dt, nm in ((psim, torch.float64, "best_sim"), (pidx, torch.int32, "best_idx")):
            if t.dtype != dt or tuple(t.shape) != (G, N) or not t.is_contiguous() or t.device != dev:
                raise ValueError(f"prior {nm} must be contiguous {dt} [G][N] on the keys' device")
        ps, pi = _ptr(psim), _ptr(pidx)
    out = {} if out is None else out
    o = {
        "keep": _need(out.get("keep"), (G, N), torch.uint8, dev, "keep"),
        "best_sim": _need(out.get("best_sim"), (G, N), torch.float64, dev, "best_sim"),
        "best_idx": _need(out.get("best_idx"), (G, N), torch.int32, dev, "best_idx"),
        "n_orphans": _need(out.get("n_orphans"), (G,), torch.int32, dev, "n_orphans"),
        "n_donors": _need(out.get("n_donors"), (G,), torch.int32, dev, "n_donors"),
        "n_swaps": _need(out.get("n_swaps"), (G,), torch.int32, dev, "n_swaps"),
        "pairs": _need(out.get("pairs"), (G, N // 2, 2), torch.int32, dev, "pairs"),
    }
    nb = workspace_bytes(OP_REPAIR, p)
    ws = _workspace(ws, nb, dev)
    wp, wn = _ws_ptr(ws)
    st = lib.twinkv_repair(ctypes.byref(p), _ptr(keys), _ptr(keep_in), ps, pi, _ptr(o["keep"]), _ptr(o["best_sim"]),
                           _ptr(o["best_idx"]), _ptr(o["n_orphans"]), _ptr(o["n_donors"]), _ptr(o["n_swaps"]),
                           _ptr(o["pairs"]) if N >= 2 else ctypes.c_void_p(0), wp, wn, _stream(),
                           _marks(events, REPAIR_PHASES))
    _check(st, "twinkv_repair")
    o["ws"] = ws
    return o


def gather_kv(keys, values, kept_idx, offsets, out=None, events=None, total=None):
    """Packed cache of the retained positions: the rows kept_idx[off[g]:off[g+1]]
    of every head g, in that order, for keys (and values unless None).
    ``offsets``: int64 [G+1] prefix sums of the per-head counts, on the host
    (copied to the device) or on the keys' device; ``total`` (optional) is
    offsets[G], which saves reading device offsets back.  Returns out_keys (and
    out_values) [total][d] device tensors of the inputs' dtypes, plus the
    device offsets under "offsets"."""
    lib = load()
    keys = _as_bf16_bits(keys, "keys")
    G, N, d = keys.shape
    dev = keys.device
    if values is not None:
        values = _as_bf16_bits(values, "values")
        if values.shape != keys.shape:
            raise ValueError("keys and values must have the same shape")
    off = torch.as_tensor(offsets, dtype=torch.int64)
    if off.numel() != G + 1:
        raise ValueError("offsets must have G + 1 entries")
    off_dev = off if off.device == dev else off.to(dev)
    if total is None:
        total = int(off[-1]) if off.device.type == "cpu" else int(off_dev[-1].item())
    total = int(total)
    if kept_idx.dtype != torch.int32 or kept_idx.device != dev or not kept_idx.is_contiguous() \
            or kept_idx.numel() < total:
        raise ValueError("kept_idx must be a contiguous int32 device tensor with at least total entries")
    out = {} if out is None else out
    ok = _need(out.get("keys"), (total, d), keys.dtype, dev, "out keys")
    ov = _need(out.get("values"), (total, d), values.dtype, dev, "out values") if values is not None else None
    p = params(G, N, d, 0.0, 0, 0, 0)  # gather reads only G, N, d
    st = lib.twinkv_gather_kv(ctypes.byref(p), _ptr(keys), _ptr(values), _ptr(kept_idx), _ptr(off_dev), total,
                              _ptr(ok) if total else ctypes.c_void_p(0),
                              (_ptr(ov) if total else ctypes.c_void_p(0)) if values is not None else ctypes.c_void_p(0),
                              _stream(), _marks(events, GATHER_PHASES))
    _check(st, "twinkv_gather_kv")
    return {"keys": ok, "values": ov, "offsets": off_dev, "total": total}


def allocate(keys, queries, heads_per_layer, budget, sink=4, recent=64, pool=7, out=None, ws=None, events=None):
    """Per-head capacities of every layer from prefix attention (Equation 5).

    keys: bf16 [G][N][d]; queries: bf16 [G][Gq][W][d], the post-RoPE queries of
    the last W prefix positions of the Gq query heads sharing each KV head.
    Consecutive groups of ``heads_per_layer`` heads share the per-head
    ``budget``.  Returns capacity (int32 [G]), g_count (int32 [G]) and the
    pooled scores z (float32 [G][N]) as device tensors, plus the workspace."""
    lib = load()
    keys = _as_bf16_bits(keys, "keys")
    G, N, d = keys.shape
    dev = keys.device
    if queries.dtype not in (torch.bfloat16, torch.int16, torch.uint16) or not queries.is_cuda \
            or not queries.is_contiguous() or queries.dim() != 4 or queries.shape[0] != G or queries.shape[3] != d:
        raise ValueError("queries must be a contiguous bf16 device tensor [G][Gq][W][d]")
    Gq, W = int(queries.shape[1]), int(queries.shape[2])
    H = int(heads_per_layer)
    p = params(G, N, d, 0.0, 0, sink, recent)
    out = {} if out is None else out
    o = {
        "capacity": _need(out.get("capacity"), (G,), torch.int32, dev, "capacity"),
        "g_count": _need(out.get("g_count"), (G,), torch.int32, dev, "g_count"),
        "z": _need(out.get("z"), (G, N), torch.float32, dev, "z"),
    }
    nb = int(lib.twinkv_allocate_workspace_bytes(ctypes.byref(p), H, Gq, W, int(pool), int(budget)))
    ws = _workspace(ws, nb, dev)
    wp, wn = _ws_ptr(ws)
    st = lib.twinkv_allocate(ctypes.byref(p), H, Gq, W, int(pool), int(budget), _ptr(keys), _ptr(queries),
                             _ptr(o["capacity"]), _ptr(o["g_count"]), _ptr(o["z"]), wp, wn, _stream(),
                             _marks(events, ALLOC_PHASES))
    _check(st, "twinkv_allocate")
    o["ws"] = ws
    return o


def variant_score(count_t, energy_t, variant, perm=None, out=None, events=None):
    """Selection keys (score, tie) of a score variant ("twin", "value",
    "rarity"), optionally with permuted counts (perm: int32 [G][N]); pass them
    to select() as its score and energy."""
    lib = load()
    G, N = count_t.shape
    dev = count_t.device
    if count_t.dtype != torch.int32 or not count_t.is_contiguous() or not count_t.is_cuda:
        raise ValueError("count must be a contiguous int32 device tensor [G][N]")
    if energy_t.dtype != torch.float64 or tuple(energy_t.shape) != (G, N) or energy_t.device != dev \
            or not energy_t.is_contiguous():
        raise ValueError("energy must be a contiguous float64 [G][N] tensor on the counts' device")
    if perm is not None and (perm.dtype != torch.int32 or tuple(perm.shape) != (G, N) or perm.device != dev
                             or not perm.is_contiguous()):
        raise ValueError("perm must be a contiguous int32 [G][N] tensor on the counts' device")
    if variant not in VARIANTS:
        raise ValueError(f"variant must be one of {sorted(VARIANTS)}")
    out = {} if out is None else out
    sc = _need(out.get("score"), (G, N), torch.float64, dev, "score")
    tie = _need(out.get("tie"), (G, N), torch.float64, dev, "tie")
    p = params(G, N, 0, 0.0, 0)
    st = lib.twinkv_variant_score(ctypes.byref(p), VARIANTS[variant], _ptr(count_t), _ptr(energy_t), _ptr(perm),
                                  _ptr(sc), _ptr(tie), _stream(), _marks(events, VARIANT_PHASES))
    _check(st, "twinkv_variant_score")
    return {"score": sc, "tie": tie}


def count_stats(count_t, energy_t, capacity, sink=4, recent=64, keep_twin=None, keep_value=None, events=None):
    """Per-head count statistics over the unprotected positions: int64
    [G][26] counts (n, twin, six-bin histogram, kept, added, removed and three
    five-bin margin histograms) and float64 [G][2] (discount sum, value-only
    energy cut), as device tensors."""
    lib = load()
    G, N = count_t.shape
    dev = count_t.device
    if count_t.dtype != torch.int32 or not count_t.is_contiguous() or not count_t.is_cuda:
        raise ValueError("count must be a contiguous int32 device tensor [G][N]")
    if energy_t.dtype != torch.float64 or tuple(energy_t.shape) != (G, N) or energy_t.device != dev:
        raise ValueError("energy must be float64 [G][N] on the counts' device")
    if (keep_twin is None) != (keep_value is None):
        raise ValueError("give both selections or neither")
    for t, nm in ((keep_twin, "keep_twin"), (keep_value, "keep_value")):
        if t is not None and (t.dtype != torch.uint8 or tuple(t.shape) != (G, N) or t.device != dev
                              or not t.is_contiguous()):
            raise ValueError(f"{nm} must be contiguous uint8 [G][N] on the counts' device")
    cap = capacity if torch.is_tensor(capacity) and capacity.device == dev else \
        torch.as_tensor(capacity, dtype=torch.int32).to(dev)
    if cap.dtype != torch.int32 or cap.numel() != G:
        raise ValueError("capacity must be int32 [G]")
    st = torch.empty((G, STAT_INTS), dtype=torch.int64, device=dev)
    fs = torch.empty((G, 2), dtype=torch.float64, device=dev)
    p = params(G, N, 0, 0.0, 0, sink, recent)
    rc = lib.twinkv_count_stats(ctypes.byref(p), _ptr(count_t), _ptr(energy_t), _ptr(keep_twin), _ptr(keep_value),
                                _ptr(cap), _ptr(st), _ptr(fs), _stream(), _marks(events, STATS_PHASES))
    _check(rc, "twinkv_count_stats")
    return {"stats": st, "fstats": fs}
