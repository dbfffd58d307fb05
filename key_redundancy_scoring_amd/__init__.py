"""MI355X (gfx950) key-redundancy scoring: TwinKV's nonlocal key-similarity
count, best twin, value-energy score, exact-budget selection,
orphan/donor repair, the packed cache of the retained keys and values and
per-head capacities from prefix attention, computed by hand-written HIP kernels behind a C ABI
(include/twinkv.h).  This package is the thin Python binding."""
from ._lib import (  # noqa: F401
    Events,
    allocate,
    Params,
    TwinKVError,
    capacity_offsets,
    capacity_offsets_device,
    count_stats,
    gather_kv,
    header_symbols,
    load,
    params,
    repair,
    score,
    score_noalloc,
    select,
    status_string,
    uniform_capacity,
    uniform_capacity_ceil,
    variant_score,
    workspace_bytes,
)
