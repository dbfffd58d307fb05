"""MI355X (gfx950) key-redundancy scoring: TwinKV's nonlocal key-similarity
count, best twin, value-energy score, exact-budget selection and
orphan/donor repair, computed by hand-written HIP kernels behind a C ABI
(include/twinkv.h).  This package is the thin Python binding."""
from ._lib import (  # noqa: F401
    Events,
    Params,
    TwinKVError,
    capacity_offsets,
    header_symbols,
    load,
    params,
    repair,
    score,
    select,
    status_string,
    uniform_capacity,
    workspace_bytes,
)
