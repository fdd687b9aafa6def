"""MI355X (gfx950) sparse decode attention: query-aware top-k selection of KV
tokens or pages, then split-K attention over the kept entries.

The work is done by hand-written HIP kernels in libsdkv.so behind the C ABI of
include/sd.h; this package is its thin Python binding (argument marshalling
only) plus the in-tree build script.
"""

from ._lib import (  # noqa: F401
    EXPORTS,
    LIB_PATH,
    SdError,
    Selection,
    Shape,
    UNIT_PAGE,
    UNIT_TOKEN,
    alloc_workspace,
    append_page_bounds,
    alloc_workspace_entmax,
    alloc_workspace_sel,
    attend_partials,
    attend_splitk,
    bounds_shape,
    compressed_keys_shape,
    decode_step,
    decode_step_noalloc,
    decode_step_entmax,
    decode_step_sel,
    dropped_mass,
    keep_count,
    lib,
    merge_splits,
    score_compressed,
    score_pages,
    select_attend,
    select_topk,
    select_units,
    selection_capacity,
    update_compressed_keys,
    update_page_bounds,
    workspace_bytes,
    workspace_bytes_entmax,
    workspace_bytes_sel,
)
