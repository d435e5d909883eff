"""omerge: stable merges of sorted arrays, batches of merges and a stable
merge sort, on AMD MI355X (gfx950).

The work runs in hand-written HIP kernels behind a C ABI (include/omerge.h,
libomerge.so); this package is the thin Python binding over torch tensors.
"""
from .binding import (  # noqa: F401
    DESCENDING,
    KEY_F32,
    KEY_F64,
    KEY_I32,
    KEY_I64,
    KEY_U32,
    KEY_U64,
    OmergeError,
    co_rank,
    library_path,
    load_library,
    merge,
    merge_batched,
    merge_i32,
    merge_i32_direct,
    merge_i32_no_alloc,
    merge_kv,
    merge_pairs,
    merge_runs4,
    merge_segments_i32,
    merge_segments_kv,
    partition,
    partition_count,
    order_code,
    segment_length,
    sort,
    stream_copy,
)
