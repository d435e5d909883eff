"""omerge: stable merge of two sorted int32 arrays on AMD MI355X (gfx950).

The work runs in hand-written HIP kernels behind a C ABI (include/omerge.h,
libomerge.so); this package is the thin Python binding over torch tensors.
"""
from .merge import (  # noqa: F401
    OmergeError,
    co_rank,
    library_path,
    load_library,
    merge_i32,
    merge_i32_direct,
    merge_kv,
    merge_segments_i32,
    merge_segments_kv,
    partition,
    partition_count,
    segment_length,
    stream_copy,
)
