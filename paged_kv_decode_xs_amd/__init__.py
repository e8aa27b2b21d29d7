"""Paged-KV decode attention for AMD MI355X (gfx950).

The computation lives in libxs.so (hand-written HIP kernels behind the C ABI in include/xs/xs.h).
This package is its thin Python binding plus a decode-step helper that chains the three calls.
"""

from ._binding import (  # noqa: F401
    XS_BF16,
    XS_F32,
    XsError,
    library_path,
    load_library,
    num_partitions,
    xs_kv_append,
    xs_kv_append_chunk,
    xs_kv_swap_in,
    xs_kv_swap_out,
    xs_last_error,
    xs_paged_attn_decode,
    xs_paged_attn_decode_append,
    xs_paged_attn_decode_append_noalloc,
    xs_paged_attn_decode_sinks,
    xs_paged_attn_prefill,
    xs_paged_attn_prefill_sinks,
    xs_paged_attn_prefill_split,
    xs_paged_attn_reduce,
    xs_paged_attn_reduce_sinks,
    xs_step_graph_create,
    xs_step_graph_destroy,
    xs_step_graph_launch,
    xs_stream_read_probe,
    xs_version,
)
from .checks import check_device_inputs, check_prefill_inputs  # noqa: F401
from .step import DecodeStep, StepGraph, suggest_partition_size  # noqa: F401
