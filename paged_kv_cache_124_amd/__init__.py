"""PagedAttention decode for AMD Instinct MI355X (gfx950).

The work runs in libpa.so (hand-written HIP kernels and a C++ block manager,
C ABI in ``include/pa.h``).  This package is its thin Python binding: the
functions below have the names of the C entry points and only marshal
arguments.
"""

from ._lib import (  # noqa: F401
    PA_BF16,
    PA_F32,
    PA_FP8_E4M3,
    PA_OK,
    BlockManager,
    PAError,
    lib,
    pa_append_kv,
    pa_append_kv_args,
    pa_append_kv_fp8,
    pa_append_kv_fp8_args,
    pa_append_step,
    pa_append_step_args,
    pa_append_step_fp8,
    pa_append_step_fp8_args,
    pa_copy_blocks,
    pa_copy_blocks_args,
    pa_copy_blocks_fp8,
    pa_copy_blocks_fp8_args,
    pa_decode,
    pa_decode_args,
    pa_decode_fp8,
    pa_decode_fp8_args,
    pa_decode_partition_tokens,
    pa_decode_shared,
    pa_decode_shared_args,
    pa_decode_shared_workspace_bytes,
    pa_decode_step,
    pa_decode_step_args,
    pa_decode_step_shared,
    pa_decode_step_shared_args,
    pa_decode_workspace_bytes,
    pa_swap_blocks,
    pa_swap_blocks_fp8,
    host_device_pointer,
    pool_shapes,
)
