"""MI355X (gfx950) paged-KV, variable-length attention step.

The product is libpa.so (HIP kernels + C ABI, include/pa.h); this package is
its thin Python binding.  Build the library with
``python -m paged_kv_varlen_reshape_amd.build``.
"""
from ._binding import (  # noqa: F401
    BlockPool,
    LIB_PATH,
    PAError,
    PA_BF16,
    PA_ERR_HIP,
    PA_ERR_INVALID,
    PA_ERR_NO_BLOCKS,
    PA_ERR_UNSUPPORTED,
    PA_ERR_WORKSPACE,
    PA_F32,
    PA_OK,
    PA_OPT_FORCE_ROWWISE,
    PA_OPT_SPLIT_TOKENS,
    PA_OPT_TARGET_ITEMS,
    PA_OPT_DECODE_BUFFERS,
    PA_OPT_DECODE_KERNEL,
    PA_K_CHUNK,
    PA_K_COUNT,
    PA_K_DECODE,
    PA_K_MERGE,
    PA_K_PLAN,
    PA_K_RESHAPE,
    KERNEL_NAMES,
    SIGNATURES,
    last_error,
    lib,
    pa_attention,
    pa_attention_workspace_size,
    pa_get_option,
    pa_measure_copy,
    pa_measure_read,
    pa_profile_enable,
    pa_profile_read,
    pa_reshape_and_cache,
    pa_set_option,
    pa_validate_metadata,
)
