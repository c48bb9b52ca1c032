"""MI355X (gfx950) forward pass of multi-round LSH attention with shared QK.

The four steps (hash, sort, chunk attention, round combine), the backward of
the last two, the layer's projections and the Reformer block's feed-forward
layer run in the HIP kernels of
liblsh_attention.so behind a C ABI (include/lsh_attention.h); this package is
its Python binding.  Build the library with
``python -m lsh_attention_02_amd.build``.
"""
from ._binding import (DEBUG_LIB_PATH, EXPORTED, LIB_PATH, debug_check_failures, load_debug_library, LSH_BF16, LSH_ERR_HIP, LSH_ERR_INVALID_ARG,  # noqa: F401
                       LSH_ERR_UNSUPPORTED, LSH_ERR_WORKSPACE, LSH_F32, LSH_FLAG_NO_DUP_CORRECTION,
                       LSH_FLAG_SAME_BUCKET, LSH_FLAG_WRAP_LOOKBACK, LSH_OK, CConfig,
                       LSHConfig, LSHError, backward_workspace, block_forward, block_inverse, forward,
                       layer_forward, load_library, lsh_ffn, lsh_ffn_workspace_bytes,
                       lsh_project_out_add,
                       lsh_attn_backward, lsh_backward_workspace_bytes, lsh_chunk_attn,
                       lsh_combine_rounds, lsh_hash, lsh_project_in, lsh_project_out, lsh_sort,
                       lsh_sort_noalloc, lsh_sort_workspace_bytes, sort_workspace,
                       SORT_NOALLOC_MAX_BYTES)
