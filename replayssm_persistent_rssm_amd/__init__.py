"""MI355X (gfx950) ReplaySSM prefix materialize.

The product is the C-ABI library ``librssm_materialize.so`` (declared in
``include/rssm_materialize.h``, ``rssm_gdn_commit.h`` and
``rssm_ssu_decode.h``); this package is its thin ctypes binding.  Importing
it requires the built library; there is no fallback.  ``librssm_pool.so``
(``include/rssm_pool.h``) is a separate placement helper for the pools,
loaded only when used.
"""
from ._binding import (  # noqa: F401
    EXPORTS, LIB_PATH, POOL_EXPORTS, POOL_LIB_PATH, pool_lib, RSSM_BF16, RSSM_F16, RSSM_F32, RSSM_F8E4M3, RSSM_I8, RSSM_ERR_HIP,
    RSSM_ERR_INVALID_ARGUMENT, RSSM_ERR_UNSUPPORTED, RSSM_OK, MaterializeCall, RssmDesc, RssmError, RssmTables,
    checkpoint_prefix_len, dtype_code, lib, make_desc, pointer_table, replayssm_materialize,
    rssm_debug_encode_rows, rssm_debug_row_scales, rssm_last_error, rssm_materialize, rssm_materialize_checkpoints,
    rssm_materialize_launch_config, RSSM_MAX_CHECKPOINTS, stride_table, rssm_gdn_commit,
    gated_delta_rule_replayssm_commit, GdnCommitCall, RssmGdnDesc, RssmGdnTables, rssm_ssu_decode,
    SsuDecodeCall, RssmSsuDesc, RssmSsuTables, RSSM_SSU_MAX_TOKENS, RSSM_SSU_MAX_REPLAY, rssm_pool_alloc,
    rssm_pool_free, use_contiguous_allocator)
