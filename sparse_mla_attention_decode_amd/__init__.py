"""MI355X (gfx950) sparse MLA attention decode.

The compute path is the HIP library libmla.so behind the C ABI in
include/mla.h; this package only loads it and marshals arguments.
"""
from ._binding import (  # noqa: F401
    MLA_KV_BF16_576, MLA_KV_FP8_656, MLA_KV_V4_584, MLA_KV_V41_528, MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED,
    MLA_ERR_WORKSPACE, MLA_ERR_HIP, MLA_ERR_NO_DEVICE, EXPORTED, DecodePlan, MlaError,
    load_library, make_shape, mla_debug_gather_dequant, mla_decode_args, mla_get_sched_meta,
    mla_get_sched_meta_len, mla_plan_sched_meta_len_host, mla_indexer_args, mla_indexer_scores,
    mla_indexer_topk, indexer_args, indexer_select,
    mla_last_error, mla_plan_sched_meta_host, mla_resolve_shape, mla_sched_meta_size, mla_shape,
    mla_dense_decode_fwd, mla_sparse_decode_fwd, mla_sparse_decode_extra_fwd, mla_extra_kv, extra_kv_args, mla_sparse_decode_noalloc, mla_splitkv_combine, mla_version, mla_workspace_size,
)
