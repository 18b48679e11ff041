"""libpagedattn: attention over a paged KV cache for a mixed varlen batch on MI355X.

The library is hand-written HIP for gfx950 behind a C ABI (``include/pagedattn.h``);
this package is its Python binding (argument marshalling only) plus the build
script.  Entry points keep their C names::

    params = make_params(num_seqs=..., num_heads=..., ...)
    plan = pa_plan_create(params, query_start_loc, seq_lens, block_table, device=0)
    ws = torch.empty(pa_plan_workspace_bytes(plan), dtype=torch.uint8, device="cuda")
    pa_forward(plan, q, kv_cache, block_table_dev, query_start_loc_dev, seq_lens_dev, out, lse, ws)
"""
from ._capi import (  # noqa: F401
    EXPORTED,
    LIB_PATH,
    PA_ARRAY_DECODE_LISTS,
    PA_ARRAY_DECODE_SPANS,
    PA_ARRAY_IS_DECODE,
    PA_ARRAY_ORDER,
    PA_ARRAY_PREFIX_BLOCKS,
    PA_ARRAY_ROW_PARTIALS,
    PA_BF16,
    PA_ERR_HIP,
    PA_ERR_INVALID_ARG,
    PA_ERR_OOM,
    PA_ERR_UNSUPPORTED,
    PA_FP32,
    PA_KV_FP8_E4M3,
    PA_KV_HND,
    PA_KV_NHD,
    PA_KV_SAME,
    PA_OK,
    PagedAttnError,
    Plan,
    lib,
    make_params,
    pa_forward,
    pa_forward_fp8,
    pa_forward_noalloc,
    pa_gather_kv,
    pa_kv_cache_shape,
    pa_kv_cache_stride_order,
    pa_last_error,
    pa_merge_states,
    pa_params,
    pa_plan_check_metadata,
    pa_plan_create,
    pa_plan_destroy,
    pa_plan_get_array,
    pa_plan_get_info,
    pa_plan_workspace_bytes,
    pa_profile_start,
    pa_profile_stop,
    pa_status_string,
    pa_write_kv,
    pa_write_kv_fp8,
)
from .device import DeviceBatch, to_device  # noqa: F401
