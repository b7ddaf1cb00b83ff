"""Split-KV paged decode attention for MI355X (gfx950).

The decode, the multi-token (prefill) route and the append that writes new tokens into the
cache run in hand-written HIP kernels behind the C ABI of ``include/skvd.h`` (``libskvd.so``, built in-tree by
``python -m quantized_kv_cache_page_amd.build``). This package is its thin Python face: ``Plan`` marshals torch tensors into those calls, and the
``skvd_*`` functions are the C-ABI entry points under the same names. ``ops`` registers the
decode, the multi-token route and the append as torch operators (``torch.ops.skvd.decode_v1``,
``decode_out_v1``, ``prefill_v1``, ``prefill_out_v1``, ``append_v1``) whose schemas declare
exactly what they write.
"""
from ._binding import (  # noqa: F401
    LIB_PATH, REDUCERS, SIGNATURES, Plan, SkvdError, last_error, lib, skvd_abi_version_py,
    skvd_decode, skvd_decode_check, skvd_decode_merge, skvd_decode_partial,
    skvd_decode_partial_timed, skvd_gather_debug,
    skvd_plan_create, skvd_plan_describe, skvd_plan_destroy, skvd_plan_get_info,
    skvd_plan_params, skvd_plan_workspace_bytes, skvd_decode_args, status_string,
    skvd_stream_read, stream_read, skvd_append, skvd_append_check, skvd_append_args,
    skvd_prefill, skvd_prefill_check, skvd_merge_states, merge_states, skvd_attention,
    STATUS_KV_LEN_CLAMPED, STATUS_PAGE_CLAMPED, skvd_decode_noalloc,
)
from . import ops  # noqa: F401,E402  (torch.ops.skvd.*)
