"""Grouped-query attention forward for AMD MI355X (gfx950).

Python face of the C ABI declared in ``include/gqa_attn.h``; the work runs in hand-written HIP
kernels in ``libgqa_attn.so``. Import fails if the library has not been built.
"""
from ._binding import (  # noqa: F401
    ABI_VERSION,
    GQAError,
    GQAValueError,
    AttnOptions,
    gqa_attn_backward,
    gqa_attn_decode,
    gqa_attn_decode_ex,
    gqa_attn_decode_noalloc,
    gqa_attn_decode_ragged,
    gqa_attn_decode_window_cache,
    gqa_attn_decode_workspace_bytes,
    gqa_attn_decode_workspace_bytes_hkv,
    GQA_SCALE_DEFAULT,
    GQA_DECODE_SCRATCH_BYTES,
    gqa_attn_prefill,
    gqa_attn_prefill_ex,
    gqa_attn_prefill_gva,
    gqa_attn_prefill_window,
    gqa_fold_kv,
    gqa_prepare_keys,
    gqa_status_string,
    header_functions,
    load_library,
    raw_library,
)

prefill = gqa_attn_prefill
decode = gqa_attn_decode
fold_kv = gqa_fold_kv
