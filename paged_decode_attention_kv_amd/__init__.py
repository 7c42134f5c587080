"""Paged INT8-KV decode attention for AMD MI355X (gfx950).

The compute path is the HIP library ``libpdakv.so`` (C ABI in
``include/pdakv.h``); this package is its thin Python binding, with one
function per C entry point, plus small device-memory helpers. Importing it
fails when the library is not built: there is no CPU or PyTorch fallback.
"""

from ._lib import (  # noqa: F401
    CAP_GFX950,
    DTYPE_BF16,
    DTYPE_F16,
    DTYPE_F32,
    EFLAG_BLOCK_RANGE,
    EFLAG_CONTEXT_RANGE,
    EFLAG_SCALE_RANGE,
    EFLAG_SLOT_RANGE,
    ERR_DTYPE,
    ERR_HIP,
    ERR_INVALID_ARG,
    ERR_NO_DEVICE,
    ERR_UNSUPPORTED,
    ERR_WORKSPACE,
    EXPORTED,
    KV_16BIT,
    KV_INT8_STATIC,
    KV_INT8_SYM,
    LIB_PATH,
    NOALLOC_SCRATCH_BYTES,
    PdakvError,
    kv_pages_swap_in,
    kv_pages_swap_out,
    kv_quant_int8_static_write,
    kv_quant_int8_sym_write,
    kv_trim_keep_sink,
    kv_write_16bit,
    paged_attn_decode_fp16,
    paged_attn_decode_fp16_append,
    paged_attn_decode_fp16_multi,
    paged_attn_decode_int8,
    paged_attn_decode_int8_append,
    paged_attn_decode_int8_multi,
    paged_attn_decode_int8_noalloc,
    paged_attn_decode_int8_static,
    paged_attn_decode_int8_static_append,
    paged_attn_decode_workspace_bytes,
    pdakv_capabilities,
    pdakv_decode_plan,
    pdakv_decode_multi_workspace_bytes,
    pdakv_decode_workspace_bytes,
    pdakv_page_bytes,
    pdakv_status_string,
    pdakv_version,
)
from .memory import (DecodeBuffers, alloc_multi_workspace, alloc_pool,  # noqa: F401
                     alloc_workspace)
