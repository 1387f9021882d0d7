"""Paged-KV FlashAttention (EXTEND and DECODE) for AMD MI355X (gfx950).

The compute lives in ``libpkv.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/pkv.h``); this package is its thin ctypes binding.
"""
from .binding import (  # noqa: F401
    PKV_BF16, PKV_DECODE, PKV_EXTEND, PKV_FP8_E4M3, PKV_SAGE_INT8, PKV_OK, PKV_EINVAL, PKV_EUNSUPPORTED,
    PKV_EWORKSPACE, PKV_EHIP, EXPORTED, LIB_PATH, STATIC_SCRATCH_BYTES, Params, Plan, PkvError, attn_decode,
    attn_decode_noalloc, attn_extend, block_sparse_table, kv_store, last_error, load_library, plan_metadata,
    workspace_size,
)
