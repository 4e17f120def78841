"""Paged KV cache decode for AMD MI355X (gfx950).

The compute lives in a HIP shared library (``libpkv.so``) behind a C ABI
declared in ``include/pkv.h``; ``paged_kv_cache_440_amd._lib`` is its thin
ctypes binding. Importing this package does not load the library: the API
names below load it on first use, and fail loudly if it was not built.
"""

_API = (
    "kv_cache_append",
    "kv_cache_append_fp8",
    "kv_cache_append_multi",
    "kv_cache_append_multi_fp8",
    "paged_attention_multi_fp8",
    "paged_attention_decode_grouped_fp8",
    "paged_attention_multi",
    "paged_attention_decode_fp8",
    "paged_attention_decode_grouped",
    "FP8_E4M3",
    "copy_blocks",
    "swap_blocks",
    "paged_attention_decode",
    "paged_attention_decode_noalloc",
    "NOALLOC_SCRATCH_BYTES",
    "paged_attention_workspace_size",
    "status_string",
    "probe_read",
    "probe_copy",
    "probe_gather",
    "probe_gather_mfma",
    "library",
    "DTYPE_CODES",
    "PARTITION_BALANCED",
    "KV_STREAM",
    "KV_REUSE",
    "PkvError",
    "set_error_word",
    "ERRBIT_TABLE",
    "ERRBIT_LENGTH",
    "ERRBIT_APPEND",
    "ERRBIT_COPY",
)

__all__ = list(_API)


def __getattr__(name):
    if name in _API:
        from . import _lib
        return getattr(_lib, name)
    raise AttributeError(name)
